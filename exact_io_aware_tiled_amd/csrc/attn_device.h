// attn_device.h -- device-side building blocks shared by the forward and
// backward attention kernels for gfx950 (CDNA4, wave64).
//
// Matrix products use the 32x32 MFMA shapes with fp32 accumulation:
//   16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}; float32: v_mfma_f32_32x32x2_f32.
// Operand convention used throughout ("one 16-byte chunk per lane"): for a
// product C[32][32] += A[32][k] * B[k][32], lane L supplies row (L % 32) of A
// and column (L % 32) of B; the contraction indices covered by one chunk are
// split between the two half-waves (h = L / 32).  Because A and B assign the
// same contraction index to the same (half, element) slot, any consistent
// assignment of indices to slots gives the same product; the kernels choose the
// assignment that matches where the data already sits.
//
// Accumulator layout of a 32x32 fp32 block (16 values per lane):
//   element e of lane L holds C[8*(e/4) + 4*h + (e%4)][L % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace eiat {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element traits: one MFMA step over a 16-byte chunk per lane, and fp32 -> T packing.
template <typename T>
struct Elt;

template <>
struct Elt<__bf16> {
  static constexpr int kBytes = 2;
  static constexpr uint32_t kSign = 0x80008000u;
  // 16 contraction indices: elements 0..7 of the chunk in each half-wave.
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32).
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

template <>
struct Elt<_Float16> {
  static constexpr int kBytes = 2;
  static constexpr uint32_t kSign = 0x80008000u;
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

template <>
struct Elt<float> {
  static constexpr int kBytes = 4;
  static constexpr uint32_t kSign = 0x80000000u;
  // Four K=2 steps: element e of the chunk in half-wave h is one contraction index.
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0,
                                               0, 0);
    return c;
  }
};

// Probability operand: the 16 fp32 values of one 32-key accumulator block (keys
// 8*(e/4) + 4*h + (e%4) of column L % 32) as MFMA chunks over those keys.
// 16-bit types: chunk s (0, 1) holds elements 8s..8s+7 -> keys 16s + 8*(i/4) + 4h + (i%4).
// float32: chunk g (0..3) holds elements 4g..4g+3     -> keys 8g + 4h + i.
template <typename T>
struct PChunks {
  static constexpr int kCount = (Elt<T>::kBytes == 2) ? 2 : 4;
  u32x4 c[kCount];
  __device__ inline void set(const f32x16& p) {
    if constexpr (Elt<T>::kBytes == 2) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w) c[s][w] = Elt<T>::pack2(p[8 * s + 2 * w], p[8 * s + 2 * w + 1]);
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int w = 0; w < 4; ++w) c[g][w] = __float_as_uint(p[4 * g + w]);
    }
  }
};

// Sum of the 16 probabilities of one accumulator block.  fp16: from the packed
// operand chunks (v_dot2 with (1, 1)), so the normaliser adds exactly the
// rounded values the value product uses; fp16 rounding (2^-11 relative) keeps
// LSE well inside its bound even for rows with very few keys.  bf16 rounding
// (2^-8) does not, so bf16 and float32 add the unrounded fp32 values (as a
// tree, to keep the dependency chain short).
template <typename T>
__device__ inline float chunk_sum(const PChunks<T>& pc, const f32x16& p, float acc) {
  if constexpr (__is_same(T, _Float16)) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t pw = pc.c[s][w];
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw), one, acc, false);
      }
    return acc;
  } else {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = p[e] + p[e + 8];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] += t[e + 4];
    return acc + ((t[0] + t[1]) + (t[2] + t[3]));
  }
}

// Load the "transposed" operand matching PChunks from an LDS row that stores 32
// consecutive keys of one output row (row-major over keys, element type T):
// chunk index ci covers the same keys as PChunks<T>::c[ci] for half-wave h.
template <typename T>
__device__ inline u32x4 keyrow_chunk(const char* row32, int ci, int h) {
  if constexpr (Elt<T>::kBytes == 2) {
    // keys 16ci + 4h + 0..3 and 16ci + 8 + 4h + 0..3 (8 bytes each)
    u32x2 lo = *reinterpret_cast<const u32x2*>(row32 + (16 * ci + 4 * h) * 2);
    u32x2 hi = *reinterpret_cast<const u32x2*>(row32 + (16 * ci + 8 + 4 * h) * 2);
    u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
    return r;
  } else {
    // keys 8ci + 4h + 0..3 (16 bytes)
    return *reinterpret_cast<const u32x4*>(row32 + (8 * ci + 4 * h) * 4);
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3) operands with E8M0 block scales: the gfx950 block-scaled
// MFMA v_mfma_scale_f32_32x32x64_f8f6f4.  Lane L supplies 32 bytes of row
// L % 32 of A (column L % 32 of B); the scale operand of lane r < 32 applies
// to bytes 0-15 of lanes r and r + 32, that of lane r + 32 to bytes 16-31 of
// both (checked on the GPU), so a lane's 32 bytes span two 32-value scale
// blocks and each lane supplies the scale of one of them.  Byte OP of each
// lane's scale word is the scale used (OP a constant operand select).
// ---------------------------------------------------------------------------
template <int OP>
__device__ inline f32x16 mma_fp8(u32x4 a_lo, u32x4 a_hi, u32x4 b_lo, u32x4 b_hi, uint32_t a_scale,
                                 uint32_t b_scale, f32x16 c) {
  const i32x8 a = {(int)a_lo[0], (int)a_lo[1], (int)a_lo[2], (int)a_lo[3],
                   (int)a_hi[0], (int)a_hi[1], (int)a_hi[2], (int)a_hi[3]};
  const i32x8 b = {(int)b_lo[0], (int)b_lo[1], (int)b_lo[2], (int)b_lo[3],
                   (int)b_hi[0], (int)b_hi[1], (int)b_hi[2], (int)b_hi[3]};
  // format 0 (fp8 e4m3) for both operands
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OP, (int)a_scale, OP,
                                                         (int)b_scale);
}

// A row's E8M0 scale bytes (D / 32 of them at p) as the scale word of half-wave
// h: byte 2c holds the scale of block 2c + h (chunk c of 64 values).
template <int D>
__device__ inline uint32_t scale_word_raw(const uint8_t* p) {
  static_assert(D == 64 || D == 128, "FP8 scores: d is 64 or 128");
  return D == 64 ? (uint32_t)*reinterpret_cast<const uint16_t*>(p)
                 : *reinterpret_cast<const uint32_t*>(p);
}
template <int D>
__device__ inline uint32_t scale_word(const uint8_t* p, int h) {
  return scale_word_raw<D>(p) >> (8 * h);
}

// Negate four e4m3 codes per word: flip the sign of every code with a nonzero
// magnitude (zero stays the code 0x00).
__device__ inline u32x4 fp8_negate(u32x4 w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] ^= ((w[i] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
  return w;
}

// Check builds (compiled into separate libraries; never the product path):
//   EIAT_LDS_POISON  every direct HBM -> LDS load first fills the 16 bytes its
//                    lane will write with all-ones (a NaN in every element
//                    type), so a tile read before its loads have landed and
//                    been published by a barrier shows up as non-finite or
//                    changed output; a correctly synchronized kernel gives
//                    bitwise the results of the normal build.
//   EIAT_ALT_TILES   other tile shapes (keys per streamed tile, query rows per
//                    dK/dV tile), for the check that results do not depend on
//                    the block size beyond rounding.
//   EIAT_WG_TIMING   the forward, dQ and dK/dV kernels record per-workgroup
//                    wall-clock stamps and hardware positions (WgStamps below;
//                    eiat_wg_times, eiat_wg_times_dq, eiat_wg_times_dkdv), for
//                    the workgroup timeline of a launch; results are unchanged.
#ifdef EIAT_ALT_TILES
constexpr bool kAltTiles = true;
#else
constexpr bool kAltTiles = false;
#endif

// Poison check build: fill this lane's 16-byte slot at LDS address `lds` and
// wait for the write, before a direct load is issued into it.
__device__ inline void poison_lds_slot(uint32_t lds) {
#ifdef EIAT_LDS_POISON
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  const u32x4 ones = {~0u, ~0u, ~0u, ~0u};
  *reinterpret_cast<lds_u32x4*>((uintptr_t)lds) = ones;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
  (void)lds;
#endif
}

// Copy rows [r0, r0 + R) of a [n][C * 16 bytes] global slice into an LDS tile
// whose rows are C 16-byte chunks plus PAD padding chunks, with the gfx950
// direct-to-LDS load (global_load_lds_dwordx4): wave instruction i writes the
// 1 KiB [1024 i, 1024 i + 1024) of the tile, lane l its 16-byte slot 64 i + l
// (placement checked on the GPU).  Slots map onto whole rows; a padding slot
// fetches a duplicate of its row's first chunk, and lanes past the last slot
// of a partly used final instruction are switched off.  Rows past n read row
// n - 1.  The data is in LDS once the issuing wave's vector-memory count has
// drained (wait_tile_loads) and a barrier has passed.
//
// The load is issued from inline assembly rather than the compiler builtin:
// the compiler cannot tell which LDS bytes such a load writes, so after the
// builtin it drains the vector-memory count before the next transposing LDS
// read (ds_read_b64_tr_b16) of ANY tile, which turns every prefetch into a
// synchronous load.  Issued this way the load is invisible to the compiler's
// wait insertion; every tile written here is read only after an explicit
// wait_tile_loads() and a barrier.  M0 (the LDS base of the load) is set in
// the same statement; no compiler-generated code in these kernels uses M0.
__device__ inline void lds_dma16(const char* src, char* lds_dst) {
  typedef char __attribute__((address_space(3)))* lds_char_t;
  const uint32_t base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_t)lds_dst);
  poison_lds_slot(base + 16 * (threadIdx.x & 63));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
#pragma clang diagnostic pop
}

template <int R, int C, int WAVES, int PAD = 1>
__device__ inline void tile_to_lds(char* lds_tile, const char* gbase, int r0, int n, int wave,
                                   int lane) {
  constexpr int kSlots = R * (C + PAD);
  constexpr int kInstr = (kSlots + 63) / 64;
#pragma unroll
  for (int i0 = 0; i0 < kInstr; i0 += WAVES) {
    const int i = i0 + wave;
    if (i0 + WAVES <= kInstr || i < kInstr) {  // wave < WAVES
      const int slot = 64 * i + lane;
      if (kSlots % 64 == 0 || slot < kSlots) {
        const int row = slot / (C + PAD), c = slot % (C + PAD);
        const int gr = min(r0 + row, n - 1);
        const char* src = gbase + (int64_t)gr * (C * 16) + (c < C ? c : 0) * 16;
        lds_dma16(src, lds_tile + 1024 * i);
      }
    }
  }
}

// The same copy with the cheaper addressing form of the direct load: a
// wave-uniform 64-bit base in SGPRs (the tile's first row) plus a per-lane
// 32-bit offset that depends only on the lane's slot and is computed once
// (init).  Per tile only scalar arithmetic and one min per instruction (the
// clamp of a tile that runs past row n - 1) change.  `wave` must be
// wave-uniform (e.g. from readfirstlane).
// XOR swizzle of unpadded 128-byte LDS rows (d = 64 at 16 bits: 8 chunks of
// 16 bytes): chunk c of tile row r is stored in slot c ^ swz_chunk(r), with
// p = bits 1..3 of r and swz_chunk = p rotated right by one bit.  The LDS
// serves a 16-byte read in passes of 16 lanes and an 8-byte read in passes of
// 32 lanes, 256 bytes over the 64 banks per pass; with the swizzle both read
// patterns of these tiles use every bank once per pass: the 16-byte A-operand
// reads (one chunk of 16 consecutive rows per pass: p runs over all eight
// values for rows of one parity) and the transposing reads (4 consecutive
// rows x 64 bytes per pass: rows r and r + 2 land in different halves of the
// row because bit 1 of r becomes bit 2 of the slot).  Padding cannot do both
// (a 16-byte pad leaves the transposing reads 2-way conflicted).  The pattern
// repeats every 16 rows.
//
// 256-byte rows (d = 128 at 16 bits, 16 chunks) take swz_chunk<16>: bits 0..1
// of r become bits 2..3 of the slot and bits 2..3 of r bits 0..1, so 16
// consecutive rows read one chunk in 16 different slots (all banks once) and
// 4 consecutive rows x 64 bytes fall in 4 different 64-byte quarters.
template <int C = 8>
__device__ inline int swz_chunk(int r) {
  static_assert(C == 8 || C == 16, "swizzled rows of 8 or 16 chunks");
  if constexpr (C == 8) {
    const int p = (r >> 1) & 7;
    return ((p & 1) << 2) | (p >> 1);
  } else {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  }
}

template <int R, int C, int WAVES, int PAD = 1, bool SWZ = false>
struct TileLoader {
  static_assert(!SWZ || ((C == 8 || C == 16) && PAD == 0), "swizzled tiles: unpadded rows");
  static constexpr int kSlots = R * (C + PAD);
  static constexpr int kInstr = (kSlots + 63) / 64;
  static constexpr int kPer = (kInstr + WAVES - 1) / WAVES;
  uint32_t off[kPer];

  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int slot = 64 * (k * WAVES + wave) + lane;
      const int row = slot / (C + PAD), c = slot % (C + PAD);
      // the slot's global chunk: the slot's own (swizzled tiles: the chunk
      // stored there), a padding slot a duplicate of chunk 0
      const int gc = SWZ ? (c ^ swz_chunk<SWZ ? C : 8>(row)) : (c < C ? c : 0);
      off[k] = (uint32_t)(row * (C * 16) + gc * 16);
    }
  }

  __device__ inline void load(char* lds_tile, const char* gbase, int r0, int n, int wave,
                              int lane) const {
    const char* g = gbase + (int64_t)r0 * (C * 16);
    typedef char __attribute__((address_space(3)))* lds_char_t;
    // One scalar base per call (this wave's first 1 KiB of the tile); the
    // instruction k adds its fixed 1024 WAVES k in the same statement, so no
    // per-instruction LDS address is kept in a scalar register.
    const uint32_t m0base = (uint32_t)(uintptr_t)(lds_char_t)(lds_tile + 1024 * wave);
    // A tile that runs past row n - 1 clamps every lane's offset to the last
    // chunk of that row: rows past n then hold copies of earlier rows' data
    // (in bounds, finite), which the kernels mask or weight by zero.  Whole
    // tiles (all but the last of a head) take the offsets as they are.
    if (r0 + R > n)
      issue<0, true>(g, m0base, (uint32_t)((n - r0) * (C * 16) - 16), wave, lane);
    else
      issue<0, false>(g, m0base, 0u, wave, lane);
  }

 private:
  template <int K, bool CLAMP>
  __device__ inline void issue(const char* g, uint32_t m0base, uint32_t lim, int wave,
                               int lane) const {
    if constexpr (K < kPer) {
      const int i = K * WAVES + wave;
      // (kPer - 1) WAVES < kInstr, so only the last instruction index can be
      // past the end for some waves (wave < WAVES)
      if (K + 1 < kPer || kInstr % WAVES == 0 || i < kInstr) {
        if (kSlots % 64 == 0 || 64 * i + lane < kSlots) {
          const uint32_t o = CLAMP ? min(off[K], lim) : off[K];
          poison_lds_slot(m0base + 1024 * WAVES * K + 16 * lane);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
          asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                       :
                       : "v"(o), "s"(g), "s"(m0base), "n"(1024 * WAVES * K)
                       : "memory", "m0", "scc");
#pragma clang diagnostic pop
        }
      }
      issue<K + 1, CLAMP>(g, m0base, lim, wave, lane);
    }
  }
};

// Wait until this wave's direct-to-LDS loads have landed.
__device__ inline void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposed operand from a row-major 16-bit tile X[r][col] (row stride
// vrow_bytes): the MFMA A-operand chunk ci (0, 1) of X^T for output rows
// [32 ob, 32 ob + 32) and the 32 contraction rows starting at kbase, with the
// contraction slots of PChunks.  Two ds_read_b64_tr_b16 per chunk.
// Lane L = 16 G + j addresses row kbase + 16 ci + 8 c + 4 (G / 2) + j / 4 and
// columns 32 ob + 16 (G % 2) + 4 (j % 4) .. + 3 for read c; within each group of
// 16 lanes the read hands lane j element (j % 4) of the rows addressed by lanes
// j / 4 + {0, 4, 8, 12} (layout checked on the GPU), i.e. lane L receives rows
// 16 ci + 8 c + 4 h + (0..3) of column 32 ob + L % 32.
__device__ inline u32x4 tr_chunk(const char* vtile, int vrow_bytes, int kbase, int ob, int ci,
                                    int lane) {
  const int G = lane >> 4, j = lane & 15;
  const int col = 32 * ob + 16 * (G & 1) + 4 * (j & 3);
  const int row = kbase + 16 * ci + 4 * (G >> 1) + (j >> 2);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const char* p0 = vtile + row * vrow_bytes + col * 2;
  const char* p1 = p0 + 8 * vrow_bytes;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  u32x4 r = {ua[0], ua[1], ub[0], ub[1]};
  return r;
}

// The reads of a swizzled tile of D 16-bit columns (rows of D / 8 chunks,
// swz_chunk<D / 8>): offsets fixed per lane, computed once.  row_read: the
// 16-byte A-operand chunk c (0 .. D / 16 - 1) of row r0 + L % 32, half h, as
// *(tile + RB r0 + row[c]) (RB = 2 D bytes per row, r0 a multiple of 16).
// tr_read: what tr_chunk(tile, RB, kbase, ob, ci, lane) reads from an
// unswizzled tile (kbase a multiple of 16).
template <int D = 64>
struct SwzReads {
  static constexpr int C = D / 8;    // chunks per row
  static constexpr int RB = 2 * D;   // bytes per row
  uint32_t row[D / 16];
  uint32_t tr[2][D / 32];
  __device__ inline void init(int lane) {
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) row[c] = RB * l32 + 16 * ((2 * c + h) ^ swz_chunk<C>(l32));
    const int G = lane >> 4, j = lane & 15;
    const int y = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int rr = 4 * (G >> 1) + (j >> 2) + 8 * r;
#pragma unroll
      for (int ob = 0; ob < D / 32; ++ob)
        tr[r][ob] = RB * rr + 16 * ((4 * ob + y) ^ swz_chunk<C>(rr)) + 8 * (j & 1);
    }
  }
  __device__ inline u32x4 row_read(const char* tile, int r0, int c) const {
    return *reinterpret_cast<const u32x4*>(tile + RB * r0 + row[c]);
  }
  __device__ inline u32x4 tr_read(const char* tile, int kbase, int ob, int ci) const {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const char* base = tile + RB * (kbase + 16 * ci);
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + tr[0][ob]));
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + tr[1][ob]));
    u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    u32x4 r = {ua[0], ua[1], ub[0], ub[1]};
    return r;
  }
};

// The value held by lane L ^ 32.  v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second; with both operands equal
// to x, lane L < 32 finds x[L + 32] in the second result and lane L >= 32 finds
// x[L - 32] in the first.
__device__ inline float wave_other_half(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// max / sum over the two half-waves (symmetric, so either result order works).
// The row maxima use IEEE maximum (v_maximum3_f32), which needs no quieting
// of its operands first, where fmaxf costs a v_max_f32 per operand that the
// compiler cannot prove canonical (the permlane results, the first score).
// Scores are finite or -inf, for which the two agree; a NaN propagates.
__device__ inline float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum of the NSB * 16 accumulator values of a lane, as four independent
// running maxima (each folds into v_maximum3) combined at the end, so the
// reduction is not one long dependency chain.
template <int NSB>
__device__ inline float tile_max(const f32x16 (&s)[NSB]) {
  float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
    for (int e = 0; e < 16; ++e) m[e & 3] = __builtin_elementwise_maximum(m[e & 3], s[sb][e]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m[0], m[1]),
                                       __builtin_elementwise_maximum(m[2], m[3]));
}

// True in every lane when `pred` holds in at least one lane of the wave.
__device__ inline bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Maximum / sum of x over the 64 lanes of the wave (result in every lane).
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return halves_max(x);
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) x += __shfl_xor(x, off, 64);
  return halves_sum(x);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ inline u32x4 zero4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Transpose four 16-byte rows (4 keys x E elements of T) into E rows of 4 keys
// and write them to LDS: row e of the output goes to dst + e * row_stride.
template <typename T>
__device__ inline void store_transposed4(char* dst, int row_stride, const u32x4 (&r)[4]) {
  if constexpr (Elt<T>::kBytes == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // column 2p: low halves; column 2p + 1: high halves
      u32x2 even = {(r[0][p] & 0xFFFFu) | (r[1][p] << 16), (r[2][p] & 0xFFFFu) | (r[3][p] << 16)};
      u32x2 odd = {(r[0][p] >> 16) | (r[1][p] & 0xFFFF0000u),
                   (r[2][p] >> 16) | (r[3][p] & 0xFFFF0000u)};
      *reinterpret_cast<u32x2*>(dst + (2 * p) * row_stride) = even;
      *reinterpret_cast<u32x2*>(dst + (2 * p + 1) * row_stride) = odd;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 col = {r[0][e], r[1][e], r[2][e], r[3][e]};
      *reinterpret_cast<u32x4*>(dst + e * row_stride) = col;
    }
  }
}

// Allowed-key membership for the three mask kinds (0 none, 1 causal, 2 window).
// ---------------------------------------------------------------------------
// Dropout mask (an extension; alphabetamath.cc, Algorithm "Exact tiled softmax
// attention with block-recomputed vector-Jacobian products": the base method
// has none, and an extension must replay the same realized mask in its
// reverse pass).  The mask is a function of the indices, regenerated wherever
// it is needed: for head bh (= b * H + h), row i and key j,
//   row key  r_i  = XXH32 of the words (seed_hi, bh, i) with seed seed_lo,
//   group    u    = XXH32 of the word (j >> 2) with seed r_i,
//   keep_ij       = byte (j & 3) of u >= thr      (drop probability thr / 256),
// and a kept weight is scaled by 256 / (256 - thr).  XXH32 is the 32-bit
// xxHash function, here for messages of one and three 32-bit words.
// ---------------------------------------------------------------------------
__device__ inline uint32_t xxh32_round(uint32_t h, uint32_t w) {
  h += w * 0xC2B2AE3Du;
  return __builtin_rotateleft32(h, 17) * 0x27D4EB2Fu;
}
__device__ inline uint32_t xxh32_final(uint32_t h) {
  h ^= h >> 15;
  h *= 0x85EBCA77u;
  h ^= h >> 13;
  h *= 0xC2B2AE3Du;
  return h ^ (h >> 16);
}
__device__ inline uint32_t drop_row_key(const DropParams& dp, uint32_t bh, uint32_t i) {
  uint32_t h = dp.seed_lo + 0x165667B1u + 12u;
  h = xxh32_round(h, dp.seed_hi);
  h = xxh32_round(h, bh);
  h = xxh32_round(h, i);
  return xxh32_final(h);
}
// The four keep bytes of key group g (keys 4g .. 4g + 3) of a row.
__device__ inline uint32_t drop_group_bytes(uint32_t row_key, uint32_t g) {
  return xxh32_final(xxh32_round(row_key + 0x165667B1u + 4u, g));
}
__device__ inline bool drop_keep(uint32_t bytes, int r, int thr) {
  return (int)((bytes >> (8 * r)) & 0xFFu) >= thr;
}

template <int MASK>
__device__ inline bool key_allowed(int q, int j, int n, int window) {
  bool ok = j < n;
  if constexpr (MASK != 0) ok = ok && (j <= q);
  if constexpr (MASK == 2) ok = ok && (j >= q - window + 1);
  return ok;
}

#ifdef EIAT_WG_TIMING
// Timing check build: for every workgroup of a kernel, the constant-rate wall
// clock (s_memrealtime) at its start, after its prologue and at its end, where
// it ran (the HW_ID register: CU, shader array and engine; XCC_ID: the XCD),
// and the shader clock counter (s_memtime) at its start and end, whose
// difference over the wall-clock difference is the engine clock the workgroup
// ran at.  Six words per workgroup, for workgroups 0 .. kWgTimingMax - 1, in a
// table of the kernel's own translation unit.
constexpr int kWgTimingMax = 1 << 16;
constexpr int kWgTimingWords = 6;
struct WgStamps {
  unsigned long long t0 = 0, c0 = 0, t1 = 0;
  __device__ void begin() {
    t0 = __builtin_amdgcn_s_memrealtime();
    c0 = __builtin_amdgcn_s_memtime();
  }
  __device__ void prologue_done() { t1 = __builtin_amdgcn_s_memrealtime(); }
  // From one thread, after a barrier that ends the workgroup's work.
  __device__ void store(unsigned long long* table, int bid) const {
    if (bid >= kWgTimingMax) return;
    const unsigned long long t2 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c2 = __builtin_amdgcn_s_memtime();
    const unsigned hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID, 32 bits
    const unsigned xcc_id = __builtin_amdgcn_s_getreg((15 << 11) | 20);  // HW_REG_XCC_ID, 16 bits
    unsigned long long* rec = table + kWgTimingWords * bid;
    rec[0] = t0;
    rec[1] = t1;
    rec[2] = t2;
    rec[3] = ((unsigned long long)xcc_id << 32) | hw_id;
    rec[4] = c0;
    rec[5] = c2;
  }
};
// Host side: copies a stamp table (the device symbol `table` of `table_bytes`)
// of the last launch to host memory `dst` (at most `bytes`) and the wall
// clock's rate in kHz to *clock_khz.  Returns a hipError_t code.
inline int wg_times_copy(const void* table, size_t table_bytes, void* dst, size_t bytes,
                         int* clock_khz) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(clock_khz, hipDeviceAttributeWallClockRate, dev);
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(dst, table, bytes < table_bytes ? bytes : table_bytes, 0,
                            hipMemcpyDeviceToHost);
  return (int)e;
}
#endif

}  // namespace eiat
