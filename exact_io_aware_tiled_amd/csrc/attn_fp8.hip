// attn_fp8.hip -- block-scaled FP8 (e4m3) query/key rows for the FP8-score
// forward, on gfx950.
//
// webturing.com.tr Principia, "Bellek Duvarinin Fizigi", section on
// FlashAttention-3: FP8 scores, with the precision loss held down by block
// scaling and "incoherent processing" (random sign multipliers).  Reading
// taken here:
//   rotation   x' = H (s * x): s a caller-given vector of +-1, H the
//              unnormalized Sylvester Walsh-Hadamard matrix of order d, so
//              rows of Q and K rotated with the same s give Q' K'^T = d Q K^T
//              (the forward then takes the scale c / d).  Sign flips alone
//              would change nothing (the code keeps the sign exactly); the
//              transform spreads a few large channels over all d values.
//   blocks     every 32 consecutive values x' of a row share a power-of-two
//              scale 2^e, e the least integer (at least -127; 0 for an
//              all-zero block) with max |x'| <= 448 2^e, stored as the byte
//              e + 127 (the E8M0 scale of the OCP microscaling format, which
//              the gfx950 block-scaled MFMA reads directly);
//   codes      the e4m3 codes nearest to x' / 2^e, ties to even (no value
//              saturates: |x' / 2^e| <= 448).
// The transform runs in float32 as butterfly stages of span 1, 2, 4, ..., d/2
// (each pair (a, b) -> (a + b, a - b)), a fixed order, so the codes are a
// deterministic function of the input.
//
// Mapping: a lane holds 8 consecutive values of a row (one 16-byte load for
// 16-bit inputs), d / 8 lanes hold a row.  Spans 1, 2, 4 are in-lane; the
// larger spans exchange with the lane whose index differs in one bit.  A
// 32-value block is 4 neighbouring lanes, so its maximum takes two exchanges.
// The kernel reads 2 (or 4) bytes and writes 1 + 1/32 bytes per value: it is
// bound by HBM bandwidth.
#include "attn_device.h"
#include "attn_internal.h"

namespace eiat {

namespace {

constexpr int kQuantThreads = 256;

// 2^-e as a float (e in [-127, 120], so 127 - e is a normal exponent field)
__device__ inline float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// The least e >= -127 with amax <= 448 2^e (0 for amax == 0).  With amax =
// f 2^x, f in [0.5, 1): e = x - 9 if f <= 0.875 (= 448 / 2^9), else x - 8.
__device__ inline int block_exponent(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int field = (int)(bits >> 23);
  if (amax == 0.0f) return 0;
  if (field == 0) return -127;  // below the normal range: far under 448 2^-127
  const int x = field - 126;
  const int e = (bits & 0x7FFFFFu) <= 0x600000u ? x - 9 : x - 8;
  return e < -127 ? -127 : e;
}

template <typename T>
__device__ inline void load8(const T* p, float (&v)[8]) {
  if constexpr (Elt<T>::kBytes == 2) {
    const u32x4 w = ldg16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = w[i] & 0xFFFFu, hi = w[i] >> 16;
      if constexpr (__is_same(T, __bf16)) {
        v[2 * i] = __uint_as_float(lo << 16);
        v[2 * i + 1] = __uint_as_float(hi << 16);
      } else {
        v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)lo);
        v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
      }
    }
  } else {
    const u32x4 a = ldg16(p), b = ldg16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
}

template <typename T, int D, bool ROT>
__global__ void __launch_bounds__(kQuantThreads)
    attn_quant_fp8_kernel(const T* __restrict__ X, const int8_t* __restrict__ signs,
                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                          int64_t rows) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPB = kQuantThreads / LPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int sub = tid % LPR;                 // values [8 sub, 8 sub + 8) of the row
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int64_t r = row < rows ? row : rows - 1;  // past the end: recompute the last row, store nothing

  float v[8];
  load8<T>(X + r * D + 8 * sub, v);
  if constexpr (ROT) {
    // sign multipliers (exact), then the in-lane butterfly stages
    const u32x2 sw = *reinterpret_cast<const u32x2*>(signs + 8 * sub);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int8_t sg = (int8_t)((sw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
      if (sg < 0) v[i] = -v[i];
    }
#pragma unroll
    for (int span = 1; span < 8; span <<= 1)
#pragma unroll
      for (int i = 0; i < 8; i += 2 * span)
#pragma unroll
        for (int j = i; j < i + span; ++j) {
          const float a = v[j], b = v[j + span];
          v[j] = a + b;
          v[j + span] = a - b;
        }
    // cross-lane stages: span 8 * bit; the lower lane of a pair keeps a + b,
    // the upper one a - b (a the lower lane's value)
#pragma unroll
    for (int bit = 1; bit < LPR; bit <<= 1) {
      const bool upper = (sub & bit) != 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __shfl_xor(v[i], bit, 64);
        v[i] = upper ? p - v[i] : v[i] + p;
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = block_exponent(amax);
  const float inv = pow2_neg(e);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * inv, v[5] * inv, 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * inv, v[7] * inv, w1, true);
  if (row < rows) {
    u32x2 w = {(uint32_t)w0, (uint32_t)w1};
    *reinterpret_cast<u32x2*>(codes + row * D + 8 * sub) = w;
    if ((sub & 3) == 0) scales[row * (D / 32) + sub / 4] = (uint8_t)(e + 127);
  }
}

template <typename T, int D>
hipError_t launch_quant_t(const QuantArgs& a) {
  constexpr int RPB = kQuantThreads / (D / 8);
  const int64_t blocks = (a.rows + RPB - 1) / RPB;
  if (a.signs)
    hipLaunchKernelGGL((attn_quant_fp8_kernel<T, D, true>), dim3((unsigned)blocks),
                       dim3(kQuantThreads), 0, a.stream, static_cast<const T*>(a.x), a.signs,
                       a.codes, a.scales, a.rows);
  else
    hipLaunchKernelGGL((attn_quant_fp8_kernel<T, D, false>), dim3((unsigned)blocks),
                       dim3(kQuantThreads), 0, a.stream, static_cast<const T*>(a.x), a.signs,
                       a.codes, a.scales, a.rows);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quant_dt(const QuantArgs& a) {
  return a.d == 64 ? launch_quant_t<T, 64>(a) : launch_quant_t<T, 128>(a);
}

// ---------------------------------------------------------------------------
// Values for FP8 weights: V quantized along the keys (the contraction index of
// P V), with the same block rule and codes as the rows above (no rotation: a
// rotation of V would have to be undone on O).  Layout written, tile-major so
// that one 64-key tile of V^T is one contiguous block:
//   codes  [bh][nt][dv][64], nt = ceil(n / 64): row r of tile t holds value
//          column r for keys 64 t .. 64 t + 63; 32-key block b (0, 1) fills
//          bytes 32 b .. 32 b + 31, key 64 t + 32 b + 8 g + 4 h + i (g, i in
//          0..3, h in 0..1) at byte 32 b + 16 h + 4 g + i -- the order in which
//          a lane of the score accumulator holds its keys, so that each lane's
//          16 bytes of a block are contiguous;
//   scales [bh][nt][dv][2]: the E8M0 scale of each 32-key block.
// Keys past n count as zero (code 0; a block with no key below n has e = 0).
// One workgroup per (head, tile): the tile goes through LDS, then thread
// (r, b) quantizes one 32-key block of column r.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float lds_elem(const char* p) {
  if constexpr (__is_same(T, __bf16))
    return __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
  else if constexpr (__is_same(T, _Float16))
    return (float)*reinterpret_cast<const _Float16*>(p);
  else
    return *reinterpret_cast<const float*>(p);
}

template <typename T, int DV>
__global__ void __launch_bounds__(2 * DV)
    attn_quant_fp8_v_kernel(const T* __restrict__ V, uint8_t* __restrict__ codes,
                            uint8_t* __restrict__ scales, int n, int nt) {
  constexpr int S = Elt<T>::kBytes;
  constexpr int ROW = DV * S + 16;  // LDS row stride, bytes
  constexpr int CPR = DV * S / 16;  // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) char tile[64 * ROW];
  const int bh = blockIdx.x / nt, t = blockIdx.x % nt;
  const int tid = threadIdx.x;
  const char* src = reinterpret_cast<const char*>(V) + ((int64_t)bh * n + (int64_t)t * 64) * DV * S;
  for (int c = tid; c < 64 * CPR; c += 2 * DV) {
    const int row = c / CPR, col = c % CPR;
    u32x4 w = zero4();
    if (t * 64 + row < n) w = ldg16(src + (int64_t)row * DV * S + col * 16);
    *reinterpret_cast<u32x4*>(tile + row * ROW + col * 16) = w;
  }
  __syncthreads();
  const int r = tid % DV, blk = tid / DV;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const int key = 32 * blk + 8 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3);
    v[p] = lds_elem<T>(tile + key * ROW + r * S);
    amax = fmaxf(amax, fabsf(v[p]));
  }
  const int e = block_exponent(amax);
  const float inv = pow2_neg(e);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q] * inv, v[4 * q + 1] * inv, 0, false);
    w[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q + 2] * inv, v[4 * q + 3] * inv, x, true);
  }
  const int64_t rowidx = ((int64_t)bh * nt + t) * DV + r;
  u32x4 lo = {w[0], w[1], w[2], w[3]}, hi = {w[4], w[5], w[6], w[7]};
  *reinterpret_cast<u32x4*>(codes + rowidx * 64 + 32 * blk) = lo;
  *reinterpret_cast<u32x4*>(codes + rowidx * 64 + 32 * blk + 16) = hi;
  scales[rowidx * 2 + blk] = (uint8_t)(e + 127);
}

template <typename T, int DV>
hipError_t launch_quant_v_t(const QuantVArgs& a) {
  const int nt = (int)((a.n + 63) / 64);
  hipLaunchKernelGGL((attn_quant_fp8_v_kernel<T, DV>), dim3((unsigned)(a.bh * nt)), dim3(2 * DV),
                     0, a.stream, static_cast<const T*>(a.v), a.codes, a.scales, (int)a.n, nt);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quant_v_dt(const QuantVArgs& a) {
  return a.dv == 64 ? launch_quant_v_t<T, 64>(a) : launch_quant_v_t<T, 128>(a);
}

}  // namespace

hipError_t launch_quant_fp8_v(const QuantVArgs& a) {
  switch (a.dtype) {
    case 0: return launch_quant_v_dt<float>(a);
    case 1: return launch_quant_v_dt<_Float16>(a);
    default: return launch_quant_v_dt<__bf16>(a);
  }
}

hipError_t launch_quant_fp8(const QuantArgs& a) {
  switch (a.dtype) {
    case 0: return launch_quant_dt<float>(a);
    case 1: return launch_quant_dt<_Float16>(a);
    default: return launch_quant_dt<__bf16>(a);
  }
}

}  // namespace eiat
