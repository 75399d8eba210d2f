// attn_fwd.hip -- exact tiled softmax attention, forward pass, for gfx950.
//
// Follows alphabetamath.cc, "Exact tiled attention and memory-aware
// differentiation": the Algorithm's forward procedure (per query row: start
// from the empty summary, for each key block skip it if no key is allowed,
// otherwise form the block's summary and copy or merge it with the running one
// using the Definition's merge; finish with Y = z / l and keep m, l), with the
// merge written as the streaming update of "The Arithmetic of Intelligence",
// ch. 12, "Streaming softmax": m' = max(m, max s), l' = l e^{m-m'} + sum e^{s-m'},
// and the weighted value sum rescaled by the same factor.
//
// Mapping to CDNA4.  A workgroup of 4 waves owns BM = 128 query rows of one
// (batch, head); each wave owns 32 rows and keeps them in registers as the B
// operand of S^T = K Q^T, so the accumulator gives every lane all the scores of
// ONE query row (16 keys per 32-key block per half-wave): the row max and row
// sum are in-lane, plus one exchange of the two half-waves (v_permlane32_swap).
// Key/value tiles of BN keys (128 for 16-bit d = 64, else 64) stream through
// LDS, double-buffered: 16-bit tiles with d >= 32 are copied HBM -> LDS
// directly (global_load_lds_dwordx4, no staging registers); the others are
// staged one tile ahead in registers.  K is read row-major as the A operand of S^T.
// For 16-bit types V is stored row-major too and read with ds_read_b64_tr_b16,
// which delivers the V^T operand of O^T += V^T P^T directly; float32 stores a
// transposed copy instead.  P = 2^(s*c*log2(e) - m) is rounded to the input type
// in registers and used directly as the B operand (no LDS round trip).  Only O
// and LSE = m + ln l go to HBM; no score block ever leaves the registers.
//
// Deviation from the pages' update, exact in real arithmetic: the running
// shift m is only raised when a block's maximum exceeds it by more than 2^8 (in
// base-2 units) for some row of the wave; otherwise the old shift is kept and no
// rescale is done.  Terms stay below 2^8 (no overflow in fp32 or in the 16-bit
// operand), and O = z / l and LSE = m + ln l do not depend on which shift was
// used, only on its consistency, as the merge identity shows.
//
// Blocks with no allowed key are not visited (causal / window tile ranges) and
// the per-element mask is applied only in blocks that straddle a boundary.
//
// FP8 modes (template F8; webturing.com.tr Principia, "Bellek Duvarinin
// Fizigi", section on FlashAttention-3): 1 forms S from e4m3 Q and K codes
// with E8M0 block scales on the block-scaled FP8 MFMA (K = 64 per
// instruction, the scales applied inside it); 2 also rounds P to e4m3 and
// forms O^T += V^T P^T from the V^T codes of attn_quant_fp8_v.  The softmax
// between the two products is the same in every mode.
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace eiat {

#ifdef EIAT_WG_TIMING
// Timing check build: per-workgroup stamps of the forward (WgStamps; the
// prologue ends when the first score block is formed).  Read with eiat_wg_times.
__device__ unsigned long long g_wg_times[kWgTimingWords * kWgTimingMax];
#endif

// F8: 0 16-bit (or float32) scores; 1 FP8 scores; 2 FP8 scores and FP8 weights
// and values (V in the tile-major layout of attn_quant_fp8_v).
template <typename T, int D, int F8 = 0>
struct FwdCfg {
  // 4 waves (128 query rows) share each K/V tile.  At 16-bit d = 128 this beat
  // 8 waves (256 rows, half the K/V loads per row) on every measured shape:
  // +3 % at n = 65536, +6 % at n = 8192, +7-18 % at n = 4096 causal, where
  // the finer grid balances better.
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * kWaves;      // query rows per workgroup
  // Keys per tile.  16-bit d = 64 streams 128-key tiles: half the barriers
  // and loop overhead per key, four independent 32-key score blocks per tile
  // (4-7 % faster at d = 64 although the 72 KiB of tiles leave room for two
  // workgroups per CU instead of three).
  // (The tile-shape check build takes 64 keys at d = 64 and 32 at d = 128.)
  static constexpr int BN = (Elt<T>::kBytes == 2 && !F8)
                                ? (kAltTiles ? (D == 128 ? 32 : 64) : (D == 64 ? 128 : 64))
                                : 64;
  static constexpr int DP = D < 32 ? 32 : D;  // value rows padded to whole 32-row blocks
  static constexpr int S = Elt<T>::kBytes;
  static constexpr bool kTr = (S == 2);       // 16-bit: V row-major + transpose reads
  static constexpr int KS = F8 ? 1 : S;       // bytes per Q / K element (FP8 scores: 1)
  // LDS bank conflicts of the 16-bit tiles loaded directly (d = 64 and 128):
  // unpadded rows with XOR-swizzled chunks (swz_chunk: conflict-free 16-byte
  // K reads and transposing V reads).  With FP8 scores the 16-bit V tiles at
  // d = 128 are swizzled too (3-8 % faster; at d = 64 1 % slower) and the FP8
  // K rows keep one padding slot.  Rows padded by one 16-byte slot otherwise.
  static constexpr bool kSwz = kTr && D >= 64 && (F8 == 0 || (F8 == 1 && D == 128));
  static constexpr int PAD = kSwz ? 0 : 1;                   // V rows (and 16-bit K rows)
  static constexpr int KPAD = (kSwz && !F8) ? 0 : 1;         // K rows
  static constexpr int KROW = D * KS + 16 * KPAD;  // K tile row stride in LDS (bytes), padded
  // V tile: row-major [BN][DP] (16-bit) or transposed [DP][BN] (float32)
  static constexpr int VROW = F8 == 2 ? 64 + 16 : (kTr ? DP * S + 16 * PAD : BN * S + 16);
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = (kTr && F8 != 2 ? BN : DP) * VROW;
  static constexpr int NCH = D * S / 32;      // d-chunks per 32x32 product (both halves)
  static constexpr int NQF = F8 ? D / 32 : NCH;  // 16-byte Q chunks per lane
  static constexpr int NOB = DP / 32;         // 32-row blocks of O^T
  static constexpr int NSB = BN / 32;         // 32-key blocks of S^T
  static constexpr int CPR = D * S / 16;      // 16-byte chunks per V row
  static constexpr int CPRK = D * KS / 16;    // 16-byte chunks per K row
  static constexpr int KCHUNKS = BN * CPRK;
  static constexpr int KPT = (KCHUNKS + kThreads - 1) / kThreads;
  // V: 16-bit stages 16-byte chunks like K; float32 stages 4-key x 16-byte tasks
  static constexpr int VTASKS = kTr ? BN * CPR : (BN / 4) * CPR;
  static constexpr int VREGS = kTr ? 1 : 4;
  static constexpr int VPT = (VTASKS + kThreads - 1) / kThreads;
  static constexpr int EPC = 16 / S;          // elements per 16-byte chunk
  // 16-bit tiles without zero-padded columns go HBM -> LDS directly
  static constexpr bool kDirect = kTr && D >= 32;
  static constexpr float kTau = 8.0f;         // lazy-rescale threshold, base-2 units
  // Two score buffers (next tile's scores issued before this tile's
  // exponentials) where the score MFMAs are long enough to hide the exp work.
  static constexpr bool kDoubleS = D >= 128;
  // Waves per SIMD the register allocation must allow (4-wave workgroups).
  // 16-bit d = 16 runs four; bf16 FP8-score kernels fit three; fp16 needs a few
  // more registers for its sums.  128-key tiles hold two workgroups per CU by
  // their LDS, so two waves: asking for three there left the sliding-window
  // kernel at one wave per SIMD (264 registers) and 28 % slower.
  static constexpr int kMinWaves =
      S == 4 ? (D >= 128 ? 1 : 2)
             : (D == 16 ? 4 : ((D >= 128 || BN == 128 || !__is_same(T, __bf16)) ? 2 : 3));
  // FP8 scores and 16-bit d = 16: exactly kMinWaves.  Left free to go higher,
  // the compiler spilled up to 126 scalar registers into vector lanes inside
  // the loop (FP8 d = 64: 4-7 % slower; d = 16: 1-5 %).
  static constexpr int kMaxWaves = (F8 || (D == 16 && S == 2)) ? kMinWaves : 8;
};

template <typename T, int D, int MASK, bool DROP, int F8>
__global__ void
    __attribute__((amdgpu_flat_work_group_size(1, FwdCfg<T, D, F8>::kThreads),
                   amdgpu_waves_per_eu(FwdCfg<T, D, F8>::kMinWaves, FwdCfg<T, D, F8>::kMaxWaves)))
    attn_fwd_kernel(const void* __restrict__ Q, const void* __restrict__ K, const T* __restrict__ V,
                    T* __restrict__ O, float* __restrict__ LSE, int n, int bh_count,
                    int num_qtiles, int window, float qk_scale, int qmode, DropParams dp,
                    const uint8_t* __restrict__ Qsc, const uint8_t* __restrict__ Ksc,
                    const uint8_t* __restrict__ Vsc) {
  using C = FwdCfg<T, D, F8>;
  constexpr int BN = C::BN;
  // LDS: two K buffers, then two V buffers.  K runs one tile ahead of V.
  __shared__ __attribute__((aligned(16))) char smem[2 * C::KBYTES + 2 * C::VBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Consecutive workgroups take consecutive heads of the same query-tile rank;
  // with masks, the heaviest query tiles (most visible keys) are issued first.
  const int bid = blockIdx.x;
#ifdef EIAT_WG_TIMING
  WgStamps wg_stamps;
  wg_stamps.begin();
#endif
  const int bh = bid % bh_count;
  int qt = bid / bh_count;
  if (MASK != 0) qt = num_qtiles - 1 - qt;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  // Dropout (DROP): this row's key of the realized mask (see attn_device.h).
  const uint32_t row_key = DROP ? drop_row_key(dp, (uint32_t)bh, (uint32_t)qrow) : 0u;

  const int64_t head = (int64_t)bh * n;
  const char* Qh = reinterpret_cast<const char*>(Q) + head * D * C::KS;
  const char* Kh = reinterpret_cast<const char*>(K) + head * D * C::KS;
  // FP8 values: tile t of this head's V^T is D rows of 64 codes at Vh + t D 64.
  const int v_tiles = (n + 63) / 64;
  const char* Vh = F8 == 2 ? reinterpret_cast<const char*>(V) + (int64_t)bh * v_tiles * D * 64
                           : reinterpret_cast<const char*>(V + head * D);

  // Key range any row of this workgroup may see; whole tiles outside it are skipped.
  int kend = n;
  if (MASK != 0) kend = min(n, q0 + C::BM);
  int kbeg = 0;
  if (MASK == 2) kbeg = max(0, q0 - window + 1);
  const int t_lo = kbeg / BN;
  const int t_hi = (kend + BN - 1) / BN;
  // Tiles in [t_in_lo, t_in_hi) need no per-element mask for any row of the
  // workgroup (every key allowed and below n); the others are boundary tiles.
  int t_in_lo = t_lo, t_in_hi = t_hi;
  if (MASK == 2) t_in_lo = max(t_lo, (q0 + C::BM - 1 - window + 1 + BN - 1) / BN);
  if (MASK != 0) t_in_hi = min(t_hi, (q0 + 1) / BN);
  t_in_hi = min(t_in_hi, n / BN);
  t_in_lo = min(t_in_lo, t_hi);
  if (t_in_hi < t_in_lo) t_in_hi = t_in_lo;

  // This wave's query rows as MFMA B-operand chunks: lane L holds row qw0 + L%32,
  // d-bytes [32c + 16h, 32c + 16h + 16).  The sign of c is folded into Q
  // (qmode 1), and c = 0 is taken as Q = 0 with a unit exponent scale (qmode 2).
  // Rows past n read row n - 1 (never stored).
  //
  // FP8 scores (F8): Q and K are e4m3 codes with one E8M0 scale byte per 32
  // values.  One block-scaled MFMA (K = 64) takes 32 bytes per lane: lane L
  // supplies bytes [64 c + 16 h, +16) and [64 c + 32 + 16 h, +16) of its row
  // for chunk c, and the scale of that row's 32-value block 2 c + h (the
  // hardware applies the scale of lane r to bytes 0-15 of lanes r and r + 32,
  // and that of lane r + 32 to bytes 16-31 of both).  Each lane's scale word
  // holds its block 2 c + h in byte 2 c (operand select 2 c).
  u32x4 qf[C::NQF];
  uint32_t qsw = 0;
  {
    const int qr = min(qrow, n - 1);
    if constexpr (F8) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        qf[2 * c] = ldg16(Qh + (int64_t)qr * D + 64 * c + 16 * h);
        qf[2 * c + 1] = ldg16(Qh + (int64_t)qr * D + 64 * c + 32 + 16 * h);
      }
#pragma unroll
      for (int c = 0; c < C::NQF; ++c) {
        if (qmode == 1) qf[c] = fp8_negate(qf[c]);
        if (qmode == 2) qf[c] = zero4();
      }
      qsw = scale_word<D>(Qsc + (head + qr) * (D / 32), h);
    } else {
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        qf[c] = ldg16(Qh + (int64_t)qr * D * C::S + 32 * c + 16 * h);
        if (qmode == 1) qf[c] ^= Elt<T>::kSign;
        if (qmode == 2) qf[c] = zero4();
      }
    }
  }

  auto kbuf = [&](int t) __attribute__((always_inline)) -> char* { return smem + (t & 1) * C::KBYTES; };
  auto vbuf = [&](int t) __attribute__((always_inline)) -> char* { return smem + 2 * C::KBYTES + (t & 1) * C::VBYTES; };

  // Value columns/rows beyond D (only for D < 32) stay zero in both V buffers.
  if constexpr (C::DP > D) {
    constexpr int zrows = C::kTr ? BN : C::DP - D;
    constexpr int zper = C::kTr ? (C::DP - D) * C::S / 16 : C::VROW / 16;
    for (int idx = tid; idx < 2 * zrows * zper; idx += C::kThreads) {
      const int b = idx / (zrows * zper), rem = idx % (zrows * zper);
      const int row = rem / zper, col = rem % zper;
      char* vb = vbuf(b);
      if constexpr (C::kTr)
        *reinterpret_cast<u32x4*>(vb + row * C::VROW + D * C::S + col * 16) = zero4();
      else
        *reinterpret_cast<u32x4*>(vb + (D + row) * C::VROW + col * 16) = zero4();
    }
  }

  TileLoader<BN, C::CPR, C::kWaves, C::PAD, C::kSwz> tl;
  SwzReads<D> swz;
  if constexpr (C::kSwz) swz.init(lane);
  TileLoader<D, 4, C::kWaves> tlv;  // FP8 values: D rows of 64 codes
  if constexpr (F8 == 2) tlv.init(wave, lane);
  // FP8 values: scale words of the V^T rows this lane supplies (block h of
  // rows 32 ob + L % 32), for the tile multiplied next and the one loading.
  uint32_t vsw[C::NOB], vsw_next[C::NOB];
#pragma unroll
  for (int ob = 0; ob < C::NOB; ++ob) vsw[ob] = vsw_next[ob] = 0;
  TileLoader<BN, C::CPRK, C::kWaves> tlk;
  if constexpr (C::kDirect) {
    tl.init(wave, lane);
    if constexpr (F8) tlk.init(wave, lane);
  }
  // FP8: scale words of the K rows this lane supplies to the score MFMAs, for
  // the tile being multiplied next (ksw) and the one being loaded (ksw_next).
  uint32_t ksw[C::NSB], ksw_next[C::NSB];
#pragma unroll
  for (int sb = 0; sb < C::NSB; ++sb) ksw[sb] = ksw_next[sb] = 0;
  const uint8_t* Ksh = F8 ? Ksc + head * (D / 32) : nullptr;
  u32x4 kreg[C::kDirect ? 1 : C::KPT];
  u32x4 vreg[C::kDirect ? 1 : C::VPT][C::VREGS];

  // Rows past n are read from row n - 1: they are masked (K) or multiplied by a
  // zero probability (V), so the loads need no branch.
  auto load_k = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * BN;
    if constexpr (F8) {
      tlk.load(kbuf(t), Kh, j0, n, wave, lane);
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
        ksw_next[sb] = scale_word_raw<D>(Ksh + (int64_t)min(j0 + 32 * sb + l32, n - 1) * (D / 32));
      return;
    } else if constexpr (C::kDirect) {
      tl.load(kbuf(t), Kh, j0, n, wave, lane);
      return;
    }
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      const int c = tid + r * C::kThreads;
      if (C::KCHUNKS % C::kThreads == 0 || c < C::KCHUNKS) {
        const int key = c / C::CPRK, col = c % C::CPRK;
        const int j = min(j0 + key, n - 1);
        kreg[r] = ldg16(Kh + (int64_t)j * D * C::S + col * 16);
      }
    }
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * BN;
    if constexpr (F8 == 2) {
      tlv.load(vbuf(t), Vh + (int64_t)t * D * 64, 0, D, wave, lane);
      const uint8_t* vs = Vsc + ((int64_t)bh * v_tiles + t) * D * 2;
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob)
        vsw_next[ob] = (uint32_t)*reinterpret_cast<const uint16_t*>(vs + (32 * ob + l32) * 2);
      return;
    }
    if constexpr (C::kDirect) {
      tl.load(vbuf(t), Vh, j0, n, wave, lane);
      return;
    }
#pragma unroll
    for (int r = 0; r < C::VPT; ++r) {
      const int task = tid + r * C::kThreads;
      if (C::VTASKS % C::kThreads == 0 || task < C::VTASKS) {
        const int kq = task / C::CPR, col = task % C::CPR;
#pragma unroll
        for (int i = 0; i < C::VREGS; ++i) {
          const int j = min(j0 + C::VREGS * kq + i, n - 1);
          vreg[r][i] = ldg16(Vh + (int64_t)j * D * C::S + col * 16);
        }
      }
    }
  };
  auto store_k = [&](int t) __attribute__((always_inline)) {
    if constexpr (C::kDirect) {
      wait_tile_loads();
      return;
    }
    char* kb = kbuf(t);
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      const int c = tid + r * C::kThreads;
      if (C::KCHUNKS % C::kThreads == 0 || c < C::KCHUNKS) {
        const int key = c / C::CPRK, col = c % C::CPRK;
        *reinterpret_cast<u32x4*>(kb + key * C::KROW + col * 16) = kreg[r];
      }
    }
  };
  auto store_v = [&](int t) __attribute__((always_inline)) {
    if constexpr (C::kDirect) {
      wait_tile_loads();
      return;
    }
    char* vb = vbuf(t);
#pragma unroll
    for (int r = 0; r < C::VPT; ++r) {
      const int task = tid + r * C::kThreads;
      if (C::VTASKS % C::kThreads == 0 || task < C::VTASKS) {
        const int kq = task / C::CPR, col = task % C::CPR;
        if constexpr (C::kTr)
          *reinterpret_cast<u32x4*>(vb + kq * C::VROW + col * 16) = vreg[r][0];
        else
          store_transposed4<T>(vb + (col * C::EPC) * C::VROW + 4 * kq * C::S, C::VROW, vreg[r]);
      }
    }
  };

  // 32-key block sb of the S^T block of tile t = K_t Q_w^T (fp32 accumulate)
  auto qk_block = [&](int t, f32x16 (&s)[C::NSB], int sb) __attribute__((always_inline)) {
    const char* kb = kbuf(t);
    {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[sb][e] = 0.0f;
      if constexpr (F8) {
        const char* kr = kb + (32 * sb + l32) * C::KROW + 16 * h;
        s[sb] = mma_fp8<0>(*reinterpret_cast<const u32x4*>(kr),
                           *reinterpret_cast<const u32x4*>(kr + 32), qf[0], qf[1], ksw[sb], qsw,
                           s[sb]);
        if constexpr (D == 128)
          s[sb] = mma_fp8<2>(*reinterpret_cast<const u32x4*>(kr + 64),
                             *reinterpret_cast<const u32x4*>(kr + 96), qf[2], qf[3], ksw[sb], qsw,
                             s[sb]);
      } else {
#pragma unroll
        for (int c = 0; c < C::NCH; ++c) {
          u32x4 a;
          if constexpr (C::kSwz)
            a = swz.row_read(kb, 32 * sb, c);
          else
            a = *reinterpret_cast<const u32x4*>(kb + (32 * sb + l32) * C::KROW + 32 * c + 16 * h);
          s[sb] = Elt<T>::mma(a, qf[c], s[sb]);
        }
      }
    }
  };
  auto qk = [&](int t, f32x16 (&s)[C::NSB]) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) qk_block(t, s, sb);
  };

  // Running summary of this lane's query row.  Both half-waves keep the same
  // shift m; each keeps a partial l over its own keys (added at the end).
  float m_run = -INFINITY;
  float m_thr = -INFINITY;  // m_run + tau, the block maximum that raises the shift
  float l_run = 0.0f;
  f32x16 o[C::NOB];
#pragma unroll
  for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[ob][e] = 0.0f;

  // Merging the scores s of tile t into the running summary is split in two so
  // that the next tile's score MFMAs can be issued between the halves:
  // prep_tile masks (boundary tiles only), takes the block max and, if needed,
  // raises the shift and rescales; exp_pv_tile forms P = 2^(s c log2 e - m),
  // adds its sum to l and accumulates O^T += V^T P^T.  A tile with no allowed
  // key for some row leaves that row unchanged (its P is 0), as the
  // Algorithm's empty-block skip does.
  //
  // Boundary tiles: the 32-key blocks [sb_lo, sb_hi) of tile t that hold an
  // allowed key for at least one row of this wave (wave-uniform).  The others
  // contribute exactly nothing (every weight 0), so they are not visited.  The
  // FP8-value product covers two blocks per instruction and keeps them all.
  int sb_lo = 0, sb_hi = C::NSB;
  auto block_range = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * BN;
    int lo = 0, hi = C::NSB;
    if constexpr (F8 != 2) {
      const int last = min(n - 1, MASK != 0 ? qw0 + 31 : n - 1) - j0;  // last key any row may see
      hi = last < 0 ? 0 : min(hi, last / 32 + 1);
      if constexpr (MASK == 2) {
        const int first = qw0 - window + 1 - j0;  // first key any row may see
        if (first > 0) lo = min(hi, first / 32);
      }
    }
    sb_lo = lo;
    sb_hi = hi;
  };
  auto active = [&](int sb, auto masked) __attribute__((always_inline)) -> bool {
    if constexpr (decltype(masked)::value) return sb >= sb_lo && sb < sb_hi;
    return true;
  };
  auto prep_tile = [&](int t, f32x16 (&s)[C::NSB], auto masked) __attribute__((always_inline)) -> float {
    const int j0 = t * BN;
    float mx = -INFINITY;
    if constexpr (decltype(masked)::value) {
      block_range(t);
      float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        if (!active(sb, masked)) continue;
        // Only a block that some row of the wave sees in part needs the
        // per-element mask (on the causal diagonal one block per wave);
        // blocks whose 32 keys every row of the wave sees are taken whole.
        const int jb = j0 + 32 * sb;
        bool whole = jb + 31 < n;
        if constexpr (MASK != 0) whole = whole && jb + 31 <= qw0;
        if constexpr (MASK == 2) whole = whole && jb >= qw0 + 31 - window + 1;
        if (!whole) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = jb + 8 * (e >> 2) + 4 * h + (e & 3);
            if (!key_allowed<MASK>(qrow, j, n, window)) s[sb][e] = -INFINITY;
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) m4[e & 3] = fmaxf(m4[e & 3], s[sb][e]);
      }
      mx = halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    } else {
      // Block maximum of this row, in units of log2 (c * log2(e) folded in),
      // as a shallow tree so the reduction is not one long dependency chain.
      mx = halves_max(tile_max<C::NSB>(s));
    }
    // In the mask-free body every row has an allowed key, so mx is finite and,
    // after the update below, so is m_run: the -inf guards are only needed in
    // boundary tiles.
    float m_blk;
    if constexpr (decltype(masked)::value)
      m_blk = (mx == -INFINITY) ? -INFINITY : mx * qk_scale;
    else
      m_blk = mx * qk_scale;
    // Raise the shift (and rescale) only if some row's max grew by more than tau.
    if (wave_any(m_blk > m_thr)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) o[ob] *= alpha;
      m_run = m_new;
      m_thr = m_new + C::kTau;
    }
    // A row with no allowed key so far keeps the empty summary: shift by 0.
    if constexpr (decltype(masked)::value)
      return (m_run == -INFINITY) ? 0.0f : m_run;
    else
      return m_run;
  };
  // One 32-key block of exp_pv_tile (every mode but FP8 values).
  auto exp_pv_block = [&](int t, f32x16 (&s)[C::NSB], float m_use, auto masked, int sb)
      __attribute__((always_inline)) {
    const char* vb = vbuf(t);
    if (!active(sb, masked)) return;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[sb][e] = fast_exp2(__builtin_fmaf(s[sb][e], qk_scale, -m_use));
    PChunks<T> pc;
    if constexpr (DROP) {
      // l sums the undropped weights; then dropped weights become 0 in the
      // value product (the kept ones are scaled by 256 / (256 - thr) at the end).
      float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < 16; ++e) ps[e & 3] += s[sb][e];
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      const int jb = t * BN + 32 * sb + 4 * h;  // key of element e = 0
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t bytes = drop_group_bytes(row_key, (uint32_t)(jb + 8 * k) >> 2);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (!drop_keep(bytes, r, dp.thr)) s[sb][4 * k + r] = 0.0f;
      }
      pc.set(s[sb]);
    } else {
      pc.set(s[sb]);
      l_run = chunk_sum<T>(pc, s[sb], l_run);
    }
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) {
#pragma unroll
      for (int ci = 0; ci < PChunks<T>::kCount; ++ci) {
        u32x4 va;
        if constexpr (C::kSwz)
          va = swz.tr_read(vb, 32 * sb, ob, ci);
        else if constexpr (C::kTr)
          va = tr_chunk(vb, C::VROW, 32 * sb, ob, ci, lane);
        else
          va = keyrow_chunk<T>(vb + (32 * ob + l32) * C::VROW + 32 * sb * C::S, ci, h);
        o[ob] = Elt<T>::mma(va, pc.c[ci], o[ob]);
      }
    }
  };
  auto exp_pv_tile = [&](int t, f32x16 (&s)[C::NSB], float m_use, auto masked) __attribute__((always_inline)) {
    if constexpr (F8 == 2) {
      const char* vb = vbuf(t);
      // FP8 weights: P rounded to e4m3 with a unit scale (P <= 2^8 < 448),
      // the lane's 16 keys of each 32-key block in accumulator order, which is
      // the byte order of the V^T codes; one block-scaled MFMA per 64 keys and
      // 32 value rows.  l sums the unrounded float32 weights.
      static_assert(C::NSB == 2, "FP8 values: 64-key tiles");
      u32x4 pk[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[sb][e] = fast_exp2(__builtin_fmaf(s[sb][e], qk_scale, -m_use));
        float ts[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ts[e] = s[sb][e] + s[sb][e + 8];
#pragma unroll
        for (int e = 0; e < 4; ++e) ts[e] += ts[e + 4];
        l_run += (ts[0] + ts[1]) + (ts[2] + ts[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[sb][4 * q], s[sb][4 * q + 1], 0, false);
          pk[sb][q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[sb][4 * q + 2], s[sb][4 * q + 3],
                                                                lo, true);
        }
      }
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) {
        const char* vr = vb + (32 * ob + l32) * C::VROW + 16 * h;
        o[ob] = mma_fp8<0>(*reinterpret_cast<const u32x4*>(vr),
                           *reinterpret_cast<const u32x4*>(vr + 32), pk[0], pk[1], vsw[ob],
                           0x7F7F7F7Fu, o[ob]);
      }
      return;
    }
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) exp_pv_block(t, s, m_use, masked, sb);
  };

  // Prologue: K_lo, V_lo and K_lo+1 in LDS, S_lo in registers.
  f32x16 sc[C::kDoubleS ? 2 : 1][C::NSB];
  // FP8: the K scale words loaded with a tile become current for its product.
  // They are loaded raw and shifted to this half-wave's bytes only here, after
  // the tile loads have been waited for: an operation on them right after the
  // load would wait for every load issued before them, the whole tile prefetch
  // included (vector-memory loads retire in order).
  auto advance_ksw = [&]() __attribute__((always_inline)) {
    if constexpr (F8 != 0) {
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) ksw[sb] = ksw_next[sb] >> (8 * h);
    }
    if constexpr (F8 == 2) {
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) vsw[ob] = vsw_next[ob] >> (8 * h);
    }
  };
  if constexpr (C::kDirect && F8 == 0) {
    // All three tiles in flight together, then one wait (not two in a row).
    load_k(t_lo);
    load_v(t_lo);
    if (t_lo + 1 < t_hi) load_k(t_lo + 1);
    wait_tile_loads();
  } else {
    // Register staging holds one tile at a time; FP8 advances the K scale
    // words of tile t_lo before those of t_lo + 1 are loaded.
    load_k(t_lo);
    load_v(t_lo);
    store_k(t_lo);
    store_v(t_lo);
    advance_ksw();
    if (t_lo + 1 < t_hi) {
      load_k(t_lo + 1);
      store_k(t_lo + 1);
    }
  }
  __syncthreads();
  qk(t_lo, sc[0]);
  advance_ksw();
  __syncthreads();  // K_lo is overwritten by K_lo+2 in the first iteration
#ifdef EIAT_WG_TIMING
  wg_stamps.prologue_done();
#endif

  // Iteration t: the scores of tile t are exponentiated and multiplied into O
  // while S_{t+1} = K_{t+1} Q^T is formed; V_{t+1} and K_{t+2}, loaded from HBM
  // at the top, are stored for the next iteration.  With one score buffer
  // S_{t+1} overwrites S_t block by block after its exponentials; with two
  // (d = 128, twice the MFMA work per tile) each block of S_{t+1} goes into
  // the other buffer ahead of the same block of S_t's exponentials.  cur holds
  // S_t; nxt receives S_{t+1} (the same buffer below d = 128).
  auto iterate = [&](int t, f32x16 (&cur)[C::NSB], f32x16 (&nxt)[C::NSB], auto masked)
      __attribute__((always_inline)) {
    const bool has1 = t + 1 < t_hi, has2 = t + 2 < t_hi;
    if (has1) load_v(t + 1);
    if (has2) load_k(t + 2);
    const float m_use = prep_tile(t, cur, masked);
    // Raised priority while this wave has MFMAs to issue, so another wave's
    // softmax VALU work fills the gaps rather than delaying them.
    __builtin_amdgcn_s_setprio(1);
    // Scheduling hint for this region: interleave the LDS operand reads with
    // the MFMAs (2-10 % faster on the 16-bit forwards at n = 4096-65536, 1-5 %
    // on the FP8-value ones and 2-3 % on FP8 scores at d = 128; FP8 scores at
    // d = 64 measured 3-5 % slower with it and keep the default schedule).
    if constexpr (!(F8 == 1 && D == 64)) __builtin_amdgcn_iglp_opt(0);
    // The next tile's scores.  In the mask-free body t + 1 == t_hi reads a
    // stale buffer whose result is unused (no branch there, so the score MFMAs
    // interleave with the exponentials); a boundary tile, which is the last one
    // of every causal row block, skips them.
    auto next_scores = [&](f32x16 (&s)[C::NSB]) __attribute__((always_inline)) {
      if constexpr (decltype(masked)::value) {
        if (has1) qk(t + 1, s);
      } else {
        qk(t + 1, s);
      }
    };
    // In the mask-free 16-bit body the two products are issued block by block,
    // so that the compiler spreads the score products over the exponentials
    // (bitwise unchanged; with dropout 10 % slower at d = 64, so left out
    // there).  One score buffer: block sb of the next tile's scores right after
    // block sb's value products, whose scores are consumed by then (1-2 %
    // faster at d = 64).  Two buffers: block sb of the next tile's scores, then
    // block sb's exponentials and value products (0.5-1 % faster at d = 128).
    constexpr bool kBlockwise = !decltype(masked)::value && F8 == 0 && !DROP;
    if constexpr (kBlockwise && C::kDoubleS) {
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        qk_block(t + 1, nxt, sb);
        exp_pv_block(t, cur, m_use, masked, sb);
      }
    } else if constexpr (kBlockwise) {
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        exp_pv_block(t, cur, m_use, masked, sb);
        qk_block(t + 1, nxt, sb);
      }
    } else if constexpr (C::kDoubleS) {
      next_scores(nxt);
      exp_pv_tile(t, cur, m_use, masked);
    } else {
      exp_pv_tile(t, cur, m_use, masked);
      next_scores(nxt);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (F8 != 0) {
      // FP8: one unconditional wait for the direct tile loads.  Behind a branch
      // the compiler sank this tile's products past the wait (they touch no
      // memory), which turned the prefetch into a synchronous load (15-17 %
      // slower FP8-value forward).  The 16-bit kernels keep the branches: there
      // the products stay ahead of the wait, and the unconditional form measured
      // 3-12 % slower.
      wait_tile_loads();
    } else {
      if (has1) store_v(t + 1);
      if (has2) store_k(t + 2);
    }
    advance_ksw();
    __syncthreads();
  };
  // With two score buffers the loop is unrolled by two so that the buffers
  // swap roles without copies; `swapped` says S_t sits in sc[1] (a segment
  // that ends after an odd number of tiles), which the next segment undoes
  // with one copy.
  //
  // In the mask-free segment the tiles are taken in pairs from an even index,
  // so that each tile's LDS buffers (chosen by the tile index mod 2) are known
  // at compile time and the operand addresses fold into the LDS instructions'
  // offsets: 8-12 fewer VALU instructions per tile, 2.5 % faster at d = 64,
  // 0.5-1.5 % at d = 16 and d = 128, bitwise unchanged.  With one score
  // buffer fp16 (3 %), dropout and FP8 scores (2 %) measured slower this way
  // and keep the plain loop.
  constexpr int kB = C::kDoubleS ? 1 : 0;
  bool swapped = false;
  auto run = [&](int t, int end, auto masked) __attribute__((always_inline)) -> int {
    constexpr bool kPairs =
        !decltype(masked)::value &&
        (C::kDoubleS || (!__is_same(T, _Float16) && F8 == 0 && !DROP));
    if constexpr (C::kDoubleS) {
      if (t < end && swapped) {
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) sc[0][sb] = sc[kB][sb];
        swapped = false;
      }
      if constexpr (kPairs) {
        if (t < end) {  // (an empty segment may start at an odd index: leave t)
          if (t & 1) {
            iterate(t, sc[0], sc[kB], masked);
            ++t;
#pragma unroll
            for (int sb = 0; sb < C::NSB; ++sb) sc[0][sb] = sc[kB][sb];
          }
          int i = t >> 1;
          for (; 2 * i + 1 < end; ++i) {
            iterate(2 * i, sc[0], sc[kB], masked);
            iterate(2 * i + 1, sc[kB], sc[0], masked);
          }
          t = 2 * i;
        }
      }
      for (; t + 1 < end; t += 2) {
        iterate(t, sc[0], sc[kB], masked);
        iterate(t + 1, sc[kB], sc[0], masked);
      }
      if (t < end) {
        iterate(t, sc[0], sc[kB], masked);
        ++t;
        swapped = true;
      }
    } else {
      if constexpr (kPairs) {
        if (t < end) {  // (an empty segment may start at an odd index: leave t)
          if (t & 1) {
            iterate(t, sc[0], sc[0], masked);
            ++t;
          }
          int i = t >> 1;
          for (; 2 * i + 1 < end; ++i) {
            iterate(2 * i, sc[0], sc[0], masked);
            iterate(2 * i + 1, sc[0], sc[0], masked);
          }
          t = 2 * i;
        }
      }
      for (; t < end; ++t) iterate(t, sc[0], sc[0], masked);
    }
    return t;
  };
  int t = run(t_lo, t_in_lo, std::true_type{});
  t = run(t, t_in_hi, std::false_type{});
  run(t, t_hi, std::true_type{});

  // Epilogue: O = z / l in the input type, LSE = m + ln l (natural log).
  const float l_tot = halves_sum(l_run);
  if (qrow < n) {
    const float inv = (DROP ? dp.inv_keep : 1.0f) / l_tot;
    char* orow = reinterpret_cast<char*>(O + (head + qrow) * D);
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = 32 * ob + 8 * g + 4 * h;
        if (a0 < D) {
          if constexpr (C::S == 2) {
            u32x2 w = {Elt<T>::pack2(o[ob][4 * g] * inv, o[ob][4 * g + 1] * inv),
                       Elt<T>::pack2(o[ob][4 * g + 2] * inv, o[ob][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + a0 * C::S) = w;
          } else {
            f32x4 w = {o[ob][4 * g] * inv, o[ob][4 * g + 1] * inv, o[ob][4 * g + 2] * inv,
                       o[ob][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + a0 * C::S) = w;
          }
        }
      }
    if (h == 0) LSE[head + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
  }
#ifdef EIAT_WG_TIMING
  __syncthreads();
  if (tid == 0) wg_stamps.store(g_wg_times, bid);
#endif
}

template <typename T, int D, int MASK, bool DROP, int F8>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdCfg<T, D, F8>;
  const int num_qtiles = (int)((a.n + C::BM - 1) / C::BM);
  const int64_t blocks = (int64_t)num_qtiles * a.bh;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, MASK, DROP, F8>), dim3((unsigned)blocks),
                     dim3(C::kThreads), 0, a.stream, a.q, a.k, static_cast<const T*>(a.v),
                     static_cast<T*>(a.o), a.lse, (int)a.n, (int)a.bh, num_qtiles, (int)a.window,
                     a.qk_scale, a.qmode, a.drop, a.qscale, a.kscale, a.vscale);
  return hipGetLastError();
}

template <typename T, int D, int MASK>
static hipError_t launch_fwd_m(const FwdArgs& a) {
  if constexpr (D >= 64 && Elt<T>::kBytes == 2) {
    if (a.vscale) return launch_fwd_t<T, D, MASK, false, 2>(a);
    if (a.qscale) return launch_fwd_t<T, D, MASK, false, 1>(a);
  }
  return a.drop.thr > 0 ? launch_fwd_t<T, D, MASK, true, 0>(a)
                        : launch_fwd_t<T, D, MASK, false, 0>(a);
}

template <typename T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a) {
  switch (a.mask) {
    case 0: return launch_fwd_m<T, D, 0>(a);
    case 1: return launch_fwd_m<T, D, 1>(a);
    default: return launch_fwd_m<T, D, 2>(a);
  }
}

template <typename T>
static hipError_t launch_fwd_dt(const FwdArgs& a) {
  switch (a.d) {
    case 16: return launch_fwd_d<T, 16>(a);
    case 64: return launch_fwd_d<T, 64>(a);
    default: return launch_fwd_d<T, 128>(a);
  }
}

#ifdef EIAT_WG_TIMING
// Copies the stamps of the last forward launch (6 words per workgroup: wall
// clock at start, after the prologue and at the end, hardware ids, shader
// clock at start and end; workgroups 0 .. min(grid, 65536) - 1) to host memory
// `dst` and the wall clock's rate in kHz to *clock_khz.  Returns a hipError_t
// code.
extern "C" __attribute__((visibility("default"))) int eiat_wg_times(void* dst, size_t bytes,
                                                                    int* clock_khz) {
  return wg_times_copy(HIP_SYMBOL(g_wg_times), sizeof(g_wg_times), dst, bytes, clock_khz);
}
#endif

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.dtype) {
    case 0: return launch_fwd_dt<float>(a);
    case 1: return launch_fwd_dt<_Float16>(a);
    default: return launch_fwd_dt<__bf16>(a);
  }
}

}  // namespace eiat
