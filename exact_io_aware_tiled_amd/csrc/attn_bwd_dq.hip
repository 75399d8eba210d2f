// attn_bwd_dq.hip -- the dQ kernel of the backward pass, for gfx950.
//
// Follows alphabetamath.cc, "Exact tiled attention and memory-aware
// differentiation", the Algorithm's reverse procedure: with the forward's row
// statistics frozen (LSE_i = m_i + ln l_i, so p_ij = e^{s_ij - LSE_i}), a
// workgroup keeps 128 query rows (Q, dO, LSE and delta_i = sum_a dO_ia O_ia,
// which it forms and writes for the dK/dV kernel) in registers and streams the
// key/value tiles those rows may see through LDS, recomputing each score
// block: gamma_ij = p_ij (sum_a G_ia V_ja - delta_i), dQ_i = c sum_j gamma_ij K_j.
// No atomics: every dQ row is owned by one wave.
//
// Its own translation unit (apart from attn_bwd.hip, with the helpers both
// share in attn_bwd_common.h), so the two backward kernels compile in parallel
// and each can take its own scheduler flags (build.py).
#include "attn_bwd_common.h"
#include "attn_internal.h"

namespace eiat {

// ---------------------------------------------------------------------------
// 3. dQ: queries resident, key/value tiles streamed
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * kWaves;
  static constexpr int S = Elt<T>::kBytes;
  // keys per streamed tile (the tile-shape check build: 32 for 16-bit types)
  static constexpr int BN = ((S == 4 && D >= 128) || (S == 2 && kAltTiles)) ? 32 : 64;
  // d = 16 runs three waves per SIMD (the float32 kernels sat two registers
  // above the three-wave budget otherwise).
  static constexpr int kMinWaves = D == 16 ? 3 : 1;
  static constexpr int DP = D < 32 ? 32 : D;
  // 16-bit: the K^T operand comes from the natural K tile through transpose
  // reads; float32 keeps a transposed copy.
  static constexpr bool kTr = (S == 2);
  static constexpr bool kDirect = kTr && D >= 32;
  // LDS bank conflicts of the K and V tiles: swizzled unpadded rows at 16-bit
  // d = 64 and 128, one padding slot otherwise (as the forward's tiles,
  // attn_fwd.hip).
  static constexpr bool kSwz = kDirect && D >= 64;
  static constexpr int PAD = kSwz ? 0 : 1;
  static constexpr int NROW = (kTr ? DP : D) * S + 16 * PAD;  // K, V natural rows
  static constexpr int TROW = BN * S + 16;              // K^T rows (float32)
  static constexpr int KN = 0;
  static constexpr int KT = KN + BN * NROW;
  static constexpr int VN = KT + (kTr ? 0 : DP * TROW);
  static constexpr int BUF = VN + BN * NROW;
  static constexpr int NCH = D * S / 32;
  static constexpr int NOB = DP / 32;
  static constexpr int NSB = BN / 32;
};

#ifdef EIAT_WG_TIMING
// Timing check build: per-workgroup stamps of dQ (WgStamps; the prologue ends
// when the first key/value tile is in LDS).  Read with eiat_wg_times_dq.
__device__ unsigned long long g_wg_times_dq[kWgTimingWords * kWgTimingMax];
#endif

template <typename T, int D, int MASK, bool DROP>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(DqCfg<T, D>::kMinWaves, 8))) attn_bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const T* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ delta, T* __restrict__ dQ, int n, int bh_count, int num_qtiles,
    int window, float qk_scale, int qmode, float scale, DropParams dpar) {
  using C = DqCfg<T, D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];
  using StK = Stager<T, D, BN, C::kThreads, C::NROW, C::TROW, true, !C::kTr>;
  using StV = Stager<T, D, BN, C::kThreads, C::NROW, C::TROW, true, false>;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
#ifdef EIAT_WG_TIMING
  WgStamps wg_stamps;
  wg_stamps.begin();
#endif
  const int bh = bid % bh_count;
  int qt = bid / bh_count;
  if (MASK != 0) qt = num_qtiles - 1 - qt;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;

  const int64_t head = (int64_t)bh * n;
  const char* Qh = reinterpret_cast<const char*>(Q + head * D);
  const char* Kh = reinterpret_cast<const char*>(K + head * D);
  const char* Vh = reinterpret_cast<const char*>(V + head * D);
  const char* dOh = reinterpret_cast<const char*>(dO + head * D);

  // This row's Q and dO as B-operand chunks, and its O for delta.  Rows past n
  // read row n - 1: their weights are 0 (LSE taken as +inf) and their dQ and
  // delta are not stored.  The loads are issued here, with the first key /
  // value tile's below, and used only after those are issued, since an
  // operation on a loaded value waits for it (and for every load before it).
  u32x4 qf[C::NCH], of[C::NCH], oc[C::NCH];
  const int qr = min(qrow, n - 1);
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    qf[c] = ldg16(Qh + (int64_t)qr * D * C::S + 32 * c + 16 * h);
    of[c] = ldg16(dOh + (int64_t)qr * D * C::S + 32 * c + 16 * h);
    oc[c] = ldg16(reinterpret_cast<const char*>(O + head * D) + (int64_t)qr * D * C::S + 32 * c +
                  16 * h);
  }
  const float lse_row = LSE[head + qr];
  // Dropout (DROP): this row's key of the realized mask.
  const uint32_t row_key = DROP ? drop_row_key(dpar, (uint32_t)bh, (uint32_t)qrow) : 0u;

  int kend = n;
  if (MASK != 0) kend = min(n, q0 + C::BM);
  int kbeg = 0;
  if (MASK == 2) kbeg = max(0, q0 - window + 1);
  const int t_lo = kbeg / BN, t_hi = (kend + BN - 1) / BN;

  f32x16 dq[C::NOB];
#pragma unroll
  for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[ob][e] = 0.0f;

  for (int b = 0; b < 2; ++b) {
    if constexpr (C::kTr)
      zero_pad_cols<D, C::DP, C::S, BN, C::NROW, C::kThreads>(smem + b * C::BUF + C::KN, tid);
    else
      zero_pad_rows<D, C::DP, C::TROW, C::kThreads>(smem + b * C::BUF + C::KT, tid);
  }

  TileLoader<BN, D * C::S / 16, C::kWaves, C::PAD, C::kSwz> tl;
  if constexpr (C::kDirect) tl.init(wave, lane);
  SwzReads<D> swz;
  if constexpr (C::kSwz) swz.init(lane);
  StK sk;
  StV sv;
  auto load_tile = [&](int t) {
    if constexpr (C::kDirect) {
      char* b = smem + ((t - t_lo) & 1) * C::BUF;
      tl.load(b + C::KN, Kh, t * BN, n, wave, lane);
      tl.load(b + C::VN, Vh, t * BN, n, wave, lane);
    } else {
      sk.load(Kh, t * BN, n, tid);
      sv.load(Vh, t * BN, n, tid);
    }
  };
  auto store_tile = [&](int buf) {
    if constexpr (C::kDirect) {
      wait_tile_loads();
    } else {
      char* b = smem + buf * C::BUF;
      sk.store(b + C::KN, b + C::KT, tid);
      sv.store(b + C::VN, nullptr, tid);
    }
  };

  load_tile(t_lo);
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    if (qmode == 1) qf[c] ^= Elt<T>::kSign;
    if (qmode == 2) qf[c] = zero4();  // c = 0: every score is exactly 0
  }
  const float lse2 = qrow < n ? lse_row * kLog2e : INFINITY;
  // delta of this row from its O and dO chunks (unit 2c + h of the row is
  // chunk c of half h), summed in unit_dot's tree; written out for the dK/dV
  // kernel.
  float dlt;
  {
    float u[C::NCH];
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) u[c] = unit_dot<T>(oc[c], of[c]);
#pragma unroll
    for (int off = C::NCH / 2; off > 0; off >>= 1)
#pragma unroll
      for (int c = 0; c < off; ++c) u[c] += u[c + off];
    dlt = u[0] + __shfl_xor(u[0], 32, 64);
    if (qrow >= n) dlt = 0.0f;
    else if (h == 0) delta[head + qrow] = dlt;
  }
  store_tile(0);
  __syncthreads();
#ifdef EIAT_WG_TIMING
  wg_stamps.prologue_done();
#endif

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);
    const int j0 = t * BN;
    bool empty = false;
    if (MASK != 0) empty = j0 > qw0 + 31;
    if (MASK == 2) empty = empty || (j0 + BN - 1 < qw0 - window + 1);
    if (!empty) {
      const char* b = smem + buf * C::BUF;
      bool straddle = j0 + BN > n;
      if (MASK != 0) straddle = straddle || (j0 + BN - 1 > qw0);
      if (MASK == 2) straddle = straddle || (j0 < qw0 + 31 - window + 1);
      // S^T = K Q^T and dP^T = V dO^T for key block sb: lane holds one query
      // row, 16 keys per half (without dropout dP^T starts at -delta of the
      // lane's row, so dS = p (dP - delta) needs no subtraction afterwards)
      auto sdp = [&](int sb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.0f;
        dp[e] = DROP ? 0.0f : -dlt;
      }
      const int rk = 32 * sb + l32;
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        u32x4 ka, va;
        if constexpr (C::kSwz) {
          ka = swz.row_read(b + C::KN, 32 * sb, c);
          va = swz.row_read(b + C::VN, 32 * sb, c);
        } else {
          ka = *reinterpret_cast<const u32x4*>(b + C::KN + rk * C::NROW + 32 * c + 16 * h);
          va = *reinterpret_cast<const u32x4*>(b + C::VN + rk * C::NROW + 32 * c + 16 * h);
        }
        s = Elt<T>::mma(ka, qf[c], s);
        dp = Elt<T>::mma(va, of[c], dp);
      }
      };
      // mask, P, dS = P (dP - delta), dQ^T += K^T dS^T for key block sb
      auto rest = [&](int sb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
      if (straddle) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = j0 + 32 * sb + 8 * (e >> 2) + 4 * h + (e & 3);
          if (!key_allowed<MASK>(qrow, j, n, window)) s[e] = -INFINITY;
        }
      }
      if constexpr (DROP) {
        const int jb = j0 + 32 * sb + 4 * h;  // key of element e = 0
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t bytes = drop_group_bytes(row_key, (uint32_t)(jb + 8 * k) >> 2);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * k + r;
            const float p = fast_exp2(__builtin_fmaf(s[e], qk_scale, -lse2));
            const bool keep = drop_keep(bytes, r, dpar.thr);
            dp[e] = p * ((keep ? dp[e] * dpar.inv_keep : 0.0f) - dlt);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[e], qk_scale, -lse2));
          dp[e] = p * dp[e];
        }
      }
      PChunks<T> dsc;
      dsc.set(dp);
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) {
#pragma unroll
        for (int ci = 0; ci < PChunks<T>::kCount; ++ci) {
          u32x4 ka2;
          if constexpr (C::kSwz)
            ka2 = swz.tr_read(b + C::KN, 32 * sb, ob, ci);
          else if constexpr (C::kTr)
            ka2 = tr_chunk(b + C::KN, C::NROW, 32 * sb, ob, ci, lane);
          else
            ka2 = keyrow_chunk<T>(b + C::KT + (32 * ob + l32) * C::TROW + 32 * sb * C::S, ci, h);
          dq[ob] = Elt<T>::mma(ka2, dsc.c[ci], dq[ob]);
        }
      }
      };
      // Raised wave priority over the exponentials and dQ products of a block
      // (16-bit d >= 64), so that they go ahead of the other wave's score
      // products: 6.5 % faster at d = 128 with the pipelined loop; at d = 16
      // 12 % slower and left out.
      constexpr bool kPrio = C::kTr && D >= 64;
      auto rest_prio = [&](int sb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
        rest(sb, s, dp);
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
      };
      // At 16-bit d >= 64 the block loop is software-pipelined: the S and dP
      // products of block sb + 1 are issued before the exponentials of block
      // sb.  At d = 128 the extra registers fit the two waves per SIMD (1-2 %
      // faster); at d = 64 they cost the third wave, which without the raised
      // priority above measured 4 % slower and with it 2-4 % faster.
      if constexpr (C::kTr && D >= 64 && C::NSB > 1) {
        f32x16 s[2], dp[2];
        sdp(0, s[0], dp[0]);
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) {
          // scheduling hint: interleave LDS operand reads with the MFMAs
          __builtin_amdgcn_iglp_opt(0);
          if (sb + 1 < C::NSB) sdp(sb + 1, s[(sb + 1) & 1], dp[(sb + 1) & 1]);
          rest_prio(sb, s[sb & 1], dp[sb & 1]);
        }
      } else {
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb) {
          // scheduling hint: interleave LDS operand reads with the MFMAs
          __builtin_amdgcn_iglp_opt(0);
          f32x16 s, dp;
          sdp(sb, s, dp);
          rest_prio(sb, s, dp);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qrow < n) {
    char* dqrow = reinterpret_cast<char*>(dQ + (head + qrow) * D);
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = 32 * ob + 8 * g + 4 * h;
        if (a0 < D) {
          if constexpr (C::S == 2) {
            u32x2 w = {Elt<T>::pack2(dq[ob][4 * g] * scale, dq[ob][4 * g + 1] * scale),
                       Elt<T>::pack2(dq[ob][4 * g + 2] * scale, dq[ob][4 * g + 3] * scale)};
            *reinterpret_cast<u32x2*>(dqrow + a0 * C::S) = w;
          } else {
            f32x4 w = {dq[ob][4 * g] * scale, dq[ob][4 * g + 1] * scale,
                       dq[ob][4 * g + 2] * scale, dq[ob][4 * g + 3] * scale};
            *reinterpret_cast<f32x4*>(dqrow + a0 * C::S) = w;
          }
        }
      }
  }
#ifdef EIAT_WG_TIMING
  __syncthreads();
  if (tid == 0) wg_stamps.store(g_wg_times_dq, bid);
#endif
}

#ifdef EIAT_WG_TIMING
// Copies the stamps of the last dQ launch (layout as eiat_wg_times) to host
// memory `dst` and the wall clock's rate in kHz to *clock_khz.  Returns a
// hipError_t code.
extern "C" __attribute__((visibility("default"))) int eiat_wg_times_dq(void* dst, size_t bytes,
                                                                       int* clock_khz) {
  return wg_times_copy(HIP_SYMBOL(g_wg_times_dq), sizeof(g_wg_times_dq), dst, bytes, clock_khz);
}
#endif

// ---------------------------------------------------------------------------
// dQ launch
// ---------------------------------------------------------------------------
template <typename T, int D, int MASK, bool DROP>
static hipError_t launch_dq_t(const BwdArgs& a) {
  using C = DqCfg<T, D>;
  const int num_qtiles = (int)((a.n + C::BM - 1) / C::BM);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, MASK, DROP>),
                     dim3((unsigned)(num_qtiles * a.bh)), dim3(C::kThreads), 0, a.stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.dout),
                     static_cast<const T*>(a.o), a.lse, a.delta, static_cast<T*>(a.dq),
                     (int)a.n, (int)a.bh, num_qtiles, (int)a.window, a.qk_scale, a.qmode,
                     a.scale, a.drop);
  return hipGetLastError();
}

template <typename T, int D, int MASK>
static hipError_t launch_dq_m(const BwdArgs& a) {
  return a.drop.thr > 0 ? launch_dq_t<T, D, MASK, true>(a) : launch_dq_t<T, D, MASK, false>(a);
}

template <typename T, int D>
static hipError_t launch_dq_d(const BwdArgs& a) {
  switch (a.mask) {
    case 0: return launch_dq_m<T, D, 0>(a);
    case 1: return launch_dq_m<T, D, 1>(a);
    default: return launch_dq_m<T, D, 2>(a);
  }
}

template <typename T>
static hipError_t launch_dq_dt(const BwdArgs& a) {
  switch (a.d) {
    case 16: return launch_dq_d<T, 16>(a);
    case 64: return launch_dq_d<T, 64>(a);
    default: return launch_dq_d<T, 128>(a);
  }
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  switch (a.dtype) {
    case 0: return launch_dq_dt<float>(a);
    case 1: return launch_dq_dt<_Float16>(a);
    default: return launch_dq_dt<__bf16>(a);
  }
}

}  // namespace eiat
