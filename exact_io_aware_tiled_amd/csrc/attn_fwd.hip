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
// sum are in-lane, plus one swap of the two half-waves.  Key/value tiles of
// BN = 64 keys stream through LDS, double-buffered: K row-major, V transposed
// (V^T, keys contiguous) so that both feed the MFMA without per-element LDS
// reads.  P = 2^(s*c*log2(e) - m) is rounded to the input type in registers and
// used directly as the B operand of O^T += V^T P^T (no LDS round trip).  Only O
// and LSE = m + ln l go to HBM; no score block ever leaves the registers.
// Blocks with no allowed key are not visited (causal / window tile ranges) and
// the per-element mask is applied only in blocks that straddle a boundary.
#include "attn_device.h"
#include "attn_internal.h"

namespace eiat {

template <typename T, int D>
struct FwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * kWaves;      // query rows per workgroup
  static constexpr int BN = 64;               // keys per tile
  static constexpr int DP = D < 32 ? 32 : D;  // value rows padded to whole 32-row blocks
  static constexpr int S = Elt<T>::kBytes;
  static constexpr int KROW = D * S + 16;     // K tile row stride in LDS (bytes), padded
  static constexpr int VROW = BN * S + 16;    // V^T tile row stride in LDS (bytes), padded
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = DP * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int NCH = D * S / 32;      // d-chunks per 32x32 product (both halves)
  static constexpr int NOB = DP / 32;         // 32-row blocks of O^T
  static constexpr int NSB = BN / 32;         // 32-key blocks of S^T
  static constexpr int CPR = D * S / 16;      // 16-byte chunks per K / V row
  static constexpr int KCHUNKS = BN * CPR;
  static constexpr int VTASKS = (BN / 4) * CPR;  // 4 keys x 16 bytes each
  static constexpr int KPT = (KCHUNKS + kThreads - 1) / kThreads;
  static constexpr int VPT = (VTASKS + kThreads - 1) / kThreads;
  static constexpr int EPC = 16 / S;          // elements per 16-byte chunk
};

template <typename T, int D, int MASK>
__global__ void __launch_bounds__(256) attn_fwd_kernel(const T* __restrict__ Q,
                                                       const T* __restrict__ K,
                                                       const T* __restrict__ V,
                                                       T* __restrict__ O, float* __restrict__ LSE,
                                                       int n, int bh_count, int num_qtiles,
                                                       int window, float qk_scale, int qmode) {
  using C = FwdCfg<T, D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Consecutive workgroups take consecutive heads of the same query-tile rank;
  // with masks, the heaviest query tiles (most visible keys) are issued first.
  const int bid = blockIdx.x;
  const int bh = bid % bh_count;
  int qt = bid / bh_count;
  if (MASK != 0) qt = num_qtiles - 1 - qt;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;

  const int64_t head = (int64_t)bh * n;
  const char* Qh = reinterpret_cast<const char*>(Q + head * D);
  const char* Kh = reinterpret_cast<const char*>(K + head * D);
  const char* Vh = reinterpret_cast<const char*>(V + head * D);

  // Key range any row of this workgroup may see; whole tiles outside it are skipped.
  int kend = n;
  if (MASK != 0) kend = min(n, q0 + C::BM);
  int kbeg = 0;
  if (MASK == 2) kbeg = max(0, q0 - window + 1);
  const int t_lo = kbeg / BN;
  const int t_hi = (kend + BN - 1) / BN;

  // This wave's query rows as MFMA B-operand chunks: lane L holds row qw0 + L%32,
  // d-bytes [32c + 16h, 32c + 16h + 16).  The sign of c is folded into Q
  // (qmode 1), and c = 0 is taken as Q = 0 with a unit exponent scale (qmode 2).
  u32x4 qf[C::NCH];
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    qf[c] = qrow < n ? ldg16(Qh + (int64_t)qrow * D * C::S + 32 * c + 16 * h) : zero4();
    if (qmode == 1) qf[c] ^= Elt<T>::kSign;
    if (qmode == 2) qf[c] = zero4();
  }

  // Value rows beyond D (only for D < 32) stay zero in both buffers.
  if constexpr (C::DP > D) {
    for (int idx = tid; idx < 2 * (C::DP - D) * (C::VROW / 16); idx += C::kThreads) {
      int b = idx / ((C::DP - D) * (C::VROW / 16));
      int rem = idx % ((C::DP - D) * (C::VROW / 16));
      int row = D + rem / (C::VROW / 16);
      int col = rem % (C::VROW / 16);
      *reinterpret_cast<u32x4*>(smem + b * C::BUF + C::KBYTES + row * C::VROW + col * 16) = zero4();
    }
  }

  u32x4 kreg[C::KPT];
  u32x4 vreg[C::VPT][4];

  auto load_tile = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      const int c = tid + r * C::kThreads;
      if (c < C::KCHUNKS) {
        const int key = c / C::CPR, col = c % C::CPR;
        const int j = j0 + key;
        kreg[r] = j < n ? ldg16(Kh + (int64_t)j * D * C::S + col * 16) : zero4();
      }
    }
#pragma unroll
    for (int r = 0; r < C::VPT; ++r) {
      const int task = tid + r * C::kThreads;
      if (task < C::VTASKS) {
        const int kq = task / C::CPR, col = task % C::CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 4 * kq + i;
          vreg[r][i] = j < n ? ldg16(Vh + (int64_t)j * D * C::S + col * 16) : zero4();
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* kb = smem + buf * C::BUF;
    char* vb = kb + C::KBYTES;
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      const int c = tid + r * C::kThreads;
      if (c < C::KCHUNKS) {
        const int key = c / C::CPR, col = c % C::CPR;
        *reinterpret_cast<u32x4*>(kb + key * C::KROW + col * 16) = kreg[r];
      }
    }
#pragma unroll
    for (int r = 0; r < C::VPT; ++r) {
      const int task = tid + r * C::kThreads;
      if (task < C::VTASKS) {
        const int kq = task / C::CPR, col = task % C::CPR;
        store_transposed4<T>(vb + (col * C::EPC) * C::VROW + 4 * kq * C::S, C::VROW, vreg[r]);
      }
    }
  };

  // Running summary of this lane's query row (both half-waves keep identical m;
  // each keeps a partial l over its own keys; the partials are added at the end).
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x16 o[C::NOB];
#pragma unroll
  for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[ob][e] = 0.0f;

  load_tile(t_lo);
  store_tile(0);
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);

    const int j0 = t * BN;
    // The Algorithm's empty-block skip at wave granularity.
    bool empty = false;
    if (MASK != 0) empty = j0 > qw0 + 31;
    if (MASK == 2) empty = empty || (j0 + BN - 1 < qw0 - window + 1);

    if (!empty) {
      const char* kb = smem + buf * C::BUF;
      const char* vb = kb + C::KBYTES;

      // S^T block = K_tile Q_w^T (fp32 accumulate)
      f32x16 s[C::NSB];
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[sb][e] = 0.0f;
#pragma unroll
        for (int c = 0; c < C::NCH; ++c) {
          u32x4 a = *reinterpret_cast<const u32x4*>(kb + (32 * sb + l32) * C::KROW + 32 * c + 16 * h);
          s[sb] = Elt<T>::mma(a, qf[c], s[sb]);
        }
      }

      // Per-element mask only where the tile straddles a boundary.
      bool straddle = j0 + BN > n;
      if (MASK != 0) straddle = straddle || (j0 + BN - 1 > qw0);
      if (MASK == 2) straddle = straddle || (j0 < qw0 + 31 - window + 1);
      if (straddle) {
#pragma unroll
        for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = j0 + 32 * sb + 8 * (e >> 2) + 4 * h + (e & 3);
            if (!key_allowed<MASK>(qrow, j, n, window)) s[sb][e] = -INFINITY;
          }
      }

      // Block maximum of this row, in units of log2 (c * log2(e) folded in).
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[sb][e]);
      mx = fmaxf(mx, wave_swap_halves(mx));
      const float m_blk = (mx == -INFINITY) ? -INFINITY : mx * qk_scale;
      const float m_new = fmaxf(m_run, m_blk);
      // A row with no allowed key so far keeps the empty summary: shift by 0.
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      float rsum = 0.0f;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[sb][e], qk_scale, -m_use));
          s[sb][e] = p;
          rsum += p;
        }
      l_run = l_run * alpha + rsum;
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) o[ob] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        PChunks<T> pc;
        pc.set(s[sb]);
#pragma unroll
        for (int ob = 0; ob < C::NOB; ++ob) {
          const char* vrow = vb + (32 * ob + l32) * C::VROW + 32 * sb * C::S;
#pragma unroll
          for (int ci = 0; ci < PChunks<T>::kCount; ++ci)
            o[ob] = Elt<T>::mma(keyrow_chunk<T>(vrow, ci, h), pc.c[ci], o[ob]);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = z / l in the input type, LSE = m + ln l (natural log).
  const float l_tot = l_run + wave_swap_halves(l_run);
  if (qrow < n) {
    const float inv = 1.0f / l_tot;
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
}

template <typename T, int D, int MASK>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdCfg<T, D>;
  const int num_qtiles = (int)((a.n + C::BM - 1) / C::BM);
  const int64_t blocks = (int64_t)num_qtiles * a.bh;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, MASK>), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                     a.stream, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, (int)a.n, (int)a.bh,
                     num_qtiles, (int)a.window, a.qk_scale, a.qmode);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a) {
  switch (a.mask) {
    case 0: return launch_fwd_t<T, D, 0>(a);
    case 1: return launch_fwd_t<T, D, 1>(a);
    default: return launch_fwd_t<T, D, 2>(a);
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

hipError_t launch_fwd(const FwdArgs& a) {
  switch (a.dtype) {
    case 0: return launch_fwd_dt<float>(a);
    case 1: return launch_fwd_dt<_Float16>(a);
    default: return launch_fwd_dt<__bf16>(a);
  }
}

int64_t fwd_max_blocks_per_bh(int64_t n) { return (n + FwdCfg<float, 64>::BM - 1) / FwdCfg<float, 64>::BM; }

}  // namespace eiat
