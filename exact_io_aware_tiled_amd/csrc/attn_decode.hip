// attn_decode.hip -- decode-shaped forward for gfx950: a few new query rows per
// head against a long cache of keys and values, split over the cache.
//
// The setting is the KV cache of webturing.com.tr Principia, "Bellek Duvarinin
// Fizigi", section on the KV cache and long context: every new token attends to
// the cached keys and values of all earlier tokens, and at inference that cache
// is the memory object that streams from HBM ("The Arithmetic of
// Intelligence", ch. 12, on decoding being memory-bound and on verifying
// several new positions in one pass).  The new rows are the last nq positions
// of the sequence: row i sits at position nk - nq + i and sees the mask's key
// set for that position.  H query heads share Hkv key/value heads (query head h
// reads key/value head h / (H / Hkv)), so the G = H / Hkv heads of a group and
// their nq rows, M = G * nq <= 32 rows in all, are served by one pass over the
// group's keys and values.
//
// The arithmetic is that of alphabetamath.cc, "Exact tiled attention and
// memory-aware differentiation": each workgroup forms the stable summary
// (m, l, z) of one contiguous range of the cache (Definition "Stable summary of
// an attention key block", accumulated tile by tile with the streaming update
// of "The Arithmetic of Intelligence", ch. 12, "Streaming softmax"), and a
// second kernel merges the ranges' summaries with the Definition's merge and
// finishes O = z / l, LSE = m + ln l.  The merge is associative, so the result
// does not depend on how the cache is split.
//
// Mapping to CDNA4.  The traffic is the cache itself (Q, O and the partial
// summaries are small), so the split kernel is built to keep HBM busy: one wave
// per workgroup, each with a private ring of LDS stages fed by direct
// HBM -> LDS loads (no barriers: the wave waits on its own vector-memory count
// for the stage it needs next), and enough ranges that every CU holds several
// such waves.  The M query rows sit in registers as the B operand of
// S^T = K Q^T (lane = row, so row max and sum stay in-lane), K rows are read
// from LDS as the A operand and V through ds_read_b64_tr_b16 for
// O^T += V^T P^T, as in the prefill forward.
#include "attn_device.h"
#include "attn_internal.h"

namespace eiat {

template <typename T, int D>
struct DecCfg {
  static constexpr int S = 2;                      // bytes per element (16-bit inputs)
  static constexpr int BN = 32;                    // keys per tile
  static constexpr int CPR = D * S / 16;           // 16-byte chunks per K / V row
  static constexpr int ROW = D * S + 16;           // padded LDS row stride (bytes)
  static constexpr int TILE = BN * ROW;            // one K or V tile in LDS
  static constexpr int NSTAGE = D >= 128 ? 2 : 4;  // ring depth: ~35 KiB of LDS per wave
  static constexpr int SMEM = NSTAGE * 2 * TILE;
  static constexpr int NCH = D * S / 32;           // d-chunks per 32x32 product
  static constexpr int NOB = D / 32;               // 32-row blocks of O^T
  using Loader = TileLoader<BN, CPR, 1>;
  static constexpr int PER_STAGE = 2 * Loader::kInstr;  // direct loads per stage (K + V)
  static constexpr float kTau = 8.0f;              // lazy-rescale threshold, base-2 units
  static_assert(PER_STAGE * (NSTAGE - 1) <= 63, "vector-memory count field is 6 bits");
};

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `pending` stages (issued after the one needed) are in flight.
template <typename C>
__device__ inline void wait_stages(int pending) {
  static_assert(C::NSTAGE <= 4, "extend the switch");
  switch (pending) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<C::PER_STAGE>(); break;
    case 2: wait_vmcnt<(C::NSTAGE > 2 ? 2 : 0) * C::PER_STAGE>(); break;
    default: wait_vmcnt<(C::NSTAGE > 3 ? 3 : 0) * C::PER_STAGE>(); break;
  }
}

// Summary of one range of the cache for the M rows of one (batch, key/value
// head).  Partial outputs: z [units][nsplit][M][D] and (m, l) [units][nsplit][M],
// with m in base-2 units of the scaled scores (-inf and l = 0 for a row with no
// allowed key in the range).
template <typename T, int D, int MASK>
__global__ void __launch_bounds__(64)
    attn_decode_split_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                             const T* __restrict__ V, float* __restrict__ zpart,
                             float2* __restrict__ mlpart, int H, int Hkv, int nq, int nk, int M,
                             int nsplit, int window, float qk_scale, int qmode) {
  using C = DecCfg<T, D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];

  const int lane = threadIdx.x;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // Consecutive workgroups take consecutive ranges of one (batch, key/value
  // head), so the workgroups resident at once stream neighbouring memory.
  const int unit = blockIdx.x / nsplit;
  const int split = blockIdx.x % nsplit;
  const int b = unit / Hkv, hk = unit % Hkv;
  const int G = H / Hkv;

  // This lane's row r (lanes r >= M repeat row 0; never stored): query head
  // hk * G + r / nq, new row r % nq at position nk - nq + r % nq.
  const int r = l32 < M ? l32 : 0;
  const int hq = hk * G + r / nq, qi = r % nq;
  const int pos = nk - nq + qi;
  const char* Qr = reinterpret_cast<const char*>(Q + (((int64_t)b * H + hq) * nq + qi) * D);
  const char* Kh = reinterpret_cast<const char*>(K + (int64_t)unit * nk * D);
  const char* Vh = reinterpret_cast<const char*>(V + (int64_t)unit * nk * D);

  // Keys any of the rows may see, as 32-key tiles, divided evenly among the splits.
  int kb = 0;
  if (MASK == 2) kb = max(0, nk - nq - window + 1);
  const int tb = kb / BN, te = (nk + BN - 1) / BN;
  const int per = (te - tb + nsplit - 1) / nsplit;
  const int t0 = tb + split * per;
  const int t1 = min(te, t0 + per);

  u32x4 qf[C::NCH];
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    qf[c] = ldg16(Qr + 32 * c + 16 * h);
    if (qmode == 1) qf[c] ^= Elt<T>::kSign;
    if (qmode == 2) qf[c] = zero4();
  }

  typename C::Loader tl;
  tl.init(0, lane);
  auto kslot = [&](int s) __attribute__((always_inline)) -> char* { return smem + s * 2 * C::TILE; };
  auto issue = [&](int t, int s) __attribute__((always_inline)) {
    tl.load(kslot(s), Kh, t * BN, nk, 0, lane);
    tl.load(kslot(s) + C::TILE, Vh, t * BN, nk, 0, lane);
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[C::NOB];
#pragma unroll
  for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[ob][e] = 0.0f;

#pragma unroll
  for (int s = 0; s < C::NSTAGE - 1; ++s)
    if (t0 + s < t1) issue(t0 + s, s);

  for (int t = t0; t < t1; ++t) {
    const int u = t - t0;
    // The slot refilled below held tile t - 1: its LDS reads are complete.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t + C::NSTAGE - 1 < t1) issue(t + C::NSTAGE - 1, (u + C::NSTAGE - 1) % C::NSTAGE);
    wait_stages<C>(min(C::NSTAGE - 1, t1 - 1 - t));
    const char* kt = kslot(u % C::NSTAGE);
    const char* vt = kt + C::TILE;

    // S^T = K_t Q^T: lane = row, 16 keys per half-wave
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.0f;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
      sc = Elt<T>::mma(*reinterpret_cast<const u32x4*>(kt + l32 * C::ROW + 32 * c + 16 * h),
                       qf[c], sc);

    // Per-element mask only where some key of the tile is out of some row's set.
    const int j0 = t * BN;
    bool straddle = j0 + BN > nk;
    if (MASK != 0) straddle = straddle || (j0 + BN - 1 > nk - nq);
    if (MASK == 2) straddle = straddle || (j0 < nk - window);
    if (straddle) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (!key_allowed<MASK>(pos, j, nk, window)) sc[e] = -INFINITY;
      }
    }

    // Streaming update with the lazily raised shift (as in the prefill forward).
    f32x16 sl[1] = {sc};
    const float mx = halves_max(tile_max<1>(sl));
    const float m_blk = (mx == -INFINITY) ? -INFINITY : mx * qk_scale;
    if (wave_any(m_blk > m_run + C::kTau)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) o[ob] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = fast_exp2(__builtin_fmaf(sc[e], qk_scale, -m_use));
    PChunks<T> pc;
    pc.set(sc);
    l_run = chunk_sum<T>(pc, sc, l_run);
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
      for (int ci = 0; ci < PChunks<T>::kCount; ++ci)
        o[ob] = Elt<T>::mma(tr_chunk(vt, C::ROW, 0, ob, ci, lane), pc.c[ci], o[ob]);
  }

  const float l_tot = halves_sum(l_run);
  if (l32 < M) {
    const int64_t prow = ((int64_t)unit * nsplit + split) * M + l32;
    float* zr = zpart + prow * D;
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = 32 * ob + 8 * g + 4 * h;
        *reinterpret_cast<f32x4*>(zr + a0) =
            f32x4{o[ob][4 * g], o[ob][4 * g + 1], o[ob][4 * g + 2], o[ob][4 * g + 3]};
      }
    if (h == 0) mlpart[prow] = make_float2(m_run, l_tot);
  }
}

// Merge the nsplit range summaries of one output row with the Definition's
// merge.  The merge is associative and commutative, so it is taken in one
// step: m = max_s m_s, weights w_s = 2^(m_s - m) (0 for a range with no allowed
// key), l = sum_s w_s l_s, z = sum_s w_s z_s; then O = z / l and
// LSE = (m + log2 l) ln 2.  One workgroup of four waves per row of O: all
// threads share the ranges for m, the weights (kept in LDS) and l; each wave
// sums every output column over a quarter of the ranges (independent loads),
// and the four partial sums are added in LDS.
constexpr int kMaxSplits = 2048;
constexpr int kMergeWaves = 4;

template <typename T, int D>
__global__ void __launch_bounds__(64 * kMergeWaves)
    attn_decode_combine_kernel(const float* __restrict__ zpart, const float2* __restrict__ mlpart,
                               T* __restrict__ O, float* __restrict__ LSE, int H, int Hkv, int nq,
                               int M, int nsplit) {
  constexpr int CPL = D / 64;  // output columns per lane
  constexpr int NT = 64 * kMergeWaves;
  __shared__ float wsh[kMaxSplits];
  __shared__ float zsh[kMergeWaves][D];
  __shared__ float red[2][kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;  // ((b * H + hq) * nq + i): the row of O and LSE
  const int i = row % nq, bh = row / nq;
  const int hq = bh % H, b = bh / H;
  const int G = H / Hkv;
  const int unit = b * Hkv + hq / G;
  const int r = (hq % G) * nq + i;
  const int64_t base = (int64_t)unit * nsplit * M + r;  // summary row of range s: base + s * M

  float m = -INFINITY;
  for (int s = tid; s < nsplit; s += NT) m = fmaxf(m, mlpart[base + (int64_t)s * M].x);
  m = wave_max(m);
  if (lane == 0) red[0][wave] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) m = fmaxf(m, red[0][w]);
  float l = 0.0f;
  for (int s = tid; s < nsplit; s += NT) {
    const float2 ml = mlpart[base + (int64_t)s * M];
    const float w = (ml.x == -INFINITY) ? 0.0f : fast_exp2(ml.x - m);
    wsh[s] = w;
    l += w * ml.y;
  }
  l = wave_sum(l);
  if (lane == 0) red[1][wave] = l;
  __syncthreads();

  float z[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) z[k] = 0.0f;
  const float* zr = zpart + base * D + lane * CPL;
#pragma unroll 8
  for (int s = wave; s < nsplit; s += kMergeWaves) {
    const float w = wsh[s];
    const float* zs = zr + (int64_t)s * M * D;
#pragma unroll
    for (int k = 0; k < CPL; ++k) z[k] += w * zs[k];
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k) zsh[wave][lane * CPL + k] = z[k];
  __syncthreads();
  if (wave != 0) return;
  l = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) l += red[1][w];
  const float inv = 1.0f / l;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) acc += zsh[w][lane * CPL + k];
    z[k] = acc * inv;
  }
  T* orow = O + (int64_t)row * D + lane * CPL;
  if constexpr (CPL == 2) {
    *reinterpret_cast<uint32_t*>(orow) = Elt<T>::pack2(z[0], z[1]);
  } else {
    orow[0] = static_cast<T>(z[0]);
  }
  if (lane == 0) LSE[row] = (m + fast_log2(l)) * kLn2;
}

// Number of cache ranges per (batch, key/value head): enough ranges that the
// whole launch has about 2048 single-wave workgroups (several per CU), at most
// one per 32-key tile, and no empty range.
int decode_splits(int64_t units, int64_t nk) {
  if (units <= 0 || nk <= 0) return 1;
  const int64_t tiles = (nk + 31) / 32;
  int64_t s = (2048 + units - 1) / units;
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  const int64_t per = (tiles + s - 1) / s;
  return (int)((tiles + per - 1) / per);
}

template <typename T, int D, int MASK>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int units = (int)(a.B * a.Hkv);
  const int M = (int)(a.H / a.Hkv * a.nq);
  float* zpart = a.workspace;
  float2* mlpart = reinterpret_cast<float2*>(a.workspace + (int64_t)units * a.nsplit * M * D);
  if (a.stages & 1) {
    hipLaunchKernelGGL((attn_decode_split_kernel<T, D, MASK>),
                       dim3((unsigned)(units * a.nsplit)), dim3(64), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), zpart, mlpart, (int)a.H, (int)a.Hkv, (int)a.nq,
                       (int)a.nk, M, a.nsplit, (int)a.window, a.qk_scale, a.qmode);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.stages & 2) {
    hipLaunchKernelGGL((attn_decode_combine_kernel<T, D>), dim3((unsigned)(a.B * a.H * a.nq)),
                       dim3(64 * kMergeWaves), 0, a.stream, zpart, mlpart, static_cast<T*>(a.o), a.lse,
                       (int)a.H, (int)a.Hkv, (int)a.nq, M, a.nsplit);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  switch (a.mask) {
    case 0: return launch_decode_t<T, D, 0>(a);
    case 1: return launch_decode_t<T, D, 1>(a);
    default: return launch_decode_t<T, D, 2>(a);
  }
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
  return a.d == 64 ? launch_decode_d<T, 64>(a) : launch_decode_d<T, 128>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 1 ? launch_decode_dt<_Float16>(a) : launch_decode_dt<__bf16>(a);
}

}  // namespace eiat
