// attn_bwd.hip -- exact tiled softmax attention, backward pass, for gfx950.
//
// Follows alphabetamath.cc, "Exact tiled attention and memory-aware
// differentiation", the Algorithm's reverse procedure: with the forward's row
// statistics frozen (carried as LSE_i = m_i + ln l_i, so p_ij = e^{s_ij - LSE_i}),
//   delta_i  = sum_a G_ia Y_ia
//   gamma_ij = p_ij (sum_a G_ia V_ja - delta_i)
//   dQ_i += c gamma_ij K_j,  dK_j += c gamma_ij Q_i,  dV_j += p_ij G_i,
// recomputing every score block from Q, K instead of storing it (WebTuring
// Principia, "Bellek Duvarinin Fizigi", section on backpropagation by
// recomputation: P is rebuilt from the saved log-sum-exp).
//
// Three kernels, no atomics (deterministic):
//   1. delta: one fp32 per row from the stored O and dO (this file).
//   2. dK/dV: a workgroup keeps 128 keys of K and V in registers (32 per wave)
//      and streams the query tiles that may see them through LDS.  Scores are
//      formed as S = Q K^T so every lane holds one KEY column: P and dS then
//      feed dV^T += dO^T P and dK^T += Q^T dS straight from registers (this file).
//   3. dQ: a workgroup keeps 128 query rows (Q, dO, LSE, delta) in registers
//      and streams key/value tiles through LDS, as the forward does, with
//      dQ^T += K^T dS^T (attn_bwd_dq.hip, its own translation unit).
// The transposed operands (dO^T, Q^T, K^T) are read from the natural LDS tiles
// with ds_read_b64_tr_b16 for 16-bit types; float32 writes transposed copies
// while staging, from the same registers that hold the natural copies.
#include "attn_bwd_common.h"
#include "attn_internal.h"

namespace eiat {

// ---------------------------------------------------------------------------
// 1. delta_i = sum_a dO_ia O_ia
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_bwd_delta_kernel(const T* __restrict__ O,
                                                             const T* __restrict__ dO,
                                                             float* __restrict__ delta,
                                                             int64_t rows) {
  constexpr int S = Elt<T>::kBytes;
  constexpr int CPR = D * S / 16;  // threads (units) per row, a power of two <= 32
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / CPR;
  const int col = (int)(gt % CPR);
  float acc = 0.0f;
  if (row < rows)
    acc = unit_dot<T>(ldg16(reinterpret_cast<const char*>(O) + row * D * S + col * 16),
                      ldg16(reinterpret_cast<const char*>(dO) + row * D * S + col * 16));
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && col == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK / dV: keys resident, query tiles streamed
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkvCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BNK = 32 * kWaves;            // keys per workgroup
  // Query rows per streamed tile.  16-bit d <= 64 streams 128-row tiles: half
  // the barriers per query row and four 32-row blocks of independent MFMA work
  // per tile (8 % faster than 64 rows at d = 64; the LDS still fits two
  // workgroups per CU).  d = 128 keeps 32 rows so two workgroups fit with V in LDS.
  // (The tile-shape check build streams 64-row tiles at 16-bit d <= 64.)
  static constexpr int BMQ = D >= 128 ? 32 : (Elt<T>::kBytes == 2 && !kAltTiles ? 128 : 64);
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int S = Elt<T>::kBytes;
  // 16-bit: Q^T and dO^T operands come from the natural tiles through transpose
  // reads; float32 keeps transposed copies.
  static constexpr bool kTr = (S == 2);
  // LDS bank conflicts of the Q / dO tiles (and of the resident V rows):
  // swizzled unpadded rows at 16-bit d = 64 (as the forward's tiles,
  // attn_fwd.hip); at 16-bit d = 128, whose registers have no room for the
  // swizzle's per-lane offsets, rows padded by three 16-byte slots (16-byte
  // reads conflict-free, transposing reads 2-way); one slot otherwise.
  static constexpr bool kSwz = kTr && D == 64;
  static constexpr int PAD = kSwz ? 0 : ((kTr && D >= 128) ? 3 : 1);
  static constexpr int NROW = (kTr ? DP : D) * S + 16 * PAD;  // Q / dO natural rows
  static constexpr int TROW = BMQ * S + 16;             // Q^T / dO^T rows (float32)
  static constexpr int TBYTES = kTr ? 0 : DP * TROW;
  static constexpr int QN = 0;
  static constexpr int QT = QN + BMQ * NROW;
  static constexpr int ON = QT + TBYTES;
  static constexpr int OT = ON + BMQ * NROW;
  static constexpr int LS = OT + TBYTES;             // LSE * log2(e), BMQ floats
  static constexpr int DL = LS + BMQ * 4;            // -delta, BMQ floats
  static constexpr int RK = DL + BMQ * 4;            // dropout row keys, BMQ words
  static constexpr int BUF = RK + BMQ * 4;
  static constexpr int NCH = D * S / 32;
  static constexpr int NOB = DP / 32;
  static constexpr int NQB = BMQ / 32;
  // 16-bit tiles without zero-padded columns go HBM -> LDS directly
  static constexpr bool kDirect = kTr && D >= 32;
  // d = 128 (16-bit): the workgroup's V rows stay in LDS and are read per query
  // tile instead of being held in registers, so two waves fit per SIMD.
  static constexpr bool kVLds = kDirect && D >= 128;
  static constexpr int VRES = 2 * BUF;                 // resident V rows
  static constexpr int SMEM = 2 * BUF + (kVLds ? BNK * NROW : 0);
};

#ifdef EIAT_WG_TIMING
// Timing check build: per-workgroup stamps of dK/dV (WgStamps; the prologue
// ends when the key tile's K and V and the first query tile are in place).
// Read with eiat_wg_times_dkdv.
__device__ unsigned long long g_wg_times_dkdv[kWgTimingWords * kWgTimingMax];
#endif

template <typename T, int D, int MASK, bool DROP>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(Elt<T>::kBytes == 2 ? 2 : 1, 8))) attn_bwd_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    T* __restrict__ dK, T* __restrict__ dV, int n, int bh_count, int num_ktiles, int window,
    float qk_scale, int qmode, float scale, DropParams dpar) {
  using C = DkvCfg<T, D>;
  constexpr int BMQ = C::BMQ;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  using St = Stager<T, D, BMQ, C::kThreads, C::NROW, C::TROW, true, !C::kTr>;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
#ifdef EIAT_WG_TIMING
  WgStamps wg_stamps;
  wg_stamps.begin();
#endif
  const int bh = bid % bh_count;
  int kt = bid / bh_count;
  // Causal: key tiles near the start are seen by the most queries; issue them first.
  (void)num_ktiles;
  const int k0 = kt * C::BNK;
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;

  const int64_t head = (int64_t)bh * n;
  const char* Qh = reinterpret_cast<const char*>(Q + head * D);
  const char* Kh = reinterpret_cast<const char*>(K + head * D);
  const char* Vh = reinterpret_cast<const char*>(V + head * D);
  const char* dOh = reinterpret_cast<const char*>(dO + head * D);
  const float* LSEh = LSE + head;
  const float* Dh = delta + head;

  // This wave's 32 keys of K and V as B-operand chunks (lane: key kw0 + L%32);
  // with kVLds the V rows go to LDS instead and are read back per query tile.
  // Keys past n read row n - 1: their scores are masked (a wave with such a
  // key runs only masked tiles) and their dK/dV rows are not stored.  All the
  // loads are issued here, with the first query tile's, and waited for once:
  // the sign and zero of c (qmode) are applied after that wait, since an
  // operation on a loaded value waits for it (and for every load before it).
  u32x4 kf[C::NCH], vf[C::kVLds ? 1 : C::NCH];
  {
    const int kr = min(key, n - 1);
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      kf[c] = ldg16(Kh + (int64_t)kr * D * C::S + 32 * c + 16 * h);
      if constexpr (!C::kVLds) vf[c] = ldg16(Vh + (int64_t)kr * D * C::S + 32 * c + 16 * h);
    }
  }
  if constexpr (C::kVLds)
    tile_to_lds<32, D * C::S / 16, 1, C::PAD>(smem + C::VRES + 32 * wave * C::NROW, Vh, kw0, n, 0,
                                               lane);

  // Query rows that may see any key of this workgroup.
  int qbeg = 0, qend = n;
  if (MASK != 0) qbeg = k0;
  if (MASK == 2) qend = (int)min((int64_t)n, (int64_t)k0 + C::BNK - 1 + window);
  const int t_lo = qbeg / BMQ, t_hi = (qend + BMQ - 1) / BMQ;

  f32x16 dk[C::NOB], dv[C::NOB];
#pragma unroll
  for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[ob][e] = 0.0f;
      dv[ob][e] = 0.0f;
    }

  for (int b = 0; b < 2; ++b) {
    char* base = smem + b * C::BUF;
    if constexpr (C::kTr) {
      zero_pad_cols<D, C::DP, C::S, BMQ, C::NROW, C::kThreads>(base + C::QN, tid);
      zero_pad_cols<D, C::DP, C::S, BMQ, C::NROW, C::kThreads>(base + C::ON, tid);
    } else {
      zero_pad_rows<D, C::DP, C::TROW, C::kThreads>(base + C::QT, tid);
      zero_pad_rows<D, C::DP, C::TROW, C::kThreads>(base + C::OT, tid);
    }
  }

  TileLoader<BMQ, D * C::S / 16, C::kWaves, C::PAD, C::kSwz> tl;
  if constexpr (C::kDirect) tl.init(wave, lane);
  SwzReads<D == 128 ? 128 : 64> swz;
  if constexpr (C::kSwz) swz.init(lane);
  St sq, so;
  float4 lreg, dreg;  // LSE and delta of 4 rows as loaded (threads < BMQ / 4)
  int lrow0 = 0;      // first row of the tile those loads belong to
  u32x4 kreg;         // dropout row keys of the same 4 rows (DROP)

  auto load_tile = [&](int t) {
    const int r0 = t * BMQ;
    if constexpr (C::kDirect) {
      char* b = smem + ((t - t_lo) & 1) * C::BUF;
      tl.load(b + C::QN, Qh, r0, n, wave, lane);
      tl.load(b + C::ON, dOh, r0, n, wave, lane);
    } else {
      sq.load(Qh, r0, n, tid);
      so.load(dOh, r0, n, tid);
    }
    // LSE and delta are only loaded here; they are scaled and stored with the
    // tile (store_tile), after its loads have been waited for: using them right
    // after the load would wait for every load issued before them, the tile
    // prefetch included (vector-memory loads retire in order).
    lrow0 = r0;
    if (tid < BMQ / 4) {
      float* lr = reinterpret_cast<float*>(&lreg);
      float* dr = reinterpret_cast<float*>(&dreg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * tid + i;
        const int rc = min(r, n - 1);
        lr[i] = LSEh[rc];
        dr[i] = Dh[rc];
        if constexpr (DROP) kreg[i] = drop_row_key(dpar, (uint32_t)bh, (uint32_t)r);
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* b = smem + buf * C::BUF;
    if constexpr (C::kDirect) {
      wait_tile_loads();
    } else {
      sq.store(b + C::QN, b + C::QT, tid);
      so.store(b + C::ON, b + C::OT, tid);
    }
    if (tid < BMQ / 4) {
      const float* lr = reinterpret_cast<const float*>(&lreg);
      const float* dr = reinterpret_cast<const float*>(&dreg);
      float4 ls4, dl4;
      float* lo = reinterpret_cast<float*>(&ls4);
      float* dlo = reinterpret_cast<float*>(&dl4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = lrow0 + 4 * tid + i < n;
        // rows past n contribute nothing: p = 2^(-inf) = 0
        lo[i] = valid ? lr[i] * kLog2e : INFINITY;
        dlo[i] = valid ? -dr[i] : 0.0f;  // -delta: the dP accumulator starts from it
      }
      *reinterpret_cast<float4*>(b + C::LS + 16 * tid) = ls4;
      *reinterpret_cast<float4*>(b + C::DL + 16 * tid) = dl4;
      if constexpr (DROP) *reinterpret_cast<u32x4*>(b + C::RK + 16 * tid) = kreg;
    }
  };

  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();
  wait_tile_loads();  // the K / V chunks (when no tile was loaded)
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    if (qmode == 1) kf[c] ^= Elt<T>::kSign;
    if (qmode == 2) kf[c] = zero4();  // c = 0: every score is exactly 0
  }
#ifdef EIAT_WG_TIMING
  wg_stamps.prologue_done();
#endif

  // Query tiles [ta, tb) need no per-element mask for any key of this wave
  // (every row sees every key); the others straddle a mask boundary or hold
  // keys past n.  The three ranges run as separate loops, so the interior
  // body has no mask and no branch.
  int ta = t_lo, tb = t_hi;
  if (MASK != 0) ta = min(t_hi, max(t_lo, (kw0 + 31 + BMQ - 1) / BMQ));
  if (MASK == 2) tb = min(t_hi, (kw0 + window) / BMQ);
  if (kw0 + 32 > n) ta = t_hi;
  tb = max(tb, ta);

  auto iterate = [&](int t, auto masked) __attribute__((always_inline)) {
    const int buf = (t - t_lo) & 1;
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);
    const int qt0 = t * BMQ;

    bool empty = false;
    if (MASK != 0) empty = qt0 + BMQ - 1 < kw0;
    if (MASK == 2) empty = empty || (qt0 > kw0 + 31 + window - 1);
    if (!empty) {
      const char* b = smem + buf * C::BUF;

      // One tile, with the per-element mask compiled in or out, so that the
      // unmasked body has no branch.  At 16-bit d = 64 it is software-pipelined
      // over the 32-row blocks: the score and dP products of block qb + 1 are
      // issued before the exponentials of block qb, so that they run under them.
      const float* ls = reinterpret_cast<const float*>(b + C::LS);
      const float* dl = reinterpret_cast<const float*>(b + C::DL);  // -delta
      // S = Q K^T and dP - delta = dO V^T - delta for 32 query rows x this
      // wave's 32 keys (without dropout the dP accumulator starts at -delta of
      // its row, so dS = p (dP - delta) needs no subtraction afterwards)
      auto sdp = [&](int qb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.0f;
        if constexpr (DROP) {
#pragma unroll
          for (int e = 0; e < 16; ++e) dp[e] = 0.0f;
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 d4 = *reinterpret_cast<const float4*>(dl + 32 * qb + 8 * g + 4 * h);
            dp[4 * g] = d4.x;
            dp[4 * g + 1] = d4.y;
            dp[4 * g + 2] = d4.z;
            dp[4 * g + 3] = d4.w;
          }
        }
        const int rq = 32 * qb + l32;
#pragma unroll
        for (int c = 0; c < C::NCH; ++c) {
          u32x4 qa, oa;
          if constexpr (C::kSwz) {
            qa = swz.row_read(b + C::QN, 32 * qb, c);
            oa = swz.row_read(b + C::ON, 32 * qb, c);
          } else {
            qa = *reinterpret_cast<const u32x4*>(b + C::QN + rq * C::NROW + 32 * c + 16 * h);
            oa = *reinterpret_cast<const u32x4*>(b + C::ON + rq * C::NROW + 32 * c + 16 * h);
          }
          s = Elt<T>::mma(qa, kf[c], s);
          u32x4 vb4;
          if constexpr (C::kVLds)
            vb4 = *reinterpret_cast<const u32x4*>(smem + C::VRES + (32 * wave + l32) * C::NROW +
                                                  32 * c + 16 * h);
          else
            vb4 = vf[c];
          dp = Elt<T>::mma(oa, vb4, dp);
        }
      };
      auto rest = [&](int qb, f32x16& s, f32x16& dp, auto masked) __attribute__((always_inline)) {
        if (mask_on(masked)) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int q = qt0 + 32 * qb + 8 * (e >> 2) + 4 * h + (e & 3);
            if (!key_allowed<MASK>(q, key, n, window)) s[e] = -INFINITY;
          }
        }
        // p = 2^(s c log2 e - LSE log2 e), dS = p (dP - delta)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 l4 = *reinterpret_cast<const float4*>(ls + 32 * qb + 8 * g + 4 * h);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          float ndl[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // -delta (dropout path only)
          if constexpr (DROP) {
            const float4 d4 = *reinterpret_cast<const float4*>(dl + 32 * qb + 8 * g + 4 * h);
            ndl[0] = d4.x;
            ndl[1] = d4.y;
            ndl[2] = d4.z;
            ndl[3] = d4.w;
          }
          // Dropout (DROP): the four rows 32 qb + 8 g + 4 h + i against this
          // lane's key.  Lane t of each group of four lanes (keys 4m .. 4m + 3)
          // forms the keep bytes of row i = t for the four keys; a quad
          // broadcast hands every lane byte (key & 3) of each row's word.
          uint32_t kb[4] = {0u, 0u, 0u, 0u};
          if constexpr (DROP) {
            const int t = l32 & 3;
            const uint32_t rk = reinterpret_cast<const uint32_t*>(b + C::RK)[32 * qb + 8 * g + 4 * h + t];
            const uint32_t mine = drop_group_bytes(rk, (uint32_t)key >> 2);
            kb[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x00, 0xF, 0xF, false);
            kb[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0x55, 0xF, 0xF, false);
            kb[2] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xAA, 0xF, 0xF, false);
            kb[3] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xFF, 0xF, 0xF, false);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * g + i;
            const float p = fast_exp2(__builtin_fmaf(s[e], qk_scale, -lv[i]));
            if constexpr (DROP) {
              const bool keep = drop_keep(kb[i], key & 3, dpar.thr);
              s[e] = keep ? p : 0.0f;
              dp[e] = p * ((keep ? dp[e] * dpar.inv_keep : 0.0f) + ndl[i]);
            } else {
              s[e] = p;
              dp[e] = p * dp[e];
            }
          }
        }
        PChunks<T> pc, dsc;
        pc.set(s);
        dsc.set(dp);
#pragma unroll
        for (int ob = 0; ob < C::NOB; ++ob) {
#pragma unroll
          for (int ci = 0; ci < PChunks<T>::kCount; ++ci) {
            u32x4 oa, qa2;
            if constexpr (C::kTr) {
              if constexpr (C::kSwz) {
                oa = swz.tr_read(b + C::ON, 32 * qb, ob, ci);
                qa2 = swz.tr_read(b + C::QN, 32 * qb, ob, ci);
              } else {
                oa = tr_chunk(b + C::ON, C::NROW, 32 * qb, ob, ci, lane);
                qa2 = tr_chunk(b + C::QN, C::NROW, 32 * qb, ob, ci, lane);
              }
            } else {
              oa = keyrow_chunk<T>(b + C::OT + (32 * ob + l32) * C::TROW + 32 * qb * C::S, ci, h);
              qa2 = keyrow_chunk<T>(b + C::QT + (32 * ob + l32) * C::TROW + 32 * qb * C::S, ci, h);
            }
            dv[ob] = Elt<T>::mma(oa, pc.c[ci], dv[ob]);
            dk[ob] = Elt<T>::mma(qa2, dsc.c[ci], dk[ob]);
          }
        }
      };
      // The pipelined order holds two blocks' scores at once (32 more
      // registers): used where they are free, at 16-bit d = 64 (1 % faster);
      // d = 16 would drop from three waves per SIMD to two, float32 d = 64
      // spills, and d = 128 has one block per tile.
      constexpr bool kPipe = C::kTr && D == 64 && C::NQB > 1;
      // Raised wave priority over the exponentials and the dV/dK products of a
      // block (16-bit d >= 64), so that they go ahead of the other wave's
      // score products: dK/dV 5 % faster at d = 128, 1 % at d = 64; at d = 16
      // and for float32 it measured slower and is left out.
      constexpr bool kPrio = C::kTr && D >= 64;
      auto rest_prio = [&](int qb, f32x16& s, f32x16& dp, auto masked) __attribute__((always_inline)) {
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
        rest(qb, s, dp, masked);
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
      };
      auto tile_body = [&](auto masked) __attribute__((always_inline)) {
        if constexpr (kPipe) {
          f32x16 s[2], dp[2];
          sdp(0, s[0], dp[0]);
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            // scheduling hint: interleave LDS operand reads with the MFMAs
            __builtin_amdgcn_iglp_opt(0);
            if (qb + 1 < C::NQB) sdp(qb + 1, s[(qb + 1) & 1], dp[(qb + 1) & 1]);
            rest_prio(qb, s[qb & 1], dp[qb & 1], masked);
          }
        } else {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            // scheduling hint: interleave LDS operand reads with the MFMAs
            __builtin_amdgcn_iglp_opt(0);
            f32x16 s, dp;
            sdp(qb, s, dp);
            rest_prio(qb, s, dp, masked);
          }
        }
      };
      tile_body(masked);
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  };
  // 16-bit d <= 64: the mask compiled in or out.  d = 128 (whose registers
  // are full: the branch-free body spills there) and float32: a run-time flag.
  if constexpr (C::kTr && D <= 64) {
    for (int t = t_lo; t < ta; ++t) iterate(t, std::true_type{});
    for (int t = ta; t < tb; ++t) iterate(t, std::false_type{});
    for (int t = tb; t < t_hi; ++t) iterate(t, std::true_type{});
  } else {
    for (int t = t_lo; t < t_hi; ++t) iterate(t, t < ta || t >= tb);
  }

  // Epilogue: lane holds column `key`, rows a = 32 ob + 8 g + 4 h + (0..3).
  // With dropout, dV summed the kept weights unscaled: scale by 256 / (256 - thr).
  if constexpr (DROP) {
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) dv[ob] *= dpar.inv_keep;
  }
  if (key < n) {
    char* dkrow = reinterpret_cast<char*>(dK + (head + key) * D);
    char* dvrow = reinterpret_cast<char*>(dV + (head + key) * D);
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = 32 * ob + 8 * g + 4 * h;
        if (a0 < D) {
          if constexpr (C::S == 2) {
            u32x2 wk = {Elt<T>::pack2(dk[ob][4 * g] * scale, dk[ob][4 * g + 1] * scale),
                        Elt<T>::pack2(dk[ob][4 * g + 2] * scale, dk[ob][4 * g + 3] * scale)};
            u32x2 wv = {Elt<T>::pack2(dv[ob][4 * g], dv[ob][4 * g + 1]),
                        Elt<T>::pack2(dv[ob][4 * g + 2], dv[ob][4 * g + 3])};
            *reinterpret_cast<u32x2*>(dkrow + a0 * C::S) = wk;
            *reinterpret_cast<u32x2*>(dvrow + a0 * C::S) = wv;
          } else {
            f32x4 wk = {dk[ob][4 * g] * scale, dk[ob][4 * g + 1] * scale,
                        dk[ob][4 * g + 2] * scale, dk[ob][4 * g + 3] * scale};
            f32x4 wv = {dv[ob][4 * g], dv[ob][4 * g + 1], dv[ob][4 * g + 2], dv[ob][4 * g + 3]};
            *reinterpret_cast<f32x4*>(dkrow + a0 * C::S) = wk;
            *reinterpret_cast<f32x4*>(dvrow + a0 * C::S) = wv;
          }
        }
      }
  }
#ifdef EIAT_WG_TIMING
  __syncthreads();
  if (tid == 0) wg_stamps.store(g_wg_times_dkdv, bid);
#endif
}

#ifdef EIAT_WG_TIMING
// Copies the stamps of the last dK/dV launch (layout as eiat_wg_times) to
// host memory `dst` and the wall clock's rate in kHz to *clock_khz.  Returns a
// hipError_t code.
extern "C" __attribute__((visibility("default"))) int eiat_wg_times_dkdv(void* dst, size_t bytes,
                                                                         int* clock_khz) {
  return wg_times_copy(HIP_SYMBOL(g_wg_times_dkdv), sizeof(g_wg_times_dkdv), dst, bytes,
                       clock_khz);
}
#endif

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <typename T, int D, int MASK, bool DROP>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  const int64_t rows = a.bh * a.n;
  if (a.stages & 1) {
    constexpr int CPR = D * Elt<T>::kBytes / 16;
    const int64_t blocks = (rows * CPR + 255) / 256;
    hipLaunchKernelGGL((attn_bwd_delta_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, static_cast<const T*>(a.o), static_cast<const T*>(a.dout),
                       a.delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dQ (which also writes delta) runs before dK/dV, which reads it
  if (a.stages & 4) {
    hipError_t e = launch_bwd_dq(a);  // dQ unit
    if (e != hipSuccess) return e;
  }
  if (a.stages & 2) {
    using C = DkvCfg<T, D>;
    const int num_ktiles = (int)((a.n + C::BNK - 1) / C::BNK);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, MASK, DROP>),
                       dim3((unsigned)(num_ktiles * a.bh)), dim3(C::kThreads), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.delta,
                       static_cast<T*>(a.dk), static_cast<T*>(a.dv), (int)a.n, (int)a.bh,
                       num_ktiles, (int)a.window, a.qk_scale, a.qmode, a.scale, a.drop);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D, int MASK>
static hipError_t launch_bwd_m(const BwdArgs& a) {
  return a.drop.thr > 0 ? launch_bwd_t<T, D, MASK, true>(a) : launch_bwd_t<T, D, MASK, false>(a);
}

template <typename T, int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  switch (a.mask) {
    case 0: return launch_bwd_m<T, D, 0>(a);
    case 1: return launch_bwd_m<T, D, 1>(a);
    default: return launch_bwd_m<T, D, 2>(a);
  }
}

template <typename T>
static hipError_t launch_bwd_dt(const BwdArgs& a) {
  switch (a.d) {
    case 16: return launch_bwd_d<T, 16>(a);
    case 64: return launch_bwd_d<T, 64>(a);
    default: return launch_bwd_d<T, 128>(a);
  }
}

hipError_t launch_bwd(const BwdArgs& a) {
  switch (a.dtype) {
    case 0: return launch_bwd_dt<float>(a);
    case 1: return launch_bwd_dt<_Float16>(a);
    default: return launch_bwd_dt<__bf16>(a);
  }
}


}  // namespace eiat
