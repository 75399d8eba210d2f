// attn_api.hip -- the C ABI entry points declared in include/eiat_attn.h:
// argument validation (on the host, before any HIP call), the mapping of the
// scale c onto the kernels' exponent scale, and dispatch to the kernels.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/eiat_attn.h"
#include "attn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

eiat_status fail(eiat_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

eiat_status ok() {
  g_last_error[0] = '\0';
  return EIAT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int dtype) { return dtype == EIAT_F32 ? 4 : 2; }

// [p, p + bytes) and [r, r + rbytes) share at least one byte.
bool overlaps(const void* p, size_t bytes, const void* r, size_t rbytes) {
  if (bytes == 0 || rbytes == 0) return false;
  uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(r);
  return a < b + rbytes && b < a + bytes;
}

// Checks shared by both passes.  On success fills the scale mapping and the
// clamped window, and sets *empty when there is no work.
eiat_status check_common(int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int dtype,
                         float scale, int mask, int64_t window, bool* empty, float* qk_scale,
                         int* qmode, int64_t* win_eff) {
  if (B < 0 || H < 0 || n < 0) return fail(EIAT_ERR_INVALID_ARG, "B, H and n must be >= 0");
  if (d < 1 || dv < 1) return fail(EIAT_ERR_INVALID_ARG, "d and dv must be >= 1");
  if (dtype != EIAT_F32 && dtype != EIAT_F16 && dtype != EIAT_BF16)
    return fail(EIAT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (mask != EIAT_MASK_NONE && mask != EIAT_MASK_CAUSAL && mask != EIAT_MASK_WINDOW)
    return fail(EIAT_ERR_INVALID_ARG, "unknown mask kind %d", mask);
  if (mask == EIAT_MASK_WINDOW && window < 1)
    return fail(EIAT_ERR_INVALID_ARG, "window must be >= 1 (got %lld)", (long long)window);
  if (!isfinite(scale)) return fail(EIAT_ERR_INVALID_ARG, "scale must be finite");
  if (d != dv) return fail(EIAT_ERR_UNSUPPORTED, "d != dv (%lld, %lld) has no kernel", (long long)d, (long long)dv);
  if (d != 16 && d != 64 && d != 128)
    return fail(EIAT_ERR_UNSUPPORTED, "head dim %lld has no kernel (16, 64, 128)", (long long)d);
  // Row indices are 32-bit inside the kernels; grids are at most 2^31 - 1 blocks.
  if (n > (int64_t)INT32_MAX - 1024) return fail(EIAT_ERR_UNSUPPORTED, "n too large");
  if (B > 0 && H > (int64_t)INT32_MAX / B) return fail(EIAT_ERR_UNSUPPORTED, "B * H too large");
  const int64_t bh = B * H;
  if (bh > 0 && (n + 127) / 128 > (int64_t)INT32_MAX / bh)
    return fail(EIAT_ERR_UNSUPPORTED, "grid too large");
  if (bh > 0 && n > 0 && bh > INT64_MAX / n / d / 4)
    return fail(EIAT_ERR_UNSUPPORTED, "tensor too large");
  *empty = (bh == 0 || n == 0);
  if (scale > 0.0f) {
    *qmode = 0;
    *qk_scale = (float)((double)scale * 1.4426950408889634);
  } else if (scale < 0.0f) {
    *qmode = 1;
    *qk_scale = (float)(-(double)scale * 1.4426950408889634);
  } else {
    *qmode = 2;
    *qk_scale = 1.0f;
  }
  if (!isfinite(*qk_scale)) return fail(EIAT_ERR_INVALID_ARG, "scale * log2(e) overflows float32");
  *win_eff = mask == EIAT_MASK_WINDOW ? (window < n ? window : (n > 0 ? n : 1)) : 0;
  return EIAT_OK;
}

// Dropout probability -> mask threshold (drop probability thr / 256).
eiat_status drop_params(float p_drop, uint64_t seed, eiat::DropParams* dp) {
  if (!(p_drop >= 0.0f && p_drop < 1.0f))
    return fail(EIAT_ERR_INVALID_ARG, "p_drop must be in [0, 1) (got %g)", (double)p_drop);
  long thr = lrintf(p_drop * 256.0f);
  if (thr > 255) thr = 255;
  dp->seed_lo = (uint32_t)seed;
  dp->seed_hi = (uint32_t)(seed >> 32);
  dp->thr = (int)thr;
  dp->inv_keep = (float)(256.0 / (256.0 - (double)thr));
  return EIAT_OK;
}

const eiat::DropParams kNoDrop = {0u, 0u, 0, 1.0f};

}  // namespace

static eiat_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int dtype,
                            float scale, int mask, int64_t window, const eiat::DropParams& drop,
                            void* stream) {
  bool empty = false;
  float qk_scale = 1.0f;
  int qmode = 0;
  int64_t win = 0;
  eiat_status s =
      check_common(B, H, n, d, dv, dtype, scale, mask, window, &empty, &qk_scale, &qmode, &win);
  if (s != EIAT_OK) return s;
  if (empty) return ok();
  if (!q || !k || !v || !o || !lse) return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(EIAT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t eb = elem_bytes(dtype);
  const size_t qb = (size_t)(B * H * n * d) * eb, vb = (size_t)(B * H * n * dv) * eb;
  const size_t lb = (size_t)(B * H * n) * 4;
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, qb, vb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(o, vb, ins[i], insz[i]) || overlaps(lse, lb, ins[i], insz[i]))
      return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap inputs");
  if (overlaps(o, vb, lse, lb)) return fail(EIAT_ERR_INVALID_ARG, "o and lse overlap");

  eiat::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = n;
  a.d = (int)d;
  a.dtype = dtype;
  a.mask = mask;
  a.window = win;
  a.qk_scale = qk_scale;
  a.qmode = qmode;
  a.drop = drop;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = eiat::launch_fwd(a);
  if (e != hipSuccess) return fail(EIAT_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" {

eiat_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t n, int64_t d, int64_t dv, int dtype, float scale, int mask,
                     int64_t window, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, n, d, dv, dtype, scale, mask, window, kNoDrop, stream);
}

eiat_status attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int dtype,
                             float scale, int mask, int64_t window, float p_drop, uint64_t seed,
                             void* stream) {
  eiat::DropParams dp;
  eiat_status s = drop_params(p_drop, seed, &dp);
  if (s != EIAT_OK) return s;
  return fwd_impl(q, k, v, o, lse, B, H, n, d, dv, dtype, scale, mask, window, dp, stream);
}

eiat_status attn_quant_fp8(const void* x, const int8_t* signs, uint8_t* codes, uint8_t* scales,
                           int64_t rows, int64_t d, int dtype, void* stream) {
  if (rows < 0) return fail(EIAT_ERR_INVALID_ARG, "rows must be >= 0");
  if (d < 1) return fail(EIAT_ERR_INVALID_ARG, "d must be >= 1");
  if (dtype != EIAT_F32 && dtype != EIAT_F16 && dtype != EIAT_BF16)
    return fail(EIAT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (d != 64 && d != 128)
    return fail(EIAT_ERR_UNSUPPORTED, "FP8 quantization: d %lld has no kernel (64, 128)",
                (long long)d);
  // 256 threads cover 256 * 8 / d rows per workgroup
  if ((rows + 15) / 16 > (int64_t)INT32_MAX) return fail(EIAT_ERR_UNSUPPORTED, "rows too large");
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || (signs && !aligned16(signs)))
    return fail(EIAT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t xb = (size_t)(rows * d) * elem_bytes(dtype), cb = (size_t)(rows * d),
               sb = (size_t)(rows * (d / 32));
  if (overlaps(codes, cb, x, xb) || overlaps(scales, sb, x, xb) ||
      (signs && (overlaps(codes, cb, signs, (size_t)d) || overlaps(scales, sb, signs, (size_t)d))))
    return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap inputs");
  if (overlaps(codes, cb, scales, sb)) return fail(EIAT_ERR_INVALID_ARG, "codes and scales overlap");
  eiat::QuantArgs a;
  a.x = x;
  a.signs = signs;
  a.codes = codes;
  a.scales = scales;
  a.rows = rows;
  a.d = (int)d;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = eiat::launch_quant_fp8(a);
  if (e != hipSuccess) return fail(EIAT_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
  return ok();
}

eiat_status attn_quant_fp8_v(const void* v, uint8_t* codes, uint8_t* scales, int64_t BH, int64_t n,
                           int64_t dv, int dtype, void* stream) {
  if (BH < 0 || n < 0) return fail(EIAT_ERR_INVALID_ARG, "BH and n must be >= 0");
  if (dv < 1) return fail(EIAT_ERR_INVALID_ARG, "dv must be >= 1");
  if (dtype != EIAT_F32 && dtype != EIAT_F16 && dtype != EIAT_BF16)
    return fail(EIAT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (dv != 64 && dv != 128)
    return fail(EIAT_ERR_UNSUPPORTED, "FP8 values: dv %lld has no kernel (64, 128)", (long long)dv);
  if (n > (int64_t)INT32_MAX - 64) return fail(EIAT_ERR_UNSUPPORTED, "n too large");
  const int64_t nt = (n + 63) / 64;
  if (BH > 0 && nt > (int64_t)INT32_MAX / BH) return fail(EIAT_ERR_UNSUPPORTED, "grid too large");
  if (BH == 0 || n == 0) return ok();
  if (!v || !codes || !scales) return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(v) || !aligned16(codes) || !aligned16(scales))
    return fail(EIAT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t vb = (size_t)(BH * n * dv) * elem_bytes(dtype), cb = (size_t)(BH * nt * dv * 64),
               sb = (size_t)(BH * nt * dv * 2);
  if (overlaps(codes, cb, v, vb) || overlaps(scales, sb, v, vb))
    return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap inputs");
  if (overlaps(codes, cb, scales, sb)) return fail(EIAT_ERR_INVALID_ARG, "codes and scales overlap");
  eiat::QuantVArgs a;
  a.v = v;
  a.codes = codes;
  a.scales = scales;
  a.bh = BH;
  a.n = n;
  a.dv = (int)dv;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = eiat::launch_quant_fp8_v(a);
  if (e != hipSuccess) return fail(EIAT_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
  return ok();
}

static eiat_status fwd_fp8_impl(const uint8_t* q, const uint8_t* q_scale, const uint8_t* k,
                                const uint8_t* k_scale, const void* v, const uint8_t* v_scale,
                                void* o, float* lse, int64_t B, int64_t H, int64_t n, int64_t d,
                                int64_t dv, int dtype, float scale, int mask, int64_t window,
                                void* stream);

eiat_status attn_fwd_fp8(const uint8_t* q, const uint8_t* q_scale, const uint8_t* k,
                         const uint8_t* k_scale, const void* v, void* o, float* lse, int64_t B,
                         int64_t H, int64_t n, int64_t d, int64_t dv, int dtype, float scale,
                         int mask, int64_t window, void* stream) {
  return fwd_fp8_impl(q, q_scale, k, k_scale, v, nullptr, o, lse, B, H, n, d, dv, dtype, scale,
                      mask, window, stream);
}

eiat_status attn_fwd_fp8_pv(const uint8_t* q, const uint8_t* q_scale, const uint8_t* k,
                            const uint8_t* k_scale, const uint8_t* v, const uint8_t* v_scale,
                            void* o, float* lse, int64_t B, int64_t H, int64_t n, int64_t d,
                            int64_t dv, int dtype, float scale, int mask, int64_t window,
                            void* stream) {
  if (!v_scale && B > 0 && H > 0 && n > 0)
    return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  return fwd_fp8_impl(q, q_scale, k, k_scale, v, v_scale, o, lse, B, H, n, d, dv, dtype, scale,
                      mask, window, stream);
}

static eiat_status fwd_fp8_impl(const uint8_t* q, const uint8_t* q_scale, const uint8_t* k,
                                const uint8_t* k_scale, const void* v, const uint8_t* v_scale,
                                void* o, float* lse, int64_t B, int64_t H, int64_t n, int64_t d,
                                int64_t dv, int dtype, float scale, int mask, int64_t window,
                                void* stream) {
  bool empty = false;
  float qk_scale = 1.0f;
  int qmode = 0;
  int64_t win = 0;
  eiat_status s =
      check_common(B, H, n, d, dv, dtype, scale, mask, window, &empty, &qk_scale, &qmode, &win);
  if (s != EIAT_OK) return s;
  if (dtype == EIAT_F32)
    return fail(EIAT_ERR_UNSUPPORTED, "FP8 scores: values and output are f16 or bf16");
  if (d != 64 && d != 128)
    return fail(EIAT_ERR_UNSUPPORTED, "FP8 scores: head dim %lld has no kernel (64, 128)",
                (long long)d);
  if (empty) return ok();
  if (!q || !q_scale || !k || !k_scale || !v || !o || !lse)
    return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  const void* ptrs[8] = {q, q_scale, k, k_scale, v, o, lse, v_scale ? v_scale : q};
  for (int i = 0; i < 8; ++i)
    if (!aligned16(ptrs[i])) return fail(EIAT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const int64_t nt = (n + 63) / 64;
  const size_t qb = (size_t)(B * H * n * d), sb = (size_t)(B * H * n * (d / 32)),
               ob = (size_t)(B * H * n * dv) * elem_bytes(dtype), lb = (size_t)(B * H * n) * 4;
  // values: dtype rows, or (FP8 values) codes and block scales of the tile layout
  const size_t vb = v_scale ? (size_t)(B * H * nt * dv * 64) : ob;
  const size_t vsb = v_scale ? (size_t)(B * H * nt * dv * 2) : 0;
  const void* ins[6] = {q, q_scale, k, k_scale, v, v_scale};
  const size_t insz[6] = {qb, sb, qb, sb, vb, vsb};
  for (int i = 0; i < 6; ++i)
    if (overlaps(o, ob, ins[i], insz[i]) || overlaps(lse, lb, ins[i], insz[i]))
      return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap inputs");
  if (overlaps(o, ob, lse, lb)) return fail(EIAT_ERR_INVALID_ARG, "o and lse overlap");

  eiat::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = n;
  a.d = (int)d;
  a.dtype = dtype;
  a.mask = mask;
  a.window = win;
  a.qk_scale = qk_scale;
  a.qmode = qmode;
  a.drop = kNoDrop;
  a.qscale = q_scale;
  a.kscale = k_scale;
  a.vscale = v_scale;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = eiat::launch_fwd(a);
  if (e != hipSuccess) return fail(EIAT_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t n) {
  if (B <= 0 || H <= 0 || n <= 0) return 0;
  return (size_t)B * (size_t)H * (size_t)n * sizeof(float);
}

// ---------------------------------------------------------------------------
// Scratch of attn_bwd_noalloc: the per-row delta of the backward, in a
// file-scope device array instead of a caller-passed workspace.  Each GPU the
// library runs on holds its own copy (16 MiB) until the process ends; host
// code only ever uses the per-device address from hipGetSymbolAddress (the
// array's name in host code is a stand-in, not a device address).  Every call
// on a GPU shares that GPU's copy, so calls that overlap on one GPU (several
// streams, several host threads) race on it.  Nothing in it needs to start at
// zero: the dQ kernel writes the delta of every row before the dK/dV kernel
// reads it, in stream order.
// ---------------------------------------------------------------------------
constexpr int64_t kNoAllocMaxRows = int64_t(1) << 22;  // B * H * n limit (4,194,304 rows)
static __device__ __align__(256) float scratch[kNoAllocMaxRows];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current (the entry point's first call on it).  Null on a HIP error.
float* scratch_for_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  return g_scratch_ptr[dev];
}

}  // namespace

// The backward's entry points.  scratch_ws: delta goes to this GPU's copy of
// `scratch` (attn_bwd_noalloc); workspace and workspace_bytes are then unused.
static eiat_status bwd_impl(int stages, const void* q, const void* k, const void* v,
                            const void* o, const void* dout, const float* lse, void* dq, void* dk,
                            void* dvv, void* workspace, size_t workspace_bytes, int64_t B,
                            int64_t H, int64_t n, int64_t d, int64_t dv, int dtype, float scale,
                            int mask, int64_t window, const eiat::DropParams& drop,
                            void* stream, bool scratch_ws = false) {
  bool empty = false;
  float qk_scale = 1.0f;
  int qmode = 0;
  int64_t win = 0;
  eiat_status s =
      check_common(B, H, n, d, dv, dtype, scale, mask, window, &empty, &qk_scale, &qmode, &win);
  if (s != EIAT_OK) return s;
  if (empty) return ok();
  if (scratch_ws && B * H * n > kNoAllocMaxRows)
    return fail(EIAT_ERR_UNSUPPORTED,
                "B * H * n = %lld rows exceed the %lld rows of the no-allocation scratch; use "
                "attn_bwd with a workspace", (long long)(B * H * n), (long long)kNoAllocMaxRows);
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dvv || (!scratch_ws && !workspace))
    return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dvv, scratch_ws ? q : workspace};
  for (int i = 0; i < 10; ++i)
    if (!aligned16(ptrs[i])) return fail(EIAT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!scratch_ws && workspace_bytes < attn_bwd_workspace_bytes(B, H, n))
    return fail(EIAT_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", workspace_bytes,
                attn_bwd_workspace_bytes(B, H, n));
  const size_t eb = elem_bytes(dtype);
  const size_t qb = (size_t)(B * H * n * d) * eb, vb = (size_t)(B * H * n * dv) * eb;
  const size_t lb = (size_t)(B * H * n) * 4;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t insz[6] = {qb, qb, vb, vb, vb, lb};
  void* outs[4] = {dq, dk, dvv, workspace};
  const size_t outsz[4] = {qb, qb, vb, scratch_ws ? 0 : attn_bwd_workspace_bytes(B, H, n)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j]))
        return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap inputs");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j]))
        return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap each other");
  }
  if (scratch_ws) {
    hipError_t e = hipSuccess;
    workspace = scratch_for_current_device(&e);
    if (!workspace)
      return fail(EIAT_ERR_HIP, "no-allocation scratch address: %s", hipGetErrorString(e));
  }

  eiat::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dvv;
  a.delta = static_cast<float*>(workspace);
  a.bh = B * H;
  a.n = n;
  a.d = (int)d;
  a.dtype = dtype;
  a.mask = mask;
  a.window = win;
  a.qk_scale = qk_scale;
  a.qmode = qmode;
  a.scale = scale;
  a.stages = stages;
  a.drop = drop;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = eiat::launch_bwd(a);
  if (e != hipSuccess) return fail(EIAT_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

eiat_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dvv, void* workspace,
                     size_t workspace_bytes, int64_t B, int64_t H, int64_t n, int64_t d,
                     int64_t dv, int dtype, float scale, int mask, int64_t window, void* stream) {
  return bwd_impl(6, q, k, v, o, dout, lse, dq, dk, dvv, workspace, workspace_bytes, B, H, n, d,
                  dv, dtype, scale, mask, window, kNoDrop, stream);
}

eiat_status attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dvv,
                             void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                             int64_t n, int64_t d, int64_t dv, int dtype, float scale, int mask,
                             int64_t window, float p_drop, uint64_t seed, void* stream) {
  eiat::DropParams dp;
  eiat_status s = drop_params(p_drop, seed, &dp);
  if (s != EIAT_OK) return s;
  return bwd_impl(6, q, k, v, o, dout, lse, dq, dk, dvv, workspace, workspace_bytes, B, H, n, d,
                  dv, dtype, scale, mask, window, dp, stream);
}

eiat_status attn_bwd_dropout_stage(int stage, const void* q, const void* k, const void* v,
                                   const void* o, const void* dout, const float* lse, void* dq,
                                   void* dk, void* dvv, void* workspace, size_t workspace_bytes,
                                   int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                   int dtype, float scale, int mask, int64_t window, float p_drop,
                                   uint64_t seed, void* stream) {
  if (stage < 0 || stage > 2) return fail(EIAT_ERR_INVALID_ARG, "unknown backward stage %d", stage);
  eiat::DropParams dp;
  eiat_status s = drop_params(p_drop, seed, &dp);
  if (s != EIAT_OK) return s;
  return bwd_impl(1 << stage, q, k, v, o, dout, lse, dq, dk, dvv, workspace, workspace_bytes, B, H,
                  n, d, dv, dtype, scale, mask, window, dp, stream);
}

eiat_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dvv,
                             int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv, int dtype,
                             float scale, int mask, int64_t window, void* stream) {
  return bwd_impl(6, q, k, v, o, dout, lse, dq, dk, dvv, nullptr, 0, B, H, n, d, dv, dtype, scale,
                  mask, window, kNoDrop, stream, true);
}

eiat_status attn_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dvv,
                           void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t n, int64_t d, int64_t dv, int dtype, float scale, int mask,
                           int64_t window, void* stream) {
  if (stage < 0 || stage > 2) return fail(EIAT_ERR_INVALID_ARG, "unknown backward stage %d", stage);
  return bwd_impl(1 << stage, q, k, v, o, dout, lse, dq, dk, dvv, workspace, workspace_bytes, B, H,
                  n, d, dv, dtype, scale, mask, window, kNoDrop, stream);
}

size_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t nq, int64_t nk,
                                   int64_t dv) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || nq <= 0 || nk <= 0 || dv <= 0 || H % Hkv != 0) return 0;
  const int64_t units = B * Hkv, M = H / Hkv * nq;
  const int64_t S = eiat::decode_splits(units, nk);
  return (size_t)units * (size_t)S * (size_t)M * (size_t)(dv + 2) * sizeof(float);
}

static eiat_status decode_impl(int stages, const void* q, const void* k, const void* v, void* o,
                               float* lse, void* workspace, size_t workspace_bytes, int64_t B,
                               int64_t H, int64_t Hkv, int64_t nq, int64_t nk, int64_t d,
                               int64_t dv, int dtype, float scale, int mask, int64_t window,
                               void* stream) {
  if (B < 0 || nq < 0 || nk < 0) return fail(EIAT_ERR_INVALID_ARG, "B, nq and nk must be >= 0");
  if (H < 1 || Hkv < 1) return fail(EIAT_ERR_INVALID_ARG, "H and Hkv must be >= 1");
  if (H % Hkv != 0)
    return fail(EIAT_ERR_INVALID_ARG, "H (%lld) must be a multiple of Hkv (%lld)", (long long)H,
                (long long)Hkv);
  if (nq > nk)
    return fail(EIAT_ERR_INVALID_ARG, "the nq = %lld new rows are the last of nk = %lld positions",
                (long long)nq, (long long)nk);
  if (d < 1 || dv < 1) return fail(EIAT_ERR_INVALID_ARG, "d and dv must be >= 1");
  if (dtype != EIAT_F32 && dtype != EIAT_F16 && dtype != EIAT_BF16)
    return fail(EIAT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (mask != EIAT_MASK_NONE && mask != EIAT_MASK_CAUSAL && mask != EIAT_MASK_WINDOW)
    return fail(EIAT_ERR_INVALID_ARG, "unknown mask kind %d", mask);
  if (mask == EIAT_MASK_WINDOW && window < 1)
    return fail(EIAT_ERR_INVALID_ARG, "window must be >= 1 (got %lld)", (long long)window);
  if (!isfinite(scale)) return fail(EIAT_ERR_INVALID_ARG, "scale must be finite");
  if (dtype == EIAT_F32) return fail(EIAT_ERR_UNSUPPORTED, "decode kernels take f16 or bf16");
  if (d != dv || (d != 64 && d != 128))
    return fail(EIAT_ERR_UNSUPPORTED, "decode kernels take d == dv in {64, 128}");
  if (H / Hkv * nq > 32)
    return fail(EIAT_ERR_UNSUPPORTED, "(H / Hkv) * nq = %lld rows per key/value head exceeds 32",
                (long long)(H / Hkv * nq));
  if (nk > (int64_t)INT32_MAX - 1024) return fail(EIAT_ERR_UNSUPPORTED, "nk too large");
  if (B > 0 && H > (int64_t)INT32_MAX / 64 / B) return fail(EIAT_ERR_UNSUPPORTED, "B * H too large");
  if (B * Hkv > 0 && nk > INT64_MAX / (B * Hkv) / d / 4)
    return fail(EIAT_ERR_UNSUPPORTED, "tensor too large");
  const int64_t units = B * Hkv;
  const int nsplit = eiat::decode_splits(units, nk);
  if (units * nsplit > (int64_t)INT32_MAX) return fail(EIAT_ERR_UNSUPPORTED, "grid too large");
  if (B == 0 || nq == 0) return ok();
  float qk_scale = 1.0f;
  int qmode = 0;
  if (scale > 0.0f) {
    qk_scale = (float)((double)scale * 1.4426950408889634);
  } else if (scale < 0.0f) {
    qmode = 1;
    qk_scale = (float)(-(double)scale * 1.4426950408889634);
  } else {
    qmode = 2;
  }
  if (!isfinite(qk_scale)) return fail(EIAT_ERR_INVALID_ARG, "scale * log2(e) overflows float32");
  if (!q || !k || !v || !o || !lse || !workspace)
    return fail(EIAT_ERR_INVALID_ARG, "null pointer argument");
  const void* ptrs[6] = {q, k, v, o, lse, workspace};
  for (int i = 0; i < 6; ++i)
    if (!aligned16(ptrs[i])) return fail(EIAT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t need = attn_decode_workspace_bytes(B, H, Hkv, nq, nk, dv);
  if (workspace_bytes < need)
    return fail(EIAT_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  const size_t eb = elem_bytes(dtype);
  const size_t qb = (size_t)(B * H * nq * d) * eb, kb = (size_t)(B * Hkv * nk * d) * eb;
  const size_t ob = (size_t)(B * H * nq * dv) * eb, lb = (size_t)(B * H * nq) * 4;
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, kb, kb};
  void* outs[3] = {o, lse, workspace};
  const size_t outsz[3] = {ob, lb, need};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j]))
        return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap inputs");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j]))
        return fail(EIAT_ERR_INVALID_ARG, "outputs must not overlap each other");
  }

  eiat::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.workspace = static_cast<float*>(workspace);
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.nq = nq;
  a.nk = nk;
  a.d = (int)d;
  a.dtype = dtype;
  a.mask = mask;
  a.window = mask == EIAT_MASK_WINDOW ? (window < nk ? window : nk) : 0;
  a.qk_scale = qk_scale;
  a.qmode = qmode;
  a.nsplit = nsplit;
  a.stages = stages;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = eiat::launch_decode(a);
  if (e != hipSuccess) return fail(EIAT_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

eiat_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                        int64_t Hkv, int64_t nq, int64_t nk, int64_t d, int64_t dv, int dtype,
                        float scale, int mask, int64_t window, void* stream) {
  return decode_impl(3, q, k, v, o, lse, workspace, workspace_bytes, B, H, Hkv, nq, nk, d, dv,
                     dtype, scale, mask, window, stream);
}

eiat_status attn_decode_stage(int stage, const void* q, const void* k, const void* v, void* o,
                              float* lse, void* workspace, size_t workspace_bytes, int64_t B,
                              int64_t H, int64_t Hkv, int64_t nq, int64_t nk, int64_t d,
                              int64_t dv, int dtype, float scale, int mask, int64_t window,
                              void* stream) {
  if (stage < 0 || stage > 1) return fail(EIAT_ERR_INVALID_ARG, "unknown decode stage %d", stage);
  return decode_impl(1 << stage, q, k, v, o, lse, workspace, workspace_bytes, B, H, Hkv, nq, nk,
                     d, dv, dtype, scale, mask, window, stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case EIAT_OK: return "EIAT_OK";
    case EIAT_ERR_INVALID_ARG: return "EIAT_ERR_INVALID_ARG";
    case EIAT_ERR_UNSUPPORTED: return "EIAT_ERR_UNSUPPORTED";
    case EIAT_ERR_HIP: return "EIAT_ERR_HIP";
    default: return "EIAT_UNKNOWN_STATUS";
  }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_abi_version(void) { return EIAT_ABI_VERSION; }

}  // extern "C"
