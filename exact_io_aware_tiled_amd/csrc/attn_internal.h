// attn_internal.h -- host-side launch interface between the C ABI entry points
// (attn_api.hip) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eiat {

// Dropout on the attention weights (mask definition with the device helpers
// in attn_device.h).  thr == 0 means no dropout.
struct DropParams {
  uint32_t seed_lo, seed_hi;
  int thr;          // 0..255: drop probability thr / 256
  float inv_keep;   // 256 / (256 - thr)
};

// Arguments of one forward launch, already validated by the entry point.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t bh;        // B * H
  int64_t n;
  int d;             // == dv
  int dtype;         // 0 f32, 1 f16, 2 bf16
  int mask;          // 0 none, 1 causal, 2 window
  int64_t window;    // allowed keys per row (mask 2), clamped to n
  float qk_scale;    // |c| * log2(e), or 1 when c == 0
  int qmode;         // 0: c > 0, 1: c < 0 (Q negated), 2: c == 0 (Q taken as 0)
  DropParams drop;   // drop.thr == 0: no dropout
  // FP8 scores: q and k hold e4m3 codes with E8M0 scale bytes per 32 values
  // ([bh][n][d / 32]); v, o stay in dtype (16-bit); d is 64 or 128.
  const uint8_t* qscale = nullptr;
  const uint8_t* kscale = nullptr;
  // FP8 weights and values as well (requires qscale): v holds the codes of
  // attn_quant_fp8_v's layout and vscale its block scales; o is dtype.
  const uint8_t* vscale = nullptr;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;      // workspace, bh * n floats
  int64_t bh;
  int64_t n;
  int d;
  int dtype;
  int mask;
  int64_t window;
  float qk_scale;    // as FwdArgs
  int qmode;
  float scale;       // c itself (multiplies dQ and dK)
  int stages;        // bit 0: delta, bit 1: dK/dV, bit 2: dQ and delta (run before dK/dV)
  DropParams drop;   // the forward's dropout, replayed (thr == 0: none)
  hipStream_t stream;
};

// Decode-shaped forward: nq new rows per query head against nk cached keys.
struct DecodeArgs {
  const void* q;     // [B][H][nq][d]
  const void* k;     // [B][Hkv][nk][d]
  const void* v;     // [B][Hkv][nk][d]
  void* o;           // [B][H][nq][d]
  float* lse;        // [B][H][nq]
  float* workspace;  // range summaries (attn_decode_workspace_bytes() bytes)
  int64_t B, H, Hkv, nq, nk;
  int d;             // == dv, 64 or 128
  int dtype;         // 1 f16, 2 bf16
  int mask;
  int64_t window;    // clamped to nk
  float qk_scale;    // as FwdArgs
  int qmode;
  int nsplit;        // decode_splits(B * Hkv, nk)
  int stages;        // bit 0: range summaries, bit 1: merge into O and LSE
  hipStream_t stream;
};

// Block-scaled FP8 quantization of rows (the FP8-score forward's Q and K).
struct QuantArgs {
  const void* x;          // [rows][d], dtype
  const int8_t* signs;    // [d] of +-1, or null (no rotation)
  uint8_t* codes;         // [rows][d] e4m3
  uint8_t* scales;        // [rows][d / 32] E8M0 bytes
  int64_t rows;
  int d;                  // 64 or 128
  int dtype;              // 0 f32, 1 f16, 2 bf16
  hipStream_t stream;
};

// Values for FP8 weights: V quantized along the keys into the tile-major
// layout the FP8 value product reads (see attn_fp8.hip).
struct QuantVArgs {
  const void* v;          // [bh][n][dv], dtype
  uint8_t* codes;         // [bh][ceil(n / 64)][dv][64]
  uint8_t* scales;        // [bh][ceil(n / 64)][dv][2]
  int64_t bh, n;
  int dv;                 // 64 or 128
  int dtype;              // 0 f32, 1 f16, 2 bf16
  hipStream_t stream;
};

// Cache ranges per (batch, key/value head) used by the decode kernels.
int decode_splits(int64_t units, int64_t nk);

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_quant_fp8(const QuantArgs& a);
hipError_t launch_quant_fp8_v(const QuantVArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
// The dQ kernel alone (stage bit 2); launch_bwd calls it.
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace eiat
