/*
 * eiat_attn.h -- C ABI of the exact IO-aware tiled attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is masked row-softmax attention as defined on alphabetamath.cc,
 * "Exact tiled attention and memory-aware differentiation" (Definition "Stable
 * summary of an attention key block"; Theorem "Tiled attention and its
 * recomputed reverse pass are exact"): for every batch b, head h and query row i
 *
 *     s_ij = c * sum_r Q_ir K_jr                (j in the allowed set A_i)
 *     O_i  = sum_{j in A_i} e^{s_ij} V_j / sum_{j in A_i} e^{s_ij}
 *     LSE_i = ln sum_{j in A_i} e^{s_ij}   (= m_i + ln l_i of the summary)
 *
 * and its reverse (the Algorithm "Exact tiled softmax attention with
 * block-recomputed vector-Jacobian products", reverse procedure): given the
 * upstream gradient dO = G, the gradients dQ, dK, dV of Phi = sum G * O.
 *
 * Allowed-key sets, 0-based rows i and keys j:
 *     EIAT_MASK_NONE    every key, 0 <= j < n
 *     EIAT_MASK_CAUSAL  j <= i (the diagonal is allowed)
 *     EIAT_MASK_WINDOW  max(0, i - window + 1) <= j <= i; window >= 1 counts the
 *                       allowed keys including the diagonal (window >= n is causal)
 * Every row therefore has a nonempty allowed set.
 *
 * Layout.  All tensors are contiguous, row-major, head-major:
 *     q, k, dq, dk : [B][H][n][d]       elements of `dtype`
 *     v, o, do, dv : [B][H][n][dv]      elements of `dtype`
 *     lse          : [B][H][n]          float32, natural logarithm
 * Pointers are device pointers (memory the caller allocated on the current
 * HIP device), 16-byte aligned.  The library never allocates or frees memory;
 * every buffer is owned by the caller.  Outputs must not overlap inputs.
 *
 * Execution.  Calls enqueue kernels on `stream` (a hipStream_t; NULL is the
 * null stream) and return without waiting.  Results are deterministic: the
 * same inputs give bitwise-identical outputs (no atomics).
 *
 * Errors.  The return code is the only error channel; nothing is thrown.
 * Argument errors are detected on the host before any HIP call, so they can be
 * tested without a GPU.  attn_last_error() gives a thread-local message for
 * the last non-OK return of the calling thread.
 *
 * Supported kernels: dtype F32, F16 or BF16 (fp32 accumulation in every case),
 * d == dv in {16, 64, 128}.  Scores c * q_i . k_j must be finite in float32.
 */
#ifndef EIAT_ATTN_H
#define EIAT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EIAT_ABI_VERSION 6  /* 2: adds attn_decode; 3: adds the dropout entry points;
                               4: adds attn_quant_fp8 and attn_fwd_fp8;
                               5: adds attn_quant_fp8_v and attn_fwd_fp8_pv;
                               6: adds attn_bwd_noalloc */

/* Symbols of the shared library (built with hidden default visibility). */
#if defined(__GNUC__)
#define EIAT_API __attribute__((visibility("default")))
#else
#define EIAT_API
#endif

typedef enum {
    EIAT_OK = 0,
    EIAT_ERR_INVALID_ARG = 1, /* a null pointer, a negative size, an unknown enum, window < 1,
                                 a misaligned pointer or a too-small workspace */
    EIAT_ERR_UNSUPPORTED = 2, /* valid mathematics with no kernel here (d or dv not in
                                 {16, 64, 128}, d != dv, sizes beyond int32 row indexing) */
    EIAT_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} eiat_status;

typedef enum { EIAT_F32 = 0, EIAT_F16 = 1, EIAT_BF16 = 2 } eiat_dtype;

typedef enum { EIAT_MASK_NONE = 0, EIAT_MASK_CAUSAL = 1, EIAT_MASK_WINDOW = 2 } eiat_mask;

/*
 * Forward pass: the Algorithm's forward procedure (load a query tile, stream
 * key/value tiles past it, keep the running max m, shifted normaliser l and
 * weighted value sum z, merged with the e^{m - m'} rescale; skip key tiles with
 * no allowed key).  Writes O (in `dtype`) and LSE = m + ln l (float32) only;
 * no n x n array is formed.
 *
 *   q, k, v   inputs as laid out above
 *   o, lse    outputs; lse is required (the backward consumes it)
 *   B, H, n   batch, heads, sequence length (>= 0; zero-sized calls do nothing)
 *   d, dv     head dims of q/k and of v/o
 *   dtype     element type of q, k, v and o
 *   scale     c, any finite float (c = 0 gives the mean of the allowed values)
 *   mask, window  allowed-key sets as above; window is read only for EIAT_MASK_WINDOW
 *   stream    hipStream_t or NULL
 */
EIAT_API eiat_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t H, int64_t n, int64_t d, int64_t dv, int dtype, float scale, int mask,
                     int64_t window, void *stream);

/* Bytes of device workspace attn_bwd needs: the per-row delta_i, B*H*n float32. */
EIAT_API size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t n);

/*
 * Backward pass: the Algorithm's reverse procedure with the forward's maxima
 * and normalisers frozen (carried here as lse).  First one kernel that holds a
 * query tile and streams key/value tiles (dQ); it also forms
 * delta_i = sum_a dO_ia O_ia of its rows and writes it to `workspace`.  Then one
 * that holds a key/value tile and streams the query tiles that may see it
 * (dK, dV), reading delta.  Each recomputes its score blocks from q, k and
 * lse: p_ij = e^{s_ij - LSE_i}, gamma_ij = p_ij (dO_i . V_j - delta_i),
 * dQ_i = c sum_j gamma_ij K_j, dK_j = c sum_i gamma_ij Q_i, dV_j = sum_i p_ij dO_i.
 *
 *   q, k, v, o, lse   the forward's inputs and outputs (o, lse from attn_fwd)
 *   dout              upstream gradient dO, [B][H][n][dv]
 *   dq, dk, dvv       outputs in `dtype`
 *   workspace         device memory of at least attn_bwd_workspace_bytes(B, H, n)
 *   workspace_bytes   its size
 * Other arguments as for attn_fwd and with the same values.
 */
EIAT_API eiat_status attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                     const float *lse, void *dq, void *dk, void *dvv, void *workspace,
                     size_t workspace_bytes, int64_t B, int64_t H, int64_t n, int64_t d,
                     int64_t dv, int dtype, float scale, int mask, int64_t window, void *stream);

/*
 * One step of the reverse procedure, for callers that schedule or time the
 * steps separately: stage 0 computes delta_i = sum_a dO_ia O_ia into
 * `workspace`; stage 1 computes dK and dV; stage 2 computes dQ and writes the
 * same delta into `workspace` (bit for bit what stage 0 writes).  Stage 1 reads
 * delta from `workspace`, so stage 0 or stage 2 must have run on the same
 * workspace (in stream order) first.  attn_bwd is stage 2 then stage 1.
 * Outputs a stage does not write are not read and may hold anything.  Arguments,
 * validation and errors are those of attn_bwd; an unknown stage is
 * EIAT_ERR_INVALID_ARG.
 */
EIAT_API eiat_status attn_bwd_stage(int stage, const void *q, const void *k, const void *v,
                                    const void *o, const void *dout, const float *lse, void *dq,
                                    void *dk, void *dvv, void *workspace, size_t workspace_bytes,
                                    int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                    int dtype, float scale, int mask, int64_t window,
                                    void *stream);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory around the call (code under stream or graph capture, tight
 * serving loops, harnesses that forbid allocation).  The per-row delta lives
 * instead in a fixed device array inside the library, one per GPU (16 MiB,
 * held from the first call on that GPU until the process ends), so the call
 * itself allocates nothing: it computes exactly what attn_bwd computes (same
 * kernels, bitwise the same dq, dk, dvv).
 *   Limit: B * H * n <= 4,194,304 rows; larger problems return
 *          EIAT_ERR_UNSUPPORTED (use attn_bwd with a workspace).
 *   Sharing: every call on a GPU uses that GPU's array, which keeps the last
 *          call's contents.  Calls that overlap in time on one GPU (different
 *          streams or host threads) race on it and must be serialized by the
 *          caller; calls on one stream are ordered by the stream.
 * Arguments, layout, validation and other errors as attn_bwd (workspace and
 * workspace_bytes are absent); a failure to look up the array's device
 * address is EIAT_ERR_HIP.
 */
EIAT_API eiat_status attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                                      const void *dout, const float *lse, void *dq, void *dk,
                                      void *dvv, int64_t B, int64_t H, int64_t n, int64_t d,
                                      int64_t dv, int dtype, float scale, int mask,
                                      int64_t window, void *stream);

/*
 * Forward and reverse with dropout on the attention weights.  The pages fix
 * only the requirement (alphabetamath.cc, Algorithm "Exact tiled softmax
 * attention with block-recomputed vector-Jacobian products", reverse
 * procedure): the base method has no dropout, and an extension must replay
 * the same realized mask in its reverse pass.  Here:
 *
 *     O_i = sum_j p_ij D_ij V_j,   D_ij = keep_ij * 256 / (256 - thr)
 *
 * with p_ij the undropped softmax weights (lse is the undropped log-normaliser)
 * and thr = round(256 * p_drop) clamped to 255 (drop probability thr / 256).
 * The realized mask is a function of (seed, b * H + h, i, j): row key
 * r_i = XXH32(seed_hi | b*H+h | i; seed_lo) (three little-endian 32-bit words,
 * XXH32 the 32-bit xxHash function), u = XXH32(j >> 2; r_i), keep_ij = byte
 * (j & 3) of u >= thr.  The reverse calls regenerate it; pass the same p_drop
 * and seed, and the o that the dropout forward wrote.  p_drop must be in
 * [0, 1); p_drop = 0 gives exactly attn_fwd / attn_bwd.  Other arguments,
 * layouts and errors as attn_fwd, attn_bwd and attn_bwd_stage.
 */
EIAT_API eiat_status attn_fwd_dropout(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t H, int64_t n, int64_t d,
                                      int64_t dv, int dtype, float scale, int mask,
                                      int64_t window, float p_drop, uint64_t seed, void *stream);

EIAT_API eiat_status attn_bwd_dropout(const void *q, const void *k, const void *v, const void *o,
                                      const void *dout, const float *lse, void *dq, void *dk,
                                      void *dvv, void *workspace, size_t workspace_bytes,
                                      int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                      int dtype, float scale, int mask, int64_t window,
                                      float p_drop, uint64_t seed, void *stream);

EIAT_API eiat_status attn_bwd_dropout_stage(int stage, const void *q, const void *k,
                                            const void *v, const void *o, const void *dout,
                                            const float *lse, void *dq, void *dk, void *dvv,
                                            void *workspace, size_t workspace_bytes, int64_t B,
                                            int64_t H, int64_t n, int64_t d, int64_t dv,
                                            int dtype, float scale, int mask, int64_t window,
                                            float p_drop, uint64_t seed, void *stream);

/*
 * Decode-shaped forward: a few new query rows per head against a long cache of
 * keys and values (the KV-cache setting of webturing.com.tr Principia,
 * "Bellek Duvarinin Fizigi", section on the KV cache and long context; the
 * rows are the dense definition above, computed as the merge of the stable
 * summaries of ranges of the cache, alphabetamath.cc Definition "Stable
 * summary of an attention key block").
 *
 *   q        [B][H][nq][d]   the last nq positions of each sequence
 *   k, v     [B][Hkv][nk][d], [B][Hkv][nk][dv]   keys and values of all nk positions
 *   o        [B][H][nq][dv]  (dtype), lse [B][H][nq] float32, natural logarithm
 *   workspace  device buffer of at least attn_decode_workspace_bytes(...) bytes;
 *            overwritten (the per-range summaries), no initial contents needed
 *
 * Row i of q sits at position nk - nq + i; its allowed keys are the mask's set
 * for that position (none: every cached key; causal: j <= nk - nq + i;
 * window: the last `window` keys up to that position).  H must be a multiple of
 * Hkv; query head h reads key/value head h / (H / Hkv) (Hkv == H: one each).
 * Requires 1 <= nq <= nk when B > 0 (B == 0 or nq == 0 does nothing).
 * Kernels: dtype F16 or BF16, d == dv in {64, 128}, (H / Hkv) * nq <= 32;
 * other valid arguments return EIAT_ERR_UNSUPPORTED.  Pointers 16-byte
 * aligned; outputs and workspace must not overlap inputs or each other.
 * Calls sharing one workspace on different streams race.
 */
EIAT_API size_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t nq,
                                            int64_t nk, int64_t dv);

EIAT_API eiat_status attn_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                                 void *workspace, size_t workspace_bytes, int64_t B, int64_t H,
                                 int64_t Hkv, int64_t nq, int64_t nk, int64_t d, int64_t dv,
                                 int dtype, float scale, int mask, int64_t window, void *stream);

/*
 * One step of attn_decode, for callers that schedule or time the steps
 * separately: stage 0 writes the summaries of the cache ranges into
 * `workspace`; stage 1 merges them into o and lse.  Same arguments and checks
 * as attn_decode (stage 1 reads the workspace stage 0 wrote for the same
 * shapes); an unknown stage returns EIAT_ERR_INVALID_ARG.
 */
EIAT_API eiat_status attn_decode_stage(int stage, const void *q, const void *k, const void *v,
                                       void *o, float *lse, void *workspace,
                                       size_t workspace_bytes, int64_t B, int64_t H, int64_t Hkv,
                                       int64_t nq, int64_t nk, int64_t d, int64_t dv, int dtype,
                                       float scale, int mask, int64_t window, void *stream);

/*
 * FP8 scores with block scaling and incoherent processing (webturing.com.tr
 * Principia, "Bellek Duvarinin Fizigi", section on FlashAttention-3: FP8, with
 * the precision loss held down by block scaling and random sign multipliers).
 *
 * attn_quant_fp8 turns rows x [rows][d] (dtype F32, F16 or BF16) into FP8
 * codes with one scale per 32 values:
 *   1. if signs is not NULL: x' = H (s * x), s_r = -1 where signs[r] < 0 and +1
 *      otherwise, H the unnormalized Sylvester Walsh-Hadamard matrix of order d
 *      (H H^T = d I), computed in float32 as butterfly stages of span 1, 2,
 *      4, ..., d/2, each pair (a, b) becoming (a + b, a - b); else x' = x;
 *   2. block b of a row (values 32 b .. 32 b + 31) gets e = the least integer
 *      >= -127 with max |x'| <= 448 * 2^e (e = 0 for an all-zero block);
 *      scales[row][b] = e + 127 (an E8M0 byte, the scale 2^e);
 *   3. codes[row][r] = the OCP FP8 e4m3 code (1 sign, 4 exponent bits with
 *      bias 7, 3 mantissa bits; largest 448) nearest to x'_r / 2^e, ties to
 *      even.
 * Rotate Q and K with the same signs: then Q' K'^T = d Q K^T, and the scale
 * for attn_fwd_fp8 is c / d.  x must be finite.  Requires d in {64, 128}
 * (other d >= 1: EIAT_ERR_UNSUPPORTED).  Device pointers, 16-byte aligned:
 * x, codes [rows][d] bytes, scales [rows][d / 32] bytes, signs [d] int8 (or
 * NULL); outputs must not overlap the inputs or each other.
 */
EIAT_API eiat_status attn_quant_fp8(const void *x, const int8_t *signs, uint8_t *codes,
                                    uint8_t *scales, int64_t rows, int64_t d, int dtype,
                                    void *stream);

/*
 * Forward with FP8 scores: the definition above with
 *     s_ij = scale * sum_r Qd_ir Kd_jr,   Qd_ir = e4m3(q[i][r]) * 2^(q_scale[i][r / 32] - 127)
 * (Kd likewise), i.e. attention of the dequantized rows, the score products
 * taken on the block-scaled FP8 matrix cores with float32 accumulation.  The
 * weights P and the value product stay in dtype (F16 or BF16) as in attn_fwd.
 *   q, k      [B][H][n][d] e4m3 codes;  q_scale, k_scale  [B][H][n][d / 32] E8M0
 *   v, o      [B][H][n][dv] dtype;      lse  [B][H][n] float32
 * Masks, errors and the rest as attn_fwd; kernels for d == dv in {64, 128}
 * and dtype F16 or BF16 (others: EIAT_ERR_UNSUPPORTED).  Codes 0x7F / 0xFF
 * (NaN) must not occur (attn_quant_fp8 never writes them).
 */
EIAT_API eiat_status attn_fwd_fp8(const uint8_t *q, const uint8_t *q_scale, const uint8_t *k,
                                  const uint8_t *k_scale, const void *v, void *o, float *lse,
                                  int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                                  int dtype, float scale, int mask, int64_t window, void *stream);

/*
 * FP8 weights and values as well (the FP8 throughput figure of the same
 * section is for both products of FlashAttention-3 in FP8).
 *
 * attn_quant_fp8_v writes v [BH][n][dv] (dtype F32, F16 or BF16), quantized
 * along the keys with the rule of attn_quant_fp8 (32-key blocks of one value
 * column, E8M0 scale, nearest e4m3 code; no rotation), in a tile-major layout:
 *   codes  [BH][nt][dv][64] bytes, nt = ceil(n / 64): row r of tile t holds
 *          value column r for keys 64 t .. 64 t + 63; key 64 t + 32 b + 8 g +
 *          4 h + i (b, h in 0..1; g, i in 0..3) is at byte 32 b + 16 h + 4 g + i
 *   scales [BH][nt][dv][2] bytes: scale of block b of row r of tile t
 * Keys past n count as zero (code 0x00; a block with no key below n has scale
 * byte 127).  Requires dv in {64, 128} (else EIAT_ERR_UNSUPPORTED).  Device
 * pointers, 16-byte aligned; outputs must not overlap v or each other.
 *
 * attn_fwd_fp8_pv is attn_fwd_fp8 with v, v_scale from attn_quant_fp8_v: the
 * value product P V runs on the block-scaled FP8 matrix cores too.  The
 * weights P are rounded to e4m3 for that product (relative error <= 2^-4, or
 * 2^-10 absolute below 2^-6 in units where the row's largest weight is >= 1);
 * the normaliser and LSE use the unrounded float32 weights.  O has dtype
 * (F16 or BF16).  Shapes, masks and errors as attn_fwd_fp8.
 */
EIAT_API eiat_status attn_quant_fp8_v(const void *v, uint8_t *codes, uint8_t *scales, int64_t BH,
                                      int64_t n, int64_t dv, int dtype, void *stream);

EIAT_API eiat_status attn_fwd_fp8_pv(const uint8_t *q, const uint8_t *q_scale, const uint8_t *k,
                                     const uint8_t *k_scale, const uint8_t *v,
                                     const uint8_t *v_scale, void *o, float *lse, int64_t B,
                                     int64_t H, int64_t n, int64_t d, int64_t dv, int dtype,
                                     float scale, int mask, int64_t window, void *stream);

/* Static string naming a status code. */
EIAT_API const char *attn_status_string(int status);

/* Thread-local detail of the calling thread's last non-OK return ("" if none). */
EIAT_API const char *attn_last_error(void);

/* EIAT_ABI_VERSION of the built library. */
EIAT_API int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EIAT_ATTN_H */
