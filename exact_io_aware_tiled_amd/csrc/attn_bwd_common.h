// attn_bwd_common.h -- device helpers shared by the two backward translation
// units (attn_bwd.hip: delta and dK/dV; attn_bwd_dq.hip: dQ).
#pragma once

#include <type_traits>

#include "attn_device.h"

namespace eiat {

// Stage ROWS consecutive rows of a [n][D] slice into LDS: a natural copy (row
// stride NROW bytes) and/or a transposed copy (DP rows of ROWS elements, stride
// TROW bytes).  Each task is 4 rows x 16 bytes; rows >= n read as zero.
template <typename T, int D, int ROWS, int THREADS, int NROW, int TROW, bool NAT, bool TR>
struct Stager {
  static constexpr int S = Elt<T>::kBytes;
  static constexpr int CPR = D * S / 16;
  static constexpr int EPC = 16 / S;
  static constexpr int TASKS = (ROWS / 4) * CPR;
  static constexpr int PT = (TASKS + THREADS - 1) / THREADS;
  u32x4 reg[PT][4];

  __device__ inline void load(const char* base, int r0, int n, int tid) {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int task = tid + p * THREADS;
      if (task < TASKS) {
        const int rq = task / CPR, col = task % CPR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + 4 * rq + i;
          reg[p][i] = r < n ? ldg16(base + (int64_t)r * D * S + col * 16) : zero4();
        }
      }
    }
  }

  __device__ inline void store(char* nat, char* tr, int tid) {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int task = tid + p * THREADS;
      if (task < TASKS) {
        const int rq = task / CPR, col = task % CPR;
        if constexpr (NAT) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(nat + (4 * rq + i) * NROW + col * 16) = reg[p][i];
        }
        if constexpr (TR) store_transposed4<T>(tr + (col * EPC) * TROW + 4 * rq * S, TROW, reg[p]);
      }
    }
  }
};

// Zero columns [D, DP) of every row of a natural tile (only when D < 32): the
// transpose reads of output rows [D, DP) then see zeros.
template <int D, int DP, int S, int ROWS, int NROW, int THREADS>
__device__ inline void zero_pad_cols(char* nat, int tid) {
  if constexpr (DP > D) {
    constexpr int per_row = (DP - D) * S / 16;
    for (int idx = tid; idx < ROWS * per_row; idx += THREADS)
      *reinterpret_cast<u32x4*>(nat + (idx / per_row) * NROW + D * S + (idx % per_row) * 16) = zero4();
  }
}

// Zero rows [D, DP) of a transposed tile (only when D < 32).
template <int D, int DP, int TROW, int THREADS>
__device__ inline void zero_pad_rows(char* tr, int tid) {
  if constexpr (DP > D) {
    constexpr int per_row = TROW / 16;
    for (int idx = tid; idx < (DP - D) * per_row; idx += THREADS)
      *reinterpret_cast<u32x4*>(tr + (D + idx / per_row) * TROW + (idx % per_row) * 16) = zero4();
  }
}

// Dot product of one 16-byte unit of an O row with the same unit of its dO row:
// fused multiply-adds in element order, starting from zero.  A row's delta is
// the sum of its units' dots in a fixed tree: unit u is first added to unit
// u ^ (units / 2), then u ^ (units / 4), ..., and last u ^ 1.  The delta kernel
// and the dQ kernel both follow it, so they give the same bits.
template <typename T>
__device__ inline float unit_dot(const u32x4& a, const u32x4& b) {
  float acc = 0.0f;
  if constexpr (Elt<T>::kBytes == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float a0, a1, b0, b1;
      if constexpr (__is_same(T, __bf16)) {
        a0 = __uint_as_float(a[w] << 16);
        a1 = __uint_as_float(a[w] & 0xFFFF0000u);
        b0 = __uint_as_float(b[w] << 16);
        b1 = __uint_as_float(b[w] & 0xFFFF0000u);
      } else {
        // copy the elements out first: a bit-cast applied directly to a vector
        // element was compiled into a read of element 0
        const uint32_t aw = a[w], bw = b[w];
        const f16x2 ah = __builtin_bit_cast(f16x2, aw), bh = __builtin_bit_cast(f16x2, bw);
        a0 = (float)ah[0];
        a1 = (float)ah[1];
        b0 = (float)bh[0];
        b1 = (float)bh[1];
      }
      acc = __builtin_fmaf(a0, b0, acc);
      acc = __builtin_fmaf(a1, b1, acc);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_fmaf(__uint_as_float(a[w]), __uint_as_float(b[w]), acc);
  }
  return acc;
}

// Whether a tile body applies the per-element mask: a compile-time flag
// (std::true_type / std::false_type) or a run-time one (bool).
__device__ inline bool mask_on(bool m) { return m; }
template <bool B>
__device__ constexpr bool mask_on(std::integral_constant<bool, B>) { return B; }

}  // namespace eiat
