// Row helpers of the cache writers: loading a source row into the lane
// layout of the writers and the fp32 FWHT over it.
//
// A row of D elements is spread over D/16 consecutive lanes; lane l holds
// elements 8l .. 8l+7 and D/2 + 8l .. D/2 + 8l + 7 (x[0..7] and x[8..15]).
// Butterfly strides 1, 2, 4 run inside each half of the lane, strides
// 8 .. D/4 pair lanes whose index differs by stride/8, and stride D/2 pairs
// the two halves: strides run 1 -> D/2, the order that fixes the fp32
// rounding of every sum.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

// 8 consecutive source elements -> fp32
template <int DT>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t elem, float x[8]) {
  if constexpr (DT == TQ_DT_BF16 || DT == TQ_DT_F16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == TQ_DT_BF16) {
        x[2 * k] = bf16_lo(ws[k]);
        x[2 * k + 1] = bf16_hi(ws[k]);
      } else {
        x[2 * k] = half_lo(ws[k]);
        x[2 * k + 1] = half_hi(ws[k]);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// FWHT of a row held as two 8-element halves per lane over LPR lanes (sg[k]
// = +1 / -1 for the lower / upper lane of lane distance 2^k).
template <int LPR>
__device__ __forceinline__ void fwht_row(float x[16], const float sg[3]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if constexpr (LPR >= 2) x[j] = butterfly16<1>(x[j], sg[0]);
    if constexpr (LPR >= 4) x[j] = butterfly16<2>(x[j], sg[1]);
    if constexpr (LPR >= 8) x[j] = butterfly16<4>(x[j], sg[2]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = x[j], b = x[j + 8];
    x[j] = a + b;
    x[j + 8] = a - b;
  }
}

}  // namespace tqk
