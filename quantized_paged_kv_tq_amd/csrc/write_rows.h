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
    const uint4 w = stream_load16(static_cast<const uint16_t*>(base) + elem);
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
// = +1 / -1 for the lower / upper lane of lane distance 2^k; LPR <= 16).
template <int LPR>
__device__ __forceinline__ void fwht_row(float x[16], const float sg[4]) {
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
    if constexpr (LPR >= 16) x[j] = butterfly16<8>(x[j], sg[3]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = x[j], b = x[j + 8];
    x[j] = a + b;
    x[j + 8] = a - b;
  }
}

// ---------------------------------------------------------------------------
// Two lanes per row (quarter layout, write_int4.hip): the cross-lane
// butterfly is a DPP fused multiply-add with the partner lane.

// x[i] += (x[i] of lane ^ 1) * s for eight values: one v_fmac_f32 with a DPP
// operand each. With s = +1 in lane 0 and -1 in lane 1 this is the
// cross-lane butterfly, except that lane 1 receives the negated difference
// x1 - x0 (exact: sign flips commute with rounding). Every lane of the wave must be
// active. The s_nop covers the wait states a DPP read needs after a VALU
// write of its operand or of EXEC.
__device__ __forceinline__ void fmac_partner8(float* x, float s) {
  asm("s_nop 4\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
      : "v"(s));
}

// In-place butterfly (a, b) -> (a + b, a - b), the two instructions kept
// together so that a butterfly holds one extra register while it runs (the
// scheduler would otherwise issue many sums ahead of their differences and
// hold all the pairs live).
__device__ __forceinline__ void bfly(float& a, float& b) {
  float u;
  asm("v_add_f32 %0, %2, %3\n\tv_sub_f32 %1, %2, %3" : "=&v"(u), "=v"(b) : "v"(a), "v"(b));
  a = u;
}

// FWHT over the quarter layout (lane q holds chunks (m mod M/2) + q M/2 +
// M (m div M/2), M = D/16) from the state after stride 1: strides 2, 4 in
// a chunk, 8 .. D/8 across lane-local chunks m ^ 1 .., D/4 across the lane
// pair (DPP, leaving lane 1 negated), D/2 across m ^ M/2 in the lane (on
// lane 1's negated values, which stays exact).
template <int D>
__device__ __forceinline__ void fwht_quarters_from_stride2(float (&x)[D / 2], int q) {
  constexpr int M = D / 16;
#pragma unroll
  for (int h = 2; h < 8; h <<= 1)
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((j & h) == 0) bfly(x[8 * m + j], x[8 * m + j + h]);
#pragma unroll
  for (int hm = 1; hm < M / 2; hm <<= 1)
#pragma unroll
    for (int m = 0; m < M; ++m)
      if ((m & hm) == 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) bfly(x[8 * m + j], x[8 * (m + hm) + j]);
  const float s = q ? -1.0f : 1.0f;
#pragma unroll
  for (int m = 0; m < M; ++m) fmac_partner8(x + 8 * m, s);
#pragma unroll
  for (int m = 0; m < M / 2; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) bfly(x[8 * m + j], x[8 * (m + M / 2) + j]);
}

// Round one fp32 value to bfloat16 (nearest even) and back with a single
// packed convert whose other half is the constant 0: the converted value
// lands in the upper 16 bits over a zero lower half, which is its fp32
// encoding.
__device__ __forceinline__ float round1_bf16(float a) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {0.0f, a};
  return u2f(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2)));
}

}  // namespace tqk
