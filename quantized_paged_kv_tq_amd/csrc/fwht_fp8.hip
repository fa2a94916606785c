// Hadamard-128 rotation + per-row power-of-two-scale FP8 quantizer
// (kpool_compress.py: fwht128_quant_fp8 and _fwht_quant_kernel).
//
// Per 128-wide bf16 row: fp32 butterflies (strides 1 -> 64), multiply by the
// fp32 value of 1/sqrt(128), round to bf16, absmax with a 1e-4 floor, scale =
// the power of two at or above absmax * fl(1/448), then E4M3 of
// clamp(x / scale, +-448). Sixteen lanes per row, eight elements per lane;
// a 256-lane workgroup handles 16 rows.
//
// The ceiling of log2 is taken exactly from the exponent bits (the value is
// a power of two iff its mantissa bits are zero); division by the power-of-
// two scale is a multiplication by its exact reciprocal.
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

__global__ __launch_bounds__(256) void fwht128_fp8_kernel(const uint16_t* __restrict__ x_bf16,
                                                          int64_t rows,
                                                          uint8_t* __restrict__ y,
                                                          float* __restrict__ scale_out) {
  const int li = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = row < rows;
  float x[8];
  if (valid) {
    const uint4 w = *reinterpret_cast<const uint4*>(x_bf16 + row * 128 + li * 8);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.0f;
  }
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & h) == 0) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = butterfly_lanes<1>(x[j], li & 1);
    x[j] = butterfly_lanes<2>(x[j], li & 2);
    x[j] = butterfly_lanes<4>(x[j], li & 4);
    x[j] = butterfly_lanes<8>(x[j], li & 8);
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = round_to_bf16(x[j] * 0.08838834764831845f);
    amax = fmaxf(amax, fabsf(x[j]));
  }
  amax = group_max<16>(amax);
  amax = (amax > 1e-4f) ? amax : 1e-4f;
  const uint32_t tb = f2u(amax * (float)(1.0 / 448.0));  // positive, normal
  const uint32_t sb = (tb & 0x7FFFFFu) ? ((tb & 0x7F800000u) + 0x00800000u) : tb;
  const float inv = u2f((254u << 23) - sb);  // exact 1 / scale
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= f32_to_e4m3_sat448(fminf(fmaxf(x[j] * inv, -448.0f), 448.0f)) << (8 * j);
    hi |= f32_to_e4m3_sat448(fminf(fmaxf(x[j + 4] * inv, -448.0f), 448.0f)) << (8 * j);
  }
  if (valid) {
    *reinterpret_cast<uint2*>(y + row * 128 + li * 8) = make_uint2(lo, hi);
    if (li == 0) scale_out[row] = u2f(sb);
  }
}

hipError_t launch_fwht128_fp8(const void* x, int64_t rows, uint8_t* y, float* scale,
                              hipStream_t st) {
  const int64_t blocks = (rows + 15) / 16;
  hipLaunchKernelGGL(fwht128_fp8_kernel, dim3((uint32_t)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), rows, y, scale);
  return hipGetLastError();
}

}  // namespace tqk
