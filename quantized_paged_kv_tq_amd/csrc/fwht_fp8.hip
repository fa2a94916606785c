// Hadamard-128 rotation + per-row power-of-two-scale FP8 quantizer
// (kpool_compress.py: fwht128_quant_fp8 and _fwht_quant_kernel).
//
// Per 128-wide bf16 row: fp32 butterflies (strides 1 -> 64), multiply by the
// fp32 value of 1/sqrt(128), round to bf16, absmax with a 1e-4 floor, scale =
// the power of two at or above absmax * fl(1/448), then E4M3 of
// clamp(x / scale, +-448). Eight lanes per row; lane l holds elements 8l..8l+7
// and 64+8l..64+8l+7 (two fully coalesced 16-byte loads per row); a 256-lane
// workgroup handles two passes of 32 rows.
//
// The ceiling of log2 is taken exactly from the exponent bits (the value is
// a power of two iff its mantissa bits are zero); division by the power-of-
// two scale is a multiplication by its exact reciprocal.
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

template <int R>
__global__ __launch_bounds__(256) void fwht128_fp8_kernel(const uint16_t* __restrict__ x_bf16,
                                                          int64_t rows,
                                                          uint8_t* __restrict__ y,
                                                          float* __restrict__ scale_out) {
  const int li = threadIdx.x & 7;  // 8 lanes per row, 16 elements per lane
  float sg[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sg[k] = (li >> k) & 1 ? -1.0f : 1.0f;
  // R passes of 32 rows; all loads are issued first
  float x[R][16];
  int64_t row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = ((int64_t)blockIdx.x * R + r) * 32 + (threadIdx.x >> 3);
    if (row[r] < rows) {
      // elements 8l .. 8l+7 and 64 + 8l .. 64 + 8l + 7
      const uint16_t* src = x_bf16 + row[r] * 128 + li * 8;
      const uint4 a = stream_load16(src);
      const uint4 b = stream_load16(src + 64);
      const uint32_t ws[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[r][2 * k] = bf16_lo(ws[k]);
        x[r][2 * k + 1] = bf16_hi(ws[k]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[r][j] = 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // strides 1, 2, 4 inside each half, 8 .. 32 across lanes, 64 between
    // the halves
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if ((j & h) == 0) {
          const float a = x[r][j], b = x[r][j + h];
          x[r][j] = a + b;
          x[r][j + h] = a - b;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[r][j] = butterfly16<1>(x[r][j], sg[0]);
      x[r][j] = butterfly16<2>(x[r][j], sg[1]);
      x[r][j] = butterfly16<4>(x[r][j], sg[2]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = x[r][j], b = x[r][j + 8];
      x[r][j] = a + b;
      x[r][j + 8] = a - b;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[r][j] = round_to_bf16_hw(x[r][j] * 0.08838834764831845f);
      amax = fmaxf(amax, fabsf(x[r][j]));
    }
    amax = group16_max<8>(amax);
    amax = (amax > 1e-4f) ? amax : 1e-4f;
    const uint32_t tb = f2u(amax * (float)(1.0 / 448.0));  // positive, normal
    const uint32_t sb = (tb & 0x7FFFFFu) ? ((tb & 0x7F800000u) + 0x00800000u) : tb;
    const float inv = u2f((254u << 23) - sb);  // exact 1 / scale
    // E4M3 by the hardware convert (round to nearest even; the operands are
    // clamped to the largest finite code first)
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = fminf(fmaxf(x[r][4 * k + j] * inv, -448.0f), 448.0f);
      uint32_t v = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
      w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], v, true);
    }
    if (row[r] < rows) {
      stream_store8(y + row[r] * 128 + li * 8, w[0], w[1]);
      stream_store8(y + row[r] * 128 + 64 + li * 8, w[2], w[3]);
      if (li == 0) stream_store4(scale_out + row[r], sb);
    }
  }
}

hipError_t launch_fwht128_fp8(const void* x, int64_t rows, uint8_t* y, float* scale,
                              hipStream_t st) {
  constexpr int R = 2;
  const int64_t blocks = (rows + 32 * R - 1) / (32 * R);
  hipLaunchKernelGGL((fwht128_fp8_kernel<R>), dim3((uint32_t)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), rows, y, scale);
  return hipGetLastError();
}

}  // namespace tqk
