// Fused randomized-Hadamard rotation + INT4 per-(token, head) cache write
// (int4_per_token_head.py: reshape_and_cache_int4, single_rht and
// _reshape_cache_int4_kernel), one pass over K and V.
//
// The pages run this as three passes (rotate K, rotate V, quantize) with the
// rotated tensors in memory; here each source row is read once, rotated in
// registers and written straight into the paged cache.
//
// Lane layout: a row of D elements is spread over D/8 consecutive lanes,
// 8 elements per lane (element i = 8 * lane_in_row + j). Butterfly strides
// 1, 2, 4 run inside a lane; strides 8 .. D/2 pair lanes whose index differs
// by stride/8. Strides run 1 -> D/2, the order that fixes the fp32 rounding.
//
// Bit exactness: compiled without fp contraction; the one fused multiply-add
// of the quantizer is explicit, division and reciprocal are IEEE.
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

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

// FWHT of a row held as 8 elements per lane over LPR lanes.
template <int LPR>
__device__ __forceinline__ void fwht_row(float x[8], int li) {
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
    if constexpr (LPR >= 2) x[j] = butterfly_lanes<1>(x[j], li & 1);
    if constexpr (LPR >= 4) x[j] = butterfly_lanes<2>(x[j], li & 2);
    if constexpr (LPR >= 8) x[j] = butterfly_lanes<4>(x[j], li & 4);
    if constexpr (LPR >= 16) x[j] = butterfly_lanes<8>(x[j], li & 8);
  }
}

// Quantize one rotated row (8 elements per lane) and store its 4 packed bytes
// per lane and the scale word.
template <int LPR>
__device__ __forceinline__ void quantize_store(const float x[8], int li, bool valid,
                                               uint8_t* __restrict__ cache_row,
                                               float* __restrict__ word_out) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, x[j]);
    mx = fmaxf(mx, x[j]);
  }
  mn = group_min<LPR>(mn);
  mx = group_max<LPR>(mx);
  float scale = (mx - mn) / 15.0f;
  scale = (scale > 1e-6f) ? scale : 1e-6f;
  // The page rounds half away from zero and clamps to [0, 15]; for a
  // negative argument both of its branches end at 0, so one truncation of
  // clamp(t + 0.5, 0, 15) gives the same integer for every t.
  const float u = -mn / scale;
  const float zp = __builtin_truncf(fminf(fmaxf(u + 0.5f, 0.0f), 15.0f));
  const float inv = 1.0f / scale;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = __builtin_fmaf(x[j], inv, zp);
    const uint32_t q = (uint32_t)fminf(fmaxf(t + 0.5f, 0.0f), 15.0f);
    packed |= q << (4 * j);
  }
  if (valid) {
    *reinterpret_cast<uint32_t*>(cache_row + 4 * li) = packed;
    if (li == 0) *word_out = u2f((f2u(scale) & 0xFFFFFFF0u) | (uint32_t)zp);
  }
}

// One workgroup of 256 lanes handles 256 / (D/8) rows; row r of the launch is
// (item = r / 2, K if r even else V), item = t * Hk + h.
template <int D, int DT>
__global__ __launch_bounds__(256) void reshape_int4_kernel(
    const void* __restrict__ key, const void* __restrict__ value,
    const int64_t* __restrict__ slots, const float* __restrict__ signs,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, int64_t total_rows, int hk, int64_t cache_slots) {
  constexpr int LPR = D / 8;
  constexpr int ROWS = 256 / LPR;
  const int li = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * ROWS + threadIdx.x / LPR;
  const bool in_range = row < total_rows;
  const int64_t item = in_range ? (row >> 1) : 0;
  const bool is_v = row & 1;
  const int64_t t = item / hk;
  const int h = (int)(item - t * hk);
  const int64_t slot = in_range ? slots[t] : -1;
  const bool valid = in_range && slot >= 0 && slot < cache_slots;

  float x[8];
  if (valid) {
    load8<DT>(is_v ? value : key, item * D + li * 8, x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.0f;
  }
  const float4 s0 = reinterpret_cast<const float4*>(signs + li * 8)[0];
  const float4 s1 = reinterpret_cast<const float4*>(signs + li * 8)[1];
  x[0] *= s0.x; x[1] *= s0.y; x[2] *= s0.z; x[3] *= s0.w;
  x[4] *= s1.x; x[5] *= s1.y; x[6] *= s1.z; x[7] *= s1.w;
  fwht_row<LPR>(x, li);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (DT == TQ_DT_BF16) x[j] = round_to_bf16(x[j]);
    else if constexpr (DT == TQ_DT_F16) x[j] = round_to_f16(x[j]);
  }
  const int64_t dst = (valid ? slot : 0) * hk + h;
  uint8_t* cache = is_v ? vc : kc;
  float* words = is_v ? vs : ks;
  quantize_store<LPR>(x, li, valid, cache + dst * (D / 2), words + dst);
}

template <int D, int DT>
static hipError_t launch_reshape(const ReshapeParams& p, hipStream_t st) {
  constexpr int ROWS = 256 / (D / 8);
  const int64_t total_rows = p.num_tokens * p.hk * 2;
  const int64_t blocks = (total_rows + ROWS - 1) / ROWS;
  hipLaunchKernelGGL((reshape_int4_kernel<D, DT>), dim3((uint32_t)blocks), dim3(256), 0, st,
                     p.key, p.value, p.slots, p.signs, p.kc, p.vc, p.ks, p.vs, total_rows,
                     p.hk, p.num_blocks * (int64_t)p.block_size);
  return hipGetLastError();
}

hipError_t launch_reshape_int4(const ReshapeParams& p, hipStream_t st) {
  if (p.d == 128) {
    if (p.dtype == TQ_DT_BF16) return launch_reshape<128, TQ_DT_BF16>(p, st);
    if (p.dtype == TQ_DT_F16) return launch_reshape<128, TQ_DT_F16>(p, st);
    return launch_reshape<128, TQ_DT_F32>(p, st);
  }
  if (p.dtype == TQ_DT_BF16) return launch_reshape<64, TQ_DT_BF16>(p, st);
  if (p.dtype == TQ_DT_F16) return launch_reshape<64, TQ_DT_F16>(p, st);
  return launch_reshape<64, TQ_DT_F32>(p, st);
}

}  // namespace tqk
