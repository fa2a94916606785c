// Fused randomized-Hadamard rotation + INT4 per-(token, head) cache write
// (int4_per_token_head.py: reshape_and_cache_int4, single_rht and
// _reshape_cache_int4_kernel), one pass over K and V.
//
// The pages run this as three passes (rotate K, rotate V, quantize) with the
// rotated tensors in memory; here each source row is read once, rotated in
// registers and written straight into the paged cache.
//
// Lane layout: a row of D elements is spread over D/16 consecutive lanes,
// 16 elements per lane (element i = 16 * lane_in_row + j). Butterfly strides
// 1, 2, 4, 8 run inside a lane; strides 16 .. D/2 pair lanes whose index
// differs by stride/16 (DPP moves). Strides run 1 -> D/2, the order that
// fixes the fp32 rounding. A lane packs its 16 codes into 8 bytes.
//
// Bit exactness: compiled without fp contraction; the one fused multiply-add
// of the quantizer is explicit, division and reciprocal are IEEE.
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

// 16 consecutive source elements -> fp32
template <int DT>
__device__ __forceinline__ void load16(const void* __restrict__ base, int64_t elem, float x[16]) {
  if constexpr (DT == TQ_DT_BF16 || DT == TQ_DT_F16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint4 a = p[0], b = p[1];
    const uint32_t ws[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
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
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = p[k];
      x[4 * k] = a.x; x[4 * k + 1] = a.y; x[4 * k + 2] = a.z; x[4 * k + 3] = a.w;
    }
  }
}

// FWHT of a row held as 16 elements per lane over LPR lanes: strides 1 .. 8
// inside the lane, then 16 .. D/2 across lanes (sg[k] = +1 / -1 for the
// lower / upper lane of lane distance 2^k).
template <int LPR>
__device__ __forceinline__ void fwht_row(float x[16], const float sg[3]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
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
}

// Quantize one rotated row (16 elements per lane) and store the lane's 8
// packed bytes and the scale word.
template <int LPR>
__device__ __forceinline__ void quantize_store(const float x[16], int li, bool valid,
                                               uint8_t* __restrict__ cache_row,
                                               float* __restrict__ word_out) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) {
    mn = fminf(mn, x[j]);
    mx = fmaxf(mx, x[j]);
  }
  mn = group16_min<LPR>(mn);
  mx = group16_max<LPR>(mx);
  float scale = (mx - mn) / 15.0f;
  scale = (scale > 1e-6f) ? scale : 1e-6f;
  // The page rounds half away from zero and clamps to [0, 15]; for a
  // negative argument both of its branches end at 0, so one truncation of
  // clamp(t + 0.5, 0, 15) gives the same integer for every t.
  const float u = -mn / scale;
  const float zp = __builtin_truncf(__builtin_amdgcn_fmed3f(u + 0.5f, 0.0f, 15.0f));
  const float inv = 1.0f / scale;
  uint32_t packed[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float t = __builtin_fmaf(x[j], inv, zp);
    const uint32_t q = (uint32_t)__builtin_amdgcn_fmed3f(t + 0.5f, 0.0f, 15.0f);
    packed[j >> 3] |= q << (4 * (j & 7));
  }
  if (valid) {
    *reinterpret_cast<uint2*>(cache_row + 8 * li) = make_uint2(packed[0], packed[1]);
    if (li == 0) *word_out = u2f((f2u(scale) & 0xFFFFFFF0u) | (uint32_t)zp);
  }
}

// One workgroup of 256 lanes handles R passes of 256 / (D/16) rows; row r
// is (item = r / 2, K if r even else V), item = t * Hk + h. Every pass's
// loads are issued before the first row is transformed.
template <int D, int DT, int R>
__global__ __launch_bounds__(256) void reshape_int4_kernel(
    const void* __restrict__ key, const void* __restrict__ value,
    const int64_t* __restrict__ slots, const float* __restrict__ signs,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, int64_t total_rows, int hk, int64_t cache_slots) {
  constexpr int LPR = D / 16;
  constexpr int ROWS = 256 / LPR;
  const int li = threadIdx.x % LPR;
  float sg[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sg[k] = (li >> k) & 1 ? -1.0f : 1.0f;

  float x[R][16];
  int64_t dst[R];
  bool valid[R], is_v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = ((int64_t)blockIdx.x * R + r) * ROWS + threadIdx.x / LPR;
    const bool in_range = row < total_rows;
    const int64_t item = in_range ? (row >> 1) : 0;
    is_v[r] = row & 1;
    const int64_t t = item / hk;
    const int h = (int)(item - t * hk);
    const int64_t slot = in_range ? slots[t] : -1;
    valid[r] = in_range && slot >= 0 && slot < cache_slots;
    dst[r] = (valid[r] ? slot : 0) * hk + h;
    if (valid[r]) {
      load16<DT>(is_v[r] ? value : key, item * D + li * 16, x[r]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[r][j] = 0.0f;
    }
  }
  float s[16];
  {
    const float4* sp = reinterpret_cast<const float4*>(signs + li * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = sp[k];
      s[4 * k] = a.x; s[4 * k + 1] = a.y; s[4 * k + 2] = a.z; s[4 * k + 3] = a.w;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[r][j] *= s[j];
    fwht_row<LPR>(x[r], sg);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (DT == TQ_DT_BF16) x[r][j] = round_to_bf16_hw(x[r][j]);
      else if constexpr (DT == TQ_DT_F16) x[r][j] = round_to_f16(x[r][j]);
    }
    uint8_t* cache = is_v[r] ? vc : kc;
    float* words = is_v[r] ? vs : ks;
    quantize_store<LPR>(x[r], li, valid[r], cache + dst[r] * (D / 2), words + dst[r]);
  }
}

template <int D, int DT>
static hipError_t launch_reshape(const ReshapeParams& p, hipStream_t st) {
  constexpr int R = 2;
  constexpr int ROWS = 256 / (D / 16);
  const int64_t total_rows = p.num_tokens * p.hk * 2;
  const int64_t blocks = (total_rows + ROWS * R - 1) / (ROWS * R);
  hipLaunchKernelGGL((reshape_int4_kernel<D, DT, R>), dim3((uint32_t)blocks), dim3(256), 0, st,
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
