// Fused randomized-Hadamard rotation + INT4 per-(token, head) cache write
// (int4_per_token_head.py: reshape_and_cache_int4, single_rht and
// _reshape_cache_int4_kernel), one pass over K and V.
//
// The pages run this as three passes (rotate K, rotate V, quantize) with the
// rotated tensors in memory; here each source row is read once, rotated in
// registers and written straight into the paged cache.
//
// Lane layout: a row of D elements is spread over D/16 consecutive lanes;
// lane l holds elements 8l .. 8l+7 and D/2 + 8l .. D/2 + 8l + 7, so that each
// of its two 16-byte loads (bf16) is part of one contiguous 128-byte span per
// row. Butterfly strides 1, 2, 4 run inside each half of the lane, strides
// 8 .. D/4 pair lanes whose index differs by stride/8 (DPP moves), and
// stride D/2 pairs the two halves inside the lane: strides run 1 -> D/2, the
// order that fixes the fp32 rounding. A lane packs its codes into two
// 4-byte words (bytes 4l and D/4 + 4l of the packed row); neighbouring
// lanes swap one word so that each stores 8 contiguous bytes.
//
// Bit exactness: compiled without fp contraction; the one fused multiply-add
// of the quantizer is explicit, division and reciprocal are IEEE.
#include "tq_device.h"
#include "tq_internal.h"
#include "write_rows.h"

namespace tqk {

// Quantize one rotated row (two 8-element halves per lane) and store the
// lane's two packed words and the scale word.
template <int D, int LPR>
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
  // Lanes 2m and 2m+1 hold bytes 8m..8m+7 of the first half as packed[0]
  // and of the second half as packed[1]; swapping one word gives lane 2m
  // the first-half 8 bytes and lane 2m+1 the second-half 8 bytes, stored
  // with one 8-byte store each.
  const bool odd = li & 1;
  const uint32_t give = odd ? packed[0] : packed[1];
  const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, 0xB1, 0xF, 0xF, false);
  const uint2 out = odd ? make_uint2(got, packed[1]) : make_uint2(packed[0], got);
  if (valid) {
    *reinterpret_cast<uint2*>(cache_row + (odd ? D / 4 : 0) + 8 * (li >> 1)) = out;
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

  // The source rows are loaded without waiting for their slots (a skipped
  // row's values are read and discarded), so both loads are in flight
  // together.
  float x[R][16];
  int64_t slot[R], dst[R];
  int head[R];
  bool valid[R], is_v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = ((int64_t)blockIdx.x * R + r) * ROWS + threadIdx.x / LPR;
    const bool in_range = row < total_rows;
    const int64_t item = in_range ? (row >> 1) : 0;
    is_v[r] = row & 1;
    // token and head of the item (32-bit division: items < 2^31)
    const uint32_t it32 = (uint32_t)item;
    const int64_t t = (int64_t)(it32 / (uint32_t)hk);
    head[r] = (int)(it32 - (uint32_t)t * (uint32_t)hk);
    slot[r] = in_range ? slots[t] : -1;
    const void* src = is_v[r] ? value : key;
    load8<DT>(src, item * D + li * 8, x[r]);
    load8<DT>(src, item * D + D / 2 + li * 8, x[r] + 8);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    valid[r] = slot[r] >= 0 && slot[r] < cache_slots;
    dst[r] = (valid[r] ? slot[r] : 0) * hk + head[r];
  }
  float s[16];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float4* sp = reinterpret_cast<const float4*>(signs + hf * (D / 2) + li * 8);
    const float4 a = sp[0], b = sp[1];
    s[8 * hf + 0] = a.x; s[8 * hf + 1] = a.y; s[8 * hf + 2] = a.z; s[8 * hf + 3] = a.w;
    s[8 * hf + 4] = b.x; s[8 * hf + 5] = b.y; s[8 * hf + 6] = b.z; s[8 * hf + 7] = b.w;
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
    quantize_store<D, LPR>(x[r], li, valid[r], cache + dst[r] * (D / 2), words + dst[r]);
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
