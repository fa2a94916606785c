// Fused randomized-Hadamard rotation + INT4 per-(token, head) cache write
// (int4_per_token_head.py: reshape_and_cache_int4, single_rht and
// _reshape_cache_int4_kernel), one pass over K and V.
//
// The pages run this as three passes (rotate K, rotate V, quantize) with the
// rotated tensors in memory; here each source row is read once, rotated in
// registers and written straight into the paged cache.
//
// Lane layout (write_rows.h, pair layout): two lanes per row; lane q holds
// the 8-element chunks 2m + q. The RHT sign flips are XOR masks on the
// packed 16-bit source words (from LDS), fused with unpacking and the
// stride-1 butterflies; the stride-8 butterflies cross the lane pair as one
// DPP fused multiply-add per element, which leaves lane 1 with the negated
// transform. The negation is folded into the row's min / max and into the
// quantizer's reciprocal (sign flips are exact), so the codes are those of
// the plain transform (the sign of an exact zero, which the negation does
// not carry, changes no code and no scale word). Each lane packs its 8 chunks into 8 words (word c of
// the packed row is chunk c); one word exchange per pair of words gives lane
// 0 the first and lane 1 the second half of the packed row.
//
// Bit exactness: the FWHT strides run 1 -> D/2 in fp32 with one rounding per
// butterfly, as the pages' transform; the file is compiled without fp
// contraction; the one fused multiply-add of the quantizer is explicit;
// division and reciprocal are IEEE.
#include "tq_device.h"
#include "tq_internal.h"
#include "write_rows.h"

namespace tqk {

namespace {

// One workgroup of 256 lanes handles 128 rows; row r is (item = r / 2, K if
// r even else V), item = t * Hk + h.
template <int D, int DT>
__global__ __launch_bounds__(256) void reshape_int4_kernel(
    const void* __restrict__ key, const void* __restrict__ value,
    const int64_t* __restrict__ slots, const float* __restrict__ signs,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, int64_t total_rows, int hk, int64_t cache_slots) {
  constexpr int M = D / 16;  // chunks per lane
  constexpr int NE = D / 2;  // elements per lane
  constexpr bool kHalf = DT == TQ_DT_BF16 || DT == TQ_DT_F16;
  // RHT signs: XOR masks of the packed 16-bit pairs, or the fp32 signs
  __shared__ __attribute__((aligned(16))) uint32_t smask[kHalf ? D / 2 : D];
  if (threadIdx.x < (kHalf ? D / 2 : D)) {
    if constexpr (kHalf) {
      const float2 sp = reinterpret_cast<const float2*>(signs)[threadIdx.x];
      smask[threadIdx.x] = (sp.x < 0.0f ? 0x8000u : 0u) | (sp.y < 0.0f ? 0x80000000u : 0u);
    } else {
      smask[threadIdx.x] = f2u(signs[threadIdx.x]);
    }
  }

  const int q = threadIdx.x & 1;
  const int64_t row = (int64_t)blockIdx.x * 128 + (threadIdx.x >> 1);
  const bool in_range = row < total_rows;
  const int64_t item = in_range ? (row >> 1) : 0;
  const bool is_v = row & 1;
  // token and head of the item (32-bit division: items < 2^31)
  const uint32_t it32 = (uint32_t)item;
  const uint32_t t = it32 / (uint32_t)hk;
  const int head = (int)(it32 - t * (uint32_t)hk);
  // the source row is loaded without waiting for the slot (a skipped row's
  // values are read and discarded)
  const int64_t slot = in_range ? slots[t] : -1;
  const char* src = static_cast<const char*>(is_v ? value : key);
  constexpr int ES = kHalf ? 2 : 4;  // source element bytes
  uint4 raw[M][kHalf ? 1 : 2];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (item * D + 8 * (2 * m + q)) * ES);
    raw[m][0] = p[0];
    if constexpr (!kHalf) raw[m][1] = p[1];
  }
  __syncthreads();  // smask

  // signs, unpacking and the stride-1 butterflies
  float x[NE];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = 2 * m + q;
    if constexpr (kHalf) {
      const uint4 mk = *reinterpret_cast<const uint4*>(&smask[4 * c]);
      const uint32_t w[4] = {raw[m][0].x ^ mk.x, raw[m][0].y ^ mk.y, raw[m][0].z ^ mk.z, raw[m][0].w ^ mk.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = DT == TQ_DT_BF16 ? bf16_lo(w[k]) : half_lo(w[k]);
        const float b = DT == TQ_DT_BF16 ? bf16_hi(w[k]) : half_hi(w[k]);
        x[8 * m + 2 * k] = a + b;
        x[8 * m + 2 * k + 1] = a - b;
      }
    } else {
      const uint4 s0 = *reinterpret_cast<const uint4*>(&smask[8 * c]);
      const uint4 s1 = *reinterpret_cast<const uint4*>(&smask[8 * c + 4]);
      const uint32_t w[8] = {raw[m][0].x, raw[m][0].y, raw[m][0].z, raw[m][0].w,
                             raw[m][1].x, raw[m][1].y, raw[m][1].z, raw[m][1].w};
      const uint32_t sg[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = u2f(w[2 * k]) * u2f(sg[2 * k]);
        const float b = u2f(w[2 * k + 1]) * u2f(sg[2 * k + 1]);
        x[8 * m + 2 * k] = a + b;
        x[8 * m + 2 * k + 1] = a - b;
      }
    }
  }
  fwht_pair_from_stride2<D>(x, q);  // lane 1 now holds the negated values

  // the source dtype's rounding of the rotated row (symmetric in sign)
  if constexpr (DT == TQ_DT_BF16) {
#pragma unroll
    for (int i = 0; i < NE; i += 2) round2_bf16(x[i], x[i + 1]);
  } else if constexpr (DT == TQ_DT_F16) {
#pragma unroll
    for (int i = 0; i < NE; ++i) x[i] = round_to_f16(x[i]);
  }

  // row minimum and maximum of the true values
  float hmn = x[0], hmx = x[0];
#pragma unroll
  for (int i = 1; i < NE; ++i) {
    hmn = fminf(hmn, x[i]);
    hmx = fmaxf(hmx, x[i]);
  }
  float mn = q ? -hmx : hmn, mx = q ? -hmn : hmx;
  mn = fminf(mn, dpp_xor<1>(mn));
  mx = fmaxf(mx, dpp_xor<1>(mx));
  float scale = (mx - mn) / 15.0f;
  scale = (scale > 1e-6f) ? scale : 1e-6f;
  // The page rounds half away from zero and clamps to [0, 15]; for a
  // negative argument both of its branches end at 0, so one truncation of
  // clamp(t + 0.5, 0, 15) gives the same integer for every t.
  const float u = -mn / scale;
  const float zp = __builtin_truncf(__builtin_amdgcn_fmed3f(u + 0.5f, 0.0f, 15.0f));
  const float inv = 1.0f / scale;
  const float invs = q ? -inv : inv;  // x * invs = (true value) * inv exactly

  uint32_t d[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    d[m] = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float tq = __builtin_fmaf(x[8 * m + j], invs, zp);
      const uint32_t code = (uint32_t)__builtin_amdgcn_fmed3f(tq + 0.5f, 0.0f, 15.0f);
      d[m] |= code << (4 * j);
    }
  }
  // word c = 2m + q of the packed row is d[m]; lane 0 stores words
  // 0 .. M-1, lane 1 words M .. 2M-1
  constexpr int H = M / 2;
  uint32_t out[M];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const uint32_t send = q ? d[k] : d[H + k];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    out[2 * k] = q ? recv : d[k];
    out[2 * k + 1] = q ? d[H + k] : recv;
  }
  if (slot >= 0 && slot < cache_slots) {
    const int64_t dst = slot * hk + head;
    uint2* o = reinterpret_cast<uint2*>((is_v ? vc : kc) + dst * (D / 2) + 4 * M * q);
#pragma unroll
    for (int k = 0; k < H; ++k) o[k] = make_uint2(out[2 * k], out[2 * k + 1]);
    if (q == 0) (is_v ? vs : ks)[dst] = u2f((f2u(scale) & 0xFFFFFFF0u) | (uint32_t)zp);
  }
}

template <int D, int DT>
hipError_t launch_reshape(const ReshapeParams& p, hipStream_t st) {
  const int64_t total_rows = p.num_tokens * p.hk * 2;
  const int64_t blocks = (total_rows + 127) / 128;
  hipLaunchKernelGGL((reshape_int4_kernel<D, DT>), dim3((uint32_t)blocks), dim3(256), 0, st,
                     p.key, p.value, p.slots, p.signs, p.kc, p.vc, p.ks, p.vs, total_rows,
                     p.hk, p.num_blocks * (int64_t)p.block_size);
  return hipGetLastError();
}

}  // namespace

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
