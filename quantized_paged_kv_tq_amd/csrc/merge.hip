// Split-KV decode, stage 2: log-sum-exp merge of the per-split partials.
//
// The TurboQuant page launches a stage-2 kernel whose body it imports
// (triton_turboquant_decode.py, "Stage 2: Reduce across KV splits"); what it
// must compute follows from stage 1's partials (acc / l, m + ln l): over the
// non-empty splits (recomputed from seq_lens exactly as stage 1 cuts them),
//   M = max lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
//   lse = M + ln(sum w_s).
// For the INT4 format the output is rotated back (int4_per_token_head.py,
// unified_attention_int4): out = rht_signs * FWHT(o) / D.
// One workgroup per (batch, query head), one lane per output dimension.
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

template <int D, bool ROTATE>
__global__ __launch_bounds__(D) void merge_kernel(DecodeParams p) {
  constexpr int CH = 16;  // splits whose loads are in flight together
  __shared__ float sh[D];
  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int d = threadIdx.x;
  int64_t seq = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  seq = seq < 0 ? 0 : (seq > cap ? cap : seq);
  const int64_t split_len = (seq + p.splits - 1) / p.splits;
  // non-empty splits are a prefix: s * split_len < seq
  const int nsplit = seq == 0 ? 0 : (int)((seq + split_len - 1) / split_len);
  const float* part = p.ws + (int64_t)bh * p.splits * (D + 1);

  // running log-sum-exp over chunks of splits (natural-log partials)
  float mx = -INFINITY, wsum = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += CH) {
    float ls[CH], pv[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int s = s0 + j;
      const bool ok = s < nsplit;
      ls[j] = ok ? part[s * (D + 1) + D] : -INFINITY;
      pv[j] = ok ? part[s * (D + 1) + d] : 0.0f;
    }
    float cm = ls[0];
#pragma unroll
    for (int j = 1; j < CH; ++j) cm = fmaxf(cm, ls[j]);
    const float nm = fmaxf(mx, cm);
    if (nm == -INFINITY) continue;
    const float sc = __expf(mx - nm);
    wsum *= sc;
    o *= sc;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float w = __expf(ls[j] - nm);
      wsum += w;
      o += w * pv[j];
    }
    mx = nm;
  }
  if (mx != -INFINITY) o /= wsum;
  if constexpr (ROTATE) {
    sh[d] = o;
    __syncthreads();
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
      const float a = sh[d], c = sh[d ^ h];
      __syncthreads();
      sh[d] = (d & h) ? (c - a) : (a + c);
      __syncthreads();
    }
    o = sh[d] * p.rht_signs[d] * (1.0f / (float)D);
  }
  p.out[(int64_t)bh * D + d] = o;
  if (p.lse && d == 0) p.lse[bh] = (mx == -INFINITY) ? -INFINITY : mx + __logf(wsum);
}

}  // namespace

hipError_t launch_merge(const DecodeParams& p, hipStream_t st) {
  const uint32_t blocks = (uint32_t)p.B * p.hq;
  const bool rot = p.key_fmt == KF_INT4;
  if (p.d == 128) {
    if (rot) hipLaunchKernelGGL((merge_kernel<128, true>), dim3(blocks), dim3(128), 0, st, p);
    else hipLaunchKernelGGL((merge_kernel<128, false>), dim3(blocks), dim3(128), 0, st, p);
  } else {
    if (rot) hipLaunchKernelGGL((merge_kernel<64, true>), dim3(blocks), dim3(64), 0, st, p);
    else hipLaunchKernelGGL((merge_kernel<64, false>), dim3(blocks), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace tqk
