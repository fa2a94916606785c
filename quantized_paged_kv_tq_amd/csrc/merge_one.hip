// Stage 2 of the multi-query (prefill) attention, whose entries are one
// query token each with a single split (int4_per_token_head.py,
// _attn_packed in its 2D mode: sinks, output scale): the log-sum-exp merge
// of the entry's pieces, the sink term, the inverse RHT out = rht_signs *
// FWHT(o) / D and the fp32 or E4M3 store.
#include "balance.h"
#include "merge_one.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

// Stage 2 for entries of one split each (the multi-query use, D = 128): one
// wave per (entry, query head), lane l holding dims l and l + 64. An entry's
// split is whole (one partial) or cut by the balanced partition into one
// piece per range it touches, found as in merge_kernel; no list, no barrier.
template <bool ROTATE>
__global__ __launch_bounds__(256) void merge_one_split_kernel(DecodeParams p) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= (int64_t)p.B * p.hq) return;  // whole waves
  const int b = (int)(bh / p.hq);
  const int h = (int)(bh - (int64_t)b * p.hq);
  const float sgn0 = ROTATE ? p.rht_signs[lane] : 1.0f;
  const float sgn1 = ROTATE ? p.rht_signs[lane + 64] : 1.0f;
  const SeqSplits q = seq_splits(p, b);
  float M = -INFINITY, wsum = 0.0f, a0 = 0.0f, a1 = 0.0f;
  auto add = [&](const float* part) {
    const float ls = part[D];
    const float v0 = part[lane], v1 = part[lane + 64];
    if (ls == -INFINITY) return;  // an empty piece
    const float nm = fmaxf(M, ls);
    const float sc = __expf(M - nm);
    const float w = __expf(ls - nm);
    wsum = wsum * sc + w;
    a0 = a0 * sc + w * v0;
    a1 = a1 * sc + w * v1;
    M = nm;
  };
  if (q.n > 0) {
    const float* whole = p.ws + bh * p.splits * (D + 1);
    if (p.nw == 0) {
      add(whole);
    } else {
      const int Pb = p.wsx[b], N = p.wsx[p.B];
      const int a = range_owner(Pb, N, p.nw), e = range_owner(Pb + q.TLast - 1, N, p.nw);
      if (a == e) {
        add(whole);
      } else {
        const int kvh = h / p.g;
        const int grp = kvh / p.wgh;
        const int hw = h - grp * p.wgh * p.g;  // head index within its workgroup
        for (int w = a; w <= e; ++w) {
          const int lo = range_lo(w, N, p.nw);
          if (lo == range_lo(w + 1, N, p.nw)) continue;  // empty range
          // the first owner holds the split as its last piece (slot 1)
          // unless its range starts with it; later owners as their first
          const int slot = (w == a && Pb != lo) ? 1 : 0;
          add(p.wsp + ((((int64_t)grp * p.nw + w) * 2 + slot) * ((int64_t)p.wgh * p.g) + hw) * (D + 1));
        }
      }
    }
  }
  float o0 = 0.0f, o1 = 0.0f;
  if (wsum > 0.0f) {
    o0 = a0 / wsum;
    o1 = a1 / wsum;
    if (p.sinks) {
      const float f = wsum / (wsum + __expf(p.sinks[h] - M));
      o0 *= f;
      o1 *= f;
    }
  }
  if constexpr (ROTATE) {
    // inverse RHT: FWHT strides 1 .. 32 across lanes, 64 inside the lane
    o0 = butterfly_lanes<1>(o0, lane & 1);   o1 = butterfly_lanes<1>(o1, lane & 1);
    o0 = butterfly_lanes<2>(o0, lane & 2);   o1 = butterfly_lanes<2>(o1, lane & 2);
    o0 = butterfly_lanes<4>(o0, lane & 4);   o1 = butterfly_lanes<4>(o1, lane & 4);
    o0 = butterfly_lanes<8>(o0, lane & 8);   o1 = butterfly_lanes<8>(o1, lane & 8);
    o0 = butterfly_lanes<16>(o0, lane & 16); o1 = butterfly_lanes<16>(o1, lane & 16);
    o0 = butterfly_lanes<32>(o0, lane & 32); o1 = butterfly_lanes<32>(o1, lane & 32);
    const float u = o0 + o1, v = o0 - o1;
    o0 = u * sgn0 * (1.0f / (float)D);
    o1 = v * sgn1 * (1.0f / (float)D);
  }
  if (p.out_fp8) {
    const float inv = 1.0f / p.output_scale[0];
    const float v0 = fminf(fmaxf(o0 * inv, -448.0f), 448.0f);
    const float v1 = fminf(fmaxf(o1 * inv, -448.0f), 448.0f);
    p.out_fp8[bh * D + lane] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v0, v0, 0, false) & 0xFFu);
    p.out_fp8[bh * D + lane + 64] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v1, v1, 0, false) & 0xFFu);
  } else {
    p.out[bh * D + lane] = o0;
    p.out[bh * D + lane + 64] = o1;
  }
  if (p.lse && lane == 0) p.lse[bh] = (wsum > 0.0f) ? M + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_merge_one_split(const DecodeParams& p, hipStream_t st) {
  if (p.d != 128 || p.splits != 1) return hipErrorNotSupported;
  const int64_t rows = (int64_t)p.B * p.hq;
  const uint32_t blocks = (uint32_t)((rows + 3) / 4);
  if (p.key_fmt == KF_INT4)
    hipLaunchKernelGGL((merge_one_split_kernel<true>), dim3(blocks), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((merge_one_split_kernel<false>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace tqk
