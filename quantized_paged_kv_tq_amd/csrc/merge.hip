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
#include "balance.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

template <int D, bool ROTATE>
__global__ __launch_bounds__(D) void merge_kernel(DecodeParams p) {
  constexpr int CH = 16;  // partials whose loads are in flight together
  constexpr int kMaxParts = kWaveBudget + 256;  // nw + S bounds the list
  __shared__ float sh[D];
  __shared__ uint32_t rows[kMaxParts];  // partial rows of ws, in merge order
  __shared__ int cnt_scan[D];
  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int h = bh - b * p.hq;
  const int d = threadIdx.x;
  const SeqSplits q = seq_splits(p, b);
  const int nsplit = q.n;  // non-empty splits are a prefix: s * split_len < seq

  // ---- the list of partial rows to merge ----
  int nparts;
  if (p.nw == 0) {
    // one partial per non-empty split: rows (b, h, s)
    for (int s = d; s < nsplit; s += D) rows[s] = (uint32_t)((int64_t)bh * p.splits + s);
    nparts = nsplit;
  } else {
    // balanced layout: the tile list position of this sequence and the
    // total, as stage 1 computed them
    const int Pb = p.wsx[b], N = p.wsx[p.B];
    const int kvh = h / p.g;
    const int grp = kvh / p.wgh;
    const int hw = h - grp * p.wgh * p.g;  // head index within its workgroup
    const int64_t whole_rows = (int64_t)p.B * p.hq * p.splits;
    // entries of the splits d, d + D, ... (S <= 256)
    constexpr int SPT = (256 + D - 1) / D;
    int cnt[SPT], wa[SPT], ea[SPT], A_[SPT];
    for (int i = 0; i < SPT; ++i) {
      cnt[i] = 0;
      wa[i] = 0;
      ea[i] = 0;
      A_[i] = 0;
      const int s = d + i * D;
      if (s < nsplit) {
        const int A = Pb + s * q.TL;
        const int nt = (s == nsplit - 1) ? q.TLast : q.TL;
        const int a = range_owner(A, N, p.nw), e = range_owner(A + nt - 1, N, p.nw);
        // workgroups with a non-empty range in [a, e] (all of them when N >= nw)
        int c = e - a + 1;
        if (N < p.nw && c > 1) {
          c = 0;
          for (int w = a; w <= e; ++w) c += range_lo(w, N, p.nw) < range_lo(w + 1, N, p.nw);
        }
        cnt[i] = c;
        wa[i] = a;
        ea[i] = e;
        A_[i] = A;
      }
    }
    // exclusive scan of per-thread counts
    int mine = 0;
    for (int i = 0; i < SPT; ++i) mine += cnt[i];
    cnt_scan[d] = mine;
    __syncthreads();
    for (int off = 1; off < D; off <<= 1) {
      const int v = d >= off ? cnt_scan[d - off] : 0;
      __syncthreads();
      cnt_scan[d] += v;
      __syncthreads();
    }
    nparts = cnt_scan[D - 1] < kMaxParts ? cnt_scan[D - 1] : kMaxParts;
    int pos = d ? cnt_scan[d - 1] : 0;
    // thread d lists the partials of splits d, d + D, ... (any merge order)
    for (int i = 0; i < SPT; ++i) {
      const int s = d + i * D;
      if (s >= nsplit) continue;
      if (cnt[i] == 1) {
        if (pos < kMaxParts) rows[pos] = (uint32_t)((int64_t)bh * p.splits + s);
        ++pos;
      } else {
        for (int w = wa[i]; w <= ea[i]; ++w) {
          if (range_lo(w, N, p.nw) == range_lo(w + 1, N, p.nw)) continue;  // empty range
          const int slot = (w == wa[i] && A_[i] != range_lo(w, N, p.nw)) ? 1 : 0;
          const int64_t prow = whole_rows +
              (((int64_t)grp * p.nw + w) * 2 + slot) * ((int64_t)p.wgh * p.g) + hw;
          if (pos < kMaxParts) rows[pos] = (uint32_t)prow;
          ++pos;
        }
      }
    }
  }
  __syncthreads();

  // running log-sum-exp over chunks of partials (natural-log lse)
  float mx = -INFINITY, wsum = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < nparts; s0 += CH) {
    float ls[CH], pv[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int s = s0 + j;
      const bool ok = s < nparts;
      const float* part = p.ws + (int64_t)rows[ok ? s : 0] * (D + 1);
      ls[j] = ok ? part[D] : -INFINITY;
      pv[j] = ok ? part[d] : 0.0f;
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
