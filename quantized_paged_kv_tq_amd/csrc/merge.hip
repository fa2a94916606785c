// Split-KV decode, stage 2: log-sum-exp merge of the per-split partials.
//
// The TurboQuant page launches a stage-2 kernel whose body it imports
// (triton_turboquant_decode.py, "Stage 2: Reduce across KV splits"); what it
// must compute follows from stage 1's partials (acc / l, m + ln l): over the
// non-empty splits (recomputed from seq_lens exactly as stage 1 cuts them),
//   M = max lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
//   lse = M + ln(sum w_s).
// For the INT4 format the output is rotated back (int4_per_token_head.py,
// unified_attention_int4): out = rht_signs * FWHT(o) / D. Used for the
// multi-query (prefill) attention, a sink term joins the denominator and the
// output may be stored as E4M3 codes (int4_per_token_head.py, _attn_packed:
// sinks, output scale).
// One workgroup per (batch, query head), one lane per output dimension.
#include "balance.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

template <int D, bool ROTATE, int PG>
__global__ __launch_bounds__(D * PG) void merge_kernel(DecodeParams p) {
  constexpr int NT = D * PG;  // PG groups of D threads share the partials
  constexpr int CH = 16;      // partial rows whose loads are in flight together
  constexpr int kMaxParts = kWaveBudget + 256;  // nw + S bounds the list
  __shared__ uint32_t rows[kMaxParts];  // partial rows of ws, in merge order
  __shared__ int wave_tot[NT / 64];
  __shared__ float acc_l[PG][D];
  __shared__ float st_l[PG][2];  // running (max, weight sum) per group
  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int h = bh - b * p.hq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the inverse-rotation sign is loaded with the first round trip, not after
  // the merge
  const float sgn = ROTATE ? p.rht_signs[tid % D] : 1.0f;
  const SeqSplits q = seq_splits(p, b);
  const int nsplit = q.n;  // non-empty splits are a prefix: s * split_len < seq

  // ---- the list of partial rows to merge ----
  int nparts;
  if (p.nw == 0) {
    // one partial per non-empty split: rows (b, h, s)
    for (int s = tid; s < nsplit; s += NT) rows[s] = (uint32_t)((int64_t)bh * p.splits + s);
    nparts = nsplit;
  } else {
    // balanced layout: the tile-list position of this sequence and the
    // total, as stage 1 computed them
    const int Pb = p.wsx[b], N = p.wsx[p.B];
    const int kvh = h / p.g;
    const int grp = kvh / p.wgh;
    const int hw = h - grp * p.wgh * p.g;  // head index within its workgroup
    const int64_t whole_rows = (int64_t)p.B * p.hq * p.splits;
    // entries of the splits tid, tid + NT, ... (S <= 256)
    constexpr int SPT = (256 + NT - 1) / NT;
    int cnt[SPT], wa[SPT], ea[SPT], A_[SPT];
    int mine = 0;
    for (int i = 0; i < SPT; ++i) {
      cnt[i] = 0;
      wa[i] = 0;
      ea[i] = 0;
      A_[i] = 0;
      const int s = tid + i * NT;
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
        mine += c;
      }
    }
    // exclusive scan of the per-thread counts: across the wave, then waves
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off);
      if (lane >= off) incl += u;
    }
    if (lane == 63) wave_tot[tid >> 6] = incl;
    __syncthreads();
    int total = 0, before = 0;
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      total += wave_tot[w2];
      before += w2 < (tid >> 6) ? wave_tot[w2] : 0;
    }
    nparts = total < kMaxParts ? total : kMaxParts;
    int pos = before + incl - mine;
    // thread tid lists the partials of splits tid, tid + NT, ... (any order)
    for (int i = 0; i < SPT; ++i) {
      const int s = tid + i * NT;
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

  // ---- running log-sum-exp per group: group pg takes partials pg, pg+PG,
  // ..., CH of them in flight at a time (lse and value together) ----
  const int d = tid % D, pg = tid / D;
  float mx = -INFINITY, ws = 0.0f, acc = 0.0f;
  for (int s0 = pg; s0 < nparts; s0 += CH * PG) {
    float ls[CH], pv[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int s = s0 + j * PG;
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
    ws *= sc;
    acc *= sc;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float w = __expf(ls[j] - nm);
      ws += w;
      acc += w * pv[j];
    }
    mx = nm;
  }
  acc_l[pg][d] = acc;
  if (d == 0) {
    st_l[pg][0] = mx;
    st_l[pg][1] = ws;
  }
  __syncthreads();
  // combine the groups' states
  float M = -INFINITY;
#pragma unroll
  for (int g2 = 0; g2 < PG; ++g2) M = fmaxf(M, st_l[g2][0]);
  float wsum = 0.0f, o = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int g2 = 0; g2 < PG; ++g2) {
      const float a = __expf(st_l[g2][0] - M);  // 0 for an empty group
      wsum += st_l[g2][1] * a;
      o += acc_l[g2][d] * a;
    }
  }
  // the first group (threads < D) stores the row; the others only take
  // part in the barriers below
  if (wsum > 0.0f) o /= wsum;
  // a sink joins the denominator: sum_s e^{lse_s} o_s / (sum_s e^{lse_s} +
  // e^{sink}); a row with no visible key stays 0
  if (p.sinks && wsum > 0.0f) o *= wsum / (wsum + __expf(p.sinks[h] - M));
  if constexpr (ROTATE) {
    // inverse RHT: FWHT over D (strides 1 .. 32 inside the wave, 64 through
    // LDS), then signs and 1/D
    o = butterfly_lanes<1>(o, d & 1);
    o = butterfly_lanes<2>(o, d & 2);
    o = butterfly_lanes<4>(o, d & 4);
    o = butterfly_lanes<8>(o, d & 8);
    o = butterfly_lanes<16>(o, d & 16);
    o = butterfly_lanes<32>(o, d & 32);
    if constexpr (D == 128) {
      __syncthreads();  // every group has read acc_l
      if (tid < D) acc_l[0][d] = o;
      __syncthreads();
      const float pr = acc_l[0][d ^ 64];
      o = (d & 64) ? (pr - o) : (o + pr);
    }
    o = o * sgn * (1.0f / (float)D);
  }
  if (tid < D) {
    if (p.out_fp8) {
      // E4M3 codes of clamp(out * fl(1 / output_scale), +-448), nearest even
      const float v = fminf(fmaxf(o * (1.0f / p.output_scale[0]), -448.0f), 448.0f);
      p.out_fp8[(int64_t)bh * D + d] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu);
    } else {
      p.out[(int64_t)bh * D + d] = o;
    }
    if (p.lse && d == 0) p.lse[bh] = (wsum > 0.0f) ? M + __logf(wsum) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_merge(const DecodeParams& p, hipStream_t st) {
  const uint32_t blocks = (uint32_t)p.B * p.hq;
  const bool rot = p.key_fmt == KF_INT4;
  // more thread groups per row when there are few rows to fill the chip
  const int pg = blocks >= 2048 ? 1 : (blocks >= 512 ? 2 : 4);
#define TQ_MERGE(DD, RR, PP) \
  hipLaunchKernelGGL((merge_kernel<DD, RR, PP>), dim3(blocks), dim3(DD * PP), 0, st, p)
  if (p.d == 128) {
    if (rot) {
      if (pg == 1) TQ_MERGE(128, true, 1); else if (pg == 2) TQ_MERGE(128, true, 2); else TQ_MERGE(128, true, 4);
    } else {
      if (pg == 1) TQ_MERGE(128, false, 1); else if (pg == 2) TQ_MERGE(128, false, 2); else TQ_MERGE(128, false, 4);
    }
  } else if (p.d == 64) {
    if (rot) {
      if (pg == 1) TQ_MERGE(64, true, 1); else if (pg == 2) TQ_MERGE(64, true, 2); else TQ_MERGE(64, true, 4);
    } else {
      if (pg == 1) TQ_MERGE(64, false, 1); else if (pg == 2) TQ_MERGE(64, false, 2); else TQ_MERGE(64, false, 4);
    }
  } else {
    // D = 256: the TurboQuant formats only (no inverse rotation)
    if (rot) return hipErrorNotSupported;
    if (pg == 1) TQ_MERGE(256, false, 1); else if (pg == 2) TQ_MERGE(256, false, 2); else TQ_MERGE(256, false, 4);
  }
#undef TQ_MERGE
  return hipGetLastError();
}

}  // namespace tqk
