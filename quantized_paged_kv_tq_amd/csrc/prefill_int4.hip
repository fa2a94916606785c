// INT4 multi-query (prefill) attention over the paged cache
// (int4_per_token_head.py, _attn_packed in its 2D mode, as
// unified_attention_int4 wraps it).
//
// Query i of a sequence sits at absolute position pos = (seq_len -
// query_len) + i and attends to the keys at positions [lo, min(pos + 1,
// seq_len)): causal, and with a sliding window W > 0 (W = 1 +
// window_size[0]) lo = pos - W + 1. Scores are (sm_scale / D) q'.k' with the
// zero point of the INT4 key folded in; a positive softcap c maps s to
// c tanh(s / c). A sink joins the softmax denominator only. The output is the
// inverse RHT of the softmax-weighted mean of the dequantized values,
// s * FWHT(o') / D, stored as fp32 or as E4M3 codes of clamp(out /
// output_scale, +-448).
//
// One workgroup (4 waves) per (query token, kv head, head chunk): the query
// heads of the chunk are rotated once into LDS, every token of the visible
// range is decoded by D/8 lanes holding 8 dimensions each, each lane group
// keeps an online softmax (base-2 units) per head, and the groups are merged
// by log-sum-exp; the epilogue adds the sink, applies the inverse rotation
// in LDS and writes the rows. The visible range's block-table slice is staged
// in LDS, and each lane group issues the raw loads of U tokens before
// decoding any of them.
#include <type_traits>

#include "prefill.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;  // headroom of the reference maximum (base-2 units)
constexpr int kMaxRangePages = 2048;  // block-table entries staged in LDS

template <int D, int G, int U>
__global__ __launch_bounds__(256) void prefill_int4_kernel(PrefillParams p) {
  constexpr int LPT = D / 8;          // lanes per token
  constexpr int TPW = 64 / LPT;       // tokens per wave step
  constexpr int NG = 4 * TPW;         // token groups per workgroup
  __shared__ float qs[G][D];
  __shared__ int pages[kMaxRangePages];
  __shared__ float red[4][G][D + 2];

  const int nchunk = (p.g + G - 1) / G;
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  // logical order: head chunk fastest, then kv head, then query token
  const int hc = lb % nchunk;
  const int kvh = (lb / nchunk) % p.hk;
  const int64_t tq = (int64_t)(lb / ((uint32_t)nchunk * p.hk));
  const int tid = threadIdx.x;
  const int h0 = kvh * p.g + hc * G;  // first query head here
  const int nh = (p.g - hc * G) < G ? (p.g - hc * G) : G;

  // ---- the query's sequence and visible key range ----
  int lo_b = 0, hi_b = p.num_seqs;  // largest b with cu[b] <= tq
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (p.cu_seqlens[mid] <= tq) lo_b = mid;
    else hi_b = mid;
  }
  const int b = lo_b;
  const int64_t q0 = p.cu_seqlens[b], q1 = p.cu_seqlens[b + 1];
  int64_t seq = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  seq = seq < 0 ? 0 : (seq > cap ? cap : seq);
  int64_t t0 = 0, t1 = 0;
  if (tq >= q0 && tq < q1) {
    const int64_t pos = seq - (q1 - q0) + (tq - q0);
    t1 = pos + 1 < seq ? pos + 1 : seq;
    if (p.window > 0 && pos - p.window + 1 > 0) t0 = pos - p.window + 1;
  }

  // ---- query prologue: load, sign, rotate ----
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D, d = i % D;
    float v = 0.0f;
    if (hh < nh) v = p.q[(tq * p.hq + h0 + hh) * D + d] * p.rht_signs[d];
    qs[hh][d] = v;
  }
  const bool staged = t1 > t0 && ((t1 - 1) / p.block_size - t0 / p.block_size + 1) <= kMaxRangePages;
  if (staged) {
    const int64_t first = t0 / p.block_size;
    const int64_t count = (t1 - 1) / p.block_size - first + 1;
    const int32_t* row = p.block_table + (int64_t)b * p.max_blocks + first;
    for (int i = tid; i < count; i += 256) pages[i] = row[i];
  }
  __syncthreads();
  for (int hstride = 1; hstride < D; hstride <<= 1) {
    for (int i = tid; i < G * D / 2; i += 256) {
      const int hh = i / (D / 2), k = i % (D / 2);
      const int lo = (k / hstride) * 2 * hstride + (k % hstride);
      const float a = qs[hh][lo], c = qs[hh][lo + hstride];
      qs[hh][lo] = a + c;
      qs[hh][lo + hstride] = a - c;
    }
    __syncthreads();
  }
  // natural-unit scores (softcap acts on them); base-2 inside the softmax
  const float qscale = p.sm_scale / (float)D;
  const bool capped = p.softcap > 0.0f;

  const int lane = tid & 63;
  const int li = lane % LPT;
  const int grp = (tid >> 6) * TPW + lane / LPT;
  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[hh][j] = qs[hh][li * 8 + j] * qscale;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[hh][j] = 0.0f;
  }

  const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
  const int bs = p.block_size;
  const int64_t pg0 = t0 / bs;

  struct Raw {
    uint32_t w[4];
    bool ok;
  };
  auto load_raw = [&](int64_t t) {
    Raw r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = 0;
    r.ok = false;
    if (t >= t1) return r;
    const int64_t page = staged ? (int64_t)pages[t / bs - pg0] : (int64_t)bt[t / bs];
    if (page < 0 || page >= p.num_blocks) return r;  // outside the pool: masked
    r.ok = true;
    const int64_t row = (page * bs + t % bs) * p.hk + kvh;
    r.w[0] = *reinterpret_cast<const uint32_t*>(p.kc + row * (D / 2) + li * 4);
    r.w[1] = f2u(p.ks[row]);
    r.w[2] = *reinterpret_cast<const uint32_t*>(p.vc + row * (D / 2) + li * 4);
    r.w[3] = f2u(p.vs[row]);
    return r;
  };

  auto consume = [&](const Raw& r) {
    if (!r.ok) return;
    float kd[8], vd[8];
    {
      const uint32_t w = r.w[0], sw = r.w[1];
      const float zp = (float)(sw & 0xFu);
#pragma unroll
      for (int j = 0; j < 8; ++j) kd[j] = (float)((w >> (4 * j)) & 0xFu) - zp;
    }
    const float kscale = u2f(r.w[1] & 0xFFFFFFF0u);
    float sc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) part += qv[hh][j] * kd[j];
      float s = group_sum<LPT>(part) * kscale;
      if (capped) s = p.softcap * tanhf(s / p.softcap);
      sc[hh] = s * kLog2e;
    }
    {
      const uint32_t w = r.w[2], sw = r.w[3];
      const float zp = (float)(sw & 0xFu);
      const float vsc = u2f(sw & 0xFFFFFFF0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) vd[j] = ((float)((w >> (4 * j)) & 0xFu) - zp) * vsc;
    }
    // m is a reference maximum: the state moves to a new one only when a
    // score exceeds it by more than 2^kTau, so the weights stay below
    // 2^kTau and most tokens take one exponential and no rescaling
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (sc[hh] > m[hh] + kTau) {
        const float alpha = exp2f(m[hh] - sc[hh]);  // 0 while m is -inf
        l[hh] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[hh][j] *= alpha;
        m[hh] = sc[hh];
      }
      const float pr = exp2f(sc[hh] - m[hh]);
      l[hh] += pr;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[hh][j] = __builtin_fmaf(pr, vd[j], acc[hh][j]);
    }
  };

  for (int64_t tb = t0 + grp; tb < t1; tb += (int64_t)U * NG) {
    Raw r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = load_raw(tb + (int64_t)u * NG);
#pragma unroll
    for (int u = 0; u < U; ++u) consume(r[u]);
  }

  // ---- merge the lane groups of each wave (log-sum-exp) ----
  auto merge = [&](auto xorc) {
    constexpr int M = decltype(xorc)::value;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mo = xor_lane<M>(m[hh]);
      const float lo = xor_lane<M>(l[hh]);
      const float mm = fmaxf(m[hh], mo);
      const float a = (mm == -INFINITY) ? 0.0f : exp2f(m[hh] - mm);
      const float ao = (mm == -INFINITY) ? 0.0f : exp2f(mo - mm);
      l[hh] = l[hh] * a + lo * ao;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[hh][j] = acc[hh][j] * a + xor_lane<M>(acc[hh][j]) * ao;
      m[hh] = mm;
    }
  };
  if constexpr (LPT <= 8) merge(std::integral_constant<int, 8>{});
  if constexpr (LPT <= 16) merge(std::integral_constant<int, 16>{});
  merge(std::integral_constant<int, 32>{});

  const int wave = tid >> 6;
  if (lane < LPT) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wave][hh][li * 8 + j] = acc[hh][j];
      if (li == 0) {
        red[wave][hh][D] = m[hh];
        red[wave][hh][D + 1] = l[hh];
      }
    }
  }
  __syncthreads();
  // ---- merge the waves, add the sink; o' into qs ----
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D, d = i % D;
    float o = 0.0f;
    if (hh < nh) {
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][hh][D]);
      if (mm != -INFINITY) {
        const float sk = p.sinks ? p.sinks[h0 + hh] * kLog2e : -INFINITY;
        const float mt = fmaxf(mm, sk);
        float lsum = p.sinks ? exp2f(sk - mt) : 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a = exp2f(red[w][hh][D] - mt);
          lsum += red[w][hh][D + 1] * a;
          o += red[w][hh][d] * a;
        }
        o = o / lsum;
      }
    }
    qs[hh][d] = o;
  }
  __syncthreads();
  // ---- inverse RHT: s * FWHT(o') / D ----
  for (int hstride = 1; hstride < D; hstride <<= 1) {
    for (int i = tid; i < G * D / 2; i += 256) {
      const int hh = i / (D / 2), k = i % (D / 2);
      const int lo = (k / hstride) * 2 * hstride + (k % hstride);
      const float a = qs[hh][lo], c = qs[hh][lo + hstride];
      qs[hh][lo] = a + c;
      qs[hh][lo + hstride] = a - c;
    }
    __syncthreads();
  }
  const float inv_d = 1.0f / (float)D;
  if (p.out) {
    for (int i = tid; i < nh * D; i += 256) {
      const int hh = i / D, d = i % D;
      p.out[(tq * p.hq + h0 + hh) * D + d] = qs[hh][d] * p.rht_signs[d] * inv_d;
    }
  } else {
    const float inv_s = 1.0f / p.output_scale[0];
    for (int i = tid; i < nh * D; i += 256) {
      const int hh = i / D, d = i % D;
      const float v = fminf(fmaxf(qs[hh][d] * p.rht_signs[d] * inv_d * inv_s, -448.0f), 448.0f);
      p.out_fp8[(tq * p.hq + h0 + hh) * D + d] =
          (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu);
    }
  }
}

// Multi-query attention as one decode entry per query token: token tq of
// sequence b at position pos sees keys [t0, t1) (t1 = min(pos + 1, seq), t0
// = pos - W + 1 under a window), so entry i = tq - begin is a decode of
// t1 - t0 keys read from block-table row b from token t0 on. Tokens with no
// visible key (or outside every sequence) get length 0 (their output is 0).
__global__ __launch_bounds__(256) void prefill_plan_kernel(PrefillParams p, int64_t begin, int n,
                                                           int32_t* lens, int32_t* rows,
                                                           int32_t* offs) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t tq = begin + i;
  int lo_b = 0, hi_b = p.num_seqs;  // largest b with cu[b] <= tq
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (p.cu_seqlens[mid] <= tq) lo_b = mid;
    else hi_b = mid;
  }
  const int b = lo_b;
  const int64_t q0 = p.cu_seqlens[b], q1 = p.cu_seqlens[b + 1];
  int64_t seq = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  seq = seq < 0 ? 0 : (seq > cap ? cap : seq);
  int64_t t0 = 0, t1 = 0;
  if (tq >= q0 && tq < q1) {
    const int64_t pos = seq - (q1 - q0) + (tq - q0);
    t1 = pos + 1 < seq ? pos + 1 : seq;
    if (p.window > 0 && pos - p.window + 1 > 0) t0 = pos - p.window + 1;
  }
  const bool any = t1 > t0;
  lens[i] = any ? (int32_t)(t1 - t0) : 0;
  rows[i] = b;
  offs[i] = any ? (int32_t)t0 : 0;
}

template <int D>
hipError_t launch_d(const PrefillParams& p, hipStream_t st) {
  const int G = p.g <= 1 ? 1 : (p.g <= 2 ? 2 : (p.g <= 4 ? 4 : 8));
  const int chunks = (p.g + G - 1) / G;
  const uint32_t blocks = (uint32_t)(p.num_tokens * p.hk * chunks);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_int4_kernel<D, 1, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((prefill_int4_kernel<D, 2, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    case 4: hipLaunchKernelGGL((prefill_int4_kernel<D, 4, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((prefill_int4_kernel<D, 8, 4>), dim3(blocks), dim3(256), 0, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_plan(const PrefillParams& p, int64_t begin, int n, int32_t* lens,
                               int32_t* rows, int32_t* offs, hipStream_t st) {
  hipLaunchKernelGGL(prefill_plan_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, p,
                     begin, n, lens, rows, offs);
  return hipGetLastError();
}

hipError_t launch_prefill_int4(const PrefillParams& p, hipStream_t st) {
  if (p.d == 128) return launch_d<128>(p, st);
  if (p.d == 64) return launch_d<64>(p, st);
  return hipErrorNotSupported;
}

}  // namespace tqk
