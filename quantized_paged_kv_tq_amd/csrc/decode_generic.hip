// Format-generic split-KV decode, stage 1, on the vector ALUs.
//
// Covers every key/value format of the library: INT4 (int4_per_token_head.py,
// _attn_packed and unified_attention_int4) and the TurboQuant combined slot
// (triton_turboquant_decode.py, _tq_decode_stage1): FP8 or 3/4-bit centroid
// keys, 3/4-bit uniform or FP8 values; D = 64, 128 or 256.
//
// One workgroup (4 waves) per (batch, kv head, head chunk, split). The query
// heads that share the kv head (up to G of them) are rotated/scaled once into
// LDS. Each token is handled by D/8 lanes holding 8 dimensions each, so a
// wave walks 64/(D/8) tokens at a time; every lane group keeps its own online
// softmax state (running max m, sum l, accumulator) per head, and the groups
// are merged by log-sum-exp at the end. Scores are kept in base-2 units
// (log2(e) folded into the query), so p = exp2(s - m).
//
// Latency: the split's block-table slice is staged in LDS, and each lane
// group issues the raw loads of U tokens (aligned dwords; sub-dword fields
// are cut out with byte-align shifts) before decoding any of them.
#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // headroom of the reference maximum (base-2 units)

constexpr int kMaxSplitPages = 2048;  // block-table entries of a split staged in LDS

template <int D, int KF, int VF, int G, int U>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeParams p) {
  constexpr int LPT = D / 8;          // lanes per token
  constexpr int TPW = 64 / LPT;       // tokens per wave step
  constexpr int NG = 4 * TPW;         // token groups per workgroup
  __shared__ float qs[G][D];
  __shared__ float cen[16];
  __shared__ int pages[kMaxSplitPages];
  __shared__ float red[4][G][D + 2];

  const int nchunk = (p.g + G - 1) / G;
  const uint32_t nblk = gridDim.x;
  const uint32_t lb = xcd_logical_block(blockIdx.x, nblk);
  // logical order: split fastest, then head chunk, kv head, batch
  const int s = lb % p.splits;
  const int hc = (lb / p.splits) % nchunk;
  const int kvh = (lb / (p.splits * nchunk)) % p.hk;
  const int b = lb / (p.splits * nchunk * p.hk);

  int64_t seq = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  seq = seq < 0 ? 0 : (seq > cap ? cap : seq);
  const int64_t split_len = (seq + p.splits - 1) / p.splits;
  const int64_t t0 = split_len * s;
  const int64_t t1 = (t0 + split_len < seq) ? t0 + split_len : seq;
  if (t0 >= t1) return;  // empty split: nothing written (stage 2 skips it)

  const int tid = threadIdx.x;
  const int h0 = kvh * p.g + hc * G;               // first query head here
  const int nh = (p.g - hc * G) < G ? (p.g - hc * G) : G;

  // ---- query prologue: load, sign, rotate, fold the score constants ----
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D, d = i % D;
    float v = 0.0f;
    if (hh < nh) {
      v = p.q[((int64_t)b * p.hq + h0 + hh) * D + d];
      if constexpr (KF == KF_INT4) v *= p.rht_signs[d];
      else if constexpr (KF == KF_MSE3 || KF == KF_MSE4) {
        if (p.rot_signs) v *= p.rot_signs[d];
      }
    }
    qs[hh][d] = v;
  }
  if constexpr (KF == KF_MSE3 || KF == KF_MSE4) {
    if (tid < 16) cen[tid] = tid < (KF == KF_MSE3 ? 8 : 16) ? p.centroids[tid] : 0.0f;
  }
  {
    // this split's block-table slice (pages of tokens t0 .. t1 - 1)
    const int64_t first = t0 / p.block_size;
    const int64_t count = (t1 - 1) / p.block_size - first + 1;
    if (count <= kMaxSplitPages) {
      const int32_t* row = p.block_table + (int64_t)b * p.max_blocks + first;
      for (int i = tid; i < count; i += 256) pages[i] = row[i];
    }
  }
  __syncthreads();
  if constexpr (KF != KF_FP8) {
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
  }
  float qscale;
  if constexpr (KF == KF_INT4) qscale = p.sm_scale / (float)D * kLog2e;
  else if constexpr (KF == KF_FP8) qscale = p.sm_scale * kLog2e;
  else qscale = p.sm_scale * kLog2e / sqrtf((float)D);

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
  constexpr int KB = (KF == KF_MSE3) ? 3 : 4;  // centroid index bits
  constexpr int VB = (VF == VF_U3) ? 3 : (VF == VF_FP8 ? 8 : 4);  // value bits
  const int mse_bytes = (D * KB + 7) / 8;
  const int bs = p.block_size;
  const int64_t pg0 = t0 / bs;
  const int npg = (int)((t1 - 1) / bs - pg0 + 1);
  const bool staged = npg <= kMaxSplitPages;

  // raw words of one token for this lane (masked tokens: ok = false)
  struct Raw {
    uint32_t w[7];
    bool ok;
  };
  auto load_raw = [&](int64_t t) {
    Raw r;
#pragma unroll
    for (int i = 0; i < 7; ++i) r.w[i] = 0;
    r.ok = false;
    if (t >= t1) return r;
    const int64_t page = staged ? (int64_t)pages[t / bs - pg0] : (int64_t)bt[t / bs];
    if (page < 0 || page >= p.num_blocks) return r;
    r.ok = true;
    const int64_t row = (page * bs + t % bs) * p.hk + kvh;
    if constexpr (KF == KF_INT4) {
      r.w[0] = *reinterpret_cast<const uint32_t*>(p.kc + row * (D / 2) + li * 4);
      r.w[1] = f2u(p.ks[row]);
      r.w[2] = *reinterpret_cast<const uint32_t*>(p.vc + row * (D / 2) + li * 4);
      r.w[3] = f2u(p.vs[row]);
    } else {
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(p.kv + row * p.slot_bytes);
      if constexpr (KF == KF_FP8) {
        r.w[0] = s32[2 * li];
        r.w[1] = s32[2 * li + 1];
      } else {
        const int kb = li * KB;  // first key byte of this lane
        r.w[0] = s32[kb >> 2];
        r.w[1] = s32[(kb >> 2) + 1];
        r.w[2] = s32[mse_bytes >> 2];  // fp16 norm in the low half (mse_bytes % 4 == 0)
      }
      const int vbyte = p.kps + li * VB;
      r.w[3] = s32[vbyte >> 2];
      r.w[4] = s32[(vbyte >> 2) + 1];
      if constexpr (VF == VF_FP8) {
        // 8 codes from an unaligned byte offset span 3 dwords (centroid keys:
        // KPS = 2 mod 4, and the slot padding holds the third dword); FP8
        // keys leave the codes dword-aligned
        if (p.kps & 3) r.w[5] = s32[(vbyte >> 2) + 2];
      } else {
        const int sbyte = p.kps + p.vdb;
        r.w[5] = s32[sbyte >> 2];
        r.w[6] = s32[(sbyte >> 2) + 1];
      }
    }
    return r;
  };

  // decode one token's raw words and fold it into the online softmax
  auto consume = [&](const Raw& r) {
    if (!r.ok) return;
    float kd[8];
    float kscale;
    if constexpr (KF == KF_INT4) {
      const uint32_t w = r.w[0], sw = r.w[1];
      const float zp = (float)(sw & 0xFu);
      kscale = u2f(sw & 0xFFFFFFF0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) kd[j] = (float)((w >> (4 * j)) & 0xFu) - zp;
    } else if constexpr (KF == KF_FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kd[j] = e4m3_to_f32((r.w[0] >> (8 * j)) & 0xFFu);
        kd[j + 4] = e4m3_to_f32((r.w[1] >> (8 * j)) & 0xFFu);
      }
      kscale = 1.0f;
    } else {
      const uint32_t w = __builtin_amdgcn_alignbyte(r.w[1], r.w[0], (li * KB) & 3);
      float cs = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kd[j] = cen[(w >> (KB * j)) & ((1u << KB) - 1u)];
        cs += kd[j] * kd[j];
      }
      kscale = half_lo(r.w[2]);
      if (p.norm_correction) kscale *= 1.0f / sqrtf(group_sum<LPT>(cs) + 1e-16f);
    }
    float sc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) part += qv[hh][j] * kd[j];
      sc[hh] = group_sum<LPT>(part) * kscale;
    }

    float vd[8];
    if constexpr (VF == VF_INT4) {
      const uint32_t w = r.w[2], sw = r.w[3];
      const float zp = (float)(sw & 0xFu);
      const float vsc = u2f(sw & 0xFFFFFFF0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) vd[j] = ((float)((w >> (4 * j)) & 0xFu) - zp) * vsc;
    } else if constexpr (VF == VF_FP8) {
      const uint32_t sh = (uint32_t)(p.kps + li * VB) & 3;
      const uint32_t w0 = __builtin_amdgcn_alignbyte(r.w[4], r.w[3], sh);
      const uint32_t w1 = __builtin_amdgcn_alignbyte(r.w[5], r.w[4], sh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vd[j] = e4m3_to_f32((w0 >> (8 * j)) & 0xFFu);
        vd[j + 4] = e4m3_to_f32((w1 >> (8 * j)) & 0xFFu);
      }
    } else {
      const uint32_t w = __builtin_amdgcn_alignbyte(r.w[4], r.w[3], (p.kps + li * VB) & 3);
      const uint32_t sz = __builtin_amdgcn_alignbyte(r.w[6], r.w[5], (p.kps + p.vdb) & 3);
      const float vsc = half_lo(sz);
      const float vz = half_hi(sz);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vd[j] = (float)((w >> (VB * j)) & ((1u << VB) - 1u)) * vsc + vz;
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

  // U tokens per lane group: every raw load is issued before any decode
  for (int64_t tb = t0 + grp; tb < t1; tb += (int64_t)U * NG) {
    Raw r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = load_raw(tb + (int64_t)u * NG);
#pragma unroll
    for (int u = 0; u < U; ++u) consume(r[u]);
  }

  // ---- merge the lane groups of this wave (log-sum-exp) ----
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
  for (int i = tid; i < nh * (D + 1); i += 256) {
    const int hh = i / (D + 1), d = i % (D + 1);
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][hh][D]);
    float lsum = 0.0f, o = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = exp2f(red[w][hh][D] - mm);
        lsum += red[w][hh][D + 1] * a;
        if (d < D) o += red[w][hh][d] * a;
      }
    }
    float* dst = p.ws + (((int64_t)b * p.hq + h0 + hh) * p.splits + s) * (D + 1);
    if (d < D) dst[d] = lsum > 0.0f ? o / lsum : 0.0f;
    else dst[D] = lsum > 0.0f ? (mm + log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <int D, int KF, int VF>
hipError_t launch_g(const DecodeParams& p, hipStream_t st) {
  const int G = p.g <= 1 ? 1 : (p.g <= 2 ? 2 : (p.g <= 4 ? 4 : 8));
  const int chunks = (p.g + G - 1) / G;
  const uint32_t blocks = (uint32_t)p.B * p.hk * chunks * p.splits;
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_generic_kernel<D, KF, VF, 1, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_generic_kernel<D, KF, VF, 2, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_generic_kernel<D, KF, VF, 4, 4>), dim3(blocks), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((decode_generic_kernel<D, KF, VF, 8, 4>), dim3(blocks), dim3(256), 0, st, p); break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
  switch (p.key_fmt * 4 + p.val_fmt) {
    case KF_INT4 * 4 + VF_INT4:
      if constexpr (D == 256) return hipErrorNotSupported;  // INT4: D = 64, 128
      else return launch_g<D, KF_INT4, VF_INT4>(p, st);
    case KF_FP8 * 4 + VF_U3: return launch_g<D, KF_FP8, VF_U3>(p, st);
    case KF_FP8 * 4 + VF_U4: return launch_g<D, KF_FP8, VF_U4>(p, st);
    case KF_MSE3 * 4 + VF_U3: return launch_g<D, KF_MSE3, VF_U3>(p, st);
    case KF_MSE3 * 4 + VF_U4: return launch_g<D, KF_MSE3, VF_U4>(p, st);
    case KF_MSE4 * 4 + VF_U3: return launch_g<D, KF_MSE4, VF_U3>(p, st);
    case KF_MSE4 * 4 + VF_U4: return launch_g<D, KF_MSE4, VF_U4>(p, st);
    case KF_FP8 * 4 + VF_FP8: return launch_g<D, KF_FP8, VF_FP8>(p, st);
    case KF_MSE3 * 4 + VF_FP8: return launch_g<D, KF_MSE3, VF_FP8>(p, st);
    case KF_MSE4 * 4 + VF_FP8: return launch_g<D, KF_MSE4, VF_FP8>(p, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_decode_generic(const DecodeParams& p, hipStream_t st) {
  if (p.d == 128) return launch_d<128>(p, st);
  if (p.d == 64) return launch_d<64>(p, st);
  if (p.d == 256) return launch_d<256>(p, st);
  return hipErrorNotSupported;
}

}  // namespace tqk
