// INT4 split-KV decode, stage 1, on the CDNA4 matrix cores
// (int4_per_token_head.py: unified_attention_int4 / _attn_packed; split
// ranges and partials as triton_turboquant_decode.py, _tq_decode_stage1).
//
// Both contractions of a grouped decode step -- scores S = Q' K^T over the
// head dimension and the value sum O = P' V over tokens -- run as
// v_mfma_i32_16x16x64_i8 on exact integers:
//   * K and V nibbles (0..15) are int8 operands as they are;
//   * the rotated query q' (per head) is scaled by a power of two to an
//     integer below 2^27 and split into four balanced base-128 digits in
//     [-64, 64]; the four digit planes of four heads fill the 16 MFMA rows;
//   * the softmax weights P' = p * scale_v (p <= 1) are scaled per tile by a
//     power of two to an integer below 2^27 and split into four 7-bit digits.
// The int32 MFMA sums are exact; the digit planes are recombined in fp32
// (one rounding per tile and head), so the result carries fp32-level error
// while moving the 2*g*D multiply-adds per token off the vector ALUs.
// The zero points enter exactly in integers: q'.(n - zp) = q'.n - zp*sum(q')
// per digit plane, and sum_t P'_t (n_t - zp_t) = sum_t P'_t n_t -
// sum_t P'_t zp_t per digit plane.
//
// Work decomposition: one workgroup of W waves per (batch, split, kv head),
// with the kv head fastest and the XCD-aware renumbering, so the eight
// heads of one token row (sharing cache lines) run in one L2. Waves take
// 64-token tiles of the split in turn and are merged by log-sum-exp at the
// end. Inside a tile:
//   K side: lane (n, g) loads bytes [16g, 16g+16) of token 16s+n's 64-byte
//   key row (s = 0..3), i.e. four fully used 64-byte segments per token;
//   V side: lane (n, g) loads dword n (8 nibbles) of 16 tokens and a nibble
//   transpose (byte permutes) builds the B operands, so that column n of
//   MFMA i is output dimension 8n+i.
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// max / sum over the 16 lanes of a DPP row (lanes sharing lane / 16)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)));  // row_ror:8
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)));  // row_ror:4
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<1>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));
  v += xor_lane<2>(v);
  v += xor_lane<1>(v);
  return v;
}
__device__ __forceinline__ int row16_isum(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  return v;
}

// 2^e for an integer e in [-126, 127]
__device__ __forceinline__ float exp2i(int e) { return u2f((uint32_t)(e + 127) << 23); }

template <int NH, int W>
__global__ __launch_bounds__(64 * W) void decode_int4_mfma_kernel(DecodeParams p) {
  constexpr int NHEAD = 4 * NH;  // query heads per workgroup (padded)
  __shared__ __attribute__((aligned(16))) int32_t rows_lds[W][64];
  __shared__ __attribute__((aligned(16))) uint32_t p8_lds[W][NH][4][4][16];
  __shared__ int32_t qsum_lds[NHEAD][4];
  __shared__ float qf_lds[NHEAD];
  __shared__ int32_t qexp_lds[NHEAD];
  // prologue: rotated queries; epilogue: per-wave partials (not live together)
  __shared__ float big[(W * NHEAD * (D + 2) > NHEAD * D) ? W * NHEAD * (D + 2) : NHEAD * D];

  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int kvh = lb % p.hk;
  const int s_idx = (lb / p.hk) % p.splits;
  const int b = lb / (p.hk * p.splits);

  int64_t seq = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  seq = seq < 0 ? 0 : (seq > cap ? cap : seq);
  const int64_t split_len = (seq + p.splits - 1) / p.splits;
  const int64_t t0 = split_len * s_idx;
  const int64_t t1 = (t0 + split_len < seq) ? t0 + split_len : seq;
  if (t0 >= t1) return;  // empty split: nothing written (stage 2 skips it)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;   // n: MFMA column / row within a 16-lane group
  const int lg = lane >> 4;   // g: 16-lane group
  const int g = p.g;
  const int h0 = kvh * g;

  // ---------------- query prologue ----------------
  float* qrot = big;  // [NHEAD][D]
  for (int i = tid; i < NHEAD * D; i += 64 * W) {
    const int hh = i / D, d = i % D;
    qrot[i] = hh < g ? p.q[((int64_t)b * p.hq + h0 + hh) * D + d] * p.rht_signs[d] : 0.0f;
  }
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int i = tid; i < NHEAD * D / 2; i += 64 * W) {
      const int hh = i / (D / 2), k = i % (D / 2);
      const int lo = hh * D + (k / hs) * 2 * hs + (k % hs);
      const float a = qrot[lo], c = qrot[lo + hs];
      qrot[lo] = a + c;
      qrot[lo + hs] = a - c;
    }
    __syncthreads();
  }
  // per-head power-of-two scale: |q'| * 2^E < 2^27
  for (int hh = wave; hh < NHEAD; hh += W) {
    const float amax = group_max<64>(fmaxf(fabsf(qrot[hh * D + lane]), fabsf(qrot[hh * D + 64 + lane])));
    if (lane == 0) {
      const int e = amax > 0.0f ? (int)((f2u(amax) >> 23) & 0xFF) - 127 : 0;
      const int E = amax > 0.0f ? 26 - e : 0;
      qexp_lds[hh] = E;
      // score in base-2 units = sm_scale / D * log2(e) * 2^-E * (integer dot)
      qf_lds[hh] = p.sm_scale / (float)D * kLog2e * exp2i(-E);
    }
  }
  __syncthreads();

  // A operands of the score MFMA: lane (m = 4*h' + piece, g) holds the digit
  // `piece` of head 4r+h' for dims 32g + {16c + 8(j/2) + 2b + (j%2)}: the
  // byte order the K nibble unpack produces.
  v4i qa[NH][2];
#pragma unroll
  for (int r = 0; r < NH; ++r) {
    const int hh = 4 * r + (ln >> 2);
    const int piece = ln & 3;
    const float sc = exp2i(qexp_lds[hh]);
    int dsum = 0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      int words[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int dim = 32 * lg + 16 * c + 8 * (j >> 1) + 2 * bb + (j & 1);
          int v = (int)__builtin_rintf(qrot[hh * D + dim] * sc);
          int dg = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int dk = (k < 3) ? (((v + 64) & 127) - 64) : v;
            if (k == piece) dg = dk;
            v = (v - dk) >> 7;
          }
          dsum += dg;
          words[j] |= (dg & 0xFF) << (8 * bb);
        }
      }
      qa[r][c] = v4i{words[0], words[1], words[2], words[3]};
    }
    // sum of the digits over all D dims: reduce over the four 16-lane groups
    dsum += __builtin_amdgcn_ds_bpermute((int)((lane ^ 16) << 2), dsum);
    dsum += __builtin_amdgcn_ds_bpermute((int)((lane ^ 32) << 2), dsum);
    if (wave == 0 && lg == 0) qsum_lds[hh][piece] = dsum;
  }
  __syncthreads();
  // per-lane constants of the score side: lane (n, g) scores head 4r+g
  int qsum[NH][4];
  float qf[NH];
#pragma unroll
  for (int r = 0; r < NH; ++r) {
#pragma unroll
    for (int k = 0; k < 4; ++k) qsum[r][k] = qsum_lds[4 * r + lg][k];
    qf[r] = qf_lds[4 * r + lg];
  }

  float m[NH], l[NH], acc[NH][8];
#pragma unroll
  for (int r = 0; r < NH; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[r][i] = 0.0f;
  }

  const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
  const int64_t ntiles = (t1 - t0 + 63) / 64;
  for (int64_t tile = wave; tile < ntiles; tile += W) {
    const int64_t T0 = t0 + tile * 64;
    // ---- cache row of every token of the tile (-1: masked) ----
    {
      const int64_t tok = T0 + lane;
      int32_t row = -1;
      if (tok < t1) {
        const int64_t page = bt[tok / p.block_size];
        if (page >= 0 && page < p.num_blocks)
          row = (int32_t)((page * p.block_size + tok % p.block_size) * p.hk + kvh);
      }
      rows_lds[wave][lane] = row;
    }
    wave_sync();
    int32_t rk[4];
    int4 rv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rk[s] = rows_lds[wave][16 * s + ln];
      rv[s] = *reinterpret_cast<const int4*>(&rows_lds[wave][16 * s + 4 * lg]);
    }
    // ---- loads ----
    uint4 kraw[4];
    uint32_t ksw[4], vsw[4];
    uint32_t vraw[4][4];  // [s][k]: dword ln of token 16s + 4lg + k
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t r0 = rk[s] < 0 ? 0 : rk[s];
      kraw[s] = *reinterpret_cast<const uint4*>(p.kc + r0 * (D / 2) + 16 * lg);
      ksw[s] = f2u(p.ks[r0]);
      vsw[s] = f2u(p.vs[r0]);
      const int rr[4] = {rv[s].x, rv[s].y, rv[s].z, rv[s].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t rvk = rr[k] < 0 ? 0 : rr[k];
        vraw[s][k] = *reinterpret_cast<const uint32_t*>(p.vc + rvk * (D / 2) + 4 * ln);
      }
    }

    // ---- scores on the matrix cores ----
    float sc[NH][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w4[4] = {kraw[s].x, kraw[s].y, kraw[s].z, kraw[s].w};
      int ev[4], od[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ev[k] = (int)(w4[k] & 0x0F0F0F0Fu);
        od[k] = (int)((w4[k] >> 4) & 0x0F0F0F0Fu);
      }
      const v4i kb0 = v4i{ev[0], od[0], ev[1], od[1]};
      const v4i kb1 = v4i{ev[2], od[2], ev[3], od[3]};
      const int zpki = (int)(ksw[s] & 0xFu);
      const float ksc = u2f(ksw[s] & 0xFFFFFFF0u);
#pragma unroll
      for (int r = 0; r < NH; ++r) {
        v4i c = v4i{0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][0], kb0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][1], kb1, c, 0, 0, 0);
        // lane (n, g): rows 4g..4g+3 = digits 0..3 of head 4r+g, token 16s+n
        const float d0 = (float)(c.x - zpki * qsum[r][0]);
        const float d1 = (float)(c.y - zpki * qsum[r][1]);
        const float d2 = (float)(c.z - zpki * qsum[r][2]);
        const float d3 = (float)(c.w - zpki * qsum[r][3]);
        const float dot = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(d3, 128.0f, d2), 128.0f, d1), 128.0f, d0);
        sc[r][s] = rk[s] < 0 ? -INFINITY : dot * (qf[r] * ksc);
      }
    }

    // ---- online softmax (per head = per 16-lane group) ----
    float alpha[NH], pr[NH][4];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      float tm = fmaxf(fmaxf(sc[r][0], sc[r][1]), fmaxf(sc[r][2], sc[r][3]));
      tm = row16_max(tm);
      const float mn = fmaxf(m[r], tm);
      const bool none = (mn == -INFINITY);
      alpha[r] = none ? 1.0f : __builtin_amdgcn_exp2f(m[r] - mn);
      float ps = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        pr[r][s] = none ? 0.0f : __builtin_amdgcn_exp2f(sc[r][s] - mn);
        ps += pr[r][s];
      }
      l[r] = l[r] * alpha[r] + ps;
      m[r] = mn;
    }

    // ---- value weights P' = p * scale_v as 7-bit digit planes ----
    float vsc[4];
    int zpv[4];
    float smax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      vsc[s] = u2f(vsw[s] & 0xFFFFFFF0u);
      zpv[s] = (int)(vsw[s] & 0xFu);
      if (rk[s] >= 0) smax = fmaxf(smax, vsc[s]);
    }
    smax = row16_max(smax);
    const int ev_ = smax > 0.0f ? 26 - ((int)((f2u(smax) >> 23) & 0xFF) - 127) : 0;
    const float pscale = exp2i(ev_);
    const float pinv = exp2i(-ev_);
    int zsum[NH][4];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      uint32_t dw[4] = {0, 0, 0, 0};
      int z[4] = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t pi = (uint32_t)__builtin_rintf((pr[r][s] * vsc[s]) * pscale);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t dk = (pi >> (7 * k)) & 127u;
          dw[k] |= dk << (8 * s);
          z[k] += (int)dk * zpv[s];
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p8_lds[wave][r][lg][k][ln] = dw[k];
        zsum[r][k] = row16_isum(z[k]);
      }
    }
    wave_sync();

    // ---- value MFMAs: B operands by nibble transpose ----
    // vb[i][k]: byte s = nibble i (dim 8*ln + i) of token 16s + 4lg + k
    uint32_t vb[8][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w0 = vraw[0][k], w1 = vraw[1][k], w2 = vraw[2][k], w3 = vraw[3][k];
      const uint32_t x01l = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
      const uint32_t x01h = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
      const uint32_t x23l = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
      const uint32_t x23h = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
      const uint32_t t[4] = {__builtin_amdgcn_perm(x23l, x01l, 0x05040100u),
                             __builtin_amdgcn_perm(x23l, x01l, 0x07060302u),
                             __builtin_amdgcn_perm(x23h, x01h, 0x05040100u),
                             __builtin_amdgcn_perm(x23h, x01h, 0x07060302u)};
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        vb[2 * bb][k] = t[bb] & 0x0F0F0F0Fu;
        vb[2 * bb + 1][k] = (t[bb] >> 4) & 0x0F0F0F0Fu;
      }
    }
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      // A operand: lane (m = 4h' + piece, g) reads the digit plane of head
      // 4r+h' for tokens 16s + 4g + k at byte (k, s)
      const uint4 a4 = *reinterpret_cast<const uint4*>(&p8_lds[wave][r][ln >> 2][ln & 3][4 * lg]);
      const v4i pa = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v4i vbi = v4i{(int)vb[i][0], (int)vb[i][1], (int)vb[i][2], (int)vb[i][3]};
        const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa, vbi, v4i{0, 0, 0, 0}, 0, 0, 0);
        // lane (n, g): digits 0..3 of head 4r+g, dim 8n+i
        const float e0 = (float)(c.x - zsum[r][0]);
        const float e1 = (float)(c.y - zsum[r][1]);
        const float e2 = (float)(c.z - zsum[r][2]);
        const float e3 = (float)(c.w - zsum[r][3]);
        const float val = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(e3, 128.0f, e2), 128.0f, e1), 128.0f, e0);
        acc[r][i] = __builtin_fmaf(val, pinv, acc[r][i] * alpha[r]);
      }
    }
    wave_sync();  // p8_lds / rows_lds are rewritten by the next tile
  }

  // ---------------- merge the waves, write the split partial ----------------
  __syncthreads();  // qrot (aliased by `big`) is dead from here on
  float* red = big;  // [W][NHEAD][D + 2]
#pragma unroll
  for (int r = 0; r < NH; ++r) {
    const float lt = row16_sum(l[r]);
    float* dst = red + ((wave * NHEAD) + 4 * r + lg) * (D + 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[8 * ln + i] = acc[r][i];
    if (ln == 0) {
      dst[D] = m[r];
      dst[D + 1] = lt;
    }
  }
  __syncthreads();
  for (int i = tid; i < g * (D + 1); i += 64 * W) {
    const int hh = i / (D + 1), d = i % (D + 1);
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) mm = fmaxf(mm, red[(w * NHEAD + hh) * (D + 2) + D]);
    float lsum = 0.0f, o = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float* src = red + (w * NHEAD + hh) * (D + 2);
        const float a = __builtin_amdgcn_exp2f(src[D] - mm);
        lsum += src[D + 1] * a;
        if (d < D) o += src[d] * a;
      }
    }
    float* out = p.ws + (((int64_t)b * p.hq + h0 + hh) * p.splits + s_idx) * (D + 1);
    if (d < D) out[d] = lsum > 0.0f ? o / lsum : 0.0f;
    else out[D] = lsum > 0.0f ? (mm + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <int NH, int W>
hipError_t launch(const DecodeParams& p, hipStream_t st) {
  const uint32_t blocks = (uint32_t)p.B * p.hk * p.splits;
  hipLaunchKernelGGL((decode_int4_mfma_kernel<NH, W>), dim3(blocks), dim3(64 * W), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_int4_mfma(const DecodeParams& p, hipStream_t st) {
  if (p.d != D || p.key_fmt != KF_INT4 || p.g > 16) return hipErrorNotSupported;
  // cache rows are addressed with 32-bit indices
  if (p.num_blocks * (int64_t)p.block_size * p.hk >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  // eight waves per workgroup when there are few (batch, split, kv head)
  // units, so that the grid still holds enough waves to cover HBM latency
  const int64_t units = (int64_t)p.B * p.hk * p.splits;
  const bool wide = units < 1024;
  const int nh = (p.g + 3) / 4;
  switch (nh) {
    case 1: return wide ? launch<1, 8>(p, st) : launch<1, 4>(p, st);
    case 2: return wide ? launch<2, 8>(p, st) : launch<2, 4>(p, st);
    default: return launch<4, 4>(p, st);
  }
}

}  // namespace tqk
