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

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads outside return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kMasked = 0x03FFFFFFu;  // row index whose bytes lie past any buffer
// Headroom of the value-weight fixed point: weights are taken relative to a
// reference maximum that is raised only when a tile exceeds it by more than
// 2^kTau, so p = 2^(s - m_ref) <= 2^kTau.
constexpr int kTau = 4;
constexpr int kMaxPages = 2048;  // block-table entries staged in LDS

// One workgroup per (split, batch, group of HG kv heads); W = HG * R waves:
// wave w serves kv head (group * HG + w % HG) and takes every R-th tile of
// the split starting at tile w / HG. All waves walk the same pages at the
// same pace, so the HG heads' slices of each token row are requested
// together (whole rows when HG = Hk), which keeps DRAM pages open.
template <int NH, int W>
__global__ __launch_bounds__(64 * W) void decode_int4_mfma_kernel(DecodeParams p, int HG) {
  constexpr int NHEAD = 4 * NH;  // query heads per kv head (padded)
  __shared__ __attribute__((aligned(16))) uint32_t rows_lds[W][64];
  // per wave: MFMA A-operand image of its queries (prologue), then the
  // per-tile weight digit planes
  __shared__ __attribute__((aligned(16))) uint32_t wbuf[W][NH][2][64][4];
  __shared__ int32_t pages_lds[kMaxPages];
  __shared__ float red[W][NHEAD][D + 2];

  const int R = W / HG;
  const int ngrp = p.hk / HG;
  const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  // split slowest: each XCD receives whole split indices of every sequence
  const int grp = lb % ngrp;
  const int b = (lb / ngrp) % p.B;
  const int s_idx = lb / (ngrp * p.B);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;   // n: MFMA column / row within a 16-lane group
  const int lg = lane >> 4;   // g: 16-lane group
  const int kvh = grp * HG + wave % HG;
  const int rsl = wave / HG;  // this wave's tile slice
  const int g = p.g;
  const int h0 = kvh * g;
  const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
  // the whole block-table row is staged when it fits, independently of the
  // sequence length, so that it loads in the same round trip as seq_len
  const bool row_in_lds = p.max_blocks <= kMaxPages;
  if (row_in_lds)
    for (int i = tid; i < p.max_blocks; i += 64 * W) pages_lds[i] = bt[i];
  // this wave's queries, two dims per lane, signs applied
  float qx[NHEAD][2];
#pragma unroll
  for (int hh = 0; hh < NHEAD; ++hh) {
    const bool ok = hh < g;
    const float* qrow = p.q + ((int64_t)b * p.hq + h0 + (ok ? hh : 0)) * D;
    qx[hh][0] = ok ? qrow[lane] * p.rht_signs[lane] : 0.0f;
    qx[hh][1] = ok ? qrow[lane + 64] * p.rht_signs[lane + 64] : 0.0f;
  }

  int64_t seq = p.seq_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  seq = seq < 0 ? 0 : (seq > cap ? cap : seq);
  const int64_t split_len = (seq + p.splits - 1) / p.splits;
  const int64_t t0 = split_len * s_idx;
  const int64_t t1 = (t0 + split_len < seq) ? t0 + split_len : seq;
  if (t0 >= t1) return;  // empty split (uniform): nothing written, stage 2 skips it

  const uint32_t bs = (uint32_t)p.block_size;
  const bool bs_pow2 = (bs & (bs - 1u)) == 0u;
  const int bs_shift = __builtin_ctz(bs);
  const uint32_t nrows = (uint32_t)(p.num_blocks * bs * p.hk);
  const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(p.kc, nrows * (uint32_t)(D / 2));
  const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(p.vc, nrows * (uint32_t)(D / 2));
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(p.ks, nrows * 4u);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(p.vs, nrows * 4u);
  __syncthreads();  // page list staged

  const int64_t ntiles = (t1 - t0 + 63) / 64;
  // Row index of the tile's token `lane` into rows_lds (masked: kMasked).
  auto stage_rows = [&](int64_t tile) {
    const int64_t tok = t0 + tile * 64 + lane;
    uint32_t row = kMasked;
    if (tile < ntiles && tok < t1) {
      const uint32_t t32 = (uint32_t)tok;
      const uint32_t pi = bs_pow2 ? (t32 >> bs_shift) : (t32 / bs);
      const int64_t page = row_in_lds ? pages_lds[pi] : bt[pi];
      if (page >= 0 && page < p.num_blocks)
        row = ((uint32_t)page * bs + (t32 - pi * bs)) * (uint32_t)p.hk + (uint32_t)kvh;
    }
    rows_lds[wave][lane] = row;
    wave_sync();
  };
  // key bytes + both scale words of tokens 16s+n (masked rows read 0)
  v4u kraw[4];
  uint32_t ksw[4], vsw[4], live = 0;
  auto issue_k = [&]() {
    live = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t r = rows_lds[wave][16 * s + ln];
      live |= (r != kMasked ? 1u : 0u) << s;
      kraw[s] = __builtin_amdgcn_raw_buffer_load_b128(rk_, (int)((r << 6) | (16u * lg)), 0, 0);
      ksw[s] = __builtin_amdgcn_raw_buffer_load_b32(rks, (int)(r << 2), 0, 0);
      vsw[s] = __builtin_amdgcn_raw_buffer_load_b32(rvs, (int)(r << 2), 0, 0);
    }
  };
  // value dword n of tokens 16s+4g+k
  uint32_t vraw[4][4];
  auto issue_v = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 rv = *reinterpret_cast<const uint4*>(&rows_lds[wave][16 * s + 4 * lg]);
      const uint32_t rr[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vraw[s][k] = __builtin_amdgcn_raw_buffer_load_b32(rv_, (int)((rr[k] << 6) | (4u * ln)), 0, 0);
    }
  };

  stage_rows(rsl);  // the first tile's loads overlap the query prologue
  issue_k();
  issue_v();

  // ---------------- query prologue (per wave, no barrier) ----------------
  // Rotate each head (two dims per lane), scale by a power of two to
  // integers below 2^27, split into four balanced base-128 digits and
  // scatter them into the MFMA A-operand image: lane (m = 4h' + piece, g)
  // holds, for chunk c, dword j, byte b, the digit of dim
  // 32g + 16c + 8(j/2) + 2b + (j%2) -- the order of the K unpack.
  float qsum[NH][4], qf[NH];
  {
    uint8_t* img = reinterpret_cast<uint8_t*>(&wbuf[wave][0][0][0][0]);
#pragma unroll
    for (int hh = 0; hh < NHEAD; ++hh) {
      float x0 = qx[hh][0], x1 = qx[hh][1];
      {
        const float a = x0 + x1, c = x0 - x1;
        x0 = a;
        x1 = c;
      }
      x0 = butterfly_lanes<1>(x0, lane & 1);   x1 = butterfly_lanes<1>(x1, lane & 1);
      x0 = butterfly_lanes<2>(x0, lane & 2);   x1 = butterfly_lanes<2>(x1, lane & 2);
      x0 = butterfly_lanes<4>(x0, lane & 4);   x1 = butterfly_lanes<4>(x1, lane & 4);
      x0 = butterfly_lanes<8>(x0, lane & 8);   x1 = butterfly_lanes<8>(x1, lane & 8);
      x0 = butterfly_lanes<16>(x0, lane & 16); x1 = butterfly_lanes<16>(x1, lane & 16);
      x0 = butterfly_lanes<32>(x0, lane & 32); x1 = butterfly_lanes<32>(x1, lane & 32);
      // x0 = q'[lane], x1 = q'[lane + 64]
      const float amax = group_max<64>(fmaxf(fabsf(x0), fabsf(x1)));
      const int E = amax > 0.0f ? 26 - ((int)((f2u(amax) >> 23) & 0xFF) - 127) : 0;
      const float sc = exp2i(E);
      const int r = hh >> 2, hp = hh & 3;
      float dsum[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int dim = lane + 64 * e;
        int v = (int)__builtin_rintf((e ? x1 : x0) * sc);
        const int gg = dim >> 5, o = dim & 31;
        const int c = o >> 4, j = 2 * ((o & 15) >> 3) + (o & 1), bb = (o & 7) >> 1;
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) {
          const int dk = (pc < 3) ? (((v + 64) & 127) - 64) : v;
          v = (v - dk) >> 7;
          const int L = 16 * gg + 4 * hp + pc;
          img[(((r * 2 + c) * 64 + L) * 4 + j) * 4 + bb] = (uint8_t)(dk & 0xFF);
          dsum[pc] = (e ? dsum[pc] : 0.0f) + (float)dk;
        }
      }
      // lane (n, g) scores head 4r+g: keep that head's digit sums and scale
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const float t = group_sum<64>(dsum[pc]);
        if (hp == lg) qsum[r][pc] = t;
      }
      // score in base-2 units = sm_scale / D * log2(e) * 2^-E * (integer dot)
      if (hp == lg) qf[r] = p.sm_scale / (float)D * kLog2e * exp2i(-E);
    }
  }
  wave_sync();
  v4i qa[NH][2];
#pragma unroll
  for (int r = 0; r < NH; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 w4 = *reinterpret_cast<const uint4*>(&wbuf[wave][r][c][lane][0]);
      qa[r][c] = v4i{(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w};
    }
  wave_sync();  // the image region is reused for the weight digit planes
  uint32_t(*p8)[4][4][16] = reinterpret_cast<uint32_t(*)[4][4][16]>(&wbuf[wave][0][0][0][0]);

  // Online softmax state, all relative to a reference maximum m_ref (base-2
  // units) per head and a power-of-two weight scale 2^ev shared by the wave:
  //   l     per-lane sum of 2^(s - m_ref) over the lane's tokens
  //   cacc  int32 MFMA sums of the weight digit planes times the value
  //         nibbles (lane (n, g): head 4r+g, dims 8n+i, planes 0..3)
  //   zl    per-lane sums of weight digits times value zero points
  //   acc   fp32 part folded at each flush
  float mref[NH], l[NH], acc[NH][8];
  v4i cacc[NH][8];
  int zl[NH][4];
#pragma unroll
  for (int r = 0; r < NH; ++r) {
    mref[r] = -INFINITY;
    l[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[r][i] = 0.0f;
      cacc[r][i] = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) zl[r][k] = 0;
  }
  int ev = 0;             // weight scale exponent
  float sref = 0.0f;      // value scales below sref fit the current ev
  bool empty = true;      // cacc / zl hold nothing
  int since_flush = 0;    // tiles accumulated since the last flush

  // fold cacc/zl into acc (scale 2^-ev), then rescale by alpha per head
  auto flush = [&](const float (&alpha)[NH]) {
    const float pinv = exp2i(-ev);
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      if (!empty) {
        float zs[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) zs[k] = (float)row16_isum(zl[r][k]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // digit plane minus its zero-point sum: exact small integers
          const float e0 = (float)cacc[r][i].x - zs[0];
          const float e1 = (float)cacc[r][i].y - zs[1];
          const float e2 = (float)cacc[r][i].z - zs[2];
          const float e3 = (float)cacc[r][i].w - zs[3];
          const float val = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(e3, 128.0f, e2), 128.0f, e1), 128.0f, e0);
          acc[r][i] = __builtin_fmaf(val, pinv, acc[r][i]);
          cacc[r][i] = v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) zl[r][k] = 0;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[r][i] *= alpha[r];
      l[r] *= alpha[r];
    }
    empty = true;
  };

  for (int64_t tile = rsl; tile < ntiles; tile += R) {
    // ---- scores on the matrix cores ----
    float sc[NH][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4u w4 = kraw[s];
      int evn[4], odd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        evn[k] = (int)(w4[k] & 0x0F0F0F0Fu);
        odd[k] = (int)((w4[k] >> 4) & 0x0F0F0F0Fu);
      }
      const v4i kb0 = v4i{evn[0], odd[0], evn[1], odd[1]};
      const v4i kb1 = v4i{evn[2], odd[2], evn[3], odd[3]};
      const float zpk = (float)(ksw[s] & 0xFu);
      const float ksc = u2f(ksw[s] & 0xFFFFFFF0u);
      // masked tokens: min(score, -inf) keeps the arithmetic unconditional
      const float mask = ((live >> s) & 1u) ? INFINITY : -INFINITY;
#pragma unroll
      for (int r = 0; r < NH; ++r) {
        v4i c = v4i{0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][0], kb0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][1], kb1, c, 0, 0, 0);
        // lane (n, g): rows 4g..4g+3 = digits 0..3 of head 4r+g, token 16s+n;
        // each plane minus zp * (digit sum) is an exact small integer
        const float d0 = __builtin_fmaf(-zpk, qsum[r][0], (float)c.x);
        const float d1 = __builtin_fmaf(-zpk, qsum[r][1], (float)c.y);
        const float d2 = __builtin_fmaf(-zpk, qsum[r][2], (float)c.z);
        const float d3 = __builtin_fmaf(-zpk, qsum[r][3], (float)c.w);
        const float dot = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(d3, 128.0f, d2), 128.0f, d1), 128.0f, d0);
        sc[r][s] = fminf(dot * (qf[r] * ksc), mask);
      }
    }
    float vsc[4];
    uint32_t zp4 = 0;
    float smax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      vsc[s] = u2f(vsw[s] & 0xFFFFFFF0u);
      zp4 |= (vsw[s] & 0xFu) << (8 * s);
      smax = fmaxf(smax, vsc[s]);  // masked tokens load scale 0
    }
    // the next tile's rows and key-side loads (this tile's are consumed)
    stage_rows(tile + R);
    issue_k();

    // ---- reference maximum / weight scale; flush when they move ----
    float tm[NH];
    bool move = false;
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      tm[r] = row16_max(fmaxf(fmaxf(sc[r][0], sc[r][1]), fmaxf(sc[r][2], sc[r][3])));
      move |= tm[r] > mref[r] + (float)kTau;
    }
    smax = row16_max(smax);
    // a flush also bounds the int32 digit sums (< 2^31 after 8192 tiles)
    const bool smove = smax >= sref || ++since_flush >= 8192;
    if (__builtin_amdgcn_ballot_w64(move || smove) != 0) {
      float alpha[NH];
#pragma unroll
      for (int r = 0; r < NH; ++r) {
        const float mn = fmaxf(mref[r], tm[r]);
        alpha[r] = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mref[r] - mn);
        mref[r] = mn;
      }
      flush(alpha);
      since_flush = 0;
      // ev from the largest value scale (the same in every lane): weights
      // 2^(s - m_ref) * scale <= 2^kTau * sref stay below 2^27 after 2^ev
      if (smax > 0.0f) {
        const int e = (int)((f2u(smax) >> 23) & 0xFF) - 127;
        ev = 26 - kTau - e;
        sref = exp2i(e + 1);
      }
    }

    // ---- weights relative to m_ref as 7-bit digit planes ----
    const float pscale = exp2i(ev);
    float vq[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) vq[s] = vsc[s] * pscale;
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      uint32_t dw[4] = {0, 0, 0, 0};
      float ps = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float pr = (mref[r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[r][s] - mref[r]);
        ps += pr;
        const uint32_t pi = (uint32_t)__builtin_fmaf(pr, vq[s], 0.5f);
#pragma unroll
        for (int k = 0; k < 4; ++k) dw[k] |= ((pi >> (7 * k)) & 127u) << (8 * s);
      }
      l[r] += ps;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p8[r][lg][k][ln] = dw[k];
        zl[r][k] += (int)__builtin_amdgcn_udot4(dw[k], zp4, 0u, false);
      }
    }
    empty = false;
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
    issue_v();  // next tile's value rows (staged above)
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      // A operand: lane (m = 4h' + piece, g) reads the digit plane of head
      // 4r+h' for tokens 16s + 4g + k at byte (k, s)
      const uint4 a4 = *reinterpret_cast<const uint4*>(&p8[r][ln >> 2][ln & 3][4 * lg]);
      const v4i pa = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v4i vbi = v4i{(int)vb[i][0], (int)vb[i][1], (int)vb[i][2], (int)vb[i][3]};
        cacc[r][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa, vbi, cacc[r][i], 0, 0, 0);
      }
    }
    wave_sync();  // the digit planes are rewritten by the next tile
  }
  {
    float one[NH];
#pragma unroll
    for (int r = 0; r < NH; ++r) one[r] = 1.0f;
    flush(one);
  }

  // ---------------- write the split partial ----------------
  // acc / l are relative to m_ref per head (l: per-lane partial sums)
  float lt[NH];
#pragma unroll
  for (int r = 0; r < NH; ++r) lt[r] = row16_sum(l[r]);
  if (R == 1) {
    // this wave alone covered the split for its heads
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      const int hh = 4 * r + lg;
      if (hh < g) {
        float* out = p.ws + (((int64_t)b * p.hq + h0 + hh) * p.splits + s_idx) * (D + 1);
        const float inv = lt[r] > 0.0f ? 1.0f / lt[r] : 0.0f;
        float4 o0, o1;
        o0.x = acc[r][0] * inv; o0.y = acc[r][1] * inv; o0.z = acc[r][2] * inv; o0.w = acc[r][3] * inv;
        o1.x = acc[r][4] * inv; o1.y = acc[r][5] * inv; o1.z = acc[r][6] * inv; o1.w = acc[r][7] * inv;
        float* dst = out + 8 * ln;
        dst[0] = o0.x; dst[1] = o0.y; dst[2] = o0.z; dst[3] = o0.w;
        dst[4] = o1.x; dst[5] = o1.y; dst[6] = o1.z; dst[7] = o1.w;
        if (ln == 0) out[D] = lt[r] > 0.0f ? (mref[r] + __log2f(lt[r])) * kLn2 : -INFINITY;
      }
    }
    return;
  }
  // R waves shared each head: log-sum-exp merge through LDS
#pragma unroll
  for (int r = 0; r < NH; ++r) {
    float* dst = &red[wave][4 * r + lg][0];
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[8 * ln + i] = acc[r][i];
    if (ln == 0) {
      dst[D] = mref[r];
      dst[D + 1] = lt[r];
    }
  }
  __syncthreads();
  for (int i = tid; i < HG * g * (D + 1); i += 64 * W) {
    const int hw = i / (g * (D + 1));          // wave (= head) within the group
    const int hh = (i / (D + 1)) % g, d = i % (D + 1);
    float mm = -INFINITY;
    for (int rr = 0; rr < R; ++rr) mm = fmaxf(mm, red[hw + rr * HG][hh][D]);
    float lsum = 0.0f, o = 0.0f;
    if (mm != -INFINITY) {
      for (int rr = 0; rr < R; ++rr) {
        const float* src = &red[hw + rr * HG][hh][0];
        const float a = __builtin_amdgcn_exp2f(src[D] - mm);
        lsum += src[D + 1] * a;
        if (d < D) o += src[d] * a;
      }
    }
    const int head = (grp * HG + hw) * g + hh;
    float* out = p.ws + (((int64_t)b * p.hq + head) * p.splits + s_idx) * (D + 1);
    if (d < D) out[d] = lsum > 0.0f ? o / lsum : 0.0f;
    else out[D] = lsum > 0.0f ? (mm + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <int NH, int W>
hipError_t launch(const DecodeParams& p, int hg, hipStream_t st) {
  const uint32_t blocks = (uint32_t)p.B * (p.hk / hg) * p.splits;
  hipLaunchKernelGGL((decode_int4_mfma_kernel<NH, W>), dim3(blocks), dim3(64 * W), 0, st, p, hg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_int4_mfma(const DecodeParams& p, hipStream_t st) {
  if (p.d != D || p.key_fmt != KF_INT4 || p.g > 8) return hipErrorNotSupported;
  // cache bytes are addressed with 32-bit buffer offsets
  if (p.num_blocks * (int64_t)p.block_size * p.hk * (D / 2) >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  // Heads per workgroup: as many kv heads as fit in 8 waves (whole token
  // rows for Hk <= 8), then split them into smaller groups with several
  // waves per head while there are too few workgroups to fill the chip.
  int hg = 1;
  while (hg * 2 <= 8 && p.hk % (hg * 2) == 0) hg *= 2;
  const int64_t units_per_group = (int64_t)p.B * p.splits;
  while (hg > 1 && units_per_group * (p.hk / hg) < 256) hg /= 2;
  const int nh = (p.g + 3) / 4;
  if (nh == 1) return launch<1, 8>(p, hg, st);
  return launch<2, 8>(p, hg, st);
}

}  // namespace tqk
