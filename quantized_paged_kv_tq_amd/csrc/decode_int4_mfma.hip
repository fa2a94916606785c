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
//   * the softmax weights P' = p * scale_v (p <= 2^kTau) are scaled per tile
//     by a power of two to an integer below 2^27 and split into four 7-bit
//     digits.
// The int32 MFMA sums are exact; the digit planes are recombined in fp32
// (one rounding per tile and head), so the result carries fp32-level error
// while moving the 2*g*D multiply-adds per token off the vector ALUs.
// The zero points enter exactly in integers: q'.(n - zp) = q'.n - zp*sum(q')
// per digit plane, and sum_t P'_t (n_t - zp_t) = sum_t P'_t n_t -
// sum_t P'_t zp_t per digit plane.
//
// Work decomposition (balance.h): the 64-token tiles of every split of
// every sequence form one list; workgroup w takes an equal contiguous range
// of it, so the longest sequences no longer set the kernel's duration. A
// workgroup has one wave per kv head of its group (whole token rows for
// Hk <= 8: the 64-byte head slices of a row are requested together), and
// all its waves walk the same tiles. At the start of a range (and every 64
// tiles) the workgroup resolves each tile's tokens to cache rows through
// the block table into LDS. A wave emits one partial per split its range
// touches: a whole split to the split's own slot, a cut one to the
// workgroup's piece slots; stage 2 merges both.
//
// Inside a tile:
//   K side: lane (n, g) loads bytes [16g, 16g+16) of token 16s+n's 64-byte
//   key row (s = 0..3), i.e. four fully used 64-byte segments per token;
//   V side: lane (n, g) loads dword n (8 nibbles) of 16 tokens and a nibble
//   transpose (byte permutes) builds the B operands, so that column n of
//   MFMA i is output dimension 8n+i.
// The registers of a tile are refilled with the next tile's loads as soon as
// they are consumed (keys after the scores, values after the transpose).
#include "balance.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kChunk = 64;  // tiles resolved into LDS at a time

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

// Buffer resource over [base, base + bytes): loads outside return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Narrow addressing (caches below 2 GiB): the tile table holds the byte
// offset of each token's head-0 key row, (page * bs + offset) * Hk * D/2,
// and a masked token holds kMaskedByte, past every buffer the kernel reads:
// the kv head's offset (kvh * D/2 bytes, or 4 * kvh for the scale words,
// whose offset is the row offset / 16) rides in the loads' scalar offset
// and still lands beyond the buffer end, so masked rows read 0 without a
// branch or a select.
constexpr uint32_t kMaskedByte = 0x80000000u;
// Headroom of the value-weight fixed point: weights are taken relative to a
// reference maximum that is raised only when a tile exceeds it by more than
// 2^kTau, so p = 2^(s - m_ref) <= 2^kTau.
constexpr int kTau = 4;

// tile flags in the per-chunk tile table
constexpr int kFirstOfSplit = 1;
constexpr int kLastOfSplit = 2;

// NH: MFMA row sets of four query heads per wave (a wave serves 4 * NH query
// heads of one kv head). DEPTH register sets form a ring: the loads of tile
// k + DEPTH - 1 are issued at the top of tile k. The launcher uses NH = 1 and
// DEPTH = 2 with two waves per SIMD: one wave per SIMD with NH = 2 (all of
// a kv head's query heads) and rings of 3 or 4 measured slower, the second
// wave on a SIMD hiding the first one's MFMA, LDS and DPP latencies.
//
// WIDE: 64-bit addressing for caches of 2 GiB and more (buffer offsets are
// 32-bit). The tile table then holds the head-0 row index (page * bs +
// offset) * Hk, a masked token row 0 (a valid address), and a per-tile mask
// of live tokens decides what a masked token's bytes may do: its score is
// -inf (weight 0, so its value nibbles add 0) and its value scale word is
// taken as 0.
//
// MQ: multi-query entries (prefill): entry b reads block-table row
// p.bt_row[b] from token p.tok_off[b] on, and scores may be softcapped. The
// plain decode instantiation carries none of it.
template <int W, int NH, int DEPTH, bool WIDE, bool MQ>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(DEPTH == 2 ? 2 : 1)))
void decode_int4_mfma_kernel(DecodeParams p) {
  constexpr int NHEAD = 4 * NH;  // query heads per wave (padded)
  constexpr int NT = 64 * W;
  // per wave: MFMA A-operand image of its queries (query set-up), then the
  // per-tile weight digit planes
  __shared__ __attribute__((aligned(16))) uint32_t wbuf[W][NH][2][64][4];
  // each token of the chunk's tiles: the byte offset of its head-0 key row
  // (WIDE: the row index); the DEPTH - 1 rows after the chunk's last tile
  // are all masked (the prefetch past the end)
  __shared__ __attribute__((aligned(16))) uint32_t tok_rows[kChunk + DEPTH - 1][64];
  // WIDE: live tokens of each tile (bit j: token j)
  __shared__ uint64_t tlive[WIDE ? kChunk + DEPTH - 1 : 1];
  __shared__ int4 tinfo[kChunk];  // (b, s, flags, -) per tile of the chunk
  __shared__ int scan[W];
  // fp32 accumulators of the wave's heads, lane-major (touched only when
  // the int32 MFMA sums are folded in, so they need no registers)
  __shared__ float accl[W][NH * 8][64];
  // [B + 1] tiles of the sequences before b, then [B] their clamped lengths
  extern __shared__ int prefix[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;  // n: MFMA column / row within a 16-lane group
  const int lg = lane >> 4;  // g: 16-lane group
  const int grp = blockIdx.x / p.nw;
  const int wg = blockIdx.x - grp * p.nw;
  // wave -> (kv head, sub-group of four of its query heads)
  const int qs_n = (p.g + NHEAD - 1) / NHEAD;  // sub-groups per kv head
  const int kvl = wave / qs_n;      // kv head within the workgroup
  const int qsub = wave - kvl * qs_n;
  const int kvh = grp * p.wgh + kvl;
  const int g = p.g;
  const int hq0 = NHEAD * qsub;                      // first query head of this wave within its kv head
  const int gw = g - hq0 < NHEAD ? g - hq0 : NHEAD;  // query heads of this wave
  const int h0 = kvh * g + hq0;

  // ---- sequence lengths and the prefix sums of their tile counts ----
  const int N = balance_prologue<NT>(p, prefix, prefix + p.B + 1, scan);
  if (N == 0) return;  // uniform: every sequence is empty
  const int lo = range_lo(wg, N, p.nw), hi = range_lo(wg + 1, N, p.nw);
  if (lo >= hi) return;  // uniform: an empty range

  const uint32_t bs = (uint32_t)p.block_size;
  const bool bs_pow2 = (bs & (bs - 1u)) == 0u;
  const bool capped = MQ && p.softcap > 0.0f;
  const float cap_in = kLn2 / (capped ? p.softcap : 1.0f);  // base-2 score -> y = s / c
  const float cap_out = p.softcap * kLog2e;                 // tanh -> base-2 score
  const int bs_shift = __builtin_ctz(bs);
  const uint32_t nrows = (uint32_t)(p.num_blocks * bs * p.hk);
  const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(p.kc, WIDE ? 0u : nrows * (uint32_t)(D / 2));
  const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(p.vc, WIDE ? 0u : nrows * (uint32_t)(D / 2));
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(p.ks, WIDE ? 0u : nrows * 4u);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(p.vs, WIDE ? 0u : nrows * 4u);
  // the kv head's byte offsets (wave-uniform)
  const int kvo = __builtin_amdgcn_readfirstlane(kvh * (D / 2));
  const int kvs = __builtin_amdgcn_readfirstlane(kvh * 4);
  // WIDE: per-lane 64-bit bases (kv head and lane parts folded in)
  const uint8_t* kbase = p.kc + (int64_t)kvh * (D / 2) + 16 * lg;
  const uint8_t* vbase = p.vc + (int64_t)kvh * (D / 2) + 4 * ln;
  const float* ksbase = p.ks + kvh;
  const float* vsbase = p.vs + kvh;

  // ---- registers of one tile ----
  // key bytes and both scale words of tokens 16s+n; value dword n of tokens
  // 16s+4g+k (masked rows read 0)
  struct Buf {
    v4u kraw[4];
    uint32_t ksw, vsw;  // scale words of token `lane`
    uint32_t live;
    uint32_t vraw[4][4];
  };
  auto issue = [&](Buf& B, int k) {  // k < K + DEPTH - 1: rows from K on are masked
    B.live = 0;
    if constexpr (!WIDE) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t o = tok_rows[k][16 * s + ln];
        B.live |= (o < kMaskedByte ? 1u : 0u) << s;
        B.kraw[s] = __builtin_amdgcn_raw_buffer_load_b128(rk_, (int)(o | (16u * lg)), kvo, 0);
      }
      {
        const uint32_t o = tok_rows[k][lane] >> 4;  // row * 4
        B.ksw = __builtin_amdgcn_raw_buffer_load_b32(rks, (int)o, kvs, 0);
        B.vsw = __builtin_amdgcn_raw_buffer_load_b32(rvs, (int)o, kvs, 0);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t o = tok_rows[k][16 * s + 4 * lg + kk];
          B.vraw[s][kk] = __builtin_amdgcn_raw_buffer_load_b32(rv_, (int)(o | (4u * ln)), kvo, 0);
        }
      }
    } else {
      const uint64_t lv = tlive[k];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint64_t r = tok_rows[k][16 * s + ln];
        B.live |= (uint32_t)((lv >> (16 * s + ln)) & 1u) << s;
        B.kraw[s] = *reinterpret_cast<const v4u*>(kbase + r * (D / 2));
      }
      {
        const uint64_t r = tok_rows[k][lane];
        B.ksw = __float_as_uint(ksbase[r]);
        // a masked token's value scale word counts as 0 (its row is row 0)
        B.vsw = ((lv >> lane) & 1u) ? __float_as_uint(vsbase[r]) : 0u;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint64_t r = tok_rows[k][16 * s + 4 * lg + kk];
          B.vraw[s][kk] = *reinterpret_cast<const uint32_t*>(vbase + r * (D / 2));
        }
      }
    }
  };

  // Online softmax state of the current segment (a split, or the part of
  // it inside this range), all relative to a reference maximum m_ref (base-2
  // units) per head and a power-of-two weight scale 2^ev shared by the wave:
  //   l     per-lane sum of 2^(s - m_ref) over the lane's tokens
  //   cacc  int32 MFMA sums of the weight digit planes times the value
  //         nibbles (lane (n, g): head 4r+g, dims 8n+i, planes 0..3)
  //   zl    per-lane sums of weight digits times value zero points
  //   acc   fp32 part folded at each flush (accl, in LDS)
  float mref[NH], l[NH];
  float(*acc)[64] = accl[wave];  // acc[8r + i][lane]
  v4i cacc[NH][8];
  int zl[NH][4];
  int ev = 0;           // weight scale exponent
  float sref = 0.0f;    // value scales below sref fit the current ev
  bool empty = true;    // cacc / zl hold nothing
  int since_flush = 0;  // tiles accumulated since the last flush
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      mref[r] = -INFINITY;
      l[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[8 * r + i][lane] = 0.0f;
        cacc[r][i] = v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) zl[r][k] = 0;
    }
    ev = 0;
    sref = 0.0f;
    empty = true;
    since_flush = 0;
  };
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
          acc[8 * r + i][lane] = __builtin_fmaf(val, pinv, acc[8 * r + i][lane]) * alpha[r];
          cacc[r][i] = v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) zl[r][k] = 0;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[8 * r + i][lane] *= alpha[r];
      }
      l[r] *= alpha[r];
    }
    empty = true;
  };

  // ---------------- query of sequence b ----------------
  // Rotate each head (two dims per lane), scale by a power of two to
  // integers below 2^27, split into four balanced base-128 digits and
  // scatter them into the MFMA A-operand image: lane (m = 4h' + piece, g)
  // holds, for chunk c, dword j, byte b, the digit of dim
  // 32g + 16c + 8(j/2) + 2b + (j%2) -- the order of the K unpack.
  v4i qa[NH][2];
  float qsum[NH][4], qf[NH];
  // the wave's query rows of sequence b times the RHT signs (lane: dims
  // lane and lane + 64)
  auto query_rows = [&](int b, float (&qx)[NHEAD][2]) {
#pragma unroll
    for (int hh = 0; hh < NHEAD; ++hh) {
      const bool ok = hh < gw;
      const float* qrow = p.q + ((int64_t)b * p.hq + h0 + (ok ? hh : 0)) * D;
      qx[hh][0] = ok ? qrow[lane] * p.rht_signs[lane] : 0.0f;
      qx[hh][1] = ok ? qrow[lane + 64] * p.rht_signs[lane + 64] : 0.0f;
    }
  };
  // rotate, scale and split the rows into the MFMA A-operand image
  auto query_image = [&](const float (&qx)[NHEAD][2]) {
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
    wave_sync();
#pragma unroll
    for (int r = 0; r < NH; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(&wbuf[wave][r][c][lane][0]);
        qa[r][c] = v4i{(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w};
      }
    wave_sync();  // the image region is reused for the weight digit planes
  };
  auto load_query = [&](int b) {
    float qx[NHEAD][2];
    query_rows(b, qx);
    query_image(qx);
  };
  uint32_t(*p8)[4][4][16] = reinterpret_cast<uint32_t(*)[4][4][16]>(&wbuf[wave][0][0][0][0]);

  // ---------------- segment bookkeeping ----------------
  int seg_b = -1, seg_s = 0;
  bool seg_from_start = false;  // the segment began at its split's first tile
  bool seg_to_end = false;      // ... and has reached the split's last tile
  bool seg_first = false;       // the segment is the range's first
  // write the segment's partial: a whole split to its own slot, a cut one
  // to piece slot 0 (the range's first split) or 1 (its last split)
  auto emit = [&]() {
    {
      float one[NH];
#pragma unroll
      for (int r = 0; r < NH; ++r) one[r] = 1.0f;
      flush(one);
    }
    const bool whole = seg_from_start && seg_to_end;
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      const float lt = row16_sum(l[r]);
      const int hh = 4 * r + lg;
      if (hh < gw) {
        float* out;
        if (whole)
          out = p.ws + (((int64_t)seg_b * p.hq + h0 + hh) * p.splits + seg_s) * (D + 1);
        else
          out = p.wsp + ((((int64_t)grp * p.nw + wg) * 2 + (seg_first ? 0 : 1)) * (p.wgh * g) +
                         kvl * g + hq0 + hh) * (D + 1);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        float* dst = out + 8 * ln;
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = acc[8 * r + i][lane] * inv;
        if (ln == 0) out[D] = lt > 0.0f ? (mref[r] + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  };

  // One tile: the next tile's loads go into the other register set first,
  // so they are in flight for the whole of this tile's work.
  auto process = [&](Buf& X, Buf& Y, int k, int c0) {
    const int gk = c0 + k;
    const int4 info = tinfo[k];
    if (gk == lo || (info.z & kFirstOfSplit)) {
      // a new segment begins with this tile
      // (the range's first query is set up before its first tile)
      if (gk != lo) emit();
      if (gk != lo && info.x != seg_b) load_query(info.x);
      reset();
      seg_b = info.x;
      seg_s = info.y;
      seg_from_start = (info.z & kFirstOfSplit) != 0;
      seg_first = gk == lo;
    }
    seg_to_end = (info.z & kLastOfSplit) != 0;
    issue(Y, k + DEPTH - 1);
    // Hold the workgroup's waves on one tile: the two waves of a SIMD
    // otherwise drift apart (the younger one falls behind) and a long range
    // ends with the younger waves alone. Every wave of the workgroup walks
    // the same tiles, so each reaches the barrier equally often. (The
    // multi-query entries are bound by ALU work, where the drift costs
    // nothing and the barrier does.)
    if constexpr (!MQ) __builtin_amdgcn_s_barrier();

    // scale words of tokens 16s+n from lane 16s+n
    uint32_t ksw[4], vsw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ksw[s] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * s + ln) << 2, (int)X.ksw);
      vsw[s] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * s + ln) << 2, (int)X.vsw);
    }
    // ---- scores on the matrix cores ----
    float sc[NH][4], smask[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4u w4 = X.kraw[s];
      int evn[4], odd[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        evn[kk] = (int)(w4[kk] & 0x0F0F0F0Fu);
        odd[kk] = (int)((w4[kk] >> 4) & 0x0F0F0F0Fu);
      }
      const v4i kb0 = v4i{evn[0], odd[0], evn[1], odd[1]};
      const v4i kb1 = v4i{evn[2], odd[2], evn[3], odd[3]};
      const float zpk = (float)(ksw[s] & 0xFu);
      const float ksc = u2f(ksw[s] & 0xFFFFFFF0u);
      // masked tokens: min(score, -inf) keeps the arithmetic unconditional
      const float mask = ((X.live >> s) & 1u) ? INFINITY : -INFINITY;
#pragma unroll
      for (int r = 0; r < NH; ++r) {
        v4i c = v4i{0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][0], kb0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][1], kb1, c, 0, 0, 0);
        // lane (n, g): rows 4g..4g+3 = digits 0..3 of head 4r+g, token
        // 16s+n; each plane minus zp * (digit sum) is an exact integer
        const float d0 = __builtin_fmaf(-zpk, qsum[r][0], (float)c.x);
        const float d1 = __builtin_fmaf(-zpk, qsum[r][1], (float)c.y);
        const float d2 = __builtin_fmaf(-zpk, qsum[r][2], (float)c.z);
        const float d3 = __builtin_fmaf(-zpk, qsum[r][3], (float)c.w);
        const float dot = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(d3, 128.0f, d2), 128.0f, d1), 128.0f, d0);
        sc[r][s] = dot * (qf[r] * ksc);
      }
      smask[s] = mask;
    }
    // softcap on natural-unit scores (sc is in base-2 units):
    // c tanh(x ln2 / c) log2e, tanh(y) = sign(y) (1 - 2 / (e^{2|y|} + 1))
    if (MQ && capped) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < NH; ++r) {
          const float y = sc[r][s] * cap_in;
          const float e = __builtin_amdgcn_exp2f(fabsf(y) * 2.8853900817779268f);  // e^{2|y|}
          const float t = 1.0f - 2.0f / (e + 1.0f);
          sc[r][s] = __builtin_copysignf(t, y) * cap_out;
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < NH; ++r) sc[r][s] = fminf(sc[r][s], smask[s]);
    float vsc[4];
    uint32_t zp4 = 0;
    float smax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      vsc[s] = u2f(vsw[s] & 0xFFFFFFF0u);
      zp4 |= (vsw[s] & 0xFu) << (8 * s);
      smax = fmaxf(smax, vsc[s]);  // masked tokens load scale 0
    }

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
        for (int kk = 0; kk < 4; ++kk) dw[kk] |= ((pi >> (7 * kk)) & 127u) << (8 * s);
      }
      l[r] += ps;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        p8[r][lg][kk][ln] = dw[kk];
        zl[r][kk] += (int)__builtin_amdgcn_udot4(dw[kk], zp4, 0u, false);
      }
    }
    empty = false;
    wave_sync();

    // ---- value MFMAs: B operands by nibble transpose, in two halves ----
    v4i pa[NH];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      // A operand: lane (m = 4h' + piece, g) reads the digit plane of head
      // 4r+h' for tokens 16s + 4g + kk at byte (kk, s)
      const uint4 a4 = *reinterpret_cast<const uint4*>(&p8[r][ln >> 2][ln & 3][4 * lg]);
      pa[r] = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // vb[i][kk]: byte s = nibble 4h+i (dim 8n + 4h + i) of token 16s+4g+kk
      uint32_t vb[4][4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t w0 = X.vraw[0][kk], w1 = X.vraw[1][kk], w2 = X.vraw[2][kk], w3 = X.vraw[3][kk];
        // bytes 2h and 2h+1 of the four dwords, then the 4x4 byte transpose
        const uint32_t sel = h ? 0x07030602u : 0x05010400u;
        const uint32_t x01 = __builtin_amdgcn_perm(w1, w0, sel);
        const uint32_t x23 = __builtin_amdgcn_perm(w3, w2, sel);
        const uint32_t ta = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
        const uint32_t tb = __builtin_amdgcn_perm(x23, x01, 0x07060302u);
        vb[0][kk] = ta & 0x0F0F0F0Fu;
        vb[1][kk] = (ta >> 4) & 0x0F0F0F0Fu;
        vb[2][kk] = tb & 0x0F0F0F0Fu;
        vb[3][kk] = (tb >> 4) & 0x0F0F0F0Fu;
      }
#pragma unroll
      for (int r = 0; r < NH; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4i vbi = v4i{(int)vb[i][0], (int)vb[i][1], (int)vb[i][2], (int)vb[i][3]};
          cacc[r][4 * h + i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[r], vbi, cacc[r][4 * h + i], 0, 0, 0);
        }
    }
    wave_sync();  // the digit planes are rewritten by the next tile
  };

  // The range's first query rows are requested now: their loads overlap
  // the tile table's, so the first tiles can be issued back to back once
  // the table is built (tile 0 would otherwise wait for the query).
  float q0[NHEAD][2];
  {
    int bl = 0, bh = p.B - 1;  // the sequence of tile lo, as the table finds it
    while (bl < bh) {
      const int m = (bl + bh + 1) >> 1;
      if (prefix[m] <= lo) bl = m;
      else bh = m - 1;
    }
    query_rows(bl, q0);
  }

  Buf ring[DEPTH];
  for (int c0 = lo; c0 < hi; c0 += kChunk) {
    const int K = hi - c0 < kChunk ? hi - c0 : kChunk;  // tiles of this chunk
    __syncthreads();  // the previous chunk's table is no longer read
    // ---- resolve the chunk's tiles to cache rows ----
    for (int e = tid; e < (K + DEPTH - 1) * 64; e += NT) {
      const int k = e >> 6, j = e & 63;  // k is the same across a wave
      if (k >= K) {
        tok_rows[k][j] = WIDE ? 0u : kMaskedByte;
        if (WIDE && j == 0) tlive[k] = 0;
        continue;
      }
      const int x = c0 + k;
      // sequence b: the largest with prefix[b] <= x (then x < prefix[b+1])
      int bl = 0, bh = p.B - 1;
      while (bl < bh) {
        const int m = (bl + bh + 1) >> 1;
        if (prefix[m] <= x) bl = m;
        else bh = m - 1;
      }
      const int b = bl;
      const SeqSplits q = splits_of(p, prefix[p.B + 1 + b]);
      const int r = x - prefix[b];
      int s = r / q.TL;
      if (s > q.n - 1) s = q.n - 1;
      const int t = r - s * q.TL;
      const int tok0 = s * q.L + t * kTileTokens;
      int end = s * q.L + q.L;
      if (end > q.seq) end = q.seq;
      if (end > tok0 + kTileTokens) end = tok0 + kTileTokens;
      const int tok = tok0 + j;
      uint32_t row = WIDE ? 0u : kMaskedByte;
      bool live = false;
      if (tok < end) {
        // multi-query entries read their sequence's row from an offset
        const uint32_t t32 = (uint32_t)tok + (MQ ? (uint32_t)p.tok_off[b] : 0u);
        const int64_t brow = MQ ? (int64_t)p.bt_row[b] : (int64_t)b;
        const uint32_t pi = bs_pow2 ? (t32 >> bs_shift) : (t32 / bs);
        const int64_t page = p.block_table[brow * p.max_blocks + pi];
        if (page >= 0 && page < p.num_blocks) {
          const uint32_t r = ((uint32_t)page * bs + (t32 - pi * bs)) * (uint32_t)p.hk;
          row = WIDE ? r : r * (uint32_t)(D / 2);
          live = true;
        }
      }
      tok_rows[k][j] = row;
      if constexpr (WIDE) {
        const uint64_t m = __ballot(live);  // k is the same across the wave
        if (j == 0) tlive[k] = m;
      }
      if (j == 0) {
        const int nt = (s == q.n - 1) ? q.TLast : q.TL;
        tinfo[k] = make_int4(b, s, (t == 0 ? kFirstOfSplit : 0) | (t == nt - 1 ? kLastOfSplit : 0), 0);
      }
    }
    __syncthreads();

    if (c0 == lo) query_image(q0);
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u) issue(ring[u], u);
    for (int k = 0; k < K; k += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        if (k + u >= K) break;
        process(ring[u], ring[(u + DEPTH - 1) % DEPTH], k + u, c0);
      }
    }
  }
  emit();
}

template <int W, int NH, int DEPTH>
hipError_t launch(const DecodeParams& p, hipStream_t st, bool wide) {
  const uint32_t blocks = (uint32_t)(p.hk / p.wgh) * (uint32_t)p.nw;
  const size_t lds = balance_lds_bytes(p.B);
  const bool mq = p.bt_row != nullptr;
#define TQ_I4(WD, M) \
  hipLaunchKernelGGL((decode_int4_mfma_kernel<W, NH, DEPTH, WD, M>), dim3(blocks), dim3(64 * W), lds, st, p)
  if (mq) {
    if (wide) TQ_I4(true, true); else TQ_I4(false, true);
  } else {
    if (wide) TQ_I4(true, false); else TQ_I4(false, false);
  }
#undef TQ_I4
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_int4_mfma(DecodeParams& p, hipStream_t st) {
  // up to 32 query heads per kv head: ceil(g / 4) waves of four heads each,
  // at most 8 waves per workgroup
  if (p.d != D || p.key_fmt != KF_INT4 || p.g > 32) return hipErrorNotSupported;
  // multi-query entries come with both maps; a softcap only with them
  if ((p.bt_row == nullptr) != (p.tok_off == nullptr) || (p.softcap > 0.0f && !p.bt_row))
    return hipErrorInvalidValue;
  // cache bytes below 2 GiB take 32-bit buffer offsets; larger caches the
  // 64-bit addressing variant, whose tile table holds 32-bit row indices
  const int64_t rows = p.num_blocks * (int64_t)p.block_size * p.hk;
  if (rows >= ((int64_t)1 << 32)) return hipErrorNotSupported;
  const bool wide = p.force_wide || rows * (D / 2) >= ((int64_t)1 << 31);
  // token and tile indices are 32-bit; the per-sequence tile prefix sums
  // live in LDS
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  if (cap >= ((int64_t)1 << 30) || p.B > 4096) return hipErrorNotSupported;
  const int64_t tiles_ub = (int64_t)p.B * ((cap + kTileTokens - 1) / kTileTokens + p.splits);
  if (tiles_ub >= ((int64_t)1 << 30)) return hipErrorNotSupported;
  // waves: HG kv heads x QS sub-groups of four query heads, at most 8
  const int qs = (p.g + 3) / 4;
  p.wgh = balance_heads_per_wg(p.hk, p.g);
  const int64_t nw = balance_max_wgs(p.hk, p.g);
  p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
  switch (p.wgh * qs) {
    case 1: return launch<1, 1, 2>(p, st, wide);
    case 2: return launch<2, 1, 2>(p, st, wide);
    case 3: return launch<3, 1, 2>(p, st, wide);
    case 4: return launch<4, 1, 2>(p, st, wide);
    case 5: return launch<5, 1, 2>(p, st, wide);
    case 6: return launch<6, 1, 2>(p, st, wide);
    case 7: return launch<7, 1, 2>(p, st, wide);
    case 8: return launch<8, 1, 2>(p, st, wide);
    default: return hipErrorNotSupported;
  }
}

}  // namespace tqk
