// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores, for
// 3- or 4-bit Lloyd-Max centroid keys with 3- or 4-bit uniform values
// (triton_turboquant_decode.py, _tq_decode_stage1: score = sm_scale *
// norm16 * (q_rot . c[idx]); v = idx * scale16 + zero16; online softmax;
// partials acc / l and m + ln l).
//
// Scores. A key's KB-bit index idx = b0 + 2 b1 + 4 b2 (+ 8 b3) picks c[idx];
// as a function of its bits, c is the multilinear polynomial
//   c(b) = sum over S of alpha_S * prod_{i in S} b_i   (S a subset of bits),
// alpha the Moebius transform of the table. So
//   q_rot . c[idx] = alpha_0 * sum(q_rot) + sum_{S != 0} alpha_S * (q_rot . P_S)
// with P_S the 0/1 vector of the product of the bits in S. The 2^KB - 1 dot
// products with 0/1 vectors run as v_mfma_i32_16x16x64_i8 on exact
// integers: the rotated query is scaled by 2^E to integers below 2^27 and
// split into four balanced base-128 digits (the A operand, as in the INT4
// path), the bit planes are the int8 B operand. The int32 sums are exact;
// they are combined with alpha in fp32.
//
// Values. As in the INT4 path: P' = p * scale16 is split into four 7-bit
// digit planes (A operand), the 3-bit indices unpacked to bytes are the B
// operand; the zero term sum_t p_t * zero16_t is a per-head fp32 sum added
// to every dimension at the end.
//
// Work decomposition, tile table, pieces and ping-pong register sets follow
// the INT4 path (balance.h): equal ranges of the global 64-token tile list,
// one wave per four query heads of a kv head for g <= 4. For g = 5 .. 8 one
// wave serves all query heads of its kv head (two MFMA row sets), so the
// unpacking of each tile's 3-bit keys and values, which bounds this kernel,
// is done once per kv head instead of by two waves; that wave needs more
// than 256 registers and runs alone on its SIMD. D = 256 doubles a lane's
// key and value dims (64 key and 16 value dims per lane, 4 score MFMAs per
// plane, 16 PV MFMAs); its waves serve four query heads each and run alone
// on their SIMD.
//
// A table with c[2^KB - 1 - j] = -c[j] (Lloyd-Max tables are) has only odd
// Walsh terms: 4 bit planes for KB = 3 (b0, b1, b2, b0^b1^b2), 8 for KB = 4
// (the four bits and the four parities of three of them).
//
// Slot layout: bytes [0, D KB / 8) key indices (LSB-first KB-bit stream),
// then the fp16 norm, D VB / 8 bytes of value indices (LSB-first),
// the fp16 scale and the fp16 zero. A lane's 4-bit keys stay packed: its
// bit planes are read from the nibbles of each byte, even dimensions from
// the low nibbles and odd ones from the high nibbles, and the query image
// takes the same dimension order.
#pragma once

#include <type_traits>

#include "balance.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits (round to nearest even; finite values)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kChunk = 64;  // tiles resolved into LDS at a time
constexpr int kTau = 4;     // headroom of the value-weight fixed point
// Byte offset of a masked token's slot: at or past 2^31, beyond every
// buffer (cache sizes stay below 2^31 bytes), so its loads read zeros even
// after a kv head's offset and a field offset are added.
constexpr uint32_t kMaskedByte = 0x80000000u;
// Caches of 2 GiB and more take the 64-bit addressing variant (WIDE): the
// tile table holds 64-bit byte offsets from the wave's kv-head base, and a
// masked token the offset of a static page of zeros (never written), so a
// masked token reads zeros there as the narrow variant reads zeros past the
// buffer end. The zero page covers every kv head's slot (Hk * slot bytes up
// to kZeroBytes).
constexpr int kZeroBytes = 65536;
__device__ __attribute__((aligned(256))) uint8_t g_zero_page[kZeroBytes];
constexpr int kFirstOfSplit = 1;
constexpr int kLastOfSplit = 2;
// slot offsets for KB-bit keys and VB-bit values: norm, value indices,
// and the 8-byte word pair at kScaleOff whose bytes 2..3 are the scale and
// 4..5 the zero
template <int KB, int VB, int DD>
struct SlotLayout {
  static constexpr uint32_t kNormOff = DD * KB / 8;
  static constexpr uint32_t kValOff = DD * KB / 8 + 2;
  static constexpr uint32_t kScaleOff = DD * (KB + VB) / 8;
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)));
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
__device__ __forceinline__ float exp2i(int e) { return u2f((uint32_t)(e + 127) << 23); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// four 3-bit fields (bits 0..11 of x) -> four bytes
__device__ __forceinline__ uint32_t unpack3x4(uint32_t x) {
  const uint32_t y = ((x & 0xFC0u) << 10) | (x & 0x3Fu);  // fields 2, 3 to bits 16..21
  return (y | (y << 5)) & 0x07070707u;                      // fields 1, 3 to bytes 1, 3
}
// nibbles 4h .. 4h+3 of x -> four bytes
__device__ __forceinline__ uint32_t unpack4x4(uint32_t x, int h) {
  const uint32_t t = __builtin_amdgcn_perm(x, x, h ? 0x03030202u : 0x01010000u);
  return ((t >> 4) & 0x0F000F00u) | (t & 0x000F000Fu);
}
// the subset of index bits of odd Walsh plane i: the single bits, then
// b0^b1^b2 (and, with 4 bits, b0^b1^b3, b0^b2^b3, b1^b2^b3)
__host__ __device__ constexpr int odd_plane(int i) {
  return i == 0 ? 1 : i == 1 ? 2 : i == 2 ? 4 : i == 3 ? 7 : i == 4 ? 8 : i == 5 ? 11 : i == 6 ? 13 : 14;
}
// bits [bit, bit + 12) of the little-endian value w
template <int N>
__device__ __forceinline__ uint32_t bits12(const uint32_t (&w)[N], int bit) {
  const int word = bit >> 5, sh = bit & 31;
  if (sh <= 20) return w[word] >> sh;
  return __builtin_amdgcn_alignbit(w[word + 1], w[word], (uint32_t)sh);
}

// NH: MFMA row sets of four query heads per wave; the bit planes and value
// operands of a tile are unpacked once and serve all 4 * NH heads. NH = 2
// (g = 5 .. 8, one wave per kv head) needs more than 256 registers, so it
// runs one wave per SIMD.
//
// HALF (g = 5 .. 8): two waves per kv head, each with both row sets and half
// of the head dims (wave hf: key and value dims D/2 hf .. D/2 hf + D/2 - 1),
// so each unpacks half of every tile; they add their partial scores through
// LDS once per tile (one workgroup barrier), then run the same softmax. At
// D = 128 a wave fits 256 registers, so two workgroups share a CU and their
// waves hide each other's latency; at D = 256 a wave has the shape of the
// D = 128 one-wave kernel (128 dims, two row sets) and runs alone on its
// SIMD.
template <int W, int NH, bool WIDE, int KB, int VB, int DD, bool NCORR, bool HALF = false>
__global__ __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(DD == 128 && (NH == 1 || HALF) ? 2 : 1)))
void decode_tqb_kernel(DecodeParams p) {
  constexpr int D = DD;      // head dim, 128 or 256
  constexpr int F = D / 128;  // a lane's dims per 16-lane group and token: 32 F keys, 8 F values
  static_assert(!HALF || (NH == 2 && !NCORR && VB != 8), "half-dim waves: g > 4, uniform values");
  constexpr int KC = HALF ? F : 2 * F;       // 64-dim MFMA chunks of a wave's key dims
  constexpr int VDL = HALF ? 4 * F : 8 * F;  // value dims per lane
  constexpr int FH = VDL / 4;            // groups of four value dims per lane
  using L = SlotLayout<KB, VB, DD>;
  constexpr uint32_t kNormOff = L::kNormOff, kValOff = L::kValOff, kScaleOff = L::kScaleOff;
  constexpr int NC = 1 << KB;  // centroids
  constexpr int NT = 64 * W;
  constexpr int NHEAD = 4 * NH;  // query heads per wave (padded)
  constexpr bool V8 = VB == 8;  // FP8 E4M3 values (D codes, no scale or zero)
  __shared__ __attribute__((aligned(16))) uint32_t p8[V8 ? 1 : W][NH][4][4][16];  // weight digit planes
  // V8: bf16 parts of the weights, [part][head][token] per row set
  __shared__ __attribute__((aligned(16))) uint16_t pbf[V8 ? W : 1][NH][3][4][64];
  __shared__ __attribute__((aligned(16))) uint32_t qimg[W][NH][KC][64][4];  // query digit image
  // byte offset of kv head 0's slot of each token of the chunk's tiles
  // (kMaskedByte for masked tokens and the prefetch row past the end)
  using Off = typename std::conditional<WIDE, int64_t, uint32_t>::type;
  __shared__ __attribute__((aligned(16))) Off tok_rows[kChunk + 1][64];
  __shared__ int4 tinfo[kChunk];
  __shared__ int scan[W];
  __shared__ float accl[W][NH * VDL][64];  // fp32 value accumulators, lane-major
  // HALF: partial scores [tile parity][wave][lane][4 r + s]
  __shared__ __attribute__((aligned(16))) float xs[HALF ? 2 : 1][HALF ? W : 1][64][HALF ? 4 * NH : 1];
  extern __shared__ int prefix[];  // [B + 1] tile prefix sums, then [B] lengths

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int grp = blockIdx.x / p.nw;
  const int wg = blockIdx.x - grp * p.nw;
  const int qs_n = (p.g + NHEAD - 1) / NHEAD;
  const int hf = HALF ? (wave & 1) : 0;  // HALF: the wave's half of the head dims
  const int wv = HALF ? (wave >> 1) : wave;
  const int kvl = wv / qs_n;
  const int qsub = wv - kvl * qs_n;
  const int kvh = grp * p.wgh + kvl;
  const int g = p.g;
  const int hq0 = NHEAD * qsub;
  const int gw = g - hq0 < NHEAD ? g - hq0 : NHEAD;
  const int h0 = kvh * g + hq0;

  // Coefficients of the centroid table (uniform), for the index bits
  // b = (b0, .., b_{KB-1}) as the subset mask S in 0..NC-1:
  //   al: multilinear (Moebius) form c(b) = sum_S al_S prod_{i in S} b_i;
  //   ga: Walsh form c(b) = sum_S ga_S (-1)^{popcount(b & S)}.
  // A table with c[NC - 1 - j] = -c[j] (Lloyd-Max tables are) has ga_S = 0
  // for every even |S|; then only the planes of odd |S| are needed:
  //   q . c[idx] = sum_S ga_S (sum q - 2 q . [popcount(b & S) odd]).
  // e2: Walsh form of the squared table, c(b)^2 = sum_S e2_S (-1)^{popcount(b & S)},
  // for the norm-corrected read (1 / sqrt(sum over dims of c[idx]^2 + 1e-16));
  // an antisymmetric table has a symmetric square: e2_S = 0 for odd |S|.
  // e2 (only the norm-corrected read uses it) lives in LDS, thread S
  // computing entry S.
  __shared__ float e2_s[NCORR ? NC : 1];
  float al[NC], ga[NC];
  bool anti = true;
  {
    float c[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) c[j] = p.centroids[j];
#pragma unroll
    for (int j = 0; j < NC; ++j) anti = anti && (c[NC - 1 - j] == -c[j]);
#pragma unroll
    for (int S = 0; S < NC; ++S) {
      float a = 0.0f, w = 0.0f;
#pragma unroll
      for (int T = 0; T < NC; ++T) {
        w = (__builtin_popcount(T & S) & 1) ? w - c[T] : w + c[T];
        if ((T & S) != T) continue;
        const int sign = __builtin_popcount(S ^ T) & 1;
        a = sign ? a - c[T] : a + c[T];
      }
      al[S] = a;
      ga[S] = w * (1.0f / NC);
    }
    if constexpr (NCORR) {
      const int S = threadIdx.x;
      if (S < NC) {
        float w2 = 0.0f;
#pragma unroll
        for (int T = 0; T < NC; ++T) w2 = (__builtin_popcount(T & S) & 1) ? w2 - c[T] * c[T] : w2 + c[T] * c[T];
        e2_s[S] = w2 * (1.0f / NC);
      }
      // (the prologue's barriers order these stores before any read)
    }
  }
  // Folded antisymmetric scores (kFold): each odd Walsh plane S_i gets its
  // own query image, the query scaled by gq_i = ga_{S_i} / max |ga|, so one
  // accumulator sums all planes' products and a token block takes one
  // digit recombination per row set instead of one per plane:
  //   sum_i ga_{S_i} (q . P_{S_i}) = gmax * sum_i q_i . P_{S_i},  q_i = gq_i q
  // (q_i rounded to integers at the query's 2^E scale, an error of 2^-27 of
  // the largest query element per dim and plane).
  constexpr bool kFold = KB == 3 && NH == 2 && DD == 128 && !NCORR;
  constexpr int NPF = KB == 3 ? 4 : 8;  // odd Walsh planes
  float gsum = 0.0f, gmax = 0.0f, gq[kFold ? NPF : 1];
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    gsum += ga[odd_plane(i)];
    gmax = fmaxf(gmax, fabsf(ga[odd_plane(i)]));
  }
#pragma unroll
  for (int i = 0; i < (kFold ? NPF : 1); ++i) gq[i] = gmax > 0.0f ? ga[odd_plane(i)] / gmax : 0.0f;

  // ---- sequence lengths and the prefix sums of their tile counts ----
  const int N = balance_prologue<NT>(p, prefix, prefix + p.B + 1, scan);
  if (N == 0) return;
  const int lo = range_lo(wg, N, p.nw), hi = range_lo(wg + 1, N, p.nw);
  if (lo >= hi) return;

  const uint32_t bs = (uint32_t)p.block_size;
  const bool bs_pow2 = (bs & (bs - 1u)) == 0u;
  const int bs_shift = __builtin_ctz(bs);
  const uint32_t sb = (uint32_t)p.slot_bytes;
  const uint32_t nrows = (uint32_t)(p.num_blocks * bs * p.hk);
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc(p.kv, WIDE ? 0u : nrows * sb);
  // WIDE: the wave's kv-head base and the offset of the zero page from it
  const uint8_t* kvb = p.kv + (int64_t)kvh * sb;
  const int64_t zoff = (int64_t)(g_zero_page - p.kv);
  auto ld32 = [&](Off o) -> uint32_t {
    if constexpr (WIDE) return *reinterpret_cast<const uint32_t*>(kvb + o);
    else return __builtin_amdgcn_raw_buffer_load_b32(rkv, (int)o, 0, 0);
  };
  auto ld64 = [&](Off o) -> v2u {
    if constexpr (WIDE) return *reinterpret_cast<const v2u*>(kvb + o);
    else return __builtin_amdgcn_raw_buffer_load_b64(rkv, (int)o, 0, 0);
  };
  auto ld128 = [&](Off o) -> v4u {
    if constexpr (WIDE) return *reinterpret_cast<const v4u*>(kvb + o);
    else return __builtin_amdgcn_raw_buffer_load_b128(rkv, (int)o, 0, 0);
  };
  // a token's slot is masked (it reads zeros)
  auto masked = [&](Off o) -> bool {
    if constexpr (WIDE) return o == (Off)zoff;
    else return o >= kMaskedByte;
  };
  // this lane's value bytes (dims 8F n .. 8F n + 8F - 1) start at byte
  // kValOff + VB F n; one dword load per 8 dims from byte kValOff + VB F n +
  // VB f (buffer loads take byte offsets, dword loads need not be 4-byte
  // aligned)
  // (HALF: dims 64F hf + 4F n .. +4F-1; at D = 128, 3-bit ones start at
  // bit 4 of the dword when n is odd)
  const uint32_t vbyte = HALF ? kValOff + (VB == 3 ? 24u * F * hf + ((3u * F * ln) >> 1) : 32u * F * hf + 2u * F * ln)
                              : kValOff + (uint32_t)(VB * F) * (uint32_t)ln;
  const uint32_t vsh = (HALF && F == 1 && VB == 3 && (ln & 1)) ? 4u : 0u;

  // ---- registers of one tile ----
  // key bytes [4 KB F g, 4 KB F (g + 1)) of tokens 16s + n (dims 32F g ..
  // 32F g + 32F - 1); the norm word and scale/zero words of token `lane`;
  // the dwords starting at value bytes VB F n + VB f of tokens 16s + 4g + k
  struct Buf {
    uint32_t kraw[4][HALF ? (KB * 16 * F + 31) / 32 : KB * F];
    uint32_t nw, sz0, sz1, live;
    uint32_t vraw[V8 ? 1 : 4][4][HALF ? 1 : F];
    uint32_t v8[V8 ? 2 : 1][8][2];  // V8: value bytes 8n .. 8n+7 of tokens 32h + 8g + j
  };
  const uint32_t kvh_off = (uint32_t)kvh * sb;
  auto slot_of = [&](int k, int j) -> Off { return WIDE ? tok_rows[k][j] : tok_rows[k][j] + kvh_off; };
  // keys and per-token words first; the value windows after the current
  // tile's scores (issue_v), which keeps both tiles' values from being live
  // through the score computation
  auto issue_v = [&](Buf& B, int k) {
    if constexpr (V8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const Off o = slot_of(k, 32 * h + 8 * lg + j);
          B.v8[h][j][0] = ld32(o + kValOff + 8u * ln);
          B.v8[h][j][1] = ld32(o + kValOff + 8u * ln + 4u);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const Off o = slot_of(k, 16 * s + 4 * lg + kk);
#pragma unroll
          for (int f = 0; f < (HALF ? 1 : F); ++f) B.vraw[s][kk][f] = ld32(o + vbyte + (uint32_t)(VB * f));
        }
      }
    }
  };
  auto issue = [&](Buf& B, int k) {
    B.live = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const Off o = slot_of(k, 16 * s + ln);
      B.live |= (masked(o) ? 0u : 1u) << s;
      if constexpr (HALF && F == 2) {
        // 32 dims from byte KB (16 hf + 4 g): 16 bytes of 4-bit keys, 12 of 3-bit ones
        if constexpr (KB == 4) {
          const v4u kw = ld128(o + 64u * hf + 16u * lg);
          B.kraw[s][0] = kw.x;
          B.kraw[s][1] = kw.y;
          B.kraw[s][2] = kw.z;
          B.kraw[s][3] = kw.w;
        } else {
#pragma unroll
          for (int i = 0; i < 3; ++i) B.kraw[s][i] = ld32(o + 48u * hf + 12u * lg + 4u * i);
        }
      } else if constexpr (HALF) {
        // 16 dims: 8 bytes of 4-bit keys, 6 of 3-bit ones (two dwords)
        if constexpr (KB == 4) {
          const v2u kw = ld64(o + 32u * hf + 8u * lg);
          B.kraw[s][0] = kw.x;
          B.kraw[s][1] = kw.y;
        } else {
          B.kraw[s][0] = ld32(o + 24u * hf + 6u * lg);
          B.kraw[s][1] = ld32(o + 24u * hf + 6u * lg + 4u);
        }
      } else if constexpr (KB == 4) {
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const v4u kw = ld128(o + (uint32_t)(16 * F) * lg + 16u * f);
          B.kraw[s][4 * f + 0] = kw.x;
          B.kraw[s][4 * f + 1] = kw.y;
          B.kraw[s][4 * f + 2] = kw.z;
          B.kraw[s][4 * f + 3] = kw.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 3 * F; ++i)
          B.kraw[s][i] = ld32(o + (uint32_t)(12 * F) * lg + 4u * i);
      }
    }
    {
      const Off o = slot_of(k, lane);
      B.nw = ld32(o + kNormOff);
      if constexpr (V8) {
        B.sz0 = B.sz1 = 0;
      } else {
        const v2u w = ld64(o + kScaleOff);
        B.sz0 = w.x;
        B.sz1 = w.y;
      }
    }
  };

  // ---- online softmax state of the current segment ----
  float mref[NH], l[NH], zacc[NH];  // per lane: head 4r + lg of this wave
  float(*acc)[64] = accl[wave];       // acc[8F r + i][lane]
  v4i cacc[NH][V8 ? 1 : VDL];
  // kBase (one wave per SIMD at D = 128, four waves per workgroup, narrow
  // addressing: one workgroup fills a CU, so the 16 KB of LDS per wave costs
  // no occupancy and leaves room for the prefix sums of 4096 sequences;
  // the 64-bit tile table would not): the int32
  // value sums are never cleared inside the tile loop (a conditional clear
  // costs a copy of all of them between register files every tile). A flush
  // or a reset takes their growth since the last one, cacc - cbase in
  // wrapping int32 (exact while the growth stays below 2^31, which the
  // 8192-tile flush bound keeps), and moves cbase to cacc.
  constexpr bool kBase = !V8 && NH == 2 && !HALF && DD == 128 && !NCORR && W == 4 && !WIDE;
  __shared__ __attribute__((aligned(16))) v4i cbase[kBase ? W : 1][kBase ? NH * VDL : 1][64];
  if constexpr (kBase) {
#pragma unroll
    for (int r = 0; r < NH; ++r)
#pragma unroll
      for (int i = 0; i < VDL; ++i) cacc[r][i] = v4i{0, 0, 0, 0};
  }
  auto base_at = [&](int r, int i) -> v4i& { return cbase[kBase ? wave : 0][kBase ? VDL * r + i : 0][lane]; };
  v4f facc[NH][V8 ? 8 : 1];  // V8: fp32 MFMA sums, rows 4g .. 4g+3 = head g's parts
  int ev = 0;
  float sref = 0.0f;
  bool empty = true;
  int since_flush = 0;
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      mref[r] = -INFINITY;
      l[r] = 0.0f;
      zacc[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < VDL; ++i) {
        acc[VDL * r + i][lane] = 0.0f;
        if constexpr (V8) facc[r][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        else if constexpr (kBase) base_at(r, i) = cacc[r][i];
        else cacc[r][i] = v4i{0, 0, 0, 0};
      }
    }
    ev = 0;
    sref = 0.0f;
    empty = true;
    since_flush = 0;
  };
  // fold cacc into acc (scale 2^-ev), then rescale acc, l and the zero term
  // by alpha (lane (n, g) holds head g's dims 8F n .. 8F n + 8F - 1)
  auto flush = [&](const float (&alpha)[NH]) {
    const float pinv = exp2i(-ev);
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      if (!empty) {
        if constexpr (kBase) {
          // the sums' growth since the last flush; the row set's bases are
          // all requested before any is used
          v4i old[VDL];
#pragma unroll
          for (int i = 0; i < VDL; ++i) old[i] = base_at(r, i);
#pragma unroll
          for (int i = 0; i < VDL; ++i) {
            base_at(r, i) = cacc[r][i];
            v4i cd;
#pragma unroll
            for (int c = 0; c < 4; ++c) cd[c] = (int)((uint32_t)cacc[r][i][c] - (uint32_t)old[i][c]);
            const float e0 = (float)cd.x, e1 = (float)cd.y;
            const float e2 = (float)cd.z, e3 = (float)cd.w;
            const float val = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(e3, 128.0f, e2), 128.0f, e1), 128.0f, e0);
            acc[VDL * r + i][lane] = __builtin_fmaf(val, pinv, acc[VDL * r + i][lane]) * alpha[r];
          }
        } else {
#pragma unroll
          for (int i = 0; i < VDL; ++i) {
            if constexpr (V8) {
              const float val = (facc[r][i].x + facc[r][i].y) + facc[r][i].z;
              acc[VDL * r + i][lane] = (acc[VDL * r + i][lane] + val) * alpha[r];
              facc[r][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            } else {
              const float e0 = (float)cacc[r][i].x, e1 = (float)cacc[r][i].y;
              const float e2 = (float)cacc[r][i].z, e3 = (float)cacc[r][i].w;
              const float val = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(e3, 128.0f, e2), 128.0f, e1), 128.0f, e0);
              acc[VDL * r + i][lane] = __builtin_fmaf(val, pinv, acc[VDL * r + i][lane]) * alpha[r];
              cacc[r][i] = v4i{0, 0, 0, 0};
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < VDL; ++i) acc[VDL * r + i][lane] *= alpha[r];
      }
      l[r] *= alpha[r];
      zacc[r] *= alpha[r];
    }
    empty = true;
  };

  // ---------------- query of sequence b ----------------
  // q' = FWHT(rot_signs * q) (2F dims per lane: lane + 64e), scaled by 2^E
  // to integers below 2^27 and split into four balanced base-128 digits;
  // the image for MFMA chunk kc (2F chunks of 64 dims): lane (m = 4h' +
  // piece, g), dword j, byte bb holds the digit of dim 32F g + 16kc + 4j +
  // bb (KB = 3), or of dim 32F g + 16kc + 8(j/2) + 2bb + (j%2) (KB = 4: low,
  // then high nibbles of each dword) -- the byte order of the bit planes.
  v4i qa[NH][KC];
  v4i qg[kFold ? NPF : 1][NH][KC];  // kFold: the folded images, one per odd Walsh plane
  float qsum[NH], qf[NH];  // this lane's head 4r + lg: sum of the scaled query, score scale
  // the wave's query rows of sequence b times the rotation signs
  auto query_rows = [&](int b, float (&qx)[NHEAD][2 * F]) {
    float sg[2 * F];
#pragma unroll
    for (int e = 0; e < 2 * F; ++e) sg[e] = p.rot_signs ? p.rot_signs[lane + 64 * e] : 1.0f;
#pragma unroll
    for (int hh = 0; hh < NHEAD; ++hh) {
      const bool ok = hh < gw;
      const float* qrow = p.q + ((int64_t)b * p.hq + h0 + (ok ? hh : 0)) * D;
#pragma unroll
      for (int e = 0; e < 2 * F; ++e) qx[hh][e] = ok ? qrow[lane + 64 * e] * sg[e] : 0.0f;
    }
  };
  // rotate, scale and split the rows into the MFMA A-operand image
  auto query_image = [&](const float (&qx)[NHEAD][2 * F]) {
    uint8_t* img = reinterpret_cast<uint8_t*>(&qimg[wave][0][0][0][0]);
    float xr[kFold ? NHEAD : 1][2 * F], scl[kFold ? NHEAD : 1];  // kFold: rotated rows, 2^E
#pragma unroll
    for (int hh = 0; hh < NHEAD; ++hh) {
      const int r = hh >> 2, hp = hh & 3;
      float x[2 * F];
#pragma unroll
      for (int e = 0; e < 2 * F; ++e) x[e] = qx[hh][e];
      // strides 64 (and 128) inside the lane, then 1 .. 32 across lanes
#pragma unroll
      for (int st = 1; st < 2 * F; st <<= 1)
#pragma unroll
        for (int e = 0; e < 2 * F; ++e)
          if (!(e & st)) {
            const float a = x[e] + x[e + st], c = x[e] - x[e + st];
            x[e] = a;
            x[e + st] = c;
          }
#pragma unroll
      for (int e = 0; e < 2 * F; ++e) {
        x[e] = butterfly_lanes<1>(x[e], lane & 1);
        x[e] = butterfly_lanes<2>(x[e], lane & 2);
        x[e] = butterfly_lanes<4>(x[e], lane & 4);
        x[e] = butterfly_lanes<8>(x[e], lane & 8);
        x[e] = butterfly_lanes<16>(x[e], lane & 16);
        x[e] = butterfly_lanes<32>(x[e], lane & 32);
      }
      // x[e] = q'[lane + 64 e]
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < 2 * F; ++e) am = fmaxf(am, fabsf(x[e]));
      const float amax = group_max<64>(am);
      const int E = amax > 0.0f ? 26 - ((int)((f2u(amax) >> 23) & 0xFF) - 127) : 0;
      const float sc = exp2i(E);
      if constexpr (kFold) {
        scl[hh] = sc;
#pragma unroll
        for (int e = 0; e < 2 * F; ++e) xr[hh][e] = x[e];
      }
      float dsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < 2 * F; ++e) {
        if (HALF && e / F != hf) continue;  // HALF: the wave's dims are 64F hf .. 64F hf + 64F - 1
        const int dim = lane + 64 * e;
        int v = (int)__builtin_rintf(x[e] * sc);
        const int op = HALF ? dim - 64 * F * hf : dim;  // dim within the wave's share
        const int gg = op / (16 * KC), o = op % (16 * KC);
        const int kc = o >> 4;
        const int j = KB == 4 ? 2 * ((o & 15) >> 3) + (o & 1) : (o & 15) >> 2;
        const int bb = KB == 4 ? (o & 7) >> 1 : o & 3;
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) {
          const int dk = (pc < 3) ? (((v + 64) & 127) - 64) : v;
          v = (v - dk) >> 7;
          const int L = 16 * gg + 4 * hp + pc;
          img[(((r * KC + kc) * 64 + L) * 4 + j) * 4 + bb] = (uint8_t)(dk & 0xFF);
          dsum[pc] += (float)dk;
        }
      }
      float t[4];
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) t[pc] = group_sum<64>(dsum[pc]);
      if (hp == lg) {
        qsum[r] = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(t[3], 128.0f, t[2]), 128.0f, t[1]), 128.0f, t[0]);
        // score in base-2 units = sm_scale / sqrt(D) * log2(e) * 2^-E * norm * (integer dot)
        qf[r] = p.sm_scale * (D == 128 ? 0.08838834764831845f : 0.0625f) * kLog2e * exp2i(-E);
      }
    }
    wave_sync();
#pragma unroll
    for (int r = 0; r < NH; ++r)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(&qimg[wave][r][kc][lane][0]);
        qa[r][kc] = v4i{(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w};
      }
    if constexpr (kFold) {
      // the folded images, one at a time through the same LDS area
      // byte of digit pc of dim lane + 64 e of head hh in the image
      auto img_at = [&](int hh, int e, int pc) -> uint8_t& {
        const int r = hh >> 2, hp = hh & 3;
        const int dim = lane + 64 * e;
        const int op = HALF ? dim - 64 * F * hf : dim;
        const int gg = op / (16 * KC), o = op % (16 * KC);
        const int kc = o >> 4;
        const int j = KB == 4 ? 2 * ((o & 15) >> 3) + (o & 1) : (o & 15) >> 2;
        const int bb = KB == 4 ? (o & 7) >> 1 : o & 3;
        const int L = 16 * gg + 4 * hp + pc;
        return img[(((r * KC + kc) * 64 + L) * 4 + j) * 4 + bb];
      };
#pragma unroll
      for (int i = 0; i < NPF; ++i) {
        wave_sync();  // the previous image is read before it is overwritten
#pragma unroll
        for (int hh = 0; hh < NHEAD; ++hh) {
          const float s = scl[hh] * gq[i];
#pragma unroll
          for (int e = 0; e < 2 * F; ++e) {
            if (HALF && e / F != hf) continue;
            int v = (int)__builtin_rintf(xr[hh][e] * s);
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
              const int dk = (pc < 3) ? (((v + 64) & 127) - 64) : v;
              v = (v - dk) >> 7;
              img_at(hh, e, pc) = (uint8_t)(dk & 0xFF);
            }
          }
        }
        wave_sync();
#pragma unroll
        for (int r = 0; r < NH; ++r)
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            const uint4 w4 = *reinterpret_cast<const uint4*>(&qimg[wave][r][kc][lane][0]);
            qg[i][r][kc] = v4i{(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w};
          }
      }
    }
  };
  auto load_query = [&](int b) {
    float qx[NHEAD][2 * F];
    query_rows(b, qx);
    query_image(qx);
  };

  // ---------------- segment bookkeeping ----------------
  int seg_b = -1, seg_s = 0;
  bool seg_from_start = false, seg_to_end = false, seg_first = false;
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
      const float zt = row16_sum(zacc[r]);
      const int hh = 4 * r + lg;
      if (hh < gw) {
        float* out;
        if (whole)
          out = p.ws + (((int64_t)seg_b * p.hq + h0 + hh) * p.splits + seg_s) * (D + 1);
        else
          out = p.wsp + ((((int64_t)grp * p.nw + wg) * 2 + (seg_first ? 0 : 1)) * (p.wgh * g) +
                         kvl * g + hq0 + hh) * (D + 1);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        float* dst = out + (HALF ? 64 * F * hf + 4 * F * ln : 8 * F * ln);
#pragma unroll
        for (int i = 0; i < VDL; ++i) dst[i] = (acc[VDL * r + i][lane] + zt) * inv;
        if (ln == 0 && hf == 0) out[D] = lt > 0.0f ? (mref[r] + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  };

  // ---------------- one tile ----------------
  auto process = [&](Buf& X, Buf& Y, int k, int c0) {
    const int gk = c0 + k;
    const int4 info = tinfo[k];
    if (gk == lo || (info.z & kFirstOfSplit)) {
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
    issue(Y, k + 1);
    // keep every use of X's registers after the next tile's loads
    __builtin_amdgcn_sched_barrier(0);

    // the scale and zero words of tokens 16s + n (kEarlySZ: requested
    // before the scores, so that their exchange completes under them; the
    // variants with less register room take them after)
    constexpr bool kEarlySZ = DD == 128 && !NCORR && !V8;
    uint32_t szw[V8 ? 1 : 4][2];
    auto fetch_sz = [&]() {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        szw[s][0] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * s + ln) << 2, (int)X.sz0);
        szw[s][1] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * s + ln) << 2, (int)X.sz1);
      }
    };
    if constexpr (kEarlySZ) fetch_sz();

    // ---- scores: lane (n, g) gets head 4r + g, token 16s + n ----
    float sc[NH][4];
    float nrs[HALF ? 4 : 1];  // HALF: the key norms, applied after the exchange
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float nrm = half_lo((uint32_t)__builtin_amdgcn_ds_bpermute((16 * s + ln) << 2, (int)X.nw));
      // KB = 3: index bytes of dims 32F g + 4i .. +3 (KB = 4 reads the
      // planes from the packed nibbles)
      uint32_t ix[KB == 3 ? 4 * KC : 1];
      if constexpr (KB == 3) {
#pragma unroll
        for (int i = 0; i < 4 * KC; ++i) ix[i] = unpack3x4(bits12(X.kraw[s], 12 * i));
      }
      // one bit plane at a time: 2F MFMAs (dims 32F g + 16kc + ...), then its
      // share of the dot product; lane (n, g) holds rows 4g..4g+3 = the
      // digit planes of head g, token 16s+n
      // the B operand of chunk kc for plane SS: the subset S of index bits
      // (low bits); SS >= 32: their parity, else their product
      auto plane_words = [&](auto sel, int kc) -> v4i {
        constexpr int SS = decltype(sel)::value;
        constexpr bool PAR = SS >= 32;
        constexpr int S = SS & 31;
        uint32_t pl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // bit k of each byte (KB = 3) or of each nibble (KB = 4) of x
          // is index bit k of one dimension
          uint32_t x;
          if constexpr (KB == 4) x = X.kraw[s][2 * kc + (j >> 1)];
          else x = ix[4 * kc + j];
          uint32_t m = PAR ? 0u : 0xFFFFFFFFu;
#pragma unroll
          for (int k = 0; k < KB; ++k) {
            if (!((S >> k) & 1)) continue;
            if constexpr (PAR) m ^= x >> k;
            else m &= x >> k;
          }
          pl[j] = ((KB == 4 && (j & 1)) ? m >> 4 : m) & 0x01010101u;
        }
        return v4i{(int)pl[0], (int)pl[1], (int)pl[2], (int)pl[3]};
      };
      auto plane_dot = [&](auto sel, float (&out)[NH]) {
        constexpr int SS = decltype(sel)::value;
        constexpr bool PAR = SS >= 32;
        constexpr int S = SS & 31;
        v4i c[NH];
#pragma unroll
        for (int r = 0; r < NH; ++r) c[r] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          uint32_t pl[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t x;
            if constexpr (KB == 4) x = X.kraw[s][2 * kc + (j >> 1)];
            else x = ix[4 * kc + j];
            uint32_t m = PAR ? 0u : 0xFFFFFFFFu;
#pragma unroll
            for (int k = 0; k < KB; ++k) {
              if (!((S >> k) & 1)) continue;
              if constexpr (PAR) m ^= x >> k;
              else m &= x >> k;
            }
            pl[j] = ((KB == 4 && (j & 1)) ? m >> 4 : m) & 0x01010101u;
          }
          const v4i bpl = v4i{(int)pl[0], (int)pl[1], (int)pl[2], (int)pl[3]};
#pragma unroll
          for (int r = 0; r < NH; ++r) c[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][kc], bpl, c[r], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < NH; ++r)
          out[r] = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf((float)c[r].w, 128.0f, (float)c[r].z), 128.0f,
                                                 (float)c[r].y), 128.0f, (float)c[r].x);
      };
      float dot[NH];
      float t[NH];
      if (kFold && anti) {
        // all odd planes into one accumulator, each against its folded image
        v4i c[NH];
#pragma unroll
        for (int r = 0; r < NH; ++r) c[r] = v4i{0, 0, 0, 0};
        auto fold_plane = [&](auto sel) {
          constexpr int I = decltype(sel)::value;
          constexpr int S = odd_plane(I);
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            uint32_t pl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              uint32_t x;
              if constexpr (KB == 4) x = X.kraw[s][2 * kc + (j >> 1)];
              else x = ix[4 * kc + j];
              uint32_t m = 0u;
#pragma unroll
              for (int k = 0; k < KB; ++k)
                if ((S >> k) & 1) m ^= x >> k;
              pl[j] = ((KB == 4 && (j & 1)) ? m >> 4 : m) & 0x01010101u;
            }
            const v4i bpl = v4i{(int)pl[0], (int)pl[1], (int)pl[2], (int)pl[3]};
#pragma unroll
            for (int r = 0; r < NH; ++r)
              c[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qg[kFold ? I : 0][r][kc], bpl, c[r], 0, 0, 0);
          }
        };
        fold_plane(std::integral_constant<int, 0>{});
        fold_plane(std::integral_constant<int, 1>{});
        fold_plane(std::integral_constant<int, 2>{});
        fold_plane(std::integral_constant<int, 3>{});
        if constexpr (NPF == 8) {
          fold_plane(std::integral_constant<int, 4>{});
          fold_plane(std::integral_constant<int, 5>{});
          fold_plane(std::integral_constant<int, 6>{});
          fold_plane(std::integral_constant<int, 7>{});
        }
#pragma unroll
        for (int r = 0; r < NH; ++r) {
          const float u = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf((float)c[r].w, 128.0f, (float)c[r].z), 128.0f,
                                                        (float)c[r].y), 128.0f, (float)c[r].x);
          dot[r] = __builtin_fmaf(gsum, qsum[r], -2.0f * gmax * u);
        }
      } else if (anti) {
        // odd Walsh terms: the single bits and (KB = 3) b0^b1^b2 or (KB = 4)
        // the four parities of three bits
        float tw[NH];
        float gs = 0.0f;
#pragma unroll
        for (int r = 0; r < NH; ++r) tw[r] = 0.0f;
#define TQK_WALSH(S)                                                               \
        plane_dot(std::integral_constant<int, 32 + S>{}, t);                       \
        gs += ga[S];                                                               \
        for (int r = 0; r < NH; ++r) tw[r] = __builtin_fmaf(ga[S], t[r], tw[r]);
        TQK_WALSH(1) TQK_WALSH(2) TQK_WALSH(4)
        if constexpr (KB == 3) {
          TQK_WALSH(7)
        } else {
          TQK_WALSH(8) TQK_WALSH(7) TQK_WALSH(11) TQK_WALSH(13) TQK_WALSH(14)
        }
#undef TQK_WALSH
#pragma unroll
        for (int r = 0; r < NH; ++r) dot[r] = __builtin_fmaf(gs, qsum[r], -2.0f * tw[r]);
      } else {
#pragma unroll
        for (int r = 0; r < NH; ++r) dot[r] = al[0] * qsum[r];
#define TQK_PLANE(S)                                                         \
        plane_dot(std::integral_constant<int, S>{}, t);                      \
        for (int r = 0; r < NH; ++r) dot[r] = __builtin_fmaf(al[S], t[r], dot[r]);
        TQK_PLANE(1) TQK_PLANE(2) TQK_PLANE(3) TQK_PLANE(4) TQK_PLANE(5) TQK_PLANE(6) TQK_PLANE(7)
        if constexpr (KB == 4) {
          TQK_PLANE(8) TQK_PLANE(9) TQK_PLANE(10) TQK_PLANE(11) TQK_PLANE(12) TQK_PLANE(13)
          TQK_PLANE(14) TQK_PLANE(15)
        }
#undef TQK_PLANE
      }
      const float mask = ((X.live >> s) & 1u) ? INFINITY : -INFINITY;
      if constexpr (NCORR) {
        // sum over the token's dims of c[idx]^2 = sum_S e2_S (D - 2 n_S),
        // n_S the dims whose index bits in S have odd parity: the plane
        // summed over all D dims by an MFMA against ones (every row of the
        // result is the count of token 16s + n)
        const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
        float cs = e2_s[0] * (float)D;
        auto count = [&](auto sel) -> float {
          v4i c = v4i{0, 0, 0, 0};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, plane_words(sel, kc), c, 0, 0, 0);
          return (float)c.x;
        };
#define TQK_SQ(S) cs = __builtin_fmaf(e2_s[S], (float)D - 2.0f * count(std::integral_constant<int, 32 + S>{}), cs);
        if (anti) {
          TQK_SQ(3) TQK_SQ(5) TQK_SQ(6)
          if constexpr (KB == 4) {
            TQK_SQ(9) TQK_SQ(10) TQK_SQ(12) TQK_SQ(15)
          }
        } else {
          TQK_SQ(1) TQK_SQ(2) TQK_SQ(3) TQK_SQ(4) TQK_SQ(5) TQK_SQ(6) TQK_SQ(7)
          if constexpr (KB == 4) {
            TQK_SQ(8) TQK_SQ(9) TQK_SQ(10) TQK_SQ(11) TQK_SQ(12) TQK_SQ(13) TQK_SQ(14) TQK_SQ(15)
          }
        }
#undef TQK_SQ
        nrm *= 1.0f / sqrtf(cs + 1e-16f);
      }
      if constexpr (HALF) {
        // this wave's share of the dot products, scaled after the exchange
#pragma unroll
        for (int r = 0; r < NH; ++r) sc[r][s] = dot[r];
        nrs[s] = nrm;
      } else {
#pragma unroll
        for (int r = 0; r < NH; ++r) sc[r][s] = fminf(dot[r] * (qf[r] * nrm), mask);
      }
      // one token block at a time (bounds the live bit planes)
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (HALF) {
      // add the other half's partial scores (a + b in one wave, b + a in the
      // other: the same sums, so both run the same softmax); the buffer
      // alternates with the tile, and a wave rewrites one only after the
      // next tile's barrier, which its partner reaches after reading it
      float* mine = &xs[gk & 1][wave][lane][0];
      *reinterpret_cast<float4*>(mine) = make_float4(sc[0][0], sc[0][1], sc[0][2], sc[0][3]);
      *reinterpret_cast<float4*>(mine + 4) = make_float4(sc[1][0], sc[1][1], sc[1][2], sc[1][3]);
      __syncthreads();
      const float* other = &xs[gk & 1][wave ^ 1][lane][0];
      const float4 o0 = *reinterpret_cast<const float4*>(other);
      const float4 o1 = *reinterpret_cast<const float4*>(other + 4);
      const float po[2][4] = {{o0.x, o0.y, o0.z, o0.w}, {o1.x, o1.y, o1.z, o1.w}};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float mask = ((X.live >> s) & 1u) ? INFINITY : -INFINITY;
#pragma unroll
        for (int r = 0; r < NH; ++r) sc[r][s] = fminf((sc[r][s] + po[r][s]) * (qf[r] * nrs[s]), mask);
      }
    }
    issue_v(Y, k + 1);
    __builtin_amdgcn_sched_barrier(0);
    float vsc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vz[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float smax = 0.0f;
    if constexpr (!V8) {
      if constexpr (!kEarlySZ) fetch_sz();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        vsc[s] = half_hi(szw[s][0]);
        vz[s] = half_lo(szw[s][1]);
        smax = fmaxf(smax, fabsf(vsc[s]));
      }
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
    // a flush also bounds the int32 digit sums (< 2^31 after 8192 tiles);
    // V8's fp32 sums need no fixed-point range
    const bool smove = !V8 && (smax >= sref || ++since_flush >= 8192);
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
      if (smax > 0.0f) {
        const int e = (int)((f2u(smax) >> 23) & 0xFF) - 127;
        ev = 26 - kTau - e;
        sref = exp2i(e + 1);
      }
    }

    if constexpr (V8) {
      // ---- weights in three bf16 parts, to LDS as [part][head][token] ----
#pragma unroll
      for (int r = 0; r < NH; ++r) {
        float ps = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float pr = (mref[r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[r][s] - mref[r]);
          ps += pr;
          const uint32_t bh = bf16_bits(pr);
          const float r1 = pr - u2f(bh << 16);
          const uint32_t bm = bf16_bits(r1);
          const uint32_t bl = bf16_bits(r1 - u2f(bm << 16));
          pbf[wave][r][0][lg][16 * s + ln] = (uint16_t)bh;
          pbf[wave][r][1][lg][16 * s + ln] = (uint16_t)bm;
          pbf[wave][r][2][lg][16 * s + ln] = (uint16_t)bl;
        }
        l[r] += ps;
      }
      empty = false;
      wave_sync();
      // ---- value MFMAs (exact bf16 values), one 32-token half at a time ----
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // A: lane (4h' + part, g) holds part `part` of head h''s weights of
        // tokens 32h + 8g .. 32h + 8g + 7 (part 3: zero)
        v8bf16 pa[NH];
        const int hd = ln >> 2, part = ln & 3;
#pragma unroll
        for (int r = 0; r < NH; ++r) {
          uint4 a4 = make_uint4(0u, 0u, 0u, 0u);
          if (part < 3) a4 = *reinterpret_cast<const uint4*>(&pbf[wave][r][part][hd][32 * h + 8 * lg]);
          pa[r] = __builtin_bit_cast(v8bf16, v4u{a4.x, a4.y, a4.z, a4.w});
        }
        // ob[t][i]: byte i of value bytes 8n .. 8n+7 of tokens 4t .. 4t+3
        // of this lane's eight (4x4 byte transposes)
        uint32_t ob[2][8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t d0 = X.v8[h][4 * t][q], d1 = X.v8[h][4 * t + 1][q];
            const uint32_t d2 = X.v8[h][4 * t + 2][q], d3 = X.v8[h][4 * t + 3][q];
            const uint32_t x01l = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
            const uint32_t x23l = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
            const uint32_t x01h = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
            const uint32_t x23h = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
            ob[t][4 * q + 0] = __builtin_amdgcn_perm(x23l, x01l, 0x05040100u);
            ob[t][4 * q + 1] = __builtin_amdgcn_perm(x23l, x01l, 0x07060302u);
            ob[t][4 * q + 2] = __builtin_amdgcn_perm(x23h, x01h, 0x05040100u);
            ob[t][4 * q + 3] = __builtin_amdgcn_perm(x23h, x01h, 0x07060302u);
          }
        }
        // B of MFMA i: column n = value dim 8n + i, rows = the 32 tokens
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const v2bf16 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ob[0][i], 1.0f, false);
          const v2bf16 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ob[0][i], 1.0f, true);
          const v2bf16 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ob[1][i], 1.0f, false);
          const v2bf16 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ob[1][i], 1.0f, true);
          const v8bf16 vb8 = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
#pragma unroll
          for (int r = 0; r < NH; ++r)
            facc[r][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[r], vb8, facc[r][i], 0, 0, 0);
        }
      }
      wave_sync();  // the weight parts are rewritten by the next tile
    } else {
    // ---- weights p * scale16 as 7-bit digit planes; zero term in fp32 ----
    // A negative scale16 (bytes not written by the encoder) takes signed
    // digits: the digits of p * |scale16| negated as int8.
    const float pscale = exp2i(ev);
    const bool any_neg = __builtin_amdgcn_ballot_w64(vsc[0] < 0.0f || vsc[1] < 0.0f ||
                                                     vsc[2] < 0.0f || vsc[3] < 0.0f) != 0;
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      uint32_t dw[4] = {0, 0, 0, 0};
      float ps = 0.0f, zs = 0.0f;
      float pr[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        pr[s] = (mref[r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[r][s] - mref[r]);
        ps += pr[s];
        zs = __builtin_fmaf(pr[s], vz[s], zs);
      }
      if (!any_neg) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t pi = (uint32_t)__builtin_fmaf(pr[s], vsc[s] * pscale, 0.5f);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) dw[kk] |= ((pi >> (7 * kk)) & 127u) << (8 * s);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t pi = (uint32_t)__builtin_fmaf(pr[s], fabsf(vsc[s]) * pscale, 0.5f);
          const uint32_t neg = vsc[s] < 0.0f ? 0xFFFFFFFFu : 0u;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t d = (((pi >> (7 * kk)) & 127u) ^ neg) - neg;
            dw[kk] |= (d & 255u) << (8 * s);
          }
        }
      }
      l[r] += ps;
      zacc[r] += zs;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) p8[wave][r][lg][kk][ln] = dw[kk];
    }
    empty = false;
    wave_sync();

    // ---- value MFMAs: B operands by 4x4 byte transposes ----
    // u[s]: index bytes of dims 8F n + 8f + 4h .. +3 of token 16s + 4g + kk;
    // vb[i][kk] byte s = dim 8F n + 8f + 4h + i of token 16s + 4g + kk,
    // accumulated in cacc[r][8f + 4h + i]
    v4i pa[NH];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      const uint4 a4 = *reinterpret_cast<const uint4*>(&p8[wave][r][ln >> 2][ln & 3][4 * lg]);
      pa[r] = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
    }
#pragma unroll
    for (int fh = 0; fh < FH; ++fh) {
      const int f = fh >> 1, h = fh & 1;
      uint32_t vb[4][4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t u[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t x = X.vraw[s][kk][f];
          if constexpr (HALF && F == 1) u[s] = VB == 4 ? unpack4x4(x, 0) : unpack3x4(x >> vsh);
          else if constexpr (VB == 4) u[s] = unpack4x4(x, h);
          else u[s] = unpack3x4(h ? x >> 12 : x);
        }
        const uint32_t t01l = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
        const uint32_t t01h = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
        const uint32_t t23l = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
        const uint32_t t23h = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
        vb[0][kk] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
        vb[1][kk] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
        vb[2][kk] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
        vb[3][kk] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i vbi = v4i{(int)vb[i][0], (int)vb[i][1], (int)vb[i][2], (int)vb[i][3]};
#pragma unroll
        for (int r = 0; r < NH; ++r)
          cacc[r][4 * fh + i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[r], vbi, cacc[r][4 * fh + i], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wave_sync();
    }
  };

  // The range's first query rows are requested now: their loads overlap
  // the tile table's, so tile 0 does not wait behind the query set-up.
  float q0[NHEAD][2 * F];
  {
    int bl = 0, bh = p.B - 1;  // the sequence of tile lo, as the table finds it
    while (bl < bh) {
      const int m = (bl + bh + 1) >> 1;
      if (prefix[m] <= lo) bl = m;
      else bh = m - 1;
    }
    query_rows(bl, q0);
  }

  Buf ring[2];
  for (int c0 = lo; c0 < hi; c0 += kChunk) {
    const int K = hi - c0 < kChunk ? hi - c0 : kChunk;
    __syncthreads();
    for (int e = tid; e < (K + 1) * 64; e += NT) {
      const int k = e >> 6, j = e & 63;
      if (k == K) {
        tok_rows[k][j] = WIDE ? (Off)zoff : (Off)kMaskedByte;
        continue;
      }
      const int x = c0 + k;
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
      Off row = WIDE ? (Off)zoff : (Off)kMaskedByte;
      if (tok < end) {
        const uint32_t t32 = (uint32_t)tok;
        const uint32_t pi = bs_pow2 ? (t32 >> bs_shift) : (t32 / bs);
        const int64_t page = p.block_table[(int64_t)b * p.max_blocks + pi];
        if (page >= 0 && page < p.num_blocks) {
          if constexpr (WIDE)
            row = ((int64_t)page * bs + (t32 - pi * bs)) * p.hk * (int64_t)sb;
          else
            row = ((uint32_t)page * bs + (t32 - pi * bs)) * (uint32_t)p.hk * sb;
        }
      }
      tok_rows[k][j] = row;
      if (j == 0) {
        const int nt = (s == q.n - 1) ? q.TLast : q.TL;
        tinfo[k] = make_int4(b, s, (t == 0 ? kFirstOfSplit : 0) | (t == nt - 1 ? kLastOfSplit : 0), 0);
      }
    }
    __syncthreads();
    if (c0 == lo) query_image(q0);
    issue(ring[0], 0);
    issue_v(ring[0], 0);
    // the two register sets as a ring indexed by the unrolled position (the
    // compiler keeps them apart without copies or spills)
    for (int k = 0; k < K; k += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (k + u >= K) break;
        process(ring[u], ring[u ^ 1], k + u, c0);
      }
    }
  }
  emit();
}

template <int W, int NH, int KB, int VB, int DD, bool NCORR, bool HALF = false>
hipError_t launch(const DecodeParams& p, hipStream_t st, bool wide) {
  const uint32_t blocks = (uint32_t)(p.hk / p.wgh) * (uint32_t)p.nw;
  const size_t lds = balance_lds_bytes(p.B);
  if constexpr (HALF) {
    // (narrow addressing only: the caller takes the one-wave layout for wide caches)
    hipLaunchKernelGGL((decode_tqb_kernel<W, NH, false, KB, VB, DD, false, true>), dim3(blocks), dim3(64 * W),
                       lds, st, p);
  } else if constexpr (NCORR) {
    // (the norm-corrected read has no 64-bit variant: the caller declines it)
    hipLaunchKernelGGL((decode_tqb_kernel<W, NH, false, KB, VB, DD, true>), dim3(blocks), dim3(64 * W), lds,
                       st, p);
  } else if (wide) {
    hipLaunchKernelGGL((decode_tqb_kernel<W, NH, true, KB, VB, DD, false>), dim3(blocks), dim3(64 * W), lds,
                       st, p);
  } else {
    hipLaunchKernelGGL((decode_tqb_kernel<W, NH, false, KB, VB, DD, false>), dim3(blocks), dim3(64 * W), lds,
                       st, p);
  }
  return hipGetLastError();
}

// g = 5 .. 8 at D = 128: one wave serves all query heads of a kv head
// (NH = 2), so each tile's keys and values are unpacked once instead of by
// two waves.
constexpr bool kOneWavePerKvHead = true;
// ... except, with 4-bit keys, uniform values and narrow addressing: there
// two waves share a kv head by halves of the head dims (HALF), two of them
// per SIMD. (3-bit keys keep the one-wave layout, whose folded planes come
// out ahead: the halves repeat the softmax and add a barrier per tile.) At
// D = 256 every key width takes the halves for g = 5 .. 8 with uniform values
// and narrow addressing.
constexpr bool kHalfDims = true;

template <int KB, int VB, bool NCORR>
hipError_t launch_layout128(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub);

// Waves, workgroups and the kernel variant for a shape; tiles_ub bounds the
// tile list.
template <int KB, int VB, int DD, bool NCORR>
hipError_t launch_layout(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  if constexpr (DD == 256) {
    // four query heads per wave (ceil(g / 4) waves per kv head), one wave
    // per SIMD, at most 4 waves per workgroup and per CU
    p.wgh = balance_heads_per_wg(p.hk, p.g, 4);
    const int64_t nw = balance_max_wgs(p.hk, p.g, kWaveBudget / 2);
    p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
    if constexpr (!NCORR && VB != 8) {
      if (p.g > 4 && kHalfDims && !wide) {
        // the same grid, the two waves of a kv head split by halves of the
        // head dims instead of by query heads (each unpacks half a tile)
        if (p.wgh == 1) return launch<2, 2, KB, VB, DD, false, true>(p, st, false);
        return launch<4, 2, KB, VB, DD, false, true>(p, st, false);
      }
    }
    switch (p.wgh * ((p.g + 3) / 4)) {
      case 1: return launch<1, 1, KB, VB, DD, NCORR>(p, st, wide);
      case 2: return launch<2, 1, KB, VB, DD, NCORR>(p, st, wide);
      default: return launch<4, 1, KB, VB, DD, NCORR>(p, st, wide);
    }
  } else {
    return launch_layout128<KB, VB, NCORR>(p, st, wide, tiles_ub);
  }
}

// D = 128: waves by group size
template <int KB, int VB, bool NCORR>
hipError_t launch_layout128(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  constexpr int DD = 128;
  if constexpr (!NCORR && VB != 8 && KB == 4) {
    if (p.g > 4 && kHalfDims && !wide) {
      // two waves per kv head, at most 4 per workgroup, two per SIMD
      p.wgh = balance_heads_per_wg(p.hk, p.g, 4);
      const int64_t nw = balance_max_wgs(p.hk, p.g);
      p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
      if (p.wgh == 1) return launch<2, 2, KB, VB, DD, false, true>(p, st, false);
      return launch<4, 2, KB, VB, DD, false, true>(p, st, false);
    }
  }
  if (p.g > 4 && kOneWavePerKvHead) {
    // one wave per kv head at one wave per SIMD: at most 4 waves per
    // workgroup and per CU (the piece region, sized for two waves per kv
    // head at 8 per CU, holds the same number of workgroups)
    p.wgh = balance_heads_per_wg(p.hk, 4, 4);
    const int64_t nw = balance_max_wgs(p.hk, 4, kWaveBudget / 2);
    p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
    switch (p.wgh) {
      case 1: return launch<1, 2, KB, VB, DD, NCORR>(p, st, wide);
      case 2: return launch<2, 2, KB, VB, DD, NCORR>(p, st, wide);
      default: return launch<4, 2, KB, VB, DD, NCORR>(p, st, wide);
    }
  }
  const int qs = (p.g + 3) / 4;
  p.wgh = balance_heads_per_wg(p.hk, p.g);
  const int64_t nw = balance_max_wgs(p.hk, p.g);
  p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
  switch (p.wgh * qs) {
    case 1: return launch<1, 1, KB, VB, DD, NCORR>(p, st, wide);
    case 2: return launch<2, 1, KB, VB, DD, NCORR>(p, st, wide);
    case 4: return launch<4, 1, KB, VB, DD, NCORR>(p, st, wide);
    default: return launch<8, 1, KB, VB, DD, NCORR>(p, st, wide);
  }
}

// one of the four key / value bit combinations
template <int DD, bool NCORR>
hipError_t launch_bits(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  const bool k4 = p.key_fmt == KF_MSE4, v4 = p.val_fmt == VF_U4;
  if (k4)
    return v4 ? launch_layout<4, 4, DD, NCORR>(p, st, wide, tiles_ub)
              : launch_layout<4, 3, DD, NCORR>(p, st, wide, tiles_ub);
  return v4 ? launch_layout<3, 4, DD, NCORR>(p, st, wide, tiles_ub)
            : launch_layout<3, 3, DD, NCORR>(p, st, wide, tiles_ub);
}

}  // namespace

// The launches kept in their own translation units (for build time): head
// dim 256, the norm-corrected read (narrow addressing only) at both head
// dims, and FP8 values.
hipError_t launch_decode_tqb_d256(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub);
hipError_t launch_decode_tqb_ncorr(DecodeParams& p, hipStream_t st, int64_t tiles_ub);
// FP8 values (head dim 128; the norm-corrected read with them goes to
// launch_decode_tqb_ncorr)
hipError_t launch_decode_tqb_fp8v(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub);

}  // namespace tqk
