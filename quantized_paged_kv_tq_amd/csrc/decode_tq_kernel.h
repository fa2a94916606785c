// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores, for FP8
// E4M3 keys with 4-bit uniform values (triton_turboquant_decode.py,
// _tq_decode_stage1: score = sm_scale * q . e4m3(k); v = idx * scale16 +
// zero16; online softmax; partials acc / l and m + ln l).
//
// Scores. The keys are converted to bf16 exactly (every E4M3 value is a
// bf16 value) with v_cvt_scalef32_pk_bf16_fp8. The fp32 query is split into
// three bf16 parts q = hi + mid + lo (exact to 2^-24 relative), and one
// v_mfma_f32_16x16x32_bf16 per 32 dimensions takes A rows 4h + p = part p of
// head h: the lane (n, g) of the 16x16 result then holds the three partial
// products of head g and token n, which it adds in fp32.
//
// Values. As in the INT4 path: P' = p * scale16 (p <= 2^kTau relative to a
// reference maximum) is scaled per tile by a power of two below 2^27 and
// split into four 7-bit digit planes (the A operand of
// v_mfma_i32_16x16x64_i8), the 4-bit indices are the B operand as stored,
// and the int32 sums are exact. The zero term sum_t p_t * zero16_t is a
// per-head fp32 sum added to every dimension at the end.
//
// Work decomposition, tile table, pieces and ping-pong register sets follow
// the INT4 path (balance.h): equal ranges of the global 64-token tile list,
// one wave per four query heads of a kv head for g <= 4. For g = 5 .. 8 one
// wave serves all query heads of its kv head (two MFMA row sets): each
// tile's keys are converted to bf16 and its value nibbles transposed once
// per kv head instead of by two waves, and each wave's loads are its own
// (two waves of a kv head fetched the same lines). That wave needs more
// than 256 registers and runs alone on its SIMD.
#pragma once

#include <type_traits>

#include "balance.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

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

// fp32 -> bf16 bits (round to nearest even; finite values)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// NH: MFMA row sets of four query heads per wave; a tile's keys are
// converted and its value nibbles transposed once for all 4 * NH heads. NH =
// 2 (g = 5 .. 8, one wave per kv head) needs more than 256 registers, so it
// runs one wave per SIMD.
//
// VF8: FP8 E4M3 values (D codes, no scale or zero) instead of 4-bit ones.
// Every E4M3 value is a bf16 value, so the values convert exactly; the
// weights p are split into three bf16 parts like the query, and the value
// sum runs as v_mfma_f32_16x16x32_bf16 with A rows 4h + part (weights of
// head h) and B = 32 tokens x 16 value dims, dims 8n + i for MFMA i (lane n
// loads value bytes 8n .. 8n + 7 of its tokens, and a 4x4 byte transpose
// gives byte i of 4 tokens per register).
template <int W, int NH, bool VF8, bool WIDE, int DD>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(NH == 1 && DD == 128 ? 2 : 1)))
void decode_tq_fp8_kernel(DecodeParams p) {
  constexpr int D = DD;       // head dim, 128 or 256
  constexpr int F = D / 128;  // a lane's dims per 16-lane group and token: 32 F keys, 8 F values
  // the range's first query is requested before the tile table is built
  // (not where holding it through the table build costs registers in the
  // tile loop: the 64-bit, FP8-value, two-row-set and D = 256 variants)
  constexpr bool kEarlyQuery = !WIDE && !VF8 && NH == 1 && DD == 128;
  constexpr int NT = 64 * W;
  constexpr int NHEAD = 4 * NH;  // query heads per wave (padded)
  __shared__ __attribute__((aligned(16))) uint32_t p8[VF8 ? 1 : W][NH][4][4][16];  // weight digit planes
  // VF8: bf16 parts of the weights, [part][head][token] per row set
  __shared__ __attribute__((aligned(16))) uint16_t pbf[VF8 ? W : 1][NH][3][4][64];
  // byte offset of kv head 0's slot of each token of the chunk's tiles
  // (kMaskedByte for masked tokens and the prefetch row past the end)
  using Off = typename std::conditional<WIDE, int64_t, uint32_t>::type;
  __shared__ __attribute__((aligned(16))) Off tok_rows[kChunk + 1][64];
  __shared__ int4 tinfo[kChunk];
  __shared__ int scan[W];
  __shared__ float accl[W][NH * 8 * F][64];  // fp32 value accumulators, lane-major
  extern __shared__ int prefix[];  // [B + 1] tile prefix sums, then [B] lengths

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int grp = blockIdx.x / p.nw;
  const int wg = blockIdx.x - grp * p.nw;
  const int qs_n = (p.g + NHEAD - 1) / NHEAD;
  const int kvl = wave / qs_n;
  const int qsub = wave - kvl * qs_n;
  const int kvh = grp * p.wgh + kvl;
  const int g = p.g;
  const int hq0 = NHEAD * qsub;
  const int gw = g - hq0 < NHEAD ? g - hq0 : NHEAD;
  const int h0 = kvh * g + hq0;

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
  const uint32_t voff = (uint32_t)p.kps;            // value indices
  const uint32_t soff = (uint32_t)(p.kps + p.vdb);  // fp16 scale, fp16 zero

  // ---- registers of one tile ----
  // key bytes [32F g, 32F (g + 1)) of tokens 16s + n; value dwords F n ..
  // F n + F - 1 of tokens 16s + 4g + k; the scale/zero word of token `lane`
  struct Buf {
    v4u kraw[4][2 * F];
    uint32_t sz, live;
    uint32_t vraw[4][4][F];
    uint32_t v8[2][8][2 * F];  // VF8: value bytes 8F n .. 8F n + 8F - 1 of tokens 32h + 8g + j
  };
  const uint32_t kvh_off = (uint32_t)kvh * sb;
  auto slot_of = [&](int k, int j) -> Off { return WIDE ? tok_rows[k][j] : tok_rows[k][j] + kvh_off; };
  auto issue = [&](Buf& B, int k) {
    B.live = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const Off o = slot_of(k, 16 * s + ln);
      B.live |= (masked(o) ? 0u : 1u) << s;
#pragma unroll
      for (int i = 0; i < 2 * F; ++i) B.kraw[s][i] = ld128(o + (uint32_t)(32 * F) * lg + 16u * i);
    }
    if constexpr (VF8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const Off o = slot_of(k, 32 * h + 8 * lg + j);
#pragma unroll
          for (int q = 0; q < 2 * F; ++q) B.v8[h][j][q] = ld32(o + voff + (uint32_t)(8 * F) * ln + 4u * q);
        }
      }
    } else {
      B.sz = ld32(slot_of(k, lane) + soff);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const Off o = slot_of(k, 16 * s + 4 * lg + kk);
#pragma unroll
          for (int f = 0; f < F; ++f) B.vraw[s][kk][f] = ld32(o + voff + (uint32_t)(4 * F) * ln + 4u * f);
        }
      }
    }
  };

  // ---- online softmax state of the current segment ----
  float mref[NH], l[NH], zacc[NH];  // per lane: head 4r + lg of this wave
  float(*acc)[64] = accl[wave];       // acc[8F r + i][lane]
  v4i cacc[NH][8 * F];
  v4f facc[NH][8 * F];  // VF8: fp32 MFMA sums, rows 4g .. 4g+3 = head g's parts
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
      for (int i = 0; i < 8 * F; ++i) {
        acc[8 * F * r + i][lane] = 0.0f;
        cacc[r][i] = v4i{0, 0, 0, 0};
        facc[r][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
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
#pragma unroll
        for (int i = 0; i < 8 * F; ++i) {
          if constexpr (VF8) {
            const float val = (facc[r][i].x + facc[r][i].y) + facc[r][i].z;
            acc[8 * F * r + i][lane] = (acc[8 * F * r + i][lane] + val) * alpha[r];
            facc[r][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          } else {
            const float e0 = (float)cacc[r][i].x, e1 = (float)cacc[r][i].y;
            const float e2 = (float)cacc[r][i].z, e3 = (float)cacc[r][i].w;
            const float val = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(e3, 128.0f, e2), 128.0f, e1), 128.0f, e0);
            acc[8 * F * r + i][lane] = __builtin_fmaf(val, pinv, acc[8 * F * r + i][lane]) * alpha[r];
            cacc[r][i] = v4i{0, 0, 0, 0};
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8 * F; ++i) acc[8 * F * r + i][lane] *= alpha[r];
      }
      l[r] *= alpha[r];
      zacc[r] *= alpha[r];
    }
    empty = true;
  };

  // ---------------- query of sequence b: three bf16 parts ----------------
  // A operand of MFMA kb (4F of them) for lane (m = 4h + part, g): 8 bf16
  // of dims 32F g + 8kb .. 32F g + 8kb + 7 (part 3: zero)
  v8bf16 qa[NH][4 * F];
  float qf;
  // the query dims of lane (m = 4h + part, g) for sequence b: 32F g + 8kb
  // .. 32F g + 8kb + 7 of head h, in two float4
  auto query_rows = [&](int b, float4 (&raw)[NH][4 * F][2]) {
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      const int hq = 4 * r + (ln >> 2);
      const float* qrow = p.q + ((int64_t)b * p.hq + h0 + (hq < gw ? hq : 0)) * D;
#pragma unroll
      for (int kb = 0; kb < 4 * F; ++kb) {
        raw[r][kb][0] = *reinterpret_cast<const float4*>(qrow + 32 * F * lg + 8 * kb);
        raw[r][kb][1] = *reinterpret_cast<const float4*>(qrow + 32 * F * lg + 8 * kb + 4);
      }
    }
  };
  auto query_image = [&](const float4 (&raw)[NH][4 * F][2]) {
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      const int hq = 4 * r + (ln >> 2), part = ln & 3;
      const bool ok = hq < gw && part < 3;
#pragma unroll
      for (int kb = 0; kb < 4 * F; ++kb) {
        const float4 a = raw[r][kb][0];
        const float4 c = raw[r][kb][1];
        const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          uint32_t pr[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float v = x[j + e];
            const uint32_t bh = bf16_bits(v);
            const float r1 = v - u2f(bh << 16);
            const uint32_t bm = bf16_bits(r1);
            const float r2 = r1 - u2f(bm << 16);
            const uint32_t bl = bf16_bits(r2);
            const uint32_t sel = part == 0 ? bh : (part == 1 ? bm : bl);
            pr[e] = ok ? sel : 0u;
          }
          w[j >> 1] = pr[0] | (pr[1] << 16);
        }
        qa[r][kb] = __builtin_bit_cast(v8bf16, v4u{w[0], w[1], w[2], w[3]});
      }
    }
    qf = p.sm_scale * kLog2e;
  };
  auto load_query = [&](int b) {
    float4 raw[NH][4 * F][2];
    query_rows(b, raw);
    query_image(raw);
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
        float* dst = out + 8 * F * ln;
#pragma unroll
        for (int i = 0; i < 8 * F; ++i) dst[i] = (acc[8 * F * r + i][lane] + zt) * inv;
        if (ln == 0) out[D] = lt > 0.0f ? (mref[r] + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  };

  // ---------------- one tile ----------------
  auto process = [&](Buf& X, Buf& Y, int k, int c0) {
    const int gk = c0 + k;
    const int4 info = tinfo[k];
    if (gk == lo || (info.z & kFirstOfSplit)) {
      // (with kEarlyQuery the range's first query is set up before its
      // first tile)
      if (gk != lo) emit();
      if ((!kEarlyQuery || gk != lo) && (gk == lo || info.x != seg_b)) load_query(info.x);
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

    // scale/zero words of tokens 16s + n
    uint32_t sz[4] = {0, 0, 0, 0};
    if constexpr (!VF8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) sz[s] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * s + ln) << 2, (int)X.sz);
    }

    // ---- scores: lane (n, g) gets head 4r + g, token 16s + n ----
    float sc[NH][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4f c[NH];
#pragma unroll
      for (int r = 0; r < NH; ++r) c[r] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 4 * F; ++kb) {
        // key bytes 8kb .. 8kb + 7 of this lane's 32F -> 8 bf16
        const v4u kw = X.kraw[s][kb >> 1];
        const uint32_t w0 = kw[2 * (kb & 1)], w1 = kw[2 * (kb & 1) + 1];
        const v2bf16 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        const v2bf16 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        const v2bf16 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        const v2bf16 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
        const v8bf16 kb8 = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
#pragma unroll
        for (int r = 0; r < NH; ++r) c[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][kb], kb8, c[r], 0, 0, 0);
      }
      const float mask = ((X.live >> s) & 1u) ? INFINITY : -INFINITY;
#pragma unroll
      for (int r = 0; r < NH; ++r) sc[r][s] = fminf((c[r].x + c[r].y + c[r].z) * qf, mask);
    }
    float vsc[4], vz[4];
    float smax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      vsc[s] = half_lo(sz[s]);
      vz[s] = half_hi(sz[s]);
      smax = fmaxf(smax, fabsf(vsc[s]));
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
    // (VF8: the fp32 sums need no fixed-point range)
    const bool smove = !VF8 && (smax >= sref || ++since_flush >= 8192);
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

    if constexpr (VF8) {
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
      // ---- value MFMAs, one 32-token half at a time ----
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
        // ob[t][i]: byte i of value bytes 8F n .. 8F n + 8F - 1 of tokens 4t
        // .. 4t+3 of this lane's eight (4x4 byte transposes)
        uint32_t ob[2][8 * F];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int q = 0; q < 2 * F; ++q) {
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
        // B of MFMA i: column n = value dim 8F n + i, rows = the 32 tokens
#pragma unroll
        for (int i = 0; i < 8 * F; ++i) {
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
      // The encoder's scale16 = (max - min) / levels is positive. A negative
      // one (any bytes are accepted) takes signed digits: the digits of
      // p * |scale16|, negated as int8, which the i8 MFMA sums exactly too.
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

      // ---- value MFMAs: B operands by nibble transpose, in two halves ----
      v4i pa[NH];
#pragma unroll
      for (int r = 0; r < NH; ++r) {
        const uint4 a4 = *reinterpret_cast<const uint4*>(&p8[wave][r][ln >> 2][ln & 3][4 * lg]);
        pa[r] = v4i{(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
      }
#pragma unroll
      for (int fh = 0; fh < 2 * F; ++fh) {
        // dims 8F n + 8f + 4h .. +3 (value dword f, its bytes 2h, 2h + 1)
        const int f = fh >> 1, h = fh & 1;
        uint32_t vb[4][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t w0 = X.vraw[0][kk][f], w1 = X.vraw[1][kk][f], w2 = X.vraw[2][kk][f],
                         w3 = X.vraw[3][kk][f];
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
        for (int i = 0; i < 4; ++i) {
          const v4i vbi = v4i{(int)vb[i][0], (int)vb[i][1], (int)vb[i][2], (int)vb[i][3]};
#pragma unroll
          for (int r = 0; r < NH; ++r)
            cacc[r][4 * fh + i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[r], vbi, cacc[r][4 * fh + i], 0, 0, 0);
        }
      }
      wave_sync();
    }
  };

  // The range's first query rows are requested now: their loads overlap
  // the tile table's, so tile 0 does not wait behind the query set-up.
  float4 q0[NH][4 * F][2];
  if constexpr (kEarlyQuery) {
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
    if (kEarlyQuery && c0 == lo) query_image(q0);
    issue(ring[0], 0);
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

template <int W, int NH, int DD = 128>
hipError_t launch(const DecodeParams& p, hipStream_t st, bool wide) {
  const uint32_t blocks = (uint32_t)(p.hk / p.wgh) * (uint32_t)p.nw;
  const size_t lds = balance_lds_bytes(p.B);
  if (p.val_fmt == VF_FP8) {
    if (wide)
      hipLaunchKernelGGL((decode_tq_fp8_kernel<W, NH, true, true, DD>), dim3(blocks), dim3(64 * W), lds, st, p);
    else
      hipLaunchKernelGGL((decode_tq_fp8_kernel<W, NH, true, false, DD>), dim3(blocks), dim3(64 * W), lds, st, p);
  } else {
    if (wide)
      hipLaunchKernelGGL((decode_tq_fp8_kernel<W, NH, false, true, DD>), dim3(blocks), dim3(64 * W), lds, st, p);
    else
      hipLaunchKernelGGL((decode_tq_fp8_kernel<W, NH, false, false, DD>), dim3(blocks), dim3(64 * W), lds, st, p);
  }
  return hipGetLastError();
}

}  // namespace

// The head-dim-256 launches (their own translation unit: sharing one with
// the D = 128 kernels changes how those are compiled); wide = 64-bit
// addressing.
hipError_t launch_decode_tq_d256(DecodeParams& p, hipStream_t st, bool wide);

}  // namespace tqk
