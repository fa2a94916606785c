// Fused randomized-Hadamard rotation + INT4 per-(token, head) cache write
// (int4_per_token_head.py: reshape_and_cache_int4, single_rht and
// _reshape_cache_int4_kernel), one pass over K and V.
//
// The pages run this as three passes (rotate K, rotate V, quantize) with the
// rotated tensors in memory; here each source row is read once, rotated in
// registers and written straight into the paged cache.
//
// Lane layout (write_rows.h, quarter layout): two lanes per row. The row's
// D/8 chunks of 8 elements form two halves; lane q holds the q-th quarter
// of each half. The RHT sign flips are XOR masks on the packed 16-bit
// source words (from LDS), fused with unpacking and the stride-1
// butterflies; the stride-D/4 butterfly crosses the lane pair as one DPP
// fused multiply-add per element, which leaves lane 1 with the negated
// transform (the last stride, D/2, is in-lane and keeps the negation
// exact). The negation is folded into the row's min / max and into the
// quantizer's reciprocal (sign flips are exact), so the codes are those of
// the plain transform (the sign of an exact zero, which the negation does
// not carry, changes no code and no scale word). Each lane packs its two
// quarters into code words that sit side by side with its partner's, so
// every store instruction of a lane pair writes one contiguous span, and
// every load instruction reads within one 128-byte line.
//
// Memory: a row whose slot is negative or beyond the cache is not read at
// all; code stores are non-temporal (written once, never read back here).
//
// Bit exactness: the FWHT strides run 1 -> D/2 in fp32 with one rounding per
// butterfly, as the pages' transform; the file is compiled without fp
// contraction; the one fused multiply-add of the quantizer is explicit;
// division and reciprocal are IEEE. The quantizer's clamp to [0, 15] is
// replaced by a saturating convert (the lower bound) and, on the rare rows
// whose maximum codes above 15, a cap on the values (the upper bound).
#include "tq_device.h"
#include "tq_internal.h"
#include "write_rows.h"


namespace tqk {

namespace {

struct Int4WriteArgs {
  const void* key;
  const void* value;
  const int64_t* slots;
  const float* signs;
  uint8_t* kc;
  uint8_t* vc;
  float* ks;
  float* vs;
  int64_t total_rows;
  int64_t cache_slots;
  int hk;
  uint32_t hk_magic;
  int hk_shift;
};

// One of two values (taken by value: a conditional over two fields of an
// argument struct would select between their addresses and keep the
// struct in memory).
template <class T>
__device__ __forceinline__ T pick(bool c, T x, T y) {
  return c ? x : y;
}

// Row r is (item = r / 2, K if r even else V), item = t * Hk + h. The token
// index is item / Hk by a multiply-high with a magic number
// (Granlund-Montgomery for 31-bit numerators: m = ceil(2^(31 + l) / Hk),
// l = ceil(log2 Hk), t = (item * m) >> (31 + l)); Hk = 1 passes the item
// through.
__device__ __forceinline__ uint32_t token_of(uint32_t item, const Int4WriteArgs& a) {
  return a.hk == 1 ? item : (__umulhi(item, a.hk_magic) >> a.hk_shift);
}

template <int DT>
constexpr bool half_source() { return DT == TQ_DT_BF16 || DT == TQ_DT_F16; }

// 16-byte pieces of a lane's half row: D/16 chunks of 8 elements, one piece
// per chunk for 16-bit sources and two for fp32.
template <int D, int DT>
constexpr int pieces() { return (D / 16) * (half_source<DT>() ? 1 : 2); }

// Quarter layout: the row's D/8 chunks of 8 elements form two halves of
// M = D/16 chunks; lane q holds the M/2 chunks at q * M/2 of each half, as
// lane-local chunks m = 0 .. M-1 (first half, then second).
template <int D>
__device__ __forceinline__ constexpr int chunk_of(int m, int q) {
  return (m % (D / 32)) + q * (D / 32) + (D / 16) * (m / (D / 32));
}

// Loads the slot of source row `row` and, when the row is to be stored,
// the lane's half of the row (rows past the end and rows with a negative or
// out-of-range slot read nothing: they are not stored). Returns the slot,
// -1 for rows past the end.
template <int D, int DT>
__device__ __forceinline__ int64_t load_row(uint4* raw, const Int4WriteArgs& a, int64_t row,
                                            int q) {
  constexpr int ES = half_source<DT>() ? 2 : 4;  // source element bytes
  const bool ok = row < a.total_rows;
  const uint32_t item = ok ? (uint32_t)(row >> 1) : 0u;
  const int64_t slot = ok ? a.slots[token_of(item, a)] : -1;
  const char* src = static_cast<const char*>(pick((row & 1) != 0, a.value, a.key));
  const uint4* rsrc = reinterpret_cast<const uint4*>(src + (int64_t)item * D * ES);
  constexpr int PC = pieces<D, DT>() / (D / 16);  // 16-byte pieces per chunk
  if (slot >= 0 && slot < a.cache_slots) {
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
#pragma unroll
      for (int p = 0; p < PC; ++p) raw[m * PC + p] = rsrc[chunk_of<D>(m, q) * PC + p];
  } else {
#pragma unroll
    for (int k = 0; k < pieces<D, DT>(); ++k) raw[k] = make_uint4(0u, 0u, 0u, 0u);
  }
  return slot;
}

// Sign flips, unpacking and the stride-1 butterflies of a staged row half.
template <int D, int DT>
__device__ __forceinline__ void unpack_row(const uint4 (&raw)[pieces<D, DT>()],
                                           const uint32_t* smask, int q, float (&x)[D / 2]) {
  constexpr int M = D / 16;  // chunks per lane
  constexpr bool kHalf = half_source<DT>();
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = chunk_of<D>(m, q);
    if constexpr (kHalf) {
      const uint4 mk = *reinterpret_cast<const uint4*>(&smask[4 * c]);
      const uint32_t w[4] = {raw[m].x ^ mk.x, raw[m].y ^ mk.y, raw[m].z ^ mk.z, raw[m].w ^ mk.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a0 = DT == TQ_DT_BF16 ? bf16_lo(w[k]) : half_lo(w[k]);
        const float b0 = DT == TQ_DT_BF16 ? bf16_hi(w[k]) : half_hi(w[k]);
        x[8 * m + 2 * k] = a0 + b0;
        x[8 * m + 2 * k + 1] = a0 - b0;
      }
    } else {
      const uint4 s0 = *reinterpret_cast<const uint4*>(&smask[8 * c]);
      const uint4 s1 = *reinterpret_cast<const uint4*>(&smask[8 * c + 4]);
      const uint32_t w[8] = {raw[2 * m].x, raw[2 * m].y, raw[2 * m].z, raw[2 * m].w,
                             raw[2 * m + 1].x, raw[2 * m + 1].y, raw[2 * m + 1].z, raw[2 * m + 1].w};
      const uint32_t sg[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a0 = u2f(w[2 * k]) * u2f(sg[2 * k]);
        const float b0 = u2f(w[2 * k + 1]) * u2f(sg[2 * k + 1]);
        x[8 * m + 2 * k] = a0 + b0;
        x[8 * m + 2 * k + 1] = a0 - b0;
      }
    }
  }
}

// A lane's share of one row's cache writes, held until it is stored.
template <int D>
struct RowOut {
  uint32_t d[D / 16];  // code words q * D/16 .. of the packed row
  uint32_t scale_word;
  int64_t dst;         // slot * Hk + head, or -1: nothing to store
  bool is_v;
};

template <int D>
__device__ __forceinline__ void store_row(const RowOut<D>& o, const Int4WriteArgs& a, int q) {
  constexpr int M = D / 16;
  if (o.dst >= 0) {
    uint8_t* c = pick(o.is_v, a.vc, a.kc) + o.dst * (D / 2);
    // words h * M/2 .. of the lane are code words chunk_of(h * M/2, q) ..
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint8_t* w = c + 4 * chunk_of<D>(h * (M / 2), q);
      if constexpr (M == 8)
        stream_store16(w, o.d[4 * h], o.d[4 * h + 1], o.d[4 * h + 2], o.d[4 * h + 3]);
      else
        stream_store8(w, o.d[2 * h], o.d[2 * h + 1]);
    }
    if (q == 0) pick(o.is_v, a.vs, a.ks)[o.dst] = u2f(o.scale_word);
  }
}

// Rotate (after stride 1) and quantize one row (two lanes). Every lane of
// the wave must take part (DPP exchanges and a wave vote).
template <int D, int DT>
__device__ __forceinline__ void finish_row(float (&x)[D / 2], int64_t slot,
                                           const Int4WriteArgs& a, int64_t row, int q,
                                           RowOut<D>& out) {
  constexpr int M = D / 16;  // chunks per lane
  constexpr int NE = D / 2;  // elements per lane
  fwht_quarters_from_stride2<D>(x, q);  // lane 1 now holds the negated values

  // the source dtype's rounding of the rotated row (symmetric in sign)
  if constexpr (DT == TQ_DT_BF16) {
#pragma unroll
    for (int i = 0; i < NE; ++i) x[i] = round1_bf16(x[i]);
  } else if constexpr (DT == TQ_DT_F16) {
#pragma unroll
    for (int i = 0; i < NE; ++i) x[i] = round_to_f16(x[i]);
  }

  // row minimum and maximum of the true values
  float hmn = x[0], hmx = x[0];
#pragma unroll
  for (int i = 1; i < NE; ++i) {
    hmn = fminf(hmn, x[i]);
    hmx = fmaxf(hmx, x[i]);
  }
  float mn = q ? -hmx : hmn, mx = q ? -hmn : hmx;
  mn = fminf(mn, dpp_xor<1>(mn));
  mx = fmaxf(mx, dpp_xor<1>(mx));
  float scale = (mx - mn) / 15.0f;
  scale = (scale > 1e-6f) ? scale : 1e-6f;
  // The page rounds half away from zero and clamps to [0, 15]; for a
  // negative argument both of its branches end at 0, so one truncation of
  // clamp(t + 0.5, 0, 15) gives the same integer for every t.
  const float u = -mn / scale;
  const float zp = __builtin_truncf(__builtin_amdgcn_fmed3f(u + 0.5f, 0.0f, 15.0f));
  const float inv = 1.0f / scale;
  const float invs = q ? -inv : inv;  // x * invs = (true value) * inv exactly

  // Every code of the row is at most that of its maximum (the code is
  // monotone in the value). A row whose maximum codes above 15 (rare unless
  // the row is one-signed) first has its values capped at c, a value that
  // codes to exactly 15: then min(code(x), 15) = code(min(x, c)). With c =
  // (15 - zp) * scale, c * inv + zp = 15 within 15 * 2^-23, far inside the
  // code-15 interval [14.5, 15.5). Lane 1 holds negated values, so its cap
  // is a floor at -c.
  if (!__all(__builtin_fmaf(mx, inv, zp) + 0.5f < 16.0f)) {
    const float c = fminf((15.0f - zp) * scale, 3.40282347e38f);
    const float lo = q ? -c : -INFINITY, hi = q ? INFINITY : c;
#pragma unroll
    for (int i = 0; i < NE; ++i) x[i] = __builtin_amdgcn_fmed3f(x[i], lo, hi);
  }
  // the saturating convert maps negative arguments to 0, the lower clamp
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t w = cvt_u32_sat(__builtin_fmaf(x[8 * m], invs, zp) + 0.5f);
#pragma unroll
    for (int j = 1; j < 8; ++j)
      w = lshl_or(cvt_u32_sat(__builtin_fmaf(x[8 * m + j], invs, zp) + 0.5f), 4 * j, w);
    out.d[m] = w;
  }
  out.scale_word = (f2u(scale) & 0xFFFFFFF0u) | (uint32_t)zp;
  out.is_v = row & 1;
  out.dst = -1;
  if (slot >= 0 && slot < a.cache_slots) {
    const uint32_t item = (uint32_t)(row >> 1);
    const int head = (int)(item - token_of(item, a) * (uint32_t)a.hk);
    out.dst = slot * a.hk + head;
  }
}

// One workgroup of NT lanes handles NT / 2 rows.
template <int D, int DT, int NT>
__global__ __launch_bounds__(NT) void reshape_int4_kernel(
    const void* __restrict__ key, const void* __restrict__ value,
    const int64_t* __restrict__ slots, const float* __restrict__ signs,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, int64_t total_rows, int64_t cache_slots, int hk, uint32_t hk_magic,
    int hk_shift) {
  const Int4WriteArgs a{key, value, slots, signs, kc, vc, ks, vs, total_rows, cache_slots,
                        hk, hk_magic, hk_shift};
  constexpr bool kHalf = half_source<DT>();
  constexpr int NS = kHalf ? D / 2 : D;  // sign-mask words
  // RHT signs: XOR masks of the packed 16-bit pairs, or the fp32 signs
  __shared__ __attribute__((aligned(16))) uint32_t smask[NS];
  for (int i = threadIdx.x; i < NS; i += NT) {
    if constexpr (kHalf) {
      const float2 sp = reinterpret_cast<const float2*>(a.signs)[i];
      smask[i] = (sp.x < 0.0f ? 0x8000u : 0u) | (sp.y < 0.0f ? 0x80000000u : 0u);
    } else {
      smask[i] = f2u(a.signs[i]);
    }
  }
  const int q = threadIdx.x & 1;
  const int64_t row = (int64_t)blockIdx.x * (NT / 2) + (threadIdx.x >> 1);
  uint4 raw[pieces<D, DT>()];
  const int64_t slot = load_row<D, DT>(raw, a, row, q);
  __syncthreads();  // smask
  float x[D / 2];
  unpack_row<D, DT>(raw, smask, q, x);
  RowOut<D> out;
  finish_row<D, DT>(x, slot, a, row, q, out);
  store_row<D>(out, a, q);
}

template <int D, int DT>
hipError_t launch_reshape(const ReshapeParams& p, hipStream_t st) {
  const int64_t items = p.num_tokens * p.hk;
  if (items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;  // 31-bit item index
  Int4WriteArgs a{p.key, p.value, p.slots, p.signs, p.kc, p.vc, p.ks, p.vs, items * 2,
                  p.num_blocks * (int64_t)p.block_size, p.hk, 0u, 0};
  // t = item / hk by a multiply-high (hk >= 2): l = ceil(log2 hk), m =
  // ceil(2^(31 + l) / hk) < 2^32, shift = l - 1 after the high word
  if (p.hk > 1) {
    int l = 0;
    while (((int64_t)1 << l) < p.hk) ++l;
    const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
    a.hk_magic = (uint32_t)((num + (unsigned)p.hk - 1) / (unsigned)p.hk);
    a.hk_shift = l - 1;
  }
  constexpr int NT = 256;
  const int64_t blocks = (a.total_rows + NT / 2 - 1) / (NT / 2);
  hipLaunchKernelGGL((reshape_int4_kernel<D, DT, NT>), dim3((uint32_t)blocks), dim3(NT), 0, st,
                     a.key, a.value, a.slots, a.signs, a.kc, a.vc, a.ks, a.vs, a.total_rows,
                     a.cache_slots, a.hk, a.hk_magic, a.hk_shift);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape_int4(const ReshapeParams& p, hipStream_t st) {
  if (p.d == 128) {
    if (p.dtype == TQ_DT_BF16) return launch_reshape<128, TQ_DT_BF16>(p, st);
    if (p.dtype == TQ_DT_F16) return launch_reshape<128, TQ_DT_F16>(p, st);
    return launch_reshape<128, TQ_DT_F32>(p, st);
  }
  if (p.dtype == TQ_DT_BF16) return launch_reshape<64, TQ_DT_BF16>(p, st);
  if (p.dtype == TQ_DT_F16) return launch_reshape<64, TQ_DT_F16>(p, st);
  return launch_reshape<64, TQ_DT_F32>(p, st);
}

}  // namespace tqk
