// TurboQuant combined-slot cache write: the encoder of the slot formats the
// TurboQuant decode reads (triton_turboquant_decode.py, _tq_decode_stage1,
// reads FP8 or Lloyd-Max centroid keys and uniform 3/4-bit values; the pages
// show no writer). For each (token, kv head) with a valid slot:
//   FP8 keys       e4m3(clamp(k, +-448)), D bytes;
//   centroid keys  norm = sqrt(pairwise sum of k^2), u = (FWHT(s * k) *
//                  fl(1/sqrt(D))) / norm, the rotated key divided by its
//                  norm element by element; b-bit index of the nearest
//                  centroid (ties to the lower index; norm 0: u = 0), packed
//                  LSB first, then fp16(norm);
//   values         scale = max((max - min) / (2^b - 1), 1e-6), zero = min,
//                  both rounded to fp16; index = clamp(rint((v - zero16) /
//                  scale16), 0, 2^b - 1), packed LSB first; then fp16 scale
//                  and zero; the slot's padding bytes are zeroed.
// All arithmetic is fp32 with one rounding per operation in that order
// (sums with strides 1 -> D/2, correctly rounded sqrt, IEEE division per
// element), which is what makes the bytes reproducible.
//
// Lane layout as the INT4 writer (write_rows.h): D/16 lanes per row, a lane
// holds 8 consecutive elements per half, i.e. whole bytes of a 3- or 4-bit
// stream (3 or 4 bytes per half). Key and value rows take different code,
// so each wave holds rows of one kind only: in a workgroup pass, waves 0 and
// 2 encode the keys and waves 1 and 3 the values of the same 128 / LPR
// items.
//
// Compiled without fp contraction.
#include "tq_device.h"
#include "tq_internal.h"
#include "write_rows.h"

namespace tqk {

namespace {

struct TqWriteArgs {
  const void* key;
  const void* value;
  const int64_t* slots;
  const float* centroids;
  const float* rot_signs;
  uint8_t* cache;
  int64_t total_items, cache_slots;  // items: (token, kv head) pairs
  int hk, slot_bytes;
  int key_fmt, kb, vb;  // key format, key index bits (3/4; 8 = FP8), value bits
  int kps, vdb;         // key region bytes, value index bytes
};

// LSB-first b-bit stream bytes of 8 consecutive indices (b in {3, 4}).
__device__ __forceinline__ uint32_t pack8(const uint32_t q[8], int b) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= q[j] << (b * j);
  return w;
}
__device__ __forceinline__ void store_bytes(uint8_t* dst, uint32_t w, int n) {
  for (int i = 0; i < n; ++i) dst[i] = (uint8_t)(w >> (8 * i));
}
__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Decision thresholds of the nearest-centroid search. For a table with
// c[j] < c[j+1], |c[j]| <= 1 and gaps of at least 2^-20, and |u| <= ~1 (u is
// a coordinate of a unit vector, up to rounding): the fp32 distances to two
// centroids on the same side of u differ by more than their rounding, so
// only the two centroids around u can be nearest, and between c[j] and
// c[j+1] the choice "c[j+1] strictly nearer" is monotone in u (one
// difference rounds up, the other down, as u grows). Hence the index is the
// number of thresholds T[j] <= u, with T[j] the least fp32 u in
// [c[j], c[j+1]] for which |u - c[j+1]| < |u - c[j]| in fp32, the same
// comparison, ties to the lower index, as a full scan. T[j] is found by
// bisection over the fp32 values of that interval (ordered as integers).
// The key encoder divides, u = Y / norm with Y = fl(y * fl(1/sqrt(D))), and
// the index counts the thresholds T with fl(Y / norm) >= T. Since fp32
// rounding is monotone, fl(x) >= T exactly when x >= mid (T with an even
// significand, which wins the tie at mid) or x > mid (odd), mid being the
// midpoint between T and the fp32 number below it. For norm > 0 that is
// Y >= P or Y > P with P = norm * mid, exact in fp64 (mid has at most 25
// significant bits, the norm 24). Y is an fp32 number, so the condition is
// Y >= Yc, with Yc the least fp32 number >= P (> P for odd T): seven fp32
// bounds per row replace the division of every element. bnd[j] holds mid
// and odd[j] the parity of T[j].
template <int NC>
__device__ __forceinline__ bool centroid_thresholds(const float (&cen)[NC], const float* centroids,
                                                    float (&thr)[NC - 1], double (&bnd)[NC - 1],
                                                    bool (&odd)[NC - 1]) {
  bool ok = true;
#pragma unroll
  for (int j = 0; j < NC; ++j) ok = ok && fabsf(cen[j]) <= 1.0f;
#pragma unroll
  for (int j = 0; j + 1 < NC; ++j) ok = ok && cen[j] < cen[j + 1] && cen[j + 1] - cen[j] >= 0x1p-20f;
  if (!ok) return false;  // uniform
  // lane j < NC - 1 bisects interval j
  const int lane = threadIdx.x & 63;
  const int j = lane < NC - 1 ? lane : NC - 2;
  const float a = centroids[j], b = centroids[j + 1];
  auto key = [](float f) -> uint32_t {
    const uint32_t u = f2u(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
  auto unkey = [](uint32_t k) -> float { return u2f((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); };
  uint32_t lo = key(a), hi = key(b);  // "b strictly nearer": false at a, true at b
  for (int it = 0; it < 32; ++it) {
    if (hi - lo > 1u) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      const float u = unkey(mid);
      if (fabsf(u - b) < fabsf(u - a)) hi = mid;
      else lo = mid;
    }
  }
  const float t = unkey(hi);
#pragma unroll
  for (int k = 0; k + 1 < NC; ++k) {
    thr[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), k));
    const float below = unkey(key(thr[k]) - 1u);
    bnd[k] = ((double)below + (double)thr[k]) * 0.5;  // exact
    odd[k] = (f2u(thr[k]) & 1u) != 0u;
  }
  return true;
}

// The fp32 number just above x (x finite): one step of the bit pattern.
__device__ __forceinline__ float next_up(float x) {
  if (x == 0.0f) return u2f(1u);
  return u2f(x > 0.0f ? f2u(x) + 1u : f2u(x) - 1u);
}

// The least fp32 number >= p (strict: > p), p an exact fp64 value.
__device__ __forceinline__ float f32_ceil(double p, bool strict) {
  const float f = (float)p;  // nearest
  const double fd = (double)f;
  return (strict ? fd <= p : fd < p) ? next_up(f) : f;
}

// Centroid key of one row (D/16 lanes, 16 elements per lane): norm by
// pairwise sums with strides 1 -> D/2, rotation, nearest centroid, packing.
template <int D, int KB>
__device__ __forceinline__ void encode_centroid_key(const float v[16], uint8_t* s, int li,
                                                    const float (&cen)[1 << KB], bool fast,
                                                    const double (&bnd)[(1 << KB) - 1],
                                                    const bool (&odd)[(1 << KB) - 1],
                                                    const float* rot_signs, int kps,
                                                    const float sg[4]) {
  constexpr int LPR = D / 16;
  float hs[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float q2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q2[j] = v[8 * hf + j] * v[8 * hf + j];
    q2[0] = q2[0] + q2[1];
    q2[2] = q2[2] + q2[3];
    q2[4] = q2[4] + q2[5];
    q2[6] = q2[6] + q2[7];
    q2[0] = q2[0] + q2[2];
    q2[4] = q2[4] + q2[6];
    hs[hf] = q2[0] + q2[4];
    // strides 8 .. D/4: lanes li ^ 1, li ^ 2, li ^ 4, li ^ 8; the sum of a
    // pair is the same in both lanes
    if constexpr (LPR >= 2) hs[hf] = hs[hf] + dpp_xor<1>(hs[hf]);
    if constexpr (LPR >= 4) hs[hf] = hs[hf] + dpp_xor<2>(hs[hf]);
    if constexpr (LPR >= 8) hs[hf] = hs[hf] + dpp_xor<4>(hs[hf]);
    if constexpr (LPR >= 16) hs[hf] = hs[hf] + dpp_xor<8>(hs[hf]);
  }
  const float nrm = __builtin_sqrtf(hs[0] + hs[1]);
  float y[16];
  if (rot_signs) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float4* sp = reinterpret_cast<const float4*>(rot_signs + hf * (D / 2) + li * 8);
      const float4 s0 = sp[0], s1 = sp[1];
      const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) y[8 * hf + j] = v[8 * hf + j] * ss[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = v[j];
  }
  fwht_row<LPR>(y, sg);
  // fp32 1/sqrt(D)
  const float rs = D == 128 ? 0.0883883461356163f : (D == 64 ? 0.125f : 0.0625f);
  const bool pos = nrm > 0.0f;
  uint32_t q[16];
  if (fast) {  // uniform
    // fl(Y / norm) >= T[c]  <=>  Y >= Yc[c] (see centroid_thresholds); a zero
    // norm gives u = 0: Y = 0 against the bounds for norm 1 (which are T)
    const double nd = pos ? (double)nrm : 1.0;
    float Yc[(1 << KB) - 1];
#pragma unroll
    for (int c = 0; c + 1 < (1 << KB); ++c) Yc[c] = f32_ceil(nd * bnd[c], odd[c]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float Y = pos ? y[j] * rs : 0.0f;
      uint32_t n = 0;
#pragma unroll
      for (int c = 0; c + 1 < (1 << KB); ++c) n += Y >= Yc[c] ? 1u : 0u;
      q[j] = n;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float u = pos ? (y[j] * rs) / nrm : 0.0f;
      uint32_t best = 0;
      float bd = fabsf(u - cen[0]);
#pragma unroll
      for (int c = 1; c < (1 << KB); ++c) {
        const float dc = fabsf(u - cen[c]);
        if (dc < bd) {
          bd = dc;
          best = (uint32_t)c;
        }
      }
      q[j] = best;
    }
  }
  store_bytes(s + KB * li, pack8(q, KB), KB);
  store_bytes(s + KB * (D / 16) + KB * li, pack8(q + 8, KB), KB);
  if (li == 0) *reinterpret_cast<uint16_t*>(s + kps - 2) = f16_bits(nrm);
}

// KB: key index bits (3 or 4; 8 for FP8 keys)
template <int D, int DT, int KB, int R>
__global__ __launch_bounds__(256) void write_tq_kernel(TqWriteArgs a) {
  constexpr int LPR = D / 16;
  constexpr int NC = KB == 8 ? 1 : 1 << KB;
  // the centroid table, once per workgroup (uniform: scalar registers)
  float cen[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) cen[c] = KB == 8 ? 0.0f : a.centroids[c];
  constexpr int ITEMS = 128 / LPR;  // items per pass
  const int li = threadIdx.x % LPR;
  const int wave = threadIdx.x >> 6;
  const bool values = wave & 1;  // wave-uniform
  const int it_in = (wave >> 1) * (64 / LPR) + (threadIdx.x & 63) / LPR;
  // key waves of a centroid format: decision thresholds of the table
  float thr[NC > 1 ? NC - 1 : 1];
  double bnd[NC > 1 ? NC - 1 : 1];
  bool odd[NC > 1 ? NC - 1 : 1];
  bool fast = false;
  if constexpr (KB != 8) {
    if (!values) fast = centroid_thresholds<NC>(cen, a.centroids, thr, bnd, odd);
  }
  float sg[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sg[k] = (li >> k) & 1 ? -1.0f : 1.0f;

  float x[R][16];
  int64_t slot[R];
  int head[R];
  bool is_v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t it = ((int64_t)blockIdx.x * R + r) * ITEMS + it_in;
    const bool in_range = it < a.total_items;
    const int64_t item = in_range ? it : 0;
    is_v[r] = values;
    const uint32_t it32 = (uint32_t)item;
    const int64_t t = (int64_t)(it32 / (uint32_t)a.hk);
    head[r] = (int)(it32 - (uint32_t)t * (uint32_t)a.hk);
    slot[r] = in_range ? a.slots[t] : -1;
    const void* src = is_v[r] ? a.value : a.key;
    load8<DT>(src, item * D + li * 8, x[r]);
    load8<DT>(src, item * D + D / 2 + li * 8, x[r] + 8);
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (slot[r] < 0 || slot[r] >= a.cache_slots) continue;
    uint8_t* s = a.cache + (slot[r] * a.hk + head[r]) * (int64_t)a.slot_bytes;
    const float* v = x[r];
    if (!is_v[r]) {
      if constexpr (KB == 8) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float c0 = __builtin_amdgcn_fmed3f(v[2 * j], -448.0f, 448.0f);
          const float c1 = __builtin_amdgcn_fmed3f(v[2 * j + 1], -448.0f, 448.0f);
          const uint32_t p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
          if (j & 1) w[j >> 1] |= p << 16;
          else w[j >> 1] = p;
        }
        *reinterpret_cast<uint2*>(s + 8 * li) = make_uint2(w[0], w[1]);
        *reinterpret_cast<uint2*>(s + D / 2 + 8 * li) = make_uint2(w[2], w[3]);
        continue;
      } else {
        encode_centroid_key<D, KB>(v, s, li, cen, fast, bnd, odd, a.rot_signs, a.kps, sg);
        continue;
      }
    }
    // ---- values ----
    if (a.vb == 8) {  // FP8 values (uniform): D E4M3 codes, no scale or zero
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float c0 = __builtin_amdgcn_fmed3f(v[2 * j], -448.0f, 448.0f);
        const float c1 = __builtin_amdgcn_fmed3f(v[2 * j + 1], -448.0f, 448.0f);
        const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
        if (j & 1) w[j >> 1] |= pk << 16;
        else w[j >> 1] = pk;
      }
      // the value region starts at an even byte (KPS is D or ceil(D*b/8) + 2)
      uint16_t* v0 = reinterpret_cast<uint16_t*>(s + a.kps + 8 * li);
      uint16_t* v1 = reinterpret_cast<uint16_t*>(s + a.kps + D / 2 + 8 * li);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        v0[2 * k] = (uint16_t)w[k];
        v0[2 * k + 1] = (uint16_t)(w[k] >> 16);
        v1[2 * k] = (uint16_t)w[2 + k];
        v1[2 * k + 1] = (uint16_t)(w[2 + k] >> 16);
      }
      for (int i = a.kps + a.vdb + li; i < a.slot_bytes; i += LPR) s[i] = 0;
      continue;
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) {
      mn = fminf(mn, v[j]);
      mx = fmaxf(mx, v[j]);
    }
    mn = group16_min<LPR>(mn) + 0.0f;  // a zero minimum is +0
    mx = group16_max<LPR>(mx);
    const float levels = (float)((1 << a.vb) - 1);
    float sc = (mx - mn) / levels;
    if (!(sc > 1e-6f)) sc = 1e-6f;
    const uint16_t sc16 = f16_bits(sc), z16 = f16_bits(mn);
    const float scr = (float)__builtin_bit_cast(_Float16, sc16);
    const float zr = (float)__builtin_bit_cast(_Float16, z16);
    // index = rint(fl((v - zero16) / scale16)). With t = fl(a * fl(1/scale16))
    // (a = v - zero16), |t - fl(a / scale16)| < |t| * 2^-22 (three roundings
    // of at most 2^-24 relative each), so both round to the same integer
    // unless t lies within |t| * 2^-21 of a half-integer; only then (rarely)
    // is the quotient itself computed.
    const float inv = 1.0f / scr;
    uint32_t q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = v[j] - zr;
      const float t = a * inv;
      float idx = __builtin_rintf(t);
      if (!(fabsf(t - idx) < __builtin_fmaf(fabsf(t), -0x1p-21f, 0.5f))) idx = __builtin_rintf(a / scr);
      idx = idx < 0.0f ? 0.0f : (idx > levels ? levels : idx);
      q[j] = (uint32_t)idx;
    }
    const int b = a.vb;
    uint8_t* vd = s + a.kps;
    store_bytes(vd + b * li, pack8(q, b), b);
    store_bytes(vd + b * (D / 16) + b * li, pack8(q + 8, b), b);
    if (li == 0) {
      *reinterpret_cast<uint16_t*>(vd + a.vdb) = sc16;
      *reinterpret_cast<uint16_t*>(vd + a.vdb + 2) = z16;
    }
    // padding bytes of the slot
    for (int i = a.kps + a.vdb + 4 + li; i < a.slot_bytes; i += LPR) s[i] = 0;
  }
}

template <int D, int DT>
hipError_t launch(const TqWriteArgs& a, hipStream_t st) {
  constexpr int R = 2;
  constexpr int ITEMS = 128 / (D / 16);
  const int64_t blocks = (a.total_items + ITEMS * R - 1) / (ITEMS * R);
  if (a.kb == 3)
    hipLaunchKernelGGL((write_tq_kernel<D, DT, 3, R>), dim3((uint32_t)blocks), dim3(256), 0, st, a);
  else if (a.kb == 4)
    hipLaunchKernelGGL((write_tq_kernel<D, DT, 4, R>), dim3((uint32_t)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((write_tq_kernel<D, DT, 8, R>), dim3((uint32_t)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_write_tq(const TqWriteParams& p, hipStream_t st) {
  TqWriteArgs a;
  a.key = p.key;
  a.value = p.value;
  a.slots = p.slots;
  a.centroids = p.centroids;
  a.rot_signs = p.rot_signs;
  a.cache = p.cache;
  a.total_items = p.num_tokens * p.hk;
  a.cache_slots = p.num_blocks * (int64_t)p.block_size;
  a.hk = p.hk;
  a.slot_bytes = p.slot_bytes;
  a.key_fmt = p.key_fmt;
  a.kb = p.key_fmt == KF_MSE3 ? 3 : (p.key_fmt == KF_MSE4 ? 4 : 8);
  a.vb = p.val_fmt == VF_U3 ? 3 : (p.val_fmt == VF_U4 ? 4 : 8);
  a.kps = p.kps;
  a.vdb = p.vdb;
  if (p.d == 256) {
    if (p.dtype == TQ_DT_BF16) return launch<256, TQ_DT_BF16>(a, st);
    if (p.dtype == TQ_DT_F16) return launch<256, TQ_DT_F16>(a, st);
    return launch<256, TQ_DT_F32>(a, st);
  }
  if (p.d == 128) {
    if (p.dtype == TQ_DT_BF16) return launch<128, TQ_DT_BF16>(a, st);
    if (p.dtype == TQ_DT_F16) return launch<128, TQ_DT_F16>(a, st);
    return launch<128, TQ_DT_F32>(a, st);
  }
  if (p.dtype == TQ_DT_BF16) return launch<64, TQ_DT_BF16>(a, st);
  if (p.dtype == TQ_DT_F16) return launch<64, TQ_DT_F16>(a, st);
  return launch<64, TQ_DT_F32>(a, st);
}

}  // namespace tqk
