// Device-side helpers shared by the gfx950 kernels: bit casts, rounding to
// narrow float formats, OCP E4M3 conversion and intra-wave exchanges.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqk {

__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// bfloat16 <-> fp32. Rounding is to nearest, ties to even, for finite inputs.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }
__device__ __forceinline__ float round_to_bf16(float x) {
  uint32_t u = f2u(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u2f(u & 0xFFFF0000u);
}

// IEEE binary16 <-> fp32 through the hardware converts (round to nearest
// even, fp16 denormals kept: the gfx9 default mode).
// Float -> u32 with the hardware convert, which truncates and saturates:
// every negative argument gives 0 (a C++ cast of a negative float would be
// undefined).
__device__ __forceinline__ uint32_t cvt_u32_sat(float x) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// (v << s) | w as one v_lshl_or_b32 (a chain of these packs nibbles with
// one instruction each; left to itself the compiler regroups such a chain
// into separate shifts and three-input ORs).
__device__ __forceinline__ uint32_t lshl_or(uint32_t v, int s, uint32_t w) {
  uint32_t r;
  asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "i"(s), "v"(w));
  return r;
}
__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float round_to_f16(float x) { return (float)(_Float16)x; }

// OCP FP8 E4M3FN byte -> fp32 (exact; 0x7F/0xFF are NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t sign = (b & 0x80u) << 24;
  uint32_t em = b & 0x7Fu;
  float v;
  if (em >= 8u) {
    // normal: exponent field e (1..15) -> fp32 field e + 120; 3-bit mantissa
    v = u2f(((em + (120u << 3)) << 20));
    if (em == 0x7Fu) v = __builtin_nanf("");
  } else {
    v = (float)em * 0.001953125f;  // subnormal: m * 2^-9
  }
  return u2f(f2u(v) | sign);
}

// fp32 -> OCP E4M3FN for |x| <= 448 (callers clamp first): round to nearest,
// ties to even, subnormals kept, sign of zero kept.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat448(float x) {
  uint32_t u = f2u(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {  // below 2^-6: multiples of 2^-9, exact scaling
    code = (uint32_t)__builtin_rintf(u2f(a) * 512.0f);
  } else {
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// ---------------------------------------------------------------- exchanges
// Value of lane (lane ^ M) within the wave. M = 1, 2 use DPP quad
// permutations; M = 4, 8, 16 use the swizzle crossbar in xor mode; M = 32
// uses a backward permute.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  int x = __float_as_int(v);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  } else if constexpr (M == 4 || M == 8 || M == 16) {
    r = __builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F);
  } else {
    static_assert(M == 32, "xor distance");
    r = __builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32u) << 2), x);
  }
  return __int_as_float(r);
}

template <int M>
__device__ __forceinline__ uint32_t xor_lane_u(uint32_t v) {
  return f2u(xor_lane<M>(u2f(v)));
}

// All-reduce over groups of N consecutive lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += xor_lane<1>(v);
  if constexpr (N >= 4) v += xor_lane<2>(v);
  if constexpr (N >= 8) v += xor_lane<4>(v);
  if constexpr (N >= 16) v += xor_lane<8>(v);
  if constexpr (N >= 32) v += xor_lane<16>(v);
  if constexpr (N >= 64) v += xor_lane<32>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, xor_lane<1>(v));
  if constexpr (N >= 4) v = fmaxf(v, xor_lane<2>(v));
  if constexpr (N >= 8) v = fmaxf(v, xor_lane<4>(v));
  if constexpr (N >= 16) v = fmaxf(v, xor_lane<8>(v));
  if constexpr (N >= 32) v = fmaxf(v, xor_lane<16>(v));
  if constexpr (N >= 64) v = fmaxf(v, xor_lane<32>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_min(float v) {
  if constexpr (N >= 2) v = fminf(v, xor_lane<1>(v));
  if constexpr (N >= 4) v = fminf(v, xor_lane<2>(v));
  if constexpr (N >= 8) v = fminf(v, xor_lane<4>(v));
  if constexpr (N >= 16) v = fminf(v, xor_lane<8>(v));
  if constexpr (N >= 32) v = fminf(v, xor_lane<16>(v));
  if constexpr (N >= 64) v = fminf(v, xor_lane<32>(v));
  return v;
}

// One cross-lane butterfly stage: lanes whose bit M is clear keep a + b,
// their partners keep a - b (a: value of the lower lane, b: upper lane).
template <int M>
__device__ __forceinline__ float butterfly_lanes(float x, bool upper) {
  float p = xor_lane<M>(x);
  return upper ? (p - x) : (x + p);
}

// Value of lane (lane ^ M), M in {1, 2, 4, 8}, with DPP moves only (no LDS
// crossbar). Row rotations move data to higher lanes: with row_ror:N lane i
// reads lane (i - N) mod 16. Partner i ^ 4 is i + 4 in banks 0 and 2 (lanes
// 0-3, 8-11) and i - 4 in banks 1 and 3; partner i ^ 8 is i - 8 mod 16.
template <int M>
__device__ __forceinline__ float dpp_xor(float v) {
  const int x = __float_as_int(v);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    r = __builtin_amdgcn_update_dpp(x, x, 0x12C, 0xF, 0x5, false);  // row_ror:12, banks 0, 2
    r = __builtin_amdgcn_update_dpp(r, x, 0x124, 0xF, 0xA, false);  // row_ror:4, banks 1, 3
  } else {
    static_assert(M == 8, "xor distance within a 16-lane row");
    r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
  }
  return __int_as_float(r);
}

// Butterfly between lanes i and i ^ M (M <= 8): the lane with bit M clear
// keeps x + partner, its partner keeps partner - x. sgn is +1 / -1 for
// those lanes; sgn * x is exact, so the single rounding of the fma equals
// that of the plain sum or difference.
template <int M>
__device__ __forceinline__ float butterfly16(float x, float sgn) {
  return __builtin_fmaf(sgn, x, dpp_xor<M>(x));
}

// Min / max over aligned groups of N lanes (N in {2, 4, 8, 16}) by DPP.
template <int N>
__device__ __forceinline__ float group16_max(float v) {
  if constexpr (N >= 16) v = fmaxf(v, dpp_xor<8>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_xor<4>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_xor<2>(v));
  if constexpr (N >= 2) v = fmaxf(v, dpp_xor<1>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group16_min(float v) {
  if constexpr (N >= 16) v = fminf(v, dpp_xor<8>(v));
  if constexpr (N >= 8) v = fminf(v, dpp_xor<4>(v));
  if constexpr (N >= 4) v = fminf(v, dpp_xor<2>(v));
  if constexpr (N >= 2) v = fminf(v, dpp_xor<1>(v));
  return v;
}

// Round to bfloat16 (nearest, ties to even) and back with the hardware
// convert; finite inputs.
__device__ __forceinline__ float round_to_bf16_hw(float x) {
  const __bf16 h = (__bf16)x;
  return u2f((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// Workgroup index remap for 8 XCDs: hardware dispatches workgroup i to XCD
// i % 8. Renumbering so that each XCD receives a contiguous range of
// logical indices keeps neighbouring logical workgroups (which share cache
// lines) inside one L2.
__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t bid, uint32_t nblocks) {
  const uint32_t per = nblocks / 8u, rem = nblocks % 8u;
  const uint32_t xcd = bid % 8u, k = bid / 8u;
  // XCDs < rem receive per + 1 blocks
  return (xcd < rem ? xcd * (per + 1u) : rem * (per + 1u) + (xcd - rem) * per) + k;
}

// Streaming global accesses for data touched once (source rows, written
// codes): non-temporal hints, so the lines do not displace reused ones.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 stream_load16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stream_store8(void* p, uint32_t a, uint32_t b) {
  __builtin_nontemporal_store(u32x2{a, b}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void stream_store16(void* p, uint32_t a, uint32_t b, uint32_t c,
                                               uint32_t d) {
  __builtin_nontemporal_store(u32x4{a, b, c, d}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stream_store4(void* p, uint32_t a) {
  __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
}

}  // namespace tqk
