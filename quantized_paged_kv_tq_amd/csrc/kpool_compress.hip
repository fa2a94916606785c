// Pooled-softmax key compression into the FP8 indexer page (kpool_compress.py,
// _kpool_softmax_rotate_write_cache_kernel and kpool_compress_and_write_cache).
//
// One pool of P tokens becomes one cache entry. Per dimension d the pool's
// scores plus the per-slot position bias give softmax weights over the P
// slots (max-shifted), the keys are averaged with them in fp32, the mean is
// rounded to bf16, rotated by the Hadamard-128 butterflies with the 1/sqrt(128)
// factor, rounded to bf16 again and quantized to E4M3 with one absmax scale
// (a power of two, or absmax / 448). The entry lands at its flat location:
// codes at byte 128 * t of the page, the fp32 scale at byte 128 * bs + 4 t.
//
// Lane layout: eight lanes per pool, lane l holding dimensions 8l .. 8l+7 and
// 64 + 8l .. 64 + 8l + 7, so every load and store of a pool is two fully used
// 128-byte spans and the Hadamard butterflies of strides 8 .. 32 are DPP lane
// exchanges inside the group. A 256-lane workgroup serves 32 pools per pass.
//
// Bit-exact function of the inputs: fp32 with one rounding per operation in
// slot order, the weighted sum as one fused multiply-add per slot, IEEE
// division, and e^x rounded to nearest fp32 (evaluated in double, below).
// Compiled without contraction.
#include "kpool.h"
#include "tq_device.h"
#include "tq_internal.h"
#include "write_rows.h"

namespace tqk {
namespace {

// 2^(j/256) for j = 0 .. 255, each the nearest double.
__constant__ double kExp2Frac[256] = {
    0x1.0000000000000p+0, 0x1.00b1afa5abcbfp+0, 0x1.0163da9fb3335p+0, 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0, 0x1.037d42e11bbccp+0, 0x1.04315e86e7f85p+0, 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0, 0x1.0650a0e3c1f89p+0, 0x1.0706b29ddf6dep+0, 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0, 0x1.092bdf66607e0p+0, 0x1.09e3ecac6f383p+0, 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0, 0x1.0c0f145e46c85p+0, 0x1.0cc922b7247f7p+0, 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0, 0x1.0efa55fdfa9c5p+0, 0x1.0fb66affed31bp+0, 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0, 0x1.11edbab5e2ab6p+0, 0x1.12abdc06c31ccp+0, 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0, 0x1.14e95934f312ep+0, 0x1.15a98c8a58e51p+0, 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0, 0x1.17ed48695bbc0p+0, 0x1.18af9388c8deap+0, 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1af99f8138a1cp+0, 0x1.1bbe084045cd4p+0, 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0, 0x1.1e0e75eb44027p+0, 0x1.1ed5022fcd91dp+0, 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0, 0x1.212be3578a819p+0, 0x1.21f49917ddc96p+0, 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0, 0x1.2451ffb82140ap+0, 0x1.251ce4fb2a63fp+0, 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0, 0x1.2780e341ddf29p+0, 0x1.284dfe1f56381p+0, 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0, 0x1.2ab8a66d10f13p+0, 0x1.2b87fd0dad990p+0, 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0, 0x1.2df961f641589p+0, 0x1.2ecafa93e2f56p+0, 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0, 0x1.31432edeeb2fdp+0, 0x1.32170fc4cd831p+0, 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0, 0x1.3496266e3fa2dp+0, 0x1.356c55f929ff1p+0, 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0, 0x1.37f26231e754ap+0, 0x1.38cae6d05d866p+0, 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0, 0x1.3b57fbfec6cf4p+0, 0x1.3c32dc313a8e5p+0, 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0, 0x1.3ec70df1c5175p+0, 0x1.3fa4504ac801cp+0, 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0, 0x1.423fb2709468ap+0, 0x1.431f5d950a897p+0, 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0, 0x1.45c2042a7d232p+0, 0x1.46a41ed1d0057p+0, 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0, 0x1.494e1e192aed2p+0, 0x1.4a32af0d7d3dep+0, 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0, 0x1.4ce41b817c114p+0, 0x1.4dcb299fddd0dp+0, 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0, 0x1.508417f4531eep+0, 0x1.516daa2cf6642p+0, 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0, 0x1.542e2f4f6ad27p+0, 0x1.551a4ca5d920fp+0, 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0, 0x1.57e27dbe2c4cfp+0, 0x1.58d12d497c7fdp+0, 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0, 0x1.5ba11fba87a03p+0, 0x1.5c9268a5946b7p+0, 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0, 0x1.5f6a320dceb71p+0, 0x1.605e1b976dc09p+0, 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0, 0x1.633dd1d1929fdp+0, 0x1.6434634ccc320p+0, 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0, 0x1.671c1c70833f6p+0, 0x1.68155d44ca973p+0, 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6b052fa75173ep+0, 0x1.6c012750bdabfp+0, 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0, 0x1.6ef9298593ae5p+0, 0x1.6ff7df9519484p+0, 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0, 0x1.72f8286ead08ap+0, 0x1.73f9a48a58174p+0, 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0, 0x1.77024b1ab6e09p+0, 0x1.780694fde5d3fp+0, 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0, 0x1.7b17b0976cfdbp+0, 0x1.7c1ed0130c132p+0, 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0, 0x1.7f3878491c491p+0, 0x1.80427543e1a12p+0, 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0, 0x1.8364c1eb941f7p+0, 0x1.8471a4623c7adp+0, 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0, 0x1.879cad931a436p+0, 0x1.88ac7d98a6699p+0, 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8be05bad61778p+0, 0x1.8cf3216b5448cp+0, 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0, 0x1.902fed0282c8ap+0, 0x1.9145b0b91ffc6p+0, 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0, 0x1.948b82b5f98e5p+0, 0x1.95a44cbc8520fp+0, 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0, 0x1.98f33e47a22a2p+0, 0x1.9a0f170ca07bap+0, 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0, 0x1.9d674194bb8d5p+0, 0x1.9e86319e32323p+0, 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0, 0x1.a1e7aed8eb8bbp+0, 0x1.a309bec4a2d33p+0, 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0, 0x1.a674a8af46052p+0, 0x1.a799e1330b358p+0, 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0, 0x1.ab0e521356ebap+0, 0x1.ac36bbfd3f37ap+0, 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0, 0x1.afb4ce622f2ffp+0, 0x1.b0e07298db666p+0, 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0, 0x1.b468415b749b1p+0, 0x1.b59728de5593ap+0, 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0, 0x1.b928cf22749e4p+0, 0x1.ba5b030a1064ap+0, 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0, 0x1.bdf69c3f3a207p+0, 0x1.bf2c25bd71e09p+0, 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0, 0x1.c2d1cd9fa652cp+0, 0x1.c40ab5fffd07ap+0, 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0, 0x1.c7ba88988c933p+0, 0x1.c8f6d9406e7b5p+0, 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0, 0x1.ccb0f2e6d1675p+0, 0x1.cdf0b555dc3fap+0, 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0, 0x1.d1b532b08c968p+0, 0x1.d2f87080d89f2p+0, 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0, 0x1.d6c76e862e6d3p+0, 0x1.d80e316c98398p+0, 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0, 0x1.dbe7cd63a8315p+0, 0x1.dd321f301b460p+0, 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0, 0x1.e11676b197d17p+0, 0x1.e264614f5a129p+0, 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0, 0x1.e653924676d76p+0, 0x1.e7a51fbc74c83p+0, 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0, 0x1.eb9f4867cca6ep+0, 0x1.ecf482d8e67f1p+0, 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0, 0x1.f0f9c1cb6412ap+0, 0x1.f252b376bba97p+0, 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0, 0x1.f6632798844f8p+0, 0x1.f7bfdad9cbe14p+0, 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0, 0x1.fbdba3692d514p+0, 0x1.fd3c22b8f71f1p+0, 0x1.fe9d96b2a23d9p+0,
};
// ln2 / 256 split as hi + lo: hi has 29 significant bits, so k * hi is exact
// for |k| < 2^24 and x - k * hi is exact (Cody-Waite reduction).
constexpr double kLn2By256Hi = 0x1.62e42ffp-9;
constexpr double kLn2By256Lo = -0x1.718432a1b0e26p-43;
constexpr double k256ByLn2 = 0x1.71547652b82fep+8;
constexpr double kShift = 0x1.8p52;  // its ulp is 1

// e^x rounded to the nearest fp32 for x <= 0 (Tang's table method in
// double): x = (256 m + j) ln2/256 + r with |r| <= ln2/512, e^x = 2^m *
// 2^(j/256) * e^r, e^r - 1 by its degree-4 Taylor polynomial (truncation
// below 2^-54). The double result is within about 2^-51 relative of e^x, so
// its rounding to fp32 is the correctly rounded one unless e^x lies that
// close to an fp32 rounding midpoint. Arguments are clamped to [-104, 0]:
// e^-104 < 2^-150 already rounds to 0, as e^x does below it (a NaN argument
// also gives 0). Branch-free: x * 256/ln2 + 1.5 * 2^52 rounds to an integer
// whose low word is k = 256 m + j (two's complement), and 2^m is added to
// the exponent field of the table value (2^m * 2^(j/256) >= 2^-151 stays a
// normal double).
__device__ __forceinline__ float exp_f32_rn(float xf, const double* __restrict__ tab) {
  const double x = (double)__builtin_amdgcn_fmed3f(xf, -104.0f, 0.0f);
  const double sh = __builtin_fma(x, k256ByLn2, kShift);
  const double kd = sh - kShift;
  const int k = (int)(uint32_t)__builtin_bit_cast(uint64_t, sh);
  double r = __builtin_fma(-kd, kLn2By256Hi, x);
  r = __builtin_fma(-kd, kLn2By256Lo, r);
  double q = __builtin_fma(r, 1.0 / 24.0, 1.0 / 6.0);
  q = __builtin_fma(q, r, 0.5);
  q = __builtin_fma(q, r, 1.0);
  const uint64_t tb = __builtin_bit_cast(uint64_t, tab[k & 255]);
  const uint32_t hi = (uint32_t)(tb >> 32) + ((uint32_t)(k >> 8) << 20);
  const double t = __builtin_bit_cast(double, ((uint64_t)hi << 32) | (uint32_t)tb);
  return (float)__builtin_fma(t, q * r, t);
}

typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// Scores of one slot for the lane's 16 dimensions, plus the position bias.
template <int SDT>
__device__ __forceinline__ void load_v(const void* __restrict__ score, int64_t row_elem, int e0,
                                       const float* __restrict__ ape_row, float v[16]) {
  load8<SDT>(score, row_elem + e0, v);
  load8<SDT>(score, row_elem + 64 + e0, v + 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = v[j] + ape_row[e0 + j];
    v[8 + j] = v[8 + j] + ape_row[64 + e0 + j];
  }
}

// Keys of one slot for the lane's 16 dimensions (bf16 pairs).
__device__ __forceinline__ void load_k(const uint16_t* __restrict__ k, int64_t row_elem, int e0,
                                       uint32_t w[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(k + row_elem + e0);
  const uint4 b = *reinterpret_cast<const uint4*>(k + row_elem + 64 + e0);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

__device__ __forceinline__ float kelem(const uint32_t w[8], int j) {
  return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}

// One accumulation step of slot s: p = e^(v - m), den += p, acc += k * p.
__device__ __forceinline__ void accumulate(const float v[16], const float m[16], const uint32_t kw[8],
                                           const double* tab, float den[16], float acc[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float pr = exp_f32_rn(v[j] - m[j], tab);
    den[j] = den[j] + pr;
    acc[j] = __builtin_fmaf(kelem(kw, j), pr, acc[j]);
  }
}

// Pooled mean -> Hadamard-128 -> FP8 entry, and its stores.
__device__ __forceinline__ void finish(const KpoolParams& p, int64_t pool, bool out_cache, int li,
                                      const float acc[16], const float den[16]) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = round_to_bf16_hw(acc[j] / den[j]);
  float sg[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sg[k] = (li >> k) & 1 ? -1.0f : 1.0f;
  fwht_row<8>(x, sg);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    x[j] = round_to_bf16_hw(x[j] * 0.08838834764831845f);
    amax = fmaxf(amax, fabsf(x[j]));
  }
  amax = group16_max<8>(amax);
  amax = (amax > 1e-4f) ? amax : 1e-4f;
  const float inv448 = (float)(1.0 / 448.0);
  float scale;
  float c[16];
  if (p.round_scale) {
    // the power of two at or above amax * fl(1/448), read off its bits; its
    // reciprocal is exact, so the multiplication equals the division
    const uint32_t tb = f2u(amax * inv448);
    const uint32_t sb = (tb & 0x7FFFFFu) ? ((tb & 0x7F800000u) + 0x00800000u) : tb;
    scale = u2f(sb);
    const float inv = u2f((254u << 23) - sb);
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = x[j] * inv;
  } else {
    scale = amax * inv448;
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = x[j] / scale;
  }
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = fminf(fmaxf(c[4 * k + j], -448.0f), 448.0f);
    const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false);
    w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(a[2], a[3], lo, true);
  }
  if (out_cache) {
    const int64_t l = p.loc[pool];
    const int64_t pg = l / p.block_size, off = l % p.block_size;
    uint8_t* page = p.cache + pg * ((int64_t)p.block_size * 132);
    *reinterpret_cast<u32x2_a4*>(page + off * 128 + li * 8) = u32x2_a4{w[0], w[1]};
    *reinterpret_cast<u32x2_a4*>(page + off * 128 + 64 + li * 8) = u32x2_a4{w[2], w[3]};
    if (li == 0) *reinterpret_cast<float*>(page + (int64_t)p.block_size * 128 + off * 4) = scale;
  }
  if (p.ck) {
    *reinterpret_cast<uint2*>(p.ck + pool * 128 + li * 8) = make_uint2(w[0], w[1]);
    *reinterpret_cast<uint2*>(p.ck + pool * 128 + 64 + li * 8) = make_uint2(w[2], w[3]);
    if (li == 0) p.cs[pool] = scale;
  }
}

// Does pool `pool` produce anything (in range, not masked, with an output)?
__device__ __forceinline__ bool pool_state(const KpoolParams& p, int64_t pool, bool& out_cache) {
  out_cache = false;
  if (pool >= p.n_pools) return false;
  if (p.mask && !p.mask[pool]) return false;
  if (p.cache) {
    const int64_t l = p.loc[pool];
    out_cache = l >= 0 && l < p.num_blocks * (int64_t)p.block_size;
  }
  return out_cache || p.ck != nullptr;
}

// PT > 0: pool size PT known here; the scores and keys of all slots stay in
// registers between the max pass and the accumulation pass, and the position
// bias is staged in LDS. PT == 0: any pool size; the accumulation pass
// re-reads the scores (from cache) and reads the bias from global memory.
template <int SDT, int PT>
__global__ __launch_bounds__(256) void kpool_kernel(const KpoolParams p) {
  __shared__ double tab[256];
  __shared__ float ape_s[PT > 0 ? PT * 128 : 1];
  tab[threadIdx.x] = kExp2Frac[threadIdx.x];  // 256 lanes, 256 entries
  if constexpr (PT > 0) {
    for (int i = threadIdx.x; i < PT * 128; i += 256) ape_s[i] = p.ape[i];
  }
  __syncthreads();
  const int li = threadIdx.x & 7;
  const int e0 = li * 8;
  const int P = PT > 0 ? PT : p.pool_size;
  const int64_t groups = (p.n_pools + 31) / 32;
  for (int64_t g = blockIdx.x; g < groups; g += gridDim.x) {
    const int64_t pool = g * 32 + (threadIdx.x >> 3);
    bool out_cache;
    const bool live = pool_state(p, pool, out_cache);
    const int64_t base = (live ? pool : 0) * (int64_t)P * 128;
    float m[16], den[16], acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      m[j] = -__builtin_inff();
      den[j] = 0.0f;
      acc[j] = 0.0f;
    }
    if constexpr (PT > 0) {
      float v[PT][16];
      uint32_t kw[PT][8];
#pragma unroll
      for (int s = 0; s < PT; ++s) {
        if (live) {
          load_v<SDT>(p.slot_score, base + s * 128, e0, ape_s + s * 128, v[s]);
          load_k(p.slot_k, base + s * 128, e0, kw[s]);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) v[s][j] = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) kw[s][j] = 0u;
        }
      }
#pragma unroll
      for (int s = 0; s < PT; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j) m[j] = fmaxf(m[j], v[s][j]);
#pragma unroll
      for (int s = 0; s < PT; ++s) accumulate(v[s], m, kw[s], tab, den, acc);
    } else {
      float v[16];
      uint32_t kw[8];
      for (int s = 0; s < P; ++s) {
        if (live) {
          load_v<SDT>(p.slot_score, base + s * 128, e0, p.ape + s * 128, v);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) m[j] = fmaxf(m[j], v[j]);
      }
      for (int s = 0; s < P; ++s) {
        if (live) {
          load_v<SDT>(p.slot_score, base + s * 128, e0, p.ape + s * 128, v);
          load_k(p.slot_k, base + s * 128, e0, kw);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) kw[j] = 0u;
        }
        accumulate(v, m, kw, tab, den, acc);
      }
    }
    // the eight lanes of a pool share `live`, and the lane exchanges of the
    // butterflies and the absmax stay inside those eight lanes
    if (live) finish(p, pool, out_cache, li, acc, den);
  }
}

template <int SDT>
hipError_t launch_sdt(const KpoolParams& p, hipStream_t st, dim3 grid) {
  switch (p.pool_size) {
    case 1: hipLaunchKernelGGL((kpool_kernel<SDT, 1>), grid, dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((kpool_kernel<SDT, 2>), grid, dim3(256), 0, st, p); break;
    case 4: hipLaunchKernelGGL((kpool_kernel<SDT, 4>), grid, dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((kpool_kernel<SDT, 0>), grid, dim3(256), 0, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kpool_compress(const KpoolParams& p, hipStream_t st) {
  const int64_t groups = (p.n_pools + 31) / 32;
  const dim3 grid((uint32_t)(groups < 4096 ? groups : 4096));
  switch (p.score_dtype) {
    case TQ_DT_F32: return launch_sdt<TQ_DT_F32>(p, st, grid);
    case TQ_DT_F16: return launch_sdt<TQ_DT_F16>(p, st, grid);
    default: return launch_sdt<TQ_DT_BF16>(p, st, grid);
  }
}

}  // namespace tqk
