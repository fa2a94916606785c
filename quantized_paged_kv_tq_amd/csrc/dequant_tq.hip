// Bulk dequantization of the TurboQuant combined-slot cache to fp16 K and V
// rows (triton_turboquant_decode.py, _tq_full_dequant_kv).
//
// Row (b, kv head, pos) for every pos < max_seq, read through the block
// table (page = block_table[b, pos / bs]); a page outside the pool gives a
// zero row. Keys: FP8 codes widened to fp16; centroid keys norm16 * c[idx]
// in fp32 (optionally with c scaled by 1/sqrt(sum c^2 + 1e-16) first).
// Values: 3/4-bit uniform fma(idx, scale16, zero16) in fp32; FP8 values give
// zeros, as the page's kernel does for widths other than 3 and 4. Every
// fp32 result is rounded to fp16 (nearest even).
//
// HBM-bound: D/8 lanes per row, 8 dimensions each, rows in output order so
// that each row's 2*D-byte K and V stores are contiguous 16-byte lane
// stores. Sub-dword fields are cut out of aligned dword pairs with byte-align
// shifts.
#include "prefill.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

namespace {

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// the 4 bytes at byte offset `off` of a slot (dword-aligned slot base)
__device__ __forceinline__ uint32_t bytes4(const uint8_t* slot, int off) {
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(slot);
  return __builtin_amdgcn_alignbyte(s32[(off >> 2) + 1], s32[off >> 2], (uint32_t)off & 3u);
}

template <int D, int KF, int VF>
__global__ __launch_bounds__(256) void tq_full_dequant_kernel(DequantParams p) {
  constexpr int LPT = D / 8;
  constexpr int RPB = 256 / LPT;  // rows per workgroup
  constexpr int KB = KF == KF_MSE3 ? 3 : 4;
  constexpr int VB = VF == VF_U3 ? 3 : 4;
  __shared__ float cen[16];
  if constexpr (KF != KF_FP8) {
    if (threadIdx.x < 16) cen[threadIdx.x] = threadIdx.x < (1 << KB) ? p.centroids[threadIdx.x] : 0.0f;
    __syncthreads();
  }
  const int li = threadIdx.x % LPT;
  const int64_t rows = (int64_t)p.B * p.hk * p.max_seq;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPT;
  const bool live = r < rows;
  const int64_t rr = live ? r : 0;
  const int pos = (int)(rr % p.max_seq);
  const int64_t bh = rr / p.max_seq;
  const int h = (int)(bh % p.hk);
  const int b = (int)(bh / p.hk);
  const int64_t page = p.block_table[(int64_t)b * p.max_blocks + pos / p.block_size];
  const bool ok = live && page >= 0 && page < p.num_blocks;
  const uint8_t* slot =
      p.kv + ((ok ? page : 0) * p.block_size + pos % p.block_size) * (int64_t)p.hk * p.slot_bytes +
      (int64_t)h * p.slot_bytes;
  uint32_t kw[4] = {0u, 0u, 0u, 0u}, vw[4] = {0u, 0u, 0u, 0u};
  if constexpr (KF == KF_MSE3 || KF == KF_MSE4) {
    // every lane takes part in the norm-correction sum (zeros for dead rows)
    float c[8];
    const uint32_t w = ok ? bytes4(slot, li * KB) : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = cen[(w >> (KB * j)) & ((1u << KB) - 1u)];
    if (p.norm_correction) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = ss + c[j] * c[j];
      ss = group_sum<LPT>(ss);
      const float inv = 1.0f / sqrtf(ss + 1e-16f);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = c[j] * inv;
    }
    if (ok) {
      const float nrm = half_lo(reinterpret_cast<const uint32_t*>(slot)[p.mse_bytes >> 2]);
#pragma unroll
      for (int j = 0; j < 4; ++j) kw[j] = pack_f16x2(nrm * c[2 * j], nrm * c[2 * j + 1]);
    }
  }
  if (ok) {
    if constexpr (KF == KF_FP8) {
      const uint2 w = *reinterpret_cast<const uint2*>(slot + li * 8);
      const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = ws[j >> 1] >> (16 * (j & 1));
        kw[j] = pack_f16x2(e4m3_to_f32(x & 0xFFu), e4m3_to_f32((x >> 8) & 0xFFu));
      }
    }
    if constexpr (VF == VF_U3 || VF == VF_U4) {
      const uint32_t w = bytes4(slot, p.kps + li * VB);
      const uint32_t sz = bytes4(slot, p.kps + p.vdb);
      const float sc = half_lo(sz), zr = half_hi(sz);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __builtin_fmaf((float)((w >> (VB * 2 * j)) & ((1u << VB) - 1u)), sc, zr);
        const float c2 = __builtin_fmaf((float)((w >> (VB * (2 * j + 1))) & ((1u << VB) - 1u)), sc, zr);
        vw[j] = pack_f16x2(a, c2);
      }
    }
  }
  if (live) {
    const int64_t o = r * D + li * 8;
    stream_store16(p.k_out + o, kw[0], kw[1], kw[2], kw[3]);
    stream_store16(p.v_out + o, vw[0], vw[1], vw[2], vw[3]);
  }
}

template <int D, int KF, int VF>
hipError_t launch_f(const DequantParams& p, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = (int64_t)p.B * p.hk * p.max_seq;
  const uint32_t blocks = (uint32_t)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((tq_full_dequant_kernel<D, KF, VF>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DequantParams& p, hipStream_t st) {
  switch (p.key_fmt * 4 + p.val_fmt) {
    case KF_FP8 * 4 + VF_U3: return launch_f<D, KF_FP8, VF_U3>(p, st);
    case KF_FP8 * 4 + VF_U4: return launch_f<D, KF_FP8, VF_U4>(p, st);
    case KF_FP8 * 4 + VF_FP8: return launch_f<D, KF_FP8, VF_FP8>(p, st);
    case KF_MSE3 * 4 + VF_U3: return launch_f<D, KF_MSE3, VF_U3>(p, st);
    case KF_MSE3 * 4 + VF_U4: return launch_f<D, KF_MSE3, VF_U4>(p, st);
    case KF_MSE3 * 4 + VF_FP8: return launch_f<D, KF_MSE3, VF_FP8>(p, st);
    case KF_MSE4 * 4 + VF_U3: return launch_f<D, KF_MSE4, VF_U3>(p, st);
    case KF_MSE4 * 4 + VF_U4: return launch_f<D, KF_MSE4, VF_U4>(p, st);
    case KF_MSE4 * 4 + VF_FP8: return launch_f<D, KF_MSE4, VF_FP8>(p, st);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_tq_full_dequant(const DequantParams& p, hipStream_t st) {
  if (p.d == 128) return launch_d<128>(p, st);
  if (p.d == 64) return launch_d<64>(p, st);
  if (p.d == 256) return launch_d<256>(p, st);
  return hipErrorNotSupported;
}

}  // namespace tqk
