// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores, for
// 3- or 4-bit centroid keys with 3- or 4-bit uniform values: the launches
// at head dim 128 and the entry point (the kernel is in
// decode_tqb_kernel.h).
#include "decode_tqb_kernel.h"

namespace tqk {

namespace {

// g = 5 .. 8: one wave serves all query heads of a kv head (NH = 2), so each
// tile's keys and values are unpacked once instead of by two waves.
constexpr bool kOneWavePerKvHead = true;

template <int KB, int VB>
hipError_t launch_bits(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  if (p.g > 4 && kOneWavePerKvHead) {
    // one wave per kv head at one wave per SIMD: at most 4 waves per
    // workgroup and per CU (the piece region, sized for two waves per kv
    // head at 8 per CU, holds the same number of workgroups)
    p.wgh = balance_heads_per_wg(p.hk, 4, 4);
    const int64_t nw = balance_max_wgs(p.hk, 4, kWaveBudget / 2);
    p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
    switch (p.wgh) {
      case 1: return launch<1, 2, KB, VB>(p, st, wide);
      case 2: return launch<2, 2, KB, VB>(p, st, wide);
      default: return launch<4, 2, KB, VB>(p, st, wide);
    }
  }
  const int qs = (p.g + 3) / 4;
  p.wgh = balance_heads_per_wg(p.hk, p.g);
  const int64_t nw = balance_max_wgs(p.hk, p.g);
  p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
  switch (p.wgh * qs) {
    case 1: return launch<1, 1, KB, VB>(p, st, wide);
    case 2: return launch<2, 1, KB, VB>(p, st, wide);
    case 4: return launch<4, 1, KB, VB>(p, st, wide);
    default: return launch<8, 1, KB, VB>(p, st, wide);
  }
}

}  // namespace

hipError_t launch_decode_tqb_mfma(DecodeParams& p, hipStream_t st) {
  const bool k4 = p.key_fmt == KF_MSE4, v4 = p.val_fmt == VF_U4;
  if ((p.d != 128 && p.d != 256) || (p.key_fmt != KF_MSE3 && !k4) || (p.val_fmt != VF_U3 && !v4) ||
      p.g > 8 || p.norm_correction)
    return hipErrorNotSupported;
  const int kb = k4 ? 4 : 3, vb = v4 ? 4 : 3;
  if (p.kps != p.d * kb / 8 + 2 || p.vdb != p.d * vb / 8 || p.slot_bytes % 16 != 0)
    return hipErrorNotSupported;
  // slot bytes below 2 GiB take 32-bit buffer offsets, larger caches the
  // 64-bit variant (whose zero page must cover every kv head's slot)
  const bool wide = p.force_wide ||
      p.num_blocks * (int64_t)p.block_size * p.hk * p.slot_bytes >= ((int64_t)1 << 31);
  if (wide && (int64_t)p.hk * p.slot_bytes > kZeroBytes) return hipErrorNotSupported;
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  if (cap >= ((int64_t)1 << 30) || p.B > 4096) return hipErrorNotSupported;
  const int64_t tiles_ub = (int64_t)p.B * ((cap + kTileTokens - 1) / kTileTokens + p.splits);
  if (tiles_ub >= ((int64_t)1 << 30)) return hipErrorNotSupported;
  if (p.d == 256) return launch_decode_tqb_d256(p, st, wide, tiles_ub);
  if (k4) return v4 ? launch_bits<4, 4>(p, st, wide, tiles_ub) : launch_bits<4, 3>(p, st, wide, tiles_ub);
  return v4 ? launch_bits<3, 4>(p, st, wide, tiles_ub) : launch_bits<3, 3>(p, st, wide, tiles_ub);
}

}  // namespace tqk
