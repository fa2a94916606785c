// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores, for FP8
// keys with 4-bit or FP8 values: the entry point and the launches at head
// dim 128 (the kernel is in decode_tq_kernel.h).
#include "decode_tq_kernel.h"

namespace tqk {

namespace {

// g = 5 .. 8: one wave serves all query heads of a kv head (NH = 2), so each
// tile's keys are converted once instead of by two waves.
constexpr bool kOneWavePerKvHead = true;

}  // namespace

hipError_t launch_decode_tq_mfma(DecodeParams& p, hipStream_t st) {
  if ((p.d != 128 && p.d != 256) || p.key_fmt != KF_FP8 || (p.val_fmt != VF_U4 && p.val_fmt != VF_FP8) ||
      p.g > 8)
    return hipErrorNotSupported;
  // slot bytes below 2 GiB take 32-bit buffer offsets, larger caches the
  // 64-bit variant (whose zero page must cover every kv head's slot)
  const bool wide = p.force_wide ||
      p.num_blocks * (int64_t)p.block_size * p.hk * p.slot_bytes >= ((int64_t)1 << 31);
  if (wide && (int64_t)p.hk * p.slot_bytes > kZeroBytes) return hipErrorNotSupported;
  if ((p.kps + p.vdb) % 4 != 0 || p.kps % 4 != 0 || p.slot_bytes % 16 != 0) return hipErrorNotSupported;
  const int64_t cap = (int64_t)p.max_blocks * p.block_size;
  if (cap >= ((int64_t)1 << 30) || p.B > 4096) return hipErrorNotSupported;
  const int64_t tiles_ub = (int64_t)p.B * ((cap + kTileTokens - 1) / kTileTokens + p.splits);
  if (tiles_ub >= ((int64_t)1 << 30)) return hipErrorNotSupported;
  if (p.d == 256) {
    // D = 256: four query heads per wave (ceil(g / 4) waves per kv head),
    // one wave per SIMD, at most 4 waves per workgroup and per CU
    p.wgh = balance_heads_per_wg(p.hk, p.g, 4);
    const int64_t nw = balance_max_wgs(p.hk, p.g, kWaveBudget / 2);
    p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
    return launch_decode_tq_d256(p, st, wide);
  }
  if (p.g > 4 && kOneWavePerKvHead) {
    // one wave per kv head at one wave per SIMD: at most 4 waves per
    // workgroup and per CU (the piece region, sized for two waves per kv
    // head at 8 per CU, holds the same number of workgroups)
    p.wgh = balance_heads_per_wg(p.hk, 4, 4);
    const int64_t nw = balance_max_wgs(p.hk, 4, kWaveBudget / 2);
    p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
    switch (p.wgh) {
      case 1: return launch<1, 2>(p, st, wide);
      case 2: return launch<2, 2>(p, st, wide);
      default: return launch<4, 2>(p, st, wide);
    }
  }
  const int qs = (p.g + 3) / 4;
  p.wgh = balance_heads_per_wg(p.hk, p.g);
  const int64_t nw = balance_max_wgs(p.hk, p.g);
  p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
  switch (p.wgh * qs) {
    case 1: return launch<1, 1>(p, st, wide);
    case 2: return launch<2, 1>(p, st, wide);
    case 4: return launch<4, 1>(p, st, wide);
    default: return launch<8, 1>(p, st, wide);
  }
}

}  // namespace tqk
