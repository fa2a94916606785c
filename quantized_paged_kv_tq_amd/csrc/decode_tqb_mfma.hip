// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores, for
// 3- or 4-bit centroid keys with 3- or 4-bit uniform or FP8 values: the entry
// point and the launches at head dim 128 (the kernel is in
// decode_tqb_kernel.h).
#include "decode_tqb_kernel.h"

namespace tqk {

hipError_t launch_decode_tqb_mfma(DecodeParams& p, hipStream_t st) {
  const bool k4 = p.key_fmt == KF_MSE4, v4 = p.val_fmt == VF_U4, v8 = p.val_fmt == VF_FP8;
  if ((p.d != 128 && p.d != 256) || (p.key_fmt != KF_MSE3 && !k4) ||
      (p.val_fmt != VF_U3 && !v4 && !v8) || p.g > 8)
    return hipErrorNotSupported;
  // FP8 values: head dim 128
  if (v8 && p.d != 128) return hipErrorNotSupported;
  const int kb = k4 ? 4 : 3, vb = v8 ? 8 : (v4 ? 4 : 3);
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
  if (p.norm_correction) {
    // the norm-corrected read on caches of 2 GiB and more: the generic kernel
    if (wide) return hipErrorNotSupported;
    return launch_decode_tqb_ncorr(p, st, tiles_ub);
  }
  if (v8) return launch_decode_tqb_fp8v(p, st, wide, tiles_ub);
  if (p.d == 256) return launch_decode_tqb_d256(p, st, wide, tiles_ub);
  return launch_bits<128, false>(p, st, wide, tiles_ub);
}

}  // namespace tqk
