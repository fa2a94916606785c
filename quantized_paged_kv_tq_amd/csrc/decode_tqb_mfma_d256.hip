// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores: the
// centroid-key kernel's launches at head dim 256 (decode_tqb_kernel.h).
#include "decode_tqb_kernel.h"

namespace tqk {

namespace {

template <int KB, int VB>
hipError_t launch_d256(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  // four query heads per wave (ceil(g / 4) waves per kv head), one wave per
  // SIMD, at most 4 waves per workgroup and per CU
  p.wgh = balance_heads_per_wg(p.hk, p.g, 4);
  const int64_t nw = balance_max_wgs(p.hk, p.g, kWaveBudget / 2);
  p.nw = (int)(tiles_ub < nw ? tiles_ub : nw);
  switch (p.wgh * ((p.g + 3) / 4)) {
    case 1: return launch<1, 1, KB, VB, 256>(p, st, wide);
    case 2: return launch<2, 1, KB, VB, 256>(p, st, wide);
    default: return launch<4, 1, KB, VB, 256>(p, st, wide);
  }
}

}  // namespace

hipError_t launch_decode_tqb_d256(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  const bool k4 = p.key_fmt == KF_MSE4, v4 = p.val_fmt == VF_U4;
  if (k4) return v4 ? launch_d256<4, 4>(p, st, wide, tiles_ub) : launch_d256<4, 3>(p, st, wide, tiles_ub);
  return v4 ? launch_d256<3, 4>(p, st, wide, tiles_ub) : launch_d256<3, 3>(p, st, wide, tiles_ub);
}

}  // namespace tqk
