// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores: the
// centroid-key kernel's launches for the norm-corrected read
// (triton_turboquant_decode.py, _tq_decode_stage1 with NORM_CORRECTION: the
// centroid vector scaled to unit length), at head dims 128 and 256, narrow
// addressing, with 3/4-bit or FP8 values (decode_tqb_kernel.h).
#include "decode_tqb_kernel.h"

namespace tqk {

hipError_t launch_decode_tqb_ncorr(DecodeParams& p, hipStream_t st, int64_t tiles_ub) {
  if (p.val_fmt == VF_FP8) {  // FP8 values (head dim 128)
    if (p.key_fmt == KF_MSE4) return launch_layout<4, 8, 128, true>(p, st, false, tiles_ub);
    return launch_layout<3, 8, 128, true>(p, st, false, tiles_ub);
  }
  if (p.d == 256) return launch_bits<256, true>(p, st, false, tiles_ub);
  return launch_bits<128, true>(p, st, false, tiles_ub);
}

}  // namespace tqk
