// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores: the
// centroid-key kernel's launches for FP8 E4M3 values (head dim 128;
// decode_tqb_kernel.h). The values become exact bf16 operands and the
// softmax weights three bf16 parts, summed in fp32 by the bf16 MFMA, as in
// the FP8-key kernel.
#include "decode_tqb_kernel.h"

namespace tqk {

hipError_t launch_decode_tqb_fp8v(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  if (p.key_fmt == KF_MSE4) return launch_layout<4, 8, 128, false>(p, st, wide, tiles_ub);
  return launch_layout<3, 8, 128, false>(p, st, wide, tiles_ub);
}

}  // namespace tqk
