// TurboQuant split-KV decode, stage 1, on the CDNA4 matrix cores: the
// centroid-key kernel's launches at head dim 256 (decode_tqb_kernel.h).
#include "decode_tqb_kernel.h"

namespace tqk {

hipError_t launch_decode_tqb_d256(DecodeParams& p, hipStream_t st, bool wide, int64_t tiles_ub) {
  return launch_bits<256, false>(p, st, wide, tiles_ub);
}

}  // namespace tqk
