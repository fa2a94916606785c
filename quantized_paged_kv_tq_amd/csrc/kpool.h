// Internal launch interface of the pooled-key compressor (kpool_compress.py,
// _kpool_softmax_rotate_write_cache_kernel). Arguments arrive validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqk {

struct KpoolParams {
  const uint16_t* slot_k;   // [n, P, 128] bf16
  const void* slot_score;   // [n, P, 128] in score_dtype (TQ_DT_*)
  const float* ape;         // [P, 128]
  const int64_t* loc;       // [n] flat entry index (with cache)
  const uint8_t* mask;      // [n] or null
  uint8_t* cache;           // [num_blocks, block_size, 132] or null
  uint8_t* ck;              // [n, 128] E4M3 or null
  float* cs;                // [n] or null (with ck)
  int64_t n_pools, num_blocks;
  int pool_size, block_size, score_dtype, round_scale;
};
hipError_t launch_kpool_compress(const KpoolParams& p, hipStream_t st);

}  // namespace tqk
