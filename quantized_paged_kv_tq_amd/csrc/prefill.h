// Internal launch interface of the INT4 multi-query (prefill) attention
// (int4_per_token_head.py, _attn_packed in its 2D mode). Arguments arrive
// validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqk {

struct PrefillParams {
  const float* q;             // [T, hq, d]
  const int32_t* cu_seqlens;  // [num_seqs + 1]
  const int32_t* seq_lens;    // [num_seqs]
  const int32_t* block_table; // [num_seqs, max_blocks]
  const uint8_t* kc;          // [num_blocks, bs, hk, d/2]
  const uint8_t* vc;
  const float* ks;            // [num_blocks, bs, hk] scale words
  const float* vs;
  const float* rht_signs;     // [d]
  const float* sinks;         // [hq] or null
  const float* output_scale;  // [1] or null (fp32 output)
  float* out;                 // [T, hq, d] fp32 (output_scale null)
  uint8_t* out_fp8;           // [T, hq, d] E4M3 (output_scale set)
  int64_t num_tokens, num_blocks;
  int num_seqs, hq, hk, d, g, block_size, max_blocks, window;
  float sm_scale, softcap;
};
hipError_t launch_prefill_int4(const PrefillParams& p, hipStream_t st);

}  // namespace tqk
