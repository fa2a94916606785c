// Internal launch interfaces of the prefill-side read paths: the INT4
// multi-query attention (int4_per_token_head.py, _attn_packed in its 2D
// mode) and the bulk TurboQuant dequant (triton_turboquant_decode.py,
// _tq_full_dequant_kv). Arguments arrive validated.
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
// Query tokens [begin, begin + n) as decode entries (matrix-core path): per
// entry the visible key count, the block-table row and the first key.
hipError_t launch_prefill_plan(const PrefillParams& p, int64_t begin, int n, int32_t* lens,
                               int32_t* rows, int32_t* offs, hipStream_t st);

struct DequantParams {
  const uint8_t* kv;          // [num_blocks, bs, hk, slot_bytes]
  const int32_t* block_table; // [B, max_blocks]
  const float* centroids;     // [2^key bits] (centroid keys)
  uint16_t* k_out;            // [B, hk, max_seq, d] fp16
  uint16_t* v_out;
  int64_t num_blocks;
  int B, hk, d, block_size, max_blocks, slot_bytes, key_fmt, val_fmt, norm_correction, max_seq;
  int kps, vdb, mse_bytes;    // key region, value data and index bytes of the slot
};
hipError_t launch_tq_full_dequant(const DequantParams& p, hipStream_t st);

}  // namespace tqk
