// Internal launch interface between the C ABI layer (api.hip) and the
// kernel translation units. Arguments arrive here already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define TQ_DT_F32 0
#define TQ_DT_F16 1
#define TQ_DT_BF16 2

namespace tqk {

struct ReshapeParams {
  const void* key;
  const void* value;
  const int64_t* slots;
  const float* signs;
  uint8_t* kc;
  uint8_t* vc;
  float* ks;
  float* vs;
  int64_t num_tokens;
  int64_t num_blocks;
  int hk, d, dtype, block_size;
};
hipError_t launch_reshape_int4(const ReshapeParams& p, hipStream_t st);

hipError_t launch_fwht128_fp8(const void* x, int64_t rows, uint8_t* y, float* scale,
                              hipStream_t st);

// Key/value formats (same numbering as the public header).
enum { KF_INT4 = 0, KF_FP8 = 1, KF_MSE3 = 2, KF_MSE4 = 3 };
enum { VF_INT4 = 0, VF_U3 = 1, VF_U4 = 2, VF_FP8 = 3 };

struct TqWriteParams {
  const void* key;
  const void* value;
  const int64_t* slots;
  const float* centroids;
  const float* rot_signs;
  uint8_t* cache;
  int64_t num_tokens, num_blocks;
  int hk, d, dtype, block_size, slot_bytes;
  int key_fmt, val_fmt, kps, vdb;
};
hipError_t launch_write_tq(const TqWriteParams& p, hipStream_t st);

struct DecodeParams {
  int B, hq, hk, d, g, block_size, max_blocks, splits;
  int key_fmt, val_fmt, norm_correction;
  float sm_scale;
  int64_t num_blocks;
  const float* q;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* kc;
  const uint8_t* vc;
  const float* ks;
  const float* vs;
  const float* rht_signs;
  const uint8_t* kv;
  int slot_bytes;
  int kps;       // key region bytes of a combined slot
  int vdb;       // value index bytes of a combined slot
  const float* centroids;
  const float* rot_signs;
  float* ws;     // [B, Hq, S, D+1]
  float* out;    // [B, Hq, D]
  float* lse;    // [B, Hq] or null
  // Balanced partition of the INT4 decode (balance.h), set by its launcher:
  // nw workgroups per group of wgh kv heads; 0 = one partial per split only.
  int nw, wgh;
  int force_wide;  // take the 64-bit addressing variant whatever the cache size
  float* wsp;    // piece slots [Hk / wgh][nw][2][wgh * g][D+1], after ws
  int* wsx;      // [B + 1] tile-list prefix sums (stage 1 writes, stage 2 reads)
  // Multi-query use (prefill as one decode entry per query token; INT4
  // matrix-core stage 1 and stage 2 only). Entry b reads the block table
  // row bt_row[b] from token tok_off[b] on (null: row b, from token 0).
  const int32_t* bt_row = nullptr;
  const int32_t* tok_off = nullptr;
  float softcap = 0.0f;            // > 0: score <- softcap * tanh(score / softcap)
  const float* sinks = nullptr;    // [Hq]: e^sink joins each softmax denominator
  const float* output_scale = nullptr;  // [1]: stage 2 writes E4M3 codes to out_fp8
  uint8_t* out_fp8 = nullptr;      // [B, Hq, D]
};

// Format-generic vector stage 1 (every key/value format).
hipError_t launch_decode_generic(const DecodeParams& p, hipStream_t st);
// INT4 stage 1 on the matrix cores; returns hipErrorNotSupported when the
// shape is outside what it handles (the caller then uses the generic one).
// Sets p.nw / p.wgh for stage 2.
hipError_t launch_decode_int4_mfma(DecodeParams& p, hipStream_t st);
// FP8-key / 4-bit-value TurboQuant stage 1 on the matrix cores (D = 128,
// g <= 8); hipErrorNotSupported otherwise. Sets p.nw / p.wgh for stage 2.
hipError_t launch_decode_tq_mfma(DecodeParams& p, hipStream_t st);
// 3-bit centroid-key / 3-bit-value TurboQuant stage 1 on the matrix cores
// (D = 128, g <= 8, no norm correction); hipErrorNotSupported otherwise.
// Sets p.nw / p.wgh for stage 2.
hipError_t launch_decode_tqb_mfma(DecodeParams& p, hipStream_t st);
// Stage 2: log-sum-exp merge of the split partials (+ inverse RHT for INT4).
hipError_t launch_merge(const DecodeParams& p, hipStream_t st);

}  // namespace tqk
