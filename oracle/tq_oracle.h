/*
 * CPU oracle for quantized paged-KV decode attention and its cache writers.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, obviously-correct
 * reimplementation of what the pages compute, used by the tests, by the
 * library smoke check and by the benchmark's CPU-baseline leg. The product
 * path (the HIP library) never links, loads or calls it, and it shares no
 * code, header, table or constant generator with the HIP sources.
 *
 * Sources (web pages of one vLLM fork, cited by page title and section):
 *   [tq]    triton_turboquant_decode.py  -- _tq_decode_stage1, launcher
 *   [int4]  int4_per_token_head.py       -- _reshape_cache_int4_kernel,
 *           _attn_packed, unified_attention_int4, fast_hadamard_transform,
 *           single_rht
 *   [kpool] kpool_compress.py            -- _fwht_quant_kernel,
 *           fwht128_quant_fp8
 *
 * Precision: the write paths use fp32 exactly as the pages fix it (bit-exact
 * contract); attention is evaluated in fp64 over the dequantized cache.
 */
#ifndef TQ_ORACLE_H
#define TQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar converters (round to nearest even) ---- */
uint16_t orc_f32_to_bf16(float x);
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float x);
float orc_f16_to_f32(uint16_t h);
uint8_t orc_f32_to_e4m3(float x);
float orc_e4m3_to_f32(uint8_t b);
void orc_convert(int kind, const void* in, void* out, int64_t n);

/* ---- Walsh-Hadamard ---- */
void orc_fwht_f32(float* x, int d);
void orc_fwht_f64(double* x, int d);

/* ---- INT4 per-(token, head) write path ---- */
void orc_int4_quantize_row(const float* x, int d, uint8_t* packed, float* word);
void orc_int4_dequant_row(const uint8_t* packed, float word, int d, double* out);
int orc_reshape_and_cache_int4(const void* key, const void* value, int kv_dtype,
                               int64_t num_tokens, int hk, int d,
                               const int64_t* slot_mapping, const float* signs,
                               uint8_t* key_cache, uint8_t* value_cache,
                               float* k_scale, float* v_scale,
                               int64_t num_blocks, int block_size);

/* ---- INT4 decode attention (fp64) ---- */
int orc_int4_decode(const float* q, const uint8_t* key_cache,
                    const uint8_t* value_cache, const float* k_scale,
                    const float* v_scale, const int32_t* block_table,
                    int max_blocks, const int32_t* seq_lens,
                    const float* signs, int B, int hq, int hk, int d,
                    int block_size, int num_splits, double sm_scale,
                    const int32_t* rows, int n_rows,
                    double* out, double* lse);

int orc_int4_prefill(const float* q, const uint8_t* key_cache,
                     const uint8_t* value_cache, const float* k_scale,
                     const float* v_scale, const int32_t* block_table,
                     int max_blocks, const int32_t* cu_seqlens_q,
                     const int32_t* seq_lens, int num_seqs, const float* signs,
                     int hq, int hk, int d, int block_size, double sm_scale,
                     int window, double softcap, const float* sinks,
                     double* out);

/* ---- TurboQuant combined-slot formats ---- */
int orc_tq_slot_bytes(int d, int key_fmt, int val_fmt);
void orc_lloyd_max_gaussian(int levels, double* centroids);
int orc_tq_encode(const float* key, const float* value, int64_t num_tokens,
                  int hk, int d, int key_fmt, int val_fmt,
                  const float* centroids, const float* rot_signs,
                  const int64_t* slot_mapping, uint8_t* kv_cache,
                  int64_t num_blocks, int block_size, int slot_bytes);
int orc_tq_decode(const float* q, const uint8_t* kv_cache,
                  const int32_t* block_table, int max_blocks,
                  const int32_t* seq_lens, const float* centroids,
                  const float* rot_signs, int B, int hq, int hk, int d,
                  int block_size, int slot_bytes, int key_fmt, int val_fmt,
                  int norm_correction, int num_splits, double sm_scale,
                  const int32_t* rows, int n_rows, double* out, double* lse);

int orc_tq_full_dequant(const uint8_t* kv_cache, const int32_t* block_table,
                        int max_blocks, const float* centroids, int B, int hk,
                        int d, int block_size, int64_t num_blocks,
                        int slot_bytes, int key_fmt, int val_fmt,
                        int norm_correction, int max_seq, uint16_t* k_out,
                        uint16_t* v_out);

/* ---- Hadamard-128 + power-of-two-scale FP8 ---- */
float orc_fp8_pow2_scale(float absmax);
void orc_fwht128_quant_fp8(const uint16_t* x_bf16, int64_t rows, uint8_t* y,
                           float* scale);

/* ---- pooled-softmax key compression into the FP8 indexer page ---- */
float orc_exp_f32(float x);
int orc_kpool_compress_and_write(const uint16_t* slot_k, const void* slot_score,
                                 int score_dtype, const float* ape,
                                 const int64_t* loc, const uint8_t* write_mask,
                                 int64_t n_pools, int pool_size, int head_dim,
                                 uint8_t* kv_cache, int64_t num_blocks,
                                 int block_size, int round_scale,
                                 uint8_t* compressed_k, float* compressed_scale);

#ifdef __cplusplus
}
#endif
#endif
