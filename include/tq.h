/*
 * tq.h -- C ABI of the MI355X (gfx950) quantized paged-KV decode library.
 *
 * Seven operations, each enqueued on the caller's HIP stream:
 *   tq_reshape_and_cache_int4  randomized Hadamard rotation + INT4 cache write
 *   tq_encode_and_cache        TurboQuant combined-slot cache write (FP8 or
 *                              centroid keys, uniform 3/4-bit values)
 *   tq_decode_attention        split-KV decode attention over a paged,
 *                              sub-byte-quantized cache (stage 1 + stage 2)
 *   fwht128_quant_fp8          Hadamard-128 + power-of-two-scale FP8 quantizer
 *   tq_prefill_attention_int4  multi-query (prefill) attention over the INT4
 *                              cache: causal, sliding window, softcap, sinks,
 *                              fp32 or FP8 output
 *   tq_full_dequant_kv         bulk TurboQuant slot dequant to fp16 K/V rows
 *   tq_kpool_compress_and_write_cache
 *                              pooled-softmax key compression into the FP8
 *                              indexer page
 *
 * Sources (web pages of a vLLM fork, cited by title and section):
 *   int4_per_token_head.py       reshape_and_cache_int4, unified_attention_int4,
 *                                _reshape_cache_int4_kernel, _attn_packed,
 *                                single_rht, fast_hadamard_transform
 *   triton_turboquant_decode.py  triton_turboquant_decode_attention,
 *                                _tq_decode_stage1 (and its stage-2 launch),
 *                                _tq_full_dequant_kv
 *   kpool_compress.py            fwht128_quant_fp8, _fwht_quant_kernel,
 *                                kpool_compress_and_write_cache,
 *                                _kpool_softmax_rotate_write_cache_kernel
 *
 * Conventions for every entry point
 *   - Pointers named "device" are HIP device pointers owned by the caller; the
 *     library never allocates, frees or synchronizes, and keeps no pointer
 *     after the call returns. `stream` is a hipStream_t (NULL: null stream).
 *     (tq_decode_attention_static, the variant for callers that cannot
 *     allocate, takes its workspace from a static device array of the
 *     library instead of the caller's.)
 *   - Tensors are dense and row-major in the shapes given (C order).
 *   - Return value: TQ_OK, or a negative code; nothing is launched unless
 *     TQ_OK is returned (TQ_ELAUNCH: the launch itself failed). The message of
 *     the last failure on the calling thread is tq_last_error().
 *   - Calls that write overlapping outputs race if enqueued on different
 *     streams without ordering; the library adds no ordering of its own.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_OK 0
#define TQ_EINVAL (-1)  /* invalid argument: null pointer, bad size or shape */
#define TQ_ENOTSUP (-2) /* valid but unsupported head size / format / dtype   */
#define TQ_ELAUNCH (-3) /* the HIP launch failed (hipGetLastError)            */

/* source dtypes */
#define TQ_DTYPE_F32 0
#define TQ_DTYPE_F16 1
#define TQ_DTYPE_BF16 2

/* key formats */
#define TQ_KEY_INT4 0 /* separate INT4 caches + scale words (RHT domain)     */
#define TQ_KEY_FP8 1  /* combined slot: D bytes of OCP E4M3FN                */
#define TQ_KEY_MSE3 2 /* combined slot: 3-bit centroid indices + fp16 norm    */
#define TQ_KEY_MSE4 3 /* combined slot: 4-bit centroid indices + fp16 norm    */

/* value formats */
#define TQ_VAL_INT4 0 /* separate INT4 cache + scale words (with TQ_KEY_INT4) */
#define TQ_VAL_U3 1   /* combined slot: 3-bit uniform, fp16 scale and zero    */
#define TQ_VAL_U4 2   /* combined slot: 4-bit uniform, fp16 scale and zero    */
#define TQ_VAL_FP8 3  /* combined slot: D bytes of OCP E4M3FN, no scale/zero */

/* tq_decode_args.flags */
#define TQ_FLAG_GENERIC 1u /* force the format-generic vector kernel         */
#define TQ_FLAG_WIDE 2u    /* force the 64-bit addressing variant of the    */
                           /* matrix-core kernels (taken by itself for     */
                           /* caches of 2 GiB and more); for tests          */

/* Message describing the last failed call on this thread ("" if none). */
const char* tq_last_error(void);

/* Library ABI version (incremented on incompatible changes). */
int tq_version(void);

/*
 * INT4 cache write (int4_per_token_head.py: reshape_and_cache_int4 and
 * _reshape_cache_int4_kernel). For every token t with slot_mapping[t] >= 0,
 * every kv head h, and for K and V independently:
 *   x  = fp32(src[t, h, :]) * rht_signs            (exact sign flips)
 *   x  = FWHT(x) in fp32, butterfly strides 1, 2, ..., D/2 (Sylvester order)
 *   x  = fp32(round_to_src_dtype(x))                (RNE; no-op for fp32)
 *   scale = max(fl((max x - min x) / 15), fl(1e-6))
 *   zp    = clamp(trunc(fl(-min x / scale) +- 0.5), 0, 15)
 *   q_i   = clamp(trunc(fl(fma(x_i, fl(1/scale), zp)) +- 0.5), 0, 15)
 *   cache[slot / bs, slot % bs, h, j] = q[2j] | q[2j+1] << 4
 *   scale_cache[slot / bs, slot % bs, h] = bits(scale) & ~0xF | zp
 * (+-0.5: half away from zero, as the page's where(t >= 0, t + .5, t - .5)).
 * The output bytes are a bit-exact function of the inputs.
 *
 *   key, value       device, [num_tokens, Hk, D] of kv_dtype (TQ_DTYPE_*)
 *   slot_mapping     device, [num_tokens] int64; < 0 skips the token; slots
 *                    >= num_blocks * block_size are skipped as well
 *   rht_signs        device, [D] fp32, each +1 or -1
 *   key_cache, value_cache   device, [num_blocks, block_size, Hk, D/2] u8
 *   k_scale_cache, v_scale_cache device, [num_blocks, block_size, Hk] fp32
 *   D in {64, 128}. num_tokens == 0 returns TQ_OK without launching.
 *   Alignment: key, value, rht_signs 16 B; slot_mapping, key_cache and
 *   value_cache 8 B; the scale caches 4 B (TQ_EINVAL otherwise).
 *   num_tokens * Hk < 2^31.
 *   Slots must be unique (duplicates race: an unspecified writer wins).
 */
int tq_reshape_and_cache_int4(const void* key, const void* value, int32_t kv_dtype,
                              int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, const int64_t* slot_mapping,
                              const float* rht_signs, uint8_t* key_cache,
                              uint8_t* value_cache, float* k_scale_cache,
                              float* v_scale_cache, int64_t num_blocks,
                              int32_t block_size, void* stream);

/*
 * TurboQuant combined-slot cache write: the encoder of the slot formats
 * tq_decode_attention reads (triton_turboquant_decode.py, _tq_decode_stage1
 * reads them; the pages show no writer, so the encoder below is a reading).
 * For every token t with slot_mapping[t] in [0, num_blocks * block_size)
 * and every kv head h, the slot kv_cache[slot / bs, slot % bs, h, :] is
 * rewritten from k = fp32(key[t, h, :]) and v = fp32(value[t, h, :]):
 *   TQ_KEY_FP8   bytes 0..D-1 = e4m3(clamp(k, +-448)) (RNE);
 *   TQ_KEY_MSE3 / MSE4 (b = 3 / 4):
 *     ss   = sum k_i^2 in fp32, added pairwise with strides 1, 2, ..., D/2
 *     norm = sqrt(ss) (correctly rounded)
 *     y    = FWHT(k * rot_signs) in fp32, strides 1 -> D/2 (rot_signs NULL:
 *            all +1); u_i = fl(y_i * fl(r / norm)), r = fl(1 / sqrt(D)),
 *            u = 0 when norm == 0
 *     idx_i = argmin_j |u_i - centroids[j]| (fp32; ties to the lower j),
 *            packed LSB first in ceil(D*b/8) bytes, then fp16(norm);
 *   TQ_VAL_FP8   D value bytes = e4m3(clamp(v, +-448)) (RNE) after the key
 *                region (the value-bits parameter of _tq_decode_stage1 is
 *                documented as 4 or 8 = FP8; the stage decodes only 3 and 4
 *                bits, so this layout is a reading);
 *   values (b = 3 / 4 for TQ_VAL_U3 / U4):
 *     scale = max(fl((max v - min v) / (2^b - 1)), 1e-6), zero = min v (+0
 *     for a zero minimum), both stored fp16 (RNE); idx = clamp(rint(
 *     fl(fl(v - zero16) * fl(1 / scale16))), 0, 2^b - 1), packed LSB first
 *     after the key region, then
 *     fp16 scale and fp16 zero; the remaining bytes of the slot are zeroed.
 * The slot bytes are a bit-exact function of the inputs.
 *
 *   key, value      device, [num_tokens, Hk, D] of kv_dtype (TQ_DTYPE_*)
 *   slot_mapping    device, [num_tokens] int64 (< 0 or out of range: skip)
 *   centroids       device, [2^b] fp32 (centroid keys; NULL for FP8 keys)
 *   rot_signs       device, [D] fp32 +-1, or NULL (centroid keys)
 *   kv_cache        device, [num_blocks, block_size, Hk, slot_bytes] u8,
 *                   slot_bytes >= tq_slot_bytes(D, key_fmt, val_fmt), a
 *                   multiple of 16
 *   D in {64, 128, 256}. num_tokens == 0 returns TQ_OK without launching.
 *   Alignment: key, value, rot_signs, kv_cache 16 B; slot_mapping 8 B;
 *   centroids 4 B. num_tokens * Hk < 2^31. Slots must be unique.
 */
int tq_encode_and_cache(const void* key, const void* value, int32_t kv_dtype,
                        int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t key_fmt, int32_t val_fmt, const int64_t* slot_mapping,
                        const float* centroids, const float* rot_signs, uint8_t* kv_cache,
                        int32_t slot_bytes, int64_t num_blocks, int32_t block_size,
                        void* stream);

/*
 * Decode attention, one query token per sequence.
 *
 * Stage 1 (triton_turboquant_decode.py, _tq_decode_stage1): sequence b is
 * cut into num_kv_splits ranges of split_len = ceil(seq_len / S) tokens;
 * for every non-empty split s and query head h (kv head h / (Hq / Hk)) it
 * writes  workspace[b, h, s, 0:D] = sum_t p_t v_t / l  and
 * workspace[b, h, s, D] = m + ln l  (online softmax, natural exp).
 * Stage 2 (the merge the pages launch as _fwd_kernel_stage2): log-sum-exp
 * merge of the non-empty splits into out[b, h, :] and lse[b, h].
 *
 * Token t of sequence b lives at page block_table[b, t / bs], row t % bs.
 * Key / value decoding and scoring per format:
 *   TQ_KEY_INT4 + TQ_VAL_INT4 (int4_per_token_head.py, unified_attention_int4
 *     and _attn_packed): q' = FWHT(rht_signs * q); score = sm_scale / D *
 *     q' . ((n - zp) * scale'), scale' = word & ~0xF, zp = word & 0xF;
 *     values likewise; out = rht_signs * FWHT(o') / D.
 *   TQ_KEY_FP8: score = sm_scale * q . e4m3(k).
 *   TQ_KEY_MSE3 / MSE4: q_rot = FWHT(rot_signs * q) / sqrt(D) (rot_signs may
 *     be NULL: all +1); score = sm_scale * norm16 * (q_rot . c[idx]), with
 *     c / sqrt(sum c^2 + 1e-16) when norm_correction != 0.
 *   TQ_VAL_U3 / U4: v = idx * scale16 + zero16.
 *   TQ_VAL_FP8: v = e4m3(byte).
 * Combined slot layout (TQ formats): key region (FP8: D bytes; centroid:
 * ceil(D*b/8) bytes of LSB-first b-bit indices then the fp16 norm), value
 * data (U3 / U4: ceil(D*vb/8) bytes of LSB-first indices, then fp16 scale
 * and fp16 zero; FP8: D codes), padding to
 * slot_bytes = tq_slot_bytes(D, key_fmt, val_fmt).
 *
 * Block-table entries outside [0, num_blocks) are never dereferenced (the
 * result for that sequence is then unspecified); seq_len is clamped to
 * max_blocks * block_size; seq_len == 0 gives out = 0 and lse = -inf.
 * Supported: D in {64, 128} (and 256 for the TQ formats); Hq % Hk == 0 and
 * Hq / Hk <= 64;
 * 1 <= num_kv_splits <= 256; block_size >= 1.
 */
typedef struct tq_decode_args {
  uint32_t struct_size; /* sizeof(tq_decode_args)                         */
  uint32_t flags;       /* TQ_FLAG_*                                       */
  int32_t B, Hq, Hk, D;
  int32_t block_size;
  int32_t max_blocks;    /* columns of block_table                        */
  int32_t num_kv_splits; /* S                                             */
  int32_t key_fmt, val_fmt;
  int32_t norm_correction;
  float sm_scale;        /* softmax scale, e.g. 1/sqrt(D)                 */
  int64_t num_blocks;    /* pages in the cache(s)                          */
  const float* query;          /* device [B, Hq, D] fp32                   */
  const int32_t* block_table;  /* device [B, max_blocks] int32             */
  const int32_t* seq_lens;     /* device [B] int32                         */
  /* INT4 format */
  const uint8_t* key_cache;    /* device [num_blocks, bs, Hk, D/2] u8      */
  const uint8_t* value_cache;  /* device [num_blocks, bs, Hk, D/2] u8      */
  const float* k_scale_cache;  /* device [num_blocks, bs, Hk] scale words  */
  const float* v_scale_cache;  /* device [num_blocks, bs, Hk] scale words  */
  const float* rht_signs;      /* device [D] +-1                            */
  /* TurboQuant combined-slot formats */
  const uint8_t* kv_cache;     /* device [num_blocks, bs, Hk, slot_bytes] u8 */
  int32_t slot_bytes;
  const float* centroids;      /* device [2^b] fp32 (centroid keys)        */
  const float* rot_signs;      /* device [D] +-1 or NULL (centroid keys)   */
  /* outputs */
  float* workspace; /* device scratch of the stage-1 partials, at least
                       tq_decode_workspace_bytes(B, Hq, Hk, D, S) bytes;
                       its contents on entry do not matter              */
  int64_t workspace_bytes; /* size of `workspace` in bytes (validated)   */
  float* out;       /* device [B, Hq, D] fp32                               */
  float* lse;       /* device [B, Hq] fp32, or NULL                         */
} tq_decode_args;

/*
 * Bytes of the stage-1 workspace: the per-split partials [B, Hq, S, D+1]
 * fp32 (triton_turboquant_decode.py: the stage-1 output buffer), followed by
 * the piece slots of the balanced INT4 decode, which spreads the tiles of all
 * splits evenly over the workgroups and writes a split cut between two
 * workgroups as pieces that stage 2 merges like splits (2 * nw * Hq * (D+1)
 * fp32, nw = max(1, 2048 / (Hk * ceil(Hq / Hk / 4)))). Returns 0 for invalid
 * sizes.
 */
size_t tq_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hk, int32_t D,
                                 int32_t num_kv_splits);

/*
 * Padded combined-slot size for a TurboQuant format, or -1 if invalid.
 * triton_turboquant_decode.py passes the slot width (padded_slot) and the key
 * region size (key_packed_size) in from outside: _get_layout derives only
 * the index bytes (mse_bytes = ceil(D * bits / 8), val_data_bytes), and
 * _tq_decode_stage1 reads the fp16 norm right after the key indices and the
 * fp16 scale and zero right after the value indices. The reading taken:
 * key region = D bytes (FP8 keys) or mse_bytes + 2 (centroid keys); value
 * region = val_data_bytes, + 4 for uniform values; the slot is that sum
 * rounded up to a multiple of 16 bytes.
 */
int32_t tq_slot_bytes(int32_t D, int32_t key_fmt, int32_t val_fmt);

int tq_decode_attention(const tq_decode_args* args, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as tq_decode_attention, with the stage-1 workspace taken from a
 * static device array of TQ_STATIC_WORKSPACE_BYTES inside the library
 * instead of args->workspace (args->workspace and args->workspace_bytes are
 * ignored). Each GPU that runs it holds its own copy of the array until the
 * process ends; the array's device address is looked up on the first call
 * on each device. The call allocates nothing and frees nothing.
 *   Limit: tq_decode_workspace_bytes(B, Hq, Hk, D, S) must not exceed
 *   TQ_STATIC_WORKSPACE_BYTES, else TQ_EINVAL, nothing launched, and
 *   tq_last_error() names the sizes.
 *   Contents: nothing in the array needs to start at zero (stage 1 writes
 *   every value stage 2 reads); it keeps the last call's partials.
 *   Concurrency: every call on one GPU shares that GPU's array, so calls
 *   that overlap on one GPU (several streams, or several threads) race;
 *   order them on one stream.
 * Other arguments, validation, errors and results are those of
 * tq_decode_attention.
 */
#define TQ_STATIC_WORKSPACE_BYTES ((size_t)64 << 20) /* 64 MiB per GPU */
int tq_decode_attention_static(const tq_decode_args* args, void* stream);

/*
 * Hadamard-128 + power-of-two-scale FP8 (kpool_compress.py,
 * fwht128_quant_fp8 and _fwht_quant_kernel). Per row of 128 bf16 values:
 *   x = FWHT(fp32(row)) in fp32 (strides 1..64); x = fp32(bf16(x * fl(1/sqrt 128)))
 *   scale = 2^ceil(log2(fl(max(max|x|, 1e-4) * fl(1/448))))   (exact ceiling)
 *   y = e4m3_rne(clamp(x / scale, -448, 448))    (OCP E4M3FN)
 * Bit-exact function of the input.
 *   x_bf16 device [rows, 128] bf16; y_e4m3 device [rows, 128] u8;
 *   scale device [rows] fp32. rows == 0 returns TQ_OK without launching.
 *   Alignment: x_bf16 and y_e4m3 16 B, scale 4 B (TQ_EINVAL otherwise).
 */
int fwht128_quant_fp8(const void* x_bf16, int64_t rows, uint8_t* y_e4m3,
                      float* scale, void* stream);

/*
 * Multi-query (prefill) attention over the INT4 caches (int4_per_token_head.py,
 * _attn_packed in its 2D mode as unified_attention_int4 wraps it). The query
 * tokens of num_seqs sequences are packed: sequence b owns tokens
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and has seq_lens[b] keys in the cache
 * (context + its queries, clamped to max_blocks * block_size). Query i of
 * sequence b sits at pos = seq_lens[b] - query_len + i and sees keys t with
 * t <= pos and, when window > 0, pos - t < window (window = 1 +
 * window_size[0]; 0 means none). With q' = RHT(q) = FWHT(s * q):
 *   score_t = (sm_scale / D) * q'.k'_t      (k' the dequantized rotated key)
 *   score_t <- softcap * tanh(score_t / softcap)   when softcap > 0
 *   o' = sum_t e^{score_t} v'_t / (e^{sinks[h]} + sum_t e^{score_t})
 *        (the sink term only when sinks != NULL)
 *   out = s * FWHT(o') / D;  out = e4m3_rne(clamp(out * fl(1/output_scale[0]),
 *        -448, 448)) when output_scale != NULL.
 * A query with no visible key gets out = 0. GQA: kv head = h / (Hq / Hk).
 *   query         device [num_tokens, Hq, D] f32
 *   cu_seqlens_q  device [num_seqs + 1] int32, non-decreasing, last = num_tokens
 *   seq_lens      device [num_seqs] int32
 *   block_table   device [num_seqs, max_blocks] int32; entries outside
 *                 [0, num_blocks) read as masked tokens
 *   caches        as tq_reshape_and_cache_int4 writes them
 *   rht_signs     device [D] +-1 f32
 *   sinks         device [Hq] f32 or NULL; output_scale device [1] f32 or NULL
 *   out           device [num_tokens, Hq, D]: f32, or u8 E4M3 codes when
 *                 output_scale is set
 * D = 64 or 128 (TQ_ENOTSUP otherwise). num_tokens == 0 returns TQ_OK
 * without launching.
 *
 * Paths. With a workspace of at least tq_prefill_workspace_bytes(...) bytes
 * (16-byte aligned, as are query, f32 out and both caches), D = 128 and
 * Hq / Hk <= 32, the
 * call runs on the matrix cores: each query token becomes one entry of the
 * split-KV INT4 decode (its visible keys [t0, t1) read from its sequence's
 * block-table row), in chunks of at most 4096 tokens that reuse the
 * workspace in stream order. Otherwise (no workspace, or a shape the
 * matrix-core decode does not take) a vector-ALU kernel computes the same
 * result. The workspace is scratch owned by the caller; calls that share
 * one must not overlap. Callers built against the layout without the
 * workspace fields pass struct_size = offsetof(tq_prefill_args, workspace)
 * and get the vector path.
 */
typedef struct {
  uint32_t struct_size; /* sizeof(tq_prefill_args) */
  int32_t num_seqs, Hq, Hk, D, block_size, max_blocks;
  int32_t window;       /* 1 + window_size[0]; 0: no window */
  int64_t num_tokens, num_blocks;
  float sm_scale;
  float softcap;        /* 0: none */
  const float* query;
  const int32_t* cu_seqlens_q;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const float* k_scale_cache;
  const float* v_scale_cache;
  const float* rht_signs;
  const float* sinks;
  const float* output_scale;
  void* out;
  void* workspace;          /* device scratch, or NULL (vector path) */
  int64_t workspace_bytes;
} tq_prefill_args;

int tq_prefill_attention_int4(const tq_prefill_args* args, void* stream);

/*
 * Workspace bytes that put tq_prefill_attention_int4 on the matrix cores
 * for num_tokens query tokens (0 when that path does not apply: D != 128,
 * Hq / Hk > 32, or no tokens): three int32 per token of a chunk of up to 4096
 * tokens, then the split-KV decode workspace of one chunk
 * (tq_decode_workspace_bytes with one split).
 */
size_t tq_prefill_workspace_bytes(int64_t num_tokens, int32_t Hq, int32_t Hk, int32_t D);

/*
 * Bulk dequantization of the TurboQuant combined-slot cache to fp16 rows
 * (triton_turboquant_decode.py, _tq_full_dequant_kv). For every b < B, kv
 * head h and position pos < max_seq, the slot at page block_table[b, pos /
 * block_size], row pos % block_size, head h becomes
 *   k_out[b, h, pos, :]  FP8 keys: fp16(e4m3); centroid keys:
 *                        fp16(fl32(norm16 * c[idx])), c[idx] first scaled by
 *                        1/sqrt(sum_d c^2 + 1e-16) when norm_correction
 *   v_out[b, h, pos, :]  3/4-bit values: fp16(fmaf(idx, scale16, zero16));
 *                        FP8 values: 0 (the page's kernel writes zeros for
 *                        value widths other than 3 and 4)
 * (fp16 rounding to nearest even). No sequence lengths are taken: positions
 * past a sequence read whatever page the table names; a page outside
 * [0, num_blocks) gives zero rows.
 *   kv_cache     device [num_blocks, block_size, Hk, slot_bytes] u8, 16-B aligned;
 *                slot_bytes >= tq_slot_bytes(D, key_fmt, val_fmt), a multiple of 16
 *   block_table  device [B, max_blocks] int32; max_seq <= max_blocks * block_size
 *   centroids    device [2^bits] f32 (centroid keys; else ignored)
 *   k_out, v_out device [B, Hk, max_seq, D] fp16, 16-B aligned
 * D = 64, 128 or 256. B * Hk * max_seq == 0 returns TQ_OK without launching.
 */
int tq_full_dequant_kv(const uint8_t* kv_cache, const int32_t* block_table, int32_t max_blocks,
                       const float* centroids, int32_t B, int32_t Hk, int32_t D,
                       int32_t block_size, int64_t num_blocks, int32_t slot_bytes,
                       int32_t key_fmt, int32_t val_fmt, int32_t norm_correction,
                       int32_t max_seq, void* k_out, void* v_out, void* stream);

/*
 * Pooled-softmax key compression into the FP8 indexer page (kpool_compress.py,
 * kpool_compress_and_write_cache and _kpool_softmax_rotate_write_cache_kernel).
 * One entry per pool of pool_size tokens (P). Per pool i and dimension d:
 *   v[s] = score[i,s,d] + ape[s,d]           (fp32; s = 0 .. P-1)
 *   m = max_s v[s]; p[s] = e^(v[s] - m)     (e^x rounded to nearest fp32)
 *   den = sum_s p[s]; acc = sum_s k[i,s,d] * p[s]   (fp32, slot order, the
 *                                           product-sum one fused multiply-add)
 *   x[d] = fp32(bf16(acc / den))
 * then x = fp32(bf16(FWHT(x) * fl(1/sqrt 128))) as in fwht128_quant_fp8,
 *   absmax = max(max|x|, 1e-4); scale = 2^ceil(log2(fl(absmax * fl(1/448))))
 *   when round_scale, else fl(absmax * fl(1/448));
 *   codes = e4m3_rne(clamp(x / scale, -448, 448)).
 * Bit-exact function of the inputs.
 *   slot_k      device [n_pools, pool_size, head_dim] bf16, 16-B aligned
 *   slot_score  device [n_pools, pool_size, head_dim] in score_dtype
 *               (TQ_DTYPE_F32 / F16 / BF16), 16-B aligned
 *   ape         device [pool_size, head_dim] f32 position bias, 16-B aligned
 *   loc         device [n_pools] int64 flat entry index (page = loc /
 *               block_size, row = loc % block_size); needed with kv_cache.
 *               Entries outside [0, num_blocks * block_size) are not written.
 *   write_mask  device [n_pools] u8 (0: the pool writes nothing), or NULL
 *   head_dim    must be 128 (TQ_ENOTSUP otherwise)
 *   kv_cache    device [num_blocks, block_size, head_dim + 4] u8, or NULL: a
 *               page holds the block_size entries' codes first (128 B each,
 *               row order), then their fp32 scales at byte block_size * 128
 *   round_scale nonzero: power-of-two scales
 *   compressed_k, compressed_scale
 *               device [n_pools, head_dim] E4M3 (8-B aligned) and [n_pools]
 *               f32, both or neither; every pool's entry is returned there
 *               (not allowed together with write_mask)
 * At least one of kv_cache and compressed_k is required. n_pools == 0
 * returns TQ_OK without launching. Pools with equal loc race.
 */
int tq_kpool_compress_and_write_cache(const void* slot_k, const void* slot_score,
                                      int32_t score_dtype, const float* ape, const int64_t* loc,
                                      const uint8_t* write_mask, int64_t n_pools,
                                      int32_t pool_size, int32_t head_dim, uint8_t* kv_cache,
                                      int64_t num_blocks, int32_t block_size,
                                      int32_t round_scale, uint8_t* compressed_k,
                                      float* compressed_scale, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
