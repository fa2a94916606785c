// C ABI of the library (include/tq.h): argument validation, format tables
// and dispatch to the kernel launchers. Host code only.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "tq.h"
#include "balance.h"
#include "tq_internal.h"
#include "kpool.h"
#include "merge_one.h"
#include "prefill.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int launched(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  return fail(TQ_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int key_bits(int key_fmt) { return key_fmt == TQ_KEY_MSE3 ? 3 : (key_fmt == TQ_KEY_MSE4 ? 4 : 8); }
int val_bits(int val_fmt) { return val_fmt == TQ_VAL_U3 ? 3 : (val_fmt == TQ_VAL_U4 ? 4 : 8); }

// Combined TurboQuant slot: key region, value data (indices or E4M3 codes),
// then fp16 scale and fp16 zero for uniform values.
int key_region_bytes(int d, int key_fmt) {
  if (key_fmt == TQ_KEY_FP8) return d;
  return (d * key_bits(key_fmt) + 7) / 8 + 2;
}
int value_index_bytes(int d, int val_fmt) { return (d * val_bits(val_fmt) + 7) / 8; }

// The matrix-core prefill runs query tokens as decode entries, at most the
// decode's per-call entry count at a time; its plan (three int32 per entry)
// heads the workspace.
constexpr int64_t kPrefillChunk = 4096;
size_t prefill_plan_bytes(int64_t chunk) { return ((size_t)chunk * 3 * sizeof(int32_t) + 255) / 256 * 256; }
int prefill_on_matrix_cores(const tqk::PrefillParams& pp, void* ws, hipStream_t st);

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_err; }

int tq_version(void) { return 2; }

int32_t tq_slot_bytes(int32_t D, int32_t key_fmt, int32_t val_fmt) {
  if (D <= 0 || D > 1024 || (D & (D - 1)) != 0) return -1;
  if (key_fmt < TQ_KEY_FP8 || key_fmt > TQ_KEY_MSE4) return -1;
  if (val_fmt != TQ_VAL_U3 && val_fmt != TQ_VAL_U4 && val_fmt != TQ_VAL_FP8) return -1;
  const int raw = key_region_bytes(D, key_fmt) + value_index_bytes(D, val_fmt) + (val_fmt == TQ_VAL_FP8 ? 0 : 4);
  return (raw + 15) / 16 * 16;
}

size_t tq_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hk, int32_t D, int32_t S) {
  if (B < 0 || Hq < 0 || Hk <= 0 || D < 0 || S < 0) return 0;
  // per-split partials, then the piece slots of the balanced INT4 decode:
  // [Hk / wgh][nw][2][wgh * g][D + 1] = 2 * nw * Hq * (D + 1) floats
  const size_t parts = (size_t)B * Hq * S * (D + 1);
  const int g = Hk > 0 && Hq % Hk == 0 ? Hq / Hk : 1;
  const size_t pieces = (size_t)2 * tqk::balance_max_wgs(Hk, g) * Hq * (D + 1);
  const size_t prefix = ((size_t)B + 1 + 3) / 4 * 4;  // tile-list prefix sums (int32)
  return (parts + pieces + prefix) * sizeof(float);
}

int tq_reshape_and_cache_int4(const void* key, const void* value, int32_t kv_dtype,
                              int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              const int64_t* slot_mapping, const float* rht_signs,
                              uint8_t* key_cache, uint8_t* value_cache, float* k_scale_cache,
                              float* v_scale_cache, int64_t num_blocks, int32_t block_size,
                              void* stream) {
  if (num_tokens < 0) return fail(TQ_EINVAL, "num_tokens < 0");
  if (num_kv_heads <= 0) return fail(TQ_EINVAL, "num_kv_heads must be positive");
  if (head_dim <= 0 || head_dim % 2 != 0 || (head_dim & (head_dim - 1)) != 0)
    return fail(TQ_EINVAL, "head_dim must be an even power of two (got %d)", head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(TQ_ENOTSUP, "head_dim %d not supported (64, 128)", head_dim);
  if (kv_dtype != TQ_DTYPE_F32 && kv_dtype != TQ_DTYPE_F16 && kv_dtype != TQ_DTYPE_BF16)
    return fail(TQ_ENOTSUP, "kv_dtype %d not supported", kv_dtype);
  if (block_size <= 0 || num_blocks < 0) return fail(TQ_EINVAL, "bad block_size / num_blocks");
  if (num_tokens == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  if (!key || !value || !slot_mapping || !rht_signs || !key_cache || !value_cache ||
      !k_scale_cache || !v_scale_cache)
    return fail(TQ_EINVAL, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(rht_signs, 16) ||
      !aligned(slot_mapping, 8) || !aligned(key_cache, 8) || !aligned(value_cache, 8) ||
      !aligned(k_scale_cache, 4) || !aligned(v_scale_cache, 4))
    return fail(TQ_EINVAL,
                "misaligned pointer (key/value/signs 16 B, slots and caches 8 B, scale caches 4 B)");
  if (num_tokens * num_kv_heads >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "num_tokens * num_kv_heads must be below 2^31");
  tqk::ReshapeParams p{key, value, slot_mapping, rht_signs, key_cache, value_cache,
                       k_scale_cache, v_scale_cache, num_tokens, num_blocks, num_kv_heads,
                       head_dim, kv_dtype, block_size};
  return launched(tqk::launch_reshape_int4(p, static_cast<hipStream_t>(stream)),
                  "tq_reshape_and_cache_int4");
}

int tq_encode_and_cache(const void* key, const void* value, int32_t kv_dtype,
                        int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t key_fmt, int32_t val_fmt, const int64_t* slot_mapping,
                        const float* centroids, const float* rot_signs, uint8_t* kv_cache,
                        int32_t slot_bytes, int64_t num_blocks, int32_t block_size,
                        void* stream) {
  if (num_tokens < 0) return fail(TQ_EINVAL, "num_tokens < 0");
  if (num_kv_heads <= 0) return fail(TQ_EINVAL, "num_kv_heads must be positive");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(TQ_ENOTSUP, "head_dim %d not supported (64, 128, 256)", head_dim);
  if (kv_dtype != TQ_DTYPE_F32 && kv_dtype != TQ_DTYPE_F16 && kv_dtype != TQ_DTYPE_BF16)
    return fail(TQ_ENOTSUP, "kv_dtype %d not supported", kv_dtype);
  const int sb = tq_slot_bytes(head_dim, key_fmt, val_fmt);
  if (sb < 0) return fail(TQ_EINVAL, "invalid key_fmt %d / val_fmt %d", key_fmt, val_fmt);
  if (slot_bytes < sb || slot_bytes % 16 != 0)
    return fail(TQ_EINVAL, "slot_bytes %d: need a multiple of 16 >= %d", slot_bytes, sb);
  if (block_size <= 0 || num_blocks < 0) return fail(TQ_EINVAL, "bad block_size / num_blocks");
  if (num_tokens == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  const bool centroid = key_fmt == TQ_KEY_MSE3 || key_fmt == TQ_KEY_MSE4;
  if (!key || !value || !slot_mapping || !kv_cache || (centroid && !centroids))
    return fail(TQ_EINVAL, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(kv_cache, 16) ||
      !aligned(slot_mapping, 8) || (rot_signs && !aligned(rot_signs, 16)) ||
      (centroids && !aligned(centroids, 4)))
    return fail(TQ_EINVAL,
                "misaligned pointer (key/value/kv_cache/rot_signs 16 B, slots 8 B, centroids 4 B)");
  if (num_tokens * num_kv_heads >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "num_tokens * num_kv_heads must be below 2^31");
  tqk::TqWriteParams p;
  p.key = key;
  p.value = value;
  p.slots = slot_mapping;
  p.centroids = centroids;
  p.rot_signs = centroid ? rot_signs : nullptr;
  p.cache = kv_cache;
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.hk = num_kv_heads;
  p.d = head_dim;
  p.dtype = kv_dtype;
  p.block_size = block_size;
  p.slot_bytes = slot_bytes;
  p.key_fmt = key_fmt;
  p.val_fmt = val_fmt;
  p.kps = key_region_bytes(head_dim, key_fmt);
  p.vdb = value_index_bytes(head_dim, val_fmt);
  return launched(tqk::launch_write_tq(p, static_cast<hipStream_t>(stream)), "tq_encode_and_cache");
}

int fwht128_quant_fp8(const void* x_bf16, int64_t rows, uint8_t* y_e4m3, float* scale,
                      void* stream) {
  if (rows < 0) return fail(TQ_EINVAL, "rows < 0");
  if (rows == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  if (!x_bf16 || !y_e4m3 || !scale) return fail(TQ_EINVAL, "null pointer argument");
  if (!aligned(x_bf16, 16) || !aligned(y_e4m3, 16) || !aligned(scale, 4))
    return fail(TQ_EINVAL, "misaligned pointer (x 16 B, y 16 B, scale 4 B)");
  if (rows > ((int64_t)1 << 36)) return fail(TQ_EINVAL, "rows too large");
  return launched(tqk::launch_fwht128_fp8(x_bf16, rows, y_e4m3, scale,
                                          static_cast<hipStream_t>(stream)),
                  "fwht128_quant_fp8");
}

int tq_kpool_compress_and_write_cache(const void* slot_k, const void* slot_score,
                                      int32_t score_dtype, const float* ape, const int64_t* loc,
                                      const uint8_t* write_mask, int64_t n_pools,
                                      int32_t pool_size, int32_t head_dim, uint8_t* kv_cache,
                                      int64_t num_blocks, int32_t block_size,
                                      int32_t round_scale, uint8_t* compressed_k,
                                      float* compressed_scale, void* stream) {
  if (head_dim != 128) return fail(TQ_ENOTSUP, "head_dim %d (the Hadamard-128 entry needs 128)", head_dim);
  if (n_pools < 0 || n_pools > ((int64_t)1 << 32)) return fail(TQ_EINVAL, "n_pools %lld", (long long)n_pools);
  if (pool_size < 1 || pool_size > 65536) return fail(TQ_EINVAL, "pool_size %d", pool_size);
  if (score_dtype != TQ_DTYPE_F32 && score_dtype != TQ_DTYPE_F16 && score_dtype != TQ_DTYPE_BF16)
    return fail(TQ_EINVAL, "score_dtype %d", score_dtype);
  if (!kv_cache && !compressed_k) return fail(TQ_EINVAL, "no output: kv_cache and compressed_k are both null");
  if ((compressed_k == nullptr) != (compressed_scale == nullptr))
    return fail(TQ_EINVAL, "compressed_k and compressed_scale go together");
  if (write_mask && compressed_k) return fail(TQ_EINVAL, "a write mask excludes the compressed output");
  if (kv_cache) {
    if (block_size < 1 || num_blocks < 1) return fail(TQ_EINVAL, "num_blocks %lld, block_size %d",
                                                      (long long)num_blocks, block_size);
    if (num_blocks > ((int64_t)1 << 40) / ((int64_t)block_size * 132))
      return fail(TQ_EINVAL, "cache too large");
    if (!aligned(kv_cache, 4) || !aligned(loc, 8)) return fail(TQ_EINVAL, "misaligned kv_cache (4 B) or loc (8 B)");
  }
  if (n_pools == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  if (!slot_k || !slot_score || !ape) return fail(TQ_EINVAL, "null pointer argument");
  if (kv_cache && !loc) return fail(TQ_EINVAL, "kv_cache needs loc");
  if (!aligned(slot_k, 16) || !aligned(slot_score, 16) || !aligned(ape, 16))
    return fail(TQ_EINVAL, "misaligned slot_k, slot_score or ape (16 B)");
  if (compressed_k && (!aligned(compressed_k, 8) || !aligned(compressed_scale, 4)))
    return fail(TQ_EINVAL, "misaligned compressed_k (8 B) or compressed_scale (4 B)");
  tqk::KpoolParams p;
  p.slot_k = static_cast<const uint16_t*>(slot_k);
  p.slot_score = slot_score;
  p.ape = ape;
  p.loc = loc;
  p.mask = write_mask;
  p.cache = kv_cache;
  p.ck = compressed_k;
  p.cs = compressed_scale;
  p.n_pools = n_pools;
  p.num_blocks = kv_cache ? num_blocks : 0;
  p.pool_size = pool_size;
  p.block_size = kv_cache ? block_size : 1;
  p.score_dtype = score_dtype;
  p.round_scale = round_scale ? 1 : 0;
  return launched(tqk::launch_kpool_compress(p, static_cast<hipStream_t>(stream)),
                  "tq_kpool_compress_and_write_cache");
}

size_t tq_prefill_workspace_bytes(int64_t num_tokens, int32_t Hq, int32_t Hk, int32_t D) {
  if (num_tokens <= 0 || D != 128 || Hk <= 0 || Hq < Hk || Hq % Hk != 0 || Hq / Hk > 32) return 0;
  const int64_t chunk = num_tokens < kPrefillChunk ? num_tokens : kPrefillChunk;
  return prefill_plan_bytes(chunk) + tq_decode_workspace_bytes((int32_t)chunk, Hq, Hk, D, 1);
}

int tq_prefill_attention_int4(const tq_prefill_args* a, void* stream) {
  if (!a) return fail(TQ_EINVAL, "null args");
  if (a->struct_size < offsetof(tq_prefill_args, workspace))
    return fail(TQ_EINVAL, "args.struct_size %u < %zu", a->struct_size,
                offsetof(tq_prefill_args, workspace));
  // the workspace fields exist only in the current layout
  void* const pws = a->struct_size >= sizeof(tq_prefill_args) ? a->workspace : nullptr;
  const int64_t pws_bytes = a->struct_size >= sizeof(tq_prefill_args) ? a->workspace_bytes : 0;
  if (a->num_tokens < 0 || a->num_seqs < 0) return fail(TQ_EINVAL, "negative num_tokens or num_seqs");
  if (a->D != 64 && a->D != 128) return fail(TQ_ENOTSUP, "D=%d (INT4 prefill supports 64, 128)", a->D);
  if (a->Hk < 1 || a->Hq < a->Hk || a->Hq % a->Hk != 0)
    return fail(TQ_EINVAL, "Hq=%d must be a positive multiple of Hk=%d", a->Hq, a->Hk);
  if (a->block_size < 1 || a->max_blocks < 1 || a->num_blocks < 1)
    return fail(TQ_EINVAL, "block_size, max_blocks and num_blocks must be positive");
  if (a->window < 0) return fail(TQ_EINVAL, "window %d < 0", a->window);
  if (!(a->softcap >= 0.0f) || a->softcap > 3.0e38f) return fail(TQ_EINVAL, "softcap must be finite and >= 0");
  if (!(a->sm_scale == a->sm_scale) || a->sm_scale > 3.0e38f || a->sm_scale < -3.0e38f)
    return fail(TQ_EINVAL, "sm_scale must be finite");
  if (a->num_tokens == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  if (a->num_seqs < 1) return fail(TQ_EINVAL, "num_tokens > 0 with no sequence");
  const int g = a->Hq / a->Hk;
  const int G = g <= 1 ? 1 : (g <= 2 ? 2 : (g <= 4 ? 4 : 8));
  const int64_t blocks = a->num_tokens * a->Hk * ((g + G - 1) / G);
  if (blocks > 0x7FFFFFFF) return fail(TQ_EINVAL, "num_tokens * Hk too large for one launch");
  if (!a->query || !a->cu_seqlens_q || !a->seq_lens || !a->block_table || !a->key_cache ||
      !a->value_cache || !a->k_scale_cache || !a->v_scale_cache || !a->rht_signs || !a->out)
    return fail(TQ_EINVAL, "null pointer argument");
  if (!aligned(a->key_cache, 4) || !aligned(a->value_cache, 4) || !aligned(a->query, 4) ||
      !aligned(a->k_scale_cache, 4) || !aligned(a->v_scale_cache, 4) ||
      (!a->output_scale && !aligned(a->out, 4)))
    return fail(TQ_EINVAL, "misaligned pointer (4 B)");
  tqk::PrefillParams p;
  p.q = a->query;
  p.cu_seqlens = a->cu_seqlens_q;
  p.seq_lens = a->seq_lens;
  p.block_table = a->block_table;
  p.kc = a->key_cache;
  p.vc = a->value_cache;
  p.ks = a->k_scale_cache;
  p.vs = a->v_scale_cache;
  p.rht_signs = a->rht_signs;
  p.sinks = a->sinks;
  p.output_scale = a->output_scale;
  p.out = a->output_scale ? nullptr : static_cast<float*>(a->out);
  p.out_fp8 = a->output_scale ? static_cast<uint8_t*>(a->out) : nullptr;
  p.num_tokens = a->num_tokens;
  p.num_blocks = a->num_blocks;
  p.num_seqs = a->num_seqs;
  p.hq = a->Hq;
  p.hk = a->Hk;
  p.d = a->D;
  p.g = g;
  p.block_size = a->block_size;
  p.max_blocks = a->max_blocks;
  p.window = a->window;
  p.sm_scale = a->sm_scale;
  p.softcap = a->softcap;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t need = tq_prefill_workspace_bytes(a->num_tokens, a->Hq, a->Hk, a->D);
  if (pws && need > 0 && pws_bytes >= 0 && (size_t)pws_bytes >= need && aligned(pws, 16) &&
      aligned(a->query, 16) && (a->output_scale || aligned(a->out, 16)) &&
      aligned(a->key_cache, 16) && aligned(a->value_cache, 16)) {
    const int r = prefill_on_matrix_cores(p, pws, st);
    if (r != TQ_ENOTSUP) return r;
  }
  return launched(tqk::launch_prefill_int4(p, st), "tq_prefill_attention_int4");
}

int tq_full_dequant_kv(const uint8_t* kv_cache, const int32_t* block_table, int32_t max_blocks,
                       const float* centroids, int32_t B, int32_t Hk, int32_t D,
                       int32_t block_size, int64_t num_blocks, int32_t slot_bytes,
                       int32_t key_fmt, int32_t val_fmt, int32_t norm_correction,
                       int32_t max_seq, void* k_out, void* v_out, void* stream) {
  if (D != 64 && D != 128 && D != 256) return fail(TQ_ENOTSUP, "D=%d (64, 128, 256)", D);
  if (key_fmt < TQ_KEY_FP8 || key_fmt > TQ_KEY_MSE4 || val_fmt < TQ_VAL_U3 || val_fmt > TQ_VAL_FP8)
    return fail(TQ_ENOTSUP, "key_fmt %d / val_fmt %d is not a TurboQuant slot format", key_fmt, val_fmt);
  if (B < 0 || Hk < 1 || max_seq < 0 || block_size < 1 || max_blocks < 1 || num_blocks < 1)
    return fail(TQ_EINVAL, "bad sizes");
  const int need = tq_slot_bytes(D, key_fmt, val_fmt);
  if (slot_bytes < need || slot_bytes % 16 != 0)
    return fail(TQ_EINVAL, "slot_bytes %d (need a multiple of 16 >= %d)", slot_bytes, need);
  if ((int64_t)max_seq > (int64_t)max_blocks * block_size)
    return fail(TQ_EINVAL, "max_seq %d > max_blocks * block_size", max_seq);
  const int64_t rows = (int64_t)B * Hk * max_seq;
  if (rows == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  if (rows / (256 / (D / 8)) >= 0x7FFFFFFF) return fail(TQ_EINVAL, "too many rows");
  if (!kv_cache || !block_table || !k_out || !v_out || (key_fmt != TQ_KEY_FP8 && !centroids))
    return fail(TQ_EINVAL, "null pointer argument");
  if (!aligned(kv_cache, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(TQ_EINVAL, "misaligned kv_cache, k_out or v_out (16 B)");
  tqk::DequantParams p;
  p.kv = kv_cache;
  p.block_table = block_table;
  p.centroids = centroids;
  p.k_out = static_cast<uint16_t*>(k_out);
  p.v_out = static_cast<uint16_t*>(v_out);
  p.num_blocks = num_blocks;
  p.B = B;
  p.hk = Hk;
  p.d = D;
  p.block_size = block_size;
  p.max_blocks = max_blocks;
  p.slot_bytes = slot_bytes;
  p.key_fmt = key_fmt;
  p.val_fmt = val_fmt;
  p.norm_correction = norm_correction ? 1 : 0;
  p.max_seq = max_seq;
  p.kps = key_region_bytes(D, key_fmt);
  p.vdb = value_index_bytes(D, val_fmt);
  p.mse_bytes = (D * key_bits(key_fmt) + 7) / 8;
  return launched(tqk::launch_tq_full_dequant(p, static_cast<hipStream_t>(stream)),
                  "tq_full_dequant_kv");
}

}  // extern "C"

namespace {

// tq_decode_attention with the stage-1 workspace `ws` of `ws_bytes` bytes
// (the caller's, or the library's static one); `name` labels the errors.
int decode_impl(const tq_decode_args* a, float* ws, int64_t ws_bytes, const char* name,
                void* stream) {
  if (!a) return fail(TQ_EINVAL, "null args");
  if (a->struct_size < sizeof(tq_decode_args))
    return fail(TQ_EINVAL, "args.struct_size %u < %zu", a->struct_size, sizeof(tq_decode_args));
  if (a->B < 0 || a->Hq <= 0 || a->Hk <= 0) return fail(TQ_EINVAL, "bad B / Hq / Hk");
  if (a->Hq % a->Hk != 0) return fail(TQ_EINVAL, "Hq %% Hk != 0");
  if (a->Hq / a->Hk > 64) return fail(TQ_ENOTSUP, "Hq / Hk > 64");
  if (a->D <= 0 || a->D % 2 != 0 || (a->D & (a->D - 1)) != 0)
    return fail(TQ_EINVAL, "D must be an even power of two (got %d)", a->D);
  if (a->D != 64 && a->D != 128 && !(a->D == 256 && a->key_fmt != TQ_KEY_INT4))
    return fail(TQ_ENOTSUP, "D %d not supported (64, 128; 256 for the TurboQuant formats)", a->D);
  if (a->num_kv_splits < 1 || a->num_kv_splits > 256)
    return fail(TQ_EINVAL, "num_kv_splits must be in [1, 256]");
  if (a->block_size <= 0 || a->max_blocks <= 0 || a->num_blocks <= 0)
    return fail(TQ_EINVAL, "bad block_size / max_blocks / num_blocks");
  const bool int4 = a->key_fmt == TQ_KEY_INT4;
  if (int4 != (a->val_fmt == TQ_VAL_INT4))
    return fail(TQ_ENOTSUP, "INT4 keys pair only with INT4 values");
  if (a->key_fmt < TQ_KEY_INT4 || a->key_fmt > TQ_KEY_MSE4 || a->val_fmt < TQ_VAL_INT4 ||
      a->val_fmt > TQ_VAL_FP8)
    return fail(TQ_ENOTSUP, "unknown key/value format");
  if (a->B == 0) {
    g_err[0] = '\0';
    return TQ_OK;
  }
  if (!a->query || !a->block_table || !a->seq_lens || !ws || !a->out)
    return fail(TQ_EINVAL, "null pointer argument");
  tqk::DecodeParams p{};
  if (int4) {
    if (!a->key_cache || !a->value_cache || !a->k_scale_cache || !a->v_scale_cache ||
        !a->rht_signs)
      return fail(TQ_EINVAL, "INT4 format needs key/value caches, scale caches and rht_signs");
    if (!aligned(a->key_cache, 16) || !aligned(a->value_cache, 16) ||
        !aligned(a->k_scale_cache, 4) || !aligned(a->v_scale_cache, 4))
      return fail(TQ_EINVAL, "misaligned INT4 cache pointer (16 B / 4 B)");
  } else {
    const int sb = tq_slot_bytes(a->D, a->key_fmt, a->val_fmt);
    if (!a->kv_cache) return fail(TQ_EINVAL, "TurboQuant format needs kv_cache");
    if (a->slot_bytes < sb || a->slot_bytes % 16 != 0)
      return fail(TQ_EINVAL, "slot_bytes %d: need a multiple of 16 >= %d", a->slot_bytes, sb);
    if (!aligned(a->kv_cache, 16)) return fail(TQ_EINVAL, "kv_cache must be 16-byte aligned");
    if ((a->key_fmt == TQ_KEY_MSE3 || a->key_fmt == TQ_KEY_MSE4) && !a->centroids)
      return fail(TQ_EINVAL, "centroid keys need the centroid table");
    p.kps = key_region_bytes(a->D, a->key_fmt);
    p.vdb = value_index_bytes(a->D, a->val_fmt);
  }
  if (!aligned(a->query, 16) || !aligned(ws, 16) || !aligned(a->out, 16))
    return fail(TQ_EINVAL, "query / workspace / out must be 16-byte aligned");
  {
    const size_t need = tq_decode_workspace_bytes(a->B, a->Hq, a->Hk, a->D, a->num_kv_splits);
    if (ws_bytes < 0 || (size_t)ws_bytes < need)
      return fail(TQ_EINVAL, "%s: workspace_bytes %lld < %zu", name, (long long)ws_bytes, need);
  }
  p.B = a->B; p.hq = a->Hq; p.hk = a->Hk; p.d = a->D; p.g = a->Hq / a->Hk;
  p.block_size = a->block_size; p.max_blocks = a->max_blocks; p.splits = a->num_kv_splits;
  p.key_fmt = a->key_fmt; p.val_fmt = a->val_fmt; p.norm_correction = a->norm_correction;
  p.sm_scale = a->sm_scale; p.num_blocks = a->num_blocks;
  p.q = a->query; p.block_table = a->block_table; p.seq_lens = a->seq_lens;
  p.kc = a->key_cache; p.vc = a->value_cache; p.ks = a->k_scale_cache; p.vs = a->v_scale_cache;
  p.rht_signs = a->rht_signs; p.kv = a->kv_cache; p.slot_bytes = a->slot_bytes;
  p.centroids = a->centroids; p.rot_signs = a->rot_signs;
  p.ws = ws; p.out = a->out; p.lse = a->lse;
  p.nw = 0; p.wgh = 1;
  p.force_wide = (a->flags & TQ_FLAG_WIDE) ? 1 : 0;
  p.wsp = ws + (int64_t)a->B * a->Hq * a->num_kv_splits * (a->D + 1);
  {
    const int g = a->Hq / a->Hk;
    p.wsx = reinterpret_cast<int*>(
        p.wsp + (int64_t)2 * tqk::balance_max_wgs(a->Hk, g) * a->Hq * (a->D + 1));
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorNotSupported;
  if (!(a->flags & TQ_FLAG_GENERIC)) {
    if (int4) e = tqk::launch_decode_int4_mfma(p, st);
    else if (a->key_fmt == TQ_KEY_FP8) e = tqk::launch_decode_tq_mfma(p, st);
    else e = tqk::launch_decode_tqb_mfma(p, st);
  }
  if (e == hipErrorNotSupported) e = tqk::launch_decode_generic(p, st);
  char what[96];
  snprintf(what, sizeof(what), "%s stage 1", name);
  if (e != hipSuccess) return launched(e, what);
  snprintf(what, sizeof(what), "%s stage 2", name);
  return launched(tqk::launch_merge(p, st), what);
}

// Multi-query (prefill) attention on the matrix cores: each query token is
// one entry of the split-KV INT4 decode (one split per entry), planned on
// the GPU into the workspace's head, in chunks of kPrefillChunk tokens (the
// decode's per-call entry limit). TQ_ENOTSUP when the decode declines the
// shape before anything ran; the caller then takes the vector kernel.
int prefill_on_matrix_cores(const tqk::PrefillParams& pp, void* ws, hipStream_t st) {
  const int64_t T = pp.num_tokens;
  const int64_t chunk = T < kPrefillChunk ? T : kPrefillChunk;
  int32_t* lens = static_cast<int32_t*>(ws);
  int32_t* rows = lens + chunk;
  int32_t* offs = rows + chunk;
  float* dws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + prefill_plan_bytes(chunk));
  for (int64_t begin = 0; begin < T; begin += chunk) {
    const int n = (int)(T - begin < chunk ? T - begin : chunk);
    hipError_t e = tqk::launch_prefill_plan(pp, begin, n, lens, rows, offs, st);
    if (e != hipSuccess) return launched(e, "tq_prefill_attention_int4 plan");
    tqk::DecodeParams p;
    p.B = n; p.hq = pp.hq; p.hk = pp.hk; p.d = pp.d; p.g = pp.g;
    p.block_size = pp.block_size; p.max_blocks = pp.max_blocks; p.splits = 1;
    p.key_fmt = TQ_KEY_INT4; p.val_fmt = TQ_VAL_INT4; p.norm_correction = 0;
    p.sm_scale = pp.sm_scale; p.num_blocks = pp.num_blocks;
    p.q = pp.q + begin * pp.hq * pp.d;
    p.block_table = pp.block_table; p.seq_lens = lens;
    p.kc = pp.kc; p.vc = pp.vc; p.ks = pp.ks; p.vs = pp.vs;
    p.rht_signs = pp.rht_signs; p.kv = nullptr; p.slot_bytes = 0;
    p.centroids = nullptr; p.rot_signs = nullptr;
    p.ws = dws;
    p.out = pp.out ? pp.out + begin * pp.hq * pp.d : nullptr;
    p.lse = nullptr;
    p.nw = 0; p.wgh = 1; p.force_wide = 0;
    p.wsp = dws + (int64_t)n * pp.hq * (pp.d + 1);
    p.wsx = reinterpret_cast<int*>(p.wsp + (int64_t)2 * tqk::balance_max_wgs(pp.hk, pp.g) * pp.hq *
                                               (pp.d + 1));
    p.bt_row = rows;
    p.tok_off = offs;
    p.softcap = pp.softcap;
    p.sinks = pp.sinks;
    p.output_scale = pp.output_scale;
    p.out_fp8 = pp.out_fp8 ? pp.out_fp8 + begin * pp.hq * pp.d : nullptr;
    e = tqk::launch_decode_int4_mfma(p, st);
    if (e == hipErrorNotSupported && begin == 0) return TQ_ENOTSUP;
    if (e != hipSuccess) return launched(e, "tq_prefill_attention_int4 stage 1");
    e = tqk::launch_merge_one_split(p, st);
    if (e != hipSuccess) return launched(e, "tq_prefill_attention_int4 stage 2");
  }
  g_err[0] = '\0';
  return TQ_OK;
}

// Workspace of tq_decode_attention_static: a file-scope device array. Every
// GPU that loads the library holds its own copy, at its own address, until
// the process ends. In host code `scratch` names a host-side stand-in, so
// the kernels receive the device address that hipGetSymbolAddress returns,
// looked up once per device (with that device current) and kept.
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[TQ_STATIC_WORKSPACE_BYTES / sizeof(float)];
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

int scratch_address(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TQ_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TQ_ENOTSUP, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(TQ_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_decode_attention(const tq_decode_args* a, void* stream) {
  if (!a) return fail(TQ_EINVAL, "null args");
  return decode_impl(a, a->workspace, a->workspace_bytes, "tq_decode_attention", stream);
}

int tq_decode_attention_static(const tq_decode_args* a, void* stream) {
  if (!a) return fail(TQ_EINVAL, "null args");
  if (a->struct_size >= sizeof(tq_decode_args) && a->B > 0 && a->Hq > 0 && a->Hk > 0 &&
      a->D > 0 && a->num_kv_splits > 0) {
    const size_t need = tq_decode_workspace_bytes(a->B, a->Hq, a->Hk, a->D, a->num_kv_splits);
    if (need > (size_t)TQ_STATIC_WORKSPACE_BYTES)
      return fail(TQ_EINVAL,
                  "tq_decode_attention_static: B=%d Hq=%d D=%d S=%d needs %zu workspace bytes, "
                  "above the static maximum of %zu; use tq_decode_attention with a workspace",
                  a->B, a->Hq, a->D, a->num_kv_splits, need, (size_t)TQ_STATIC_WORKSPACE_BYTES);
  }
  float* ws = nullptr;
  if (a->B > 0) {
    const int r = scratch_address(&ws);
    if (r != TQ_OK) return r;
  }
  return decode_impl(a, ws, TQ_STATIC_WORKSPACE_BYTES, "tq_decode_attention_static", stream);
}

}  // extern "C"
