/*
 * CPU oracle for quantized paged-KV decode attention and its cache writers.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, by the smoke check and by
 * the benchmark's CPU-baseline leg; never by the product path. Shares no
 * code with the HIP library. Build: gcc -O2 -std=c11 -ffp-contract=off
 * (no contraction: every fp32 operation below rounds exactly once, as
 * written; the single fused multiply-add of the INT4 quantizer is an
 * explicit fmaf call).
 *
 * Page key (cited by page title and section, never by line):
 *   [tq]    triton_turboquant_decode.py
 *   [int4]  int4_per_token_head.py
 *   [kpool] kpool_compress.py
 *
 * Where the pages are silent the reading taken is stated next to the code.
 */
#include "tq_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float u2f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* ------------------------------------------------------------------------ */
/* Scalar converters. All round to nearest, ties to even (IEEE default).     */
/* ------------------------------------------------------------------------ */

/* fp32 -> bfloat16: keep the top 16 bits after adding half an ulp of the
 * kept part, with the tie broken towards an even kept part. */
uint16_t orc_f32_to_bf16(float x) {
  uint32_t u = f2u(x);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

float orc_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* fp32 -> IEEE binary16 (1 sign, 5 exponent bits, 10 mantissa bits). */
uint16_t orc_f32_to_f16(float x) {
  uint32_t u = f2u(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  float a = fabsf(x);
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
  if (a >= 65520.0f) return (uint16_t)(sign | 0x7C00u); /* rounds to inf */
  if (a < 6.103515625e-05f) {
    /* subnormal range: units of 2^-24; the scaling is exact in fp32 and
     * nearbyintf rounds half to even. A result of 1024 is the smallest
     * normal, whose encoding is the same integer. */
    float m = nearbyintf(a * 16777216.0f);
    return (uint16_t)(sign | (uint16_t)m);
  }
  uint32_t ua = f2u(a);
  uint32_t lsb = (ua >> 13) & 1u;
  uint32_t r = (ua + 0xFFFu + lsb) >> 13; /* (exp32 << 10) | mant10 */
  r -= (uint32_t)(127 - 15) << 10;        /* rebias the exponent     */
  return (uint16_t)(sign | r);
}

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(m | 0x400), e - 25);
  return sign ? -v : v;
}

/* fp32 -> OCP FP8 E4M3FN: exponent bias 7, no infinities, a single NaN
 * mantissa pattern (S.1111.111), largest finite 448, subnormals m*2^-9.
 * Finite inputs beyond 448 saturate to +-448 (the paths below clamp to
 * +-448 before converting, so this branch only matters for direct use). */
uint8_t orc_f32_to_e4m3(float x) {
  uint8_t sign = (uint8_t)((f2u(x) >> 24) & 0x80u);
  float a = fabsf(x);
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  if (a < 0.015625f) {                /* below 2^-6: units of 2^-9 */
    float m = nearbyintf(a * 512.0f); /* 0..8; 8 encodes 2^-6 */
    return (uint8_t)(sign | (uint8_t)m);
  }
  uint32_t ua = f2u(a);
  uint32_t lsb = (ua >> 20) & 1u;
  uint32_t r = (ua + 0x7FFFFu + lsb) >> 20; /* (exp32 << 3) | mant3 */
  int32_t code = (int32_t)r - ((127 - 7) << 3);
  if (code > 0x7E) code = 0x7E; /* saturate to 448 */
  return (uint8_t)(sign | (uint8_t)code);
}

float orc_e4m3_to_f32(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int m = b & 7;
  float v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexpf((float)m, -9);
  else v = ldexpf((float)(m | 8), e - 10);
  return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard transform, unnormalized, Sylvester (natural) order.        */
/* [int4] fast_hadamard_transform, third tier: butterflies with stride       */
/* h = 1, 2, 4, ..., d/2; the element with the stride bit clear becomes      */
/* a+b, its partner a-b. Each add rounds once in the working precision.      */
/* ------------------------------------------------------------------------ */
void orc_fwht_f32(float* x, int d) {
  for (int h = 1; h < d; h <<= 1)
    for (int i = 0; i < d; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

void orc_fwht_f64(double* x, int d) {
  for (int h = 1; h < d; h <<= 1)
    for (int i = 0; i < d; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

/* ------------------------------------------------------------------------ */
/* INT4 asymmetric per-(token, head) quantizer.                              */
/* [int4] _reshape_cache_int4_kernel; pack_int4_nibbles.                     */
/* ------------------------------------------------------------------------ */

/* float -> int32 conversion of the kernel's `.to(tl.int32)`: truncation
 * toward zero, saturating at the int32 range, NaN -> 0. */
static int32_t trunc_sat(float t) {
  if (isnan(t)) return 0;
  if (t >= 2147483648.0f) return INT32_MAX;
  if (t <= -2147483648.0f) return INT32_MIN;
  return (int32_t)t;
}

/* `tl.where(t >= 0, (t + 0.5).to(int32), (t - 0.5).to(int32))` followed by
 * `.to(float32)` and a clamp to [0, 15]. */
static float round_half_away_clamp15(float t) {
  int32_t i = (t >= 0.0f) ? trunc_sat(t + 0.5f) : trunc_sat(t - 0.5f);
  float f = (float)i;
  if (f < 0.0f) f = 0.0f;
  if (f > 15.0f) f = 15.0f;
  return f;
}

/* One row of d fp32 values -> d/2 packed bytes and the scale word.
 *   scale = max((max - min) / 15, 1e-6)              (fp32, IEEE division)
 *   zp    = clamp(round_half_away(-min / scale), 0, 15)
 *   q_i   = clamp(round_half_away(x_i * (1/scale) + zp), 0, 15)
 * The multiply-add `x * inv + zp` is one fused operation (fmaf): the plain
 * reading of a Triton expression compiled with fp-contraction enabled.
 * Byte j holds q[2j] in its low nibble and q[2j+1] in its high nibble.
 * The scale word is the fp32 scale with its low four mantissa bits replaced
 * by zp. */
void orc_int4_quantize_row(const float* x, int d, uint8_t* packed, float* word) {
  float mn = INFINITY, mx = -INFINITY;
  for (int i = 0; i < d; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  float scale = (mx - mn) / 15.0f;
  if (!(scale > 1e-6f)) scale = 1e-6f;
  float u = -mn / scale;
  float zp = round_half_away_clamp15(u);
  float inv = 1.0f / scale;
  for (int j = 0; j < d / 2; ++j) {
    float qe = round_half_away_clamp15(fmaf(x[2 * j], inv, zp));
    float qo = round_half_away_clamp15(fmaf(x[2 * j + 1], inv, zp));
    packed[j] = (uint8_t)(((uint32_t)qe & 0xFu) | (((uint32_t)qo & 0xFu) << 4));
  }
  uint32_t zpi = (uint32_t)(int32_t)zp;
  *word = u2f((f2u(scale) & 0xFFFFFFF0u) | (zpi & 0xFu));
}

/* Reader side of the scale word ([int4] _attn_packed): zp = bits & 0xF,
 * scale' = float(bits & ~0xF); element value (q - zp) * scale'. */
void orc_int4_dequant_row(const uint8_t* packed, float word, int d, double* out) {
  uint32_t bits = f2u(word);
  double zp = (double)(bits & 0xFu);
  double sc = (double)u2f(bits & 0xFFFFFFF0u);
  for (int j = 0; j < d / 2; ++j) {
    out[2 * j] = ((double)(packed[j] & 0xF) - zp) * sc;
    out[2 * j + 1] = ((double)(packed[j] >> 4) - zp) * sc;
  }
}

/* Source element -> fp32. kv_dtype: 0 fp32, 1 fp16, 2 bf16. */
static float load_elem(const void* base, int kv_dtype, int64_t idx) {
  if (kv_dtype == 0) return ((const float*)base)[idx];
  if (kv_dtype == 1) return orc_f16_to_f32(((const uint16_t*)base)[idx]);
  return orc_bf16_to_f32(((const uint16_t*)base)[idx]);
}

/* Round an fp32 value to the source dtype and back (`.to(key.dtype)`). */
static float round_to_dtype(float x, int kv_dtype) {
  if (kv_dtype == 1) return orc_f16_to_f32(orc_f32_to_f16(x));
  if (kv_dtype == 2) return orc_bf16_to_f32(orc_f32_to_bf16(x));
  return x;
}

/* [int4] reshape_and_cache_int4: x <- single_rht(x.float()).to(dtype), i.e.
 * multiply by the +-1 signs, unnormalized FWHT in fp32, round to the source
 * dtype; then the per-(token, head) quantizer; write at
 * [slot // block_size, slot % block_size, head]. Negative slots are skipped
 * ([int4] _reshape_cache_int4_kernel). Slots at or beyond
 * num_blocks*block_size are skipped as well (reading: outside the cache).
 * Caches: key/value [num_blocks, block_size, hk, d/2] u8, scale words
 * [num_blocks, block_size, hk] f32. */
int orc_reshape_and_cache_int4(const void* key, const void* value, int kv_dtype,
                               int64_t num_tokens, int hk, int d,
                               const int64_t* slot_mapping, const float* signs,
                               uint8_t* key_cache, uint8_t* value_cache,
                               float* k_scale, float* v_scale,
                               int64_t num_blocks, int block_size) {
  if (d <= 0 || d > 1024 || (d & (d - 1)) != 0) return -1;
  float x[1024];
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * (int64_t)block_size) continue;
    int64_t blk = slot / block_size, off = slot % block_size;
    for (int h = 0; h < hk; ++h) {
      int64_t src = (t * hk + h) * (int64_t)d;
      int64_t dst = (blk * block_size + off) * hk + h;
      for (int pass = 0; pass < 2; ++pass) {
        const void* in = pass ? value : key;
        for (int i = 0; i < d; ++i) x[i] = load_elem(in, kv_dtype, src + i) * signs[i];
        orc_fwht_f32(x, d);
        for (int i = 0; i < d; ++i) x[i] = round_to_dtype(x[i], kv_dtype);
        uint8_t* cache = pass ? value_cache : key_cache;
        float* sc = pass ? v_scale : k_scale;
        orc_int4_quantize_row(x, d, cache + dst * (d / 2), sc + dst);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Split-KV softmax attention in fp64.                                       */
/* ------------------------------------------------------------------------ */

/* Softmax partial over tokens [t0, t1) of one (batch, query head):
 * o = sum_t e^{s_t - m} v_t / l, lse = m + ln l ([tq] _tq_decode_stage1,
 * online softmax with natural exp and the stored (acc / l, m + ln l)). The
 * scores and dequantized values are produced by the per-format callbacks. */
typedef struct {
  double (*score)(void* ctx, int64_t t);
  void (*value)(void* ctx, int64_t t, double* v);
  void* ctx;
  int d;
} token_src;

static void softmax_partial(const token_src* src, int64_t t0, int64_t t1,
                            double* o, double* lse, double* scratch_s,
                            double* scratch_v) {
  double m = -INFINITY;
  for (int64_t t = t0; t < t1; ++t) {
    scratch_s[t - t0] = src->score(src->ctx, t);
    if (scratch_s[t - t0] > m) m = scratch_s[t - t0];
  }
  double l = 0.0;
  for (int i = 0; i < src->d; ++i) o[i] = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    double p = exp(scratch_s[t - t0] - m);
    l += p;
    src->value(src->ctx, t, scratch_v);
    for (int i = 0; i < src->d; ++i) o[i] += p * scratch_v[i];
  }
  for (int i = 0; i < src->d; ++i) o[i] /= l;
  *lse = m + log(l);
}

/* Full attention for one row. num_splits == 0: one softmax over the whole
 * sequence. num_splits >= 1: the split-KV form -- split_len =
 * ceil(seq_len / S), split s covers [s*split_len, min((s+1)*split_len,
 * seq_len)) and is skipped when empty ([tq] _tq_decode_stage1, split range);
 * the non-empty partials are merged by log-sum-exp: M = max lse_s,
 * w_s = e^{lse_s - M}, o = sum w_s o_s / sum w_s, lse = M + ln sum w_s
 * (the stage-2 merge, whose body the pages import but do not show).
 * seq_len == 0 yields o = 0 and lse = -inf (reading: the pages never
 * reach it). */
static void attend_row(const token_src* src, int64_t seq_len, int num_splits,
                       double* o, double* lse) {
  int d = src->d;
  if (seq_len <= 0) {
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    *lse = -INFINITY;
    return;
  }
  double* s = malloc(sizeof(double) * (size_t)seq_len);
  double* v = malloc(sizeof(double) * (size_t)d);
  if (num_splits <= 0) {
    softmax_partial(src, 0, seq_len, o, lse, s, v);
    free(s);
    free(v);
    return;
  }
  double* os = malloc(sizeof(double) * (size_t)d * (size_t)num_splits);
  double* ls = malloc(sizeof(double) * (size_t)num_splits);
  int64_t split_len = (seq_len + num_splits - 1) / num_splits;
  int n = 0;
  for (int sp = 0; sp < num_splits; ++sp) {
    int64_t t0 = split_len * sp;
    int64_t t1 = t0 + split_len < seq_len ? t0 + split_len : seq_len;
    if (t0 >= t1) continue;
    softmax_partial(src, t0, t1, os + (size_t)n * d, ls + n, s, v);
    ++n;
  }
  double M = -INFINITY;
  for (int k = 0; k < n; ++k) if (ls[k] > M) M = ls[k];
  double wsum = 0.0;
  for (int i = 0; i < d; ++i) o[i] = 0.0;
  for (int k = 0; k < n; ++k) {
    double w = exp(ls[k] - M);
    wsum += w;
    for (int i = 0; i < d; ++i) o[i] += w * os[(size_t)k * d + i];
  }
  for (int i = 0; i < d; ++i) o[i] /= wsum;
  *lse = M + log(wsum);
  free(os);
  free(ls);
  free(s);
  free(v);
}

/* Physical page of token t ([tq] _tq_decode_stage1, page gather): the
 * block-table entry for logical page t // block_size. */
static int64_t page_of(const int32_t* bt_row, int64_t t, int block_size) {
  return bt_row[t / block_size];
}

/* ---- INT4 cache as a token source ---- */
typedef struct {
  const uint8_t *kc, *vc;
  const float *ks, *vs;
  const int32_t* bt_row;
  int block_size, hk, kvh, d;
  const double* qr;  /* rotated query, fp64 */
  double sc;         /* sm_scale / d */
  double* kbuf;
} int4_ctx;

static int64_t int4_index(const int4_ctx* c, int64_t t) {
  int64_t page = page_of(c->bt_row, t, c->block_size);
  return (page * c->block_size + t % c->block_size) * c->hk + c->kvh;
}

static double int4_score(void* p, int64_t t) {
  int4_ctx* c = p;
  int64_t idx = int4_index(c, t);
  orc_int4_dequant_row(c->kc + idx * (c->d / 2), c->ks[idx], c->d, c->kbuf);
  double dot = 0.0;
  for (int i = 0; i < c->d; ++i) dot += c->qr[i] * c->kbuf[i];
  return c->sc * dot;
}

static void int4_value(void* p, int64_t t, double* v) {
  int4_ctx* c = p;
  int64_t idx = int4_index(c, t);
  orc_int4_dequant_row(c->vc + idx * (c->d / 2), c->vs[idx], c->d, v);
}

/* [int4] unified_attention_int4 for single-token decode:
 *   q' = RHT(q) = FWHT(s * q), evaluated here in fp64 from the fp32 query;
 *   score_t = (sm_scale / d) * q' . k'_t, k'_t the dequantized rotated key;
 *   o' = softmax-weighted sum of the dequantized rotated values;
 *   out = RHT^{-1}(o') / d = s * FWHT(o') / d.
 * GQA: kv head = h / (hq / hk). rows (optional) selects flat (b*hq + h)
 * indices; out is [n_rows or B*hq, d], lse [n_rows or B*hq]. */
int orc_int4_decode(const float* q, const uint8_t* key_cache,
                    const uint8_t* value_cache, const float* k_scale,
                    const float* v_scale, const int32_t* block_table,
                    int max_blocks, const int32_t* seq_lens,
                    const float* signs, int B, int hq, int hk, int d,
                    int block_size, int num_splits, double sm_scale,
                    const int32_t* rows, int n_rows,
                    double* out, double* lse) {
  if (d <= 0 || d > 1024 || (d & (d - 1)) != 0 || hk <= 0 || hq % hk != 0)
    return -1;
  int total = rows ? n_rows : B * hq;
  double qr[1024], kbuf[1024], o[1024];
  for (int r = 0; r < total; ++r) {
    int flat = rows ? rows[r] : r;
    int b = flat / hq, h = flat % hq;
    for (int i = 0; i < d; ++i)
      qr[i] = (double)q[(size_t)flat * d + i] * (double)signs[i];
    orc_fwht_f64(qr, d);
    int4_ctx c = {key_cache, value_cache, k_scale, v_scale,
                  block_table + (size_t)b * max_blocks, block_size, hk,
                  h / (hq / hk), d, qr, sm_scale / d, kbuf};
    token_src src = {int4_score, int4_value, &c, d};
    double l;
    attend_row(&src, seq_lens[b], num_splits, o, &l);
    orc_fwht_f64(o, d);
    for (int i = 0; i < d; ++i)
      out[(size_t)r * d + i] = o[i] * (double)signs[i] / d;
    lse[r] = l;
  }
  return 0;
}

/* [int4] _attn_packed in its "2D" mode (prefill and multi-query), as
 * unified_attention_int4 wraps it. cu_seqlens_q holds num_seqs + 1 offsets
 * into the T query tokens; seq_lens the total key count of each sequence
 * (context + queries), clamped to [0, max_blocks * block_size] as in decode.
 * Query i of sequence b sits at absolute position pos = (seq_len -
 * query_len) + i and sees keys t in [0, min(pos + 1, seq_len)) (causal),
 * and, when window > 0 (window = 1 + window_size[0]), only those with
 * pos - t < window. Per visible key:
 *   s_t = (sm_scale / d) * q'.k'_t, then s_t <- c tanh(s_t / c) if c > 0;
 * with sinks, sink_h joins the denominator only (reading of the absent
 * init_softmax_M: the running max starts at sink_h with sum 1):
 *   o' = sum_t e^{s_t} v'_t / (e^{sink_h} + sum_t e^{s_t});
 * out = RHT^{-1}(o') / d = s * FWHT(o') / d. A query with no visible key
 * gets out = 0 (with or without a sink). q [T, hq, d] f32; out [T, hq, d]. */
int orc_int4_prefill(const float* q, const uint8_t* key_cache,
                     const uint8_t* value_cache, const float* k_scale,
                     const float* v_scale, const int32_t* block_table,
                     int max_blocks, const int32_t* cu_seqlens_q,
                     const int32_t* seq_lens, int num_seqs, const float* signs,
                     int hq, int hk, int d, int block_size, double sm_scale,
                     int window, double softcap, const float* sinks,
                     double* out) {
  if (d <= 0 || d > 1024 || (d & (d - 1)) != 0 || hk <= 0 || hq % hk != 0)
    return -1;
  double qr[1024], kbuf[1024], v[1024], o[1024];
  const int64_t cap = (int64_t)max_blocks * block_size;
  for (int b = 0; b < num_seqs; ++b) {
    int64_t qlen = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int64_t seq = seq_lens[b];
    if (seq < 0) seq = 0;
    if (seq > cap) seq = cap;
    for (int64_t i = 0; i < qlen; ++i) {
      int64_t tok = cu_seqlens_q[b] + i;
      int64_t pos = seq - qlen + i;
      int64_t hi = pos + 1 < seq ? pos + 1 : seq;
      int64_t lo = 0;
      if (window > 0 && pos - window + 1 > 0) lo = pos - window + 1;
      for (int h = 0; h < hq; ++h) {
        const float* qrow = q + ((size_t)tok * hq + h) * d;
        for (int k = 0; k < d; ++k) qr[k] = (double)qrow[k] * (double)signs[k];
        orc_fwht_f64(qr, d);
        int4_ctx c = {key_cache, value_cache, k_scale, v_scale,
                      block_table + (size_t)b * max_blocks, block_size, hk,
                      h / (hq / hk), d, qr, sm_scale / d, kbuf};
        double m = sinks ? (double)sinks[h] : -INFINITY;
        for (int64_t t = lo; t < hi; ++t) {
          double st = int4_score(&c, t);
          if (softcap > 0) st = softcap * tanh(st / softcap);
          if (st > m) m = st;
        }
        double l = sinks ? exp((double)sinks[h] - m) : 0.0;
        for (int k = 0; k < d; ++k) o[k] = 0.0;
        for (int64_t t = lo; t < hi; ++t) {
          double st = int4_score(&c, t);
          if (softcap > 0) st = softcap * tanh(st / softcap);
          double pt = exp(st - m);
          l += pt;
          int4_value(&c, t, v);
          for (int k = 0; k < d; ++k) o[k] += pt * v[k];
        }
        double* dst = out + ((size_t)tok * hq + h) * d;
        if (hi <= lo) {
          for (int k = 0; k < d; ++k) dst[k] = 0.0;
          continue;
        }
        for (int k = 0; k < d; ++k) o[k] /= l;
        orc_fwht_f64(o, d);
        for (int k = 0; k < d; ++k) dst[k] = o[k] * (double)signs[k] / d;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* TurboQuant combined-slot cache ([tq]).                                    */
/* key_fmt: 1 FP8 E4M3, 2 centroid 3-bit, 3 centroid 4-bit.                  */
/* val_fmt: 1 uniform 3-bit, 2 uniform 4-bit, 3 FP8 E4M3 (the stage-1        */
/* signature documents value bits "4 or 8=FP8" with D value bytes for FP8;   */
/* its body decodes only 3 and 4 bits, so FP8 values are read as D E4M3      */
/* codes with no scale or zero, like FP8 keys).                              */
/* Slot layout (reading of _tq_decode_stage1's addressing, the pages never   */
/* define key_packed_size or the padding): key region of KPS bytes (FP8: d   */
/* codes; centroid: ceil(d*b/8) bytes of indices then the fp16 norm, so      */
/* KPS = MSE_BYTES + 2), value data of ceil(d*vb/8) bytes (FP8: d), then for */
/* uniform values the fp16 scale and fp16 zero; total rounded up to 16 bytes */
/* with zero padding.                                                        */
/* ------------------------------------------------------------------------ */
static int key_bits(int key_fmt) { return key_fmt == 2 ? 3 : key_fmt == 3 ? 4 : 8; }
static int val_bits(int val_fmt) { return val_fmt == 1 ? 3 : val_fmt == 2 ? 4 : 8; }
static int key_region(int d, int key_fmt) {
  if (key_fmt == 1) return d;
  return (d * key_bits(key_fmt) + 7) / 8 + 2;
}
static int val_data_bytes(int d, int val_fmt) { return (d * val_bits(val_fmt) + 7) / 8; }

int orc_tq_slot_bytes(int d, int key_fmt, int val_fmt) {
  if (key_fmt < 1 || key_fmt > 3 || val_fmt < 1 || val_fmt > 3) return -1;
  int raw = key_region(d, key_fmt) + val_data_bytes(d, val_fmt) + (val_fmt == 3 ? 0 : 4);
  return (raw + 15) / 16 * 16;
}

/* LSB-first b-bit bit stream: index i occupies bits [b*i, b*i + b) of the
 * little-endian byte string ([tq] stage1 reads a 16-bit window starting at
 * byte (b*i)/8 and shifts right by (b*i)%8). */
static void put_bits(uint8_t* base, int i, int b, unsigned v) {
  for (int k = 0; k < b; ++k) {
    int bit = b * i + k;
    if ((v >> k) & 1u) base[bit / 8] |= (uint8_t)(1u << (bit % 8));
  }
}
static unsigned get_bits(const uint8_t* base, int i, int b) {
  int bit = b * i;
  unsigned w = base[bit / 8] | ((unsigned)base[bit / 8 + 1] << 8);
  return (w >> (bit % 8)) & ((1u << b) - 1u);
}

/* Lloyd-Max quantizer of the standard normal with `levels` cells, fp64:
 * alternate (boundaries = midpoints of adjacent centroids) and (centroid =
 * conditional mean of N(0,1) on its cell) until no centroid moves by more
 * than 1e-15. Ascending output. The pages only name a [2^b] centroid table;
 * the fixed point of this iteration is the reading taken. */
static double npdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846); }
static double ncdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }
void orc_lloyd_max_gaussian(int levels, double* c) {
  for (int i = 0; i < levels; ++i) c[i] = -2.0 + 4.0 * (i + 0.5) / levels;
  double b[65];
  for (int it = 0; it < 100000; ++it) {
    b[0] = -INFINITY;
    b[levels] = INFINITY;
    for (int i = 1; i < levels; ++i) b[i] = 0.5 * (c[i - 1] + c[i]);
    double moved = 0.0;
    for (int i = 0; i < levels; ++i) {
      double mass = ncdf(b[i + 1]) - ncdf(b[i]);
      double mean = (npdf(b[i]) - npdf(b[i + 1])) / mass;
      double dlt = fabs(mean - c[i]);
      if (dlt > moved) moved = dlt;
      c[i] = mean;
    }
    if (moved < 1e-15) break;
  }
}

/* Rotation used by the centroid key format and its query: Pi = H_d/sqrt(d),
 * optionally preceded by +-1 signs (Pi = H diag(s) / sqrt(d)). The pages
 * take Pi as an input matrix; a normalized Hadamard is the reading taken. */
static void rotate_f64(const float* x, const float* rot_signs, int d, double* y) {
  for (int i = 0; i < d; ++i)
    y[i] = (double)x[i] * (rot_signs ? (double)rot_signs[i] : 1.0);
  orc_fwht_f64(y, d);
  double nrm = 1.0 / sqrt((double)d);
  for (int i = 0; i < d; ++i) y[i] *= nrm;
}

/* Harness-side TurboQuant encoder (the pages show only the reader).
 * Keys: FP8 -> e4m3(clamp(k, +-448)); centroid -> norm = ||k||_2 stored
 * fp16, u = Pi k / norm, index = nearest centroid (ties to the lower index;
 * norm 0 gives the centroid nearest 0). Values (b bits): scale =
 * max((max-min)/(2^b-1), 1e-6) and zero = min, both stored fp16; index =
 * clamp(rint((v - zero16) / scale16), 0, 2^b-1), an IEEE division per
 * element; a zero minimum is +0.
 * Everything is fp32, each operation rounded once, in this order:
 *   ss   = sum of k_i^2, added pairwise with strides 1, 2, ..., d/2 (the
 *          order of the butterflies; see tree_sum_f32);
 *   norm = sqrt(ss) (correctly rounded);
 *   y    = FWHT(k * rot_signs) (strides 1 -> d/2);
 *   u_i  = (y_i * r) / norm, r = the fp32 rounding of 1/sqrt(d): the rotated
 *          key Pi k, then divided by its norm, element by element;
 *   index_i = argmin_j |u_i - c_j|.
 * The pages fix none of these roundings. The two divisions follow the
 * written forms u = Pi k / ||k|| and (v - zero) / scale; the summation
 * order of the norm is the reading taken, fixed so that the bytes are a
 * function of the input alone. */
static float tree_sum_f32(float* s, int d) {
  for (int h = 1; h < d; h <<= 1)
    for (int i = 0; i < d; i += 2 * h) s[i] = s[i] + s[i + h];
  return s[0];
}
int orc_tq_encode(const float* key, const float* value, int64_t num_tokens,
                  int hk, int d, int key_fmt, int val_fmt,
                  const float* centroids, const float* rot_signs,
                  const int64_t* slot_mapping, uint8_t* kv_cache,
                  int64_t num_blocks, int block_size, int slot_bytes) {
  if (d <= 0 || d > 1024 || (d & (d - 1)) != 0) return -1;
  if (orc_tq_slot_bytes(d, key_fmt, val_fmt) < 0 ||
      slot_bytes < orc_tq_slot_bytes(d, key_fmt, val_fmt))
    return -1;
  int kb = key_bits(key_fmt), vb = val_bits(val_fmt);
  int kps = key_region(d, key_fmt), vdb = val_data_bytes(d, val_fmt);
  int nc = 1 << kb;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * (int64_t)block_size) continue;
    for (int h = 0; h < hk; ++h) {
      const float* k = key + (t * hk + h) * (int64_t)d;
      const float* v = value + (t * hk + h) * (int64_t)d;
      uint8_t* s = kv_cache + (slot * hk + h) * (int64_t)slot_bytes;
      memset(s, 0, (size_t)slot_bytes);
      if (key_fmt == 1) {
        for (int i = 0; i < d; ++i) {
          float x = k[i] > 448.0f ? 448.0f : (k[i] < -448.0f ? -448.0f : k[i]);
          s[i] = orc_f32_to_e4m3(x);
        }
      } else {
        float sq[1024], y[1024];
        for (int i = 0; i < d; ++i) sq[i] = k[i] * k[i];
        const float nrm = sqrtf(tree_sum_f32(sq, d));
        const float r = (float)(1.0 / sqrt((double)d));
        for (int i = 0; i < d; ++i) y[i] = rot_signs ? k[i] * rot_signs[i] : k[i];
        orc_fwht_f32(y, d);
        for (int i = 0; i < d; ++i) {
          const float ui = nrm > 0.0f ? (y[i] * r) / nrm : 0.0f;
          int best = 0;
          float bd = fabsf(ui - centroids[0]);
          for (int j = 1; j < nc; ++j) {
            const float dj = fabsf(ui - centroids[j]);
            if (dj < bd) { bd = dj; best = j; }
          }
          put_bits(s, i, kb, (unsigned)best);
        }
        uint16_t n16 = orc_f32_to_f16(nrm);
        s[kps - 2] = (uint8_t)(n16 & 0xFF);
        s[kps - 1] = (uint8_t)(n16 >> 8);
      }
      if (val_fmt == 3) {
        for (int i = 0; i < d; ++i) {
          float x = v[i] > 448.0f ? 448.0f : (v[i] < -448.0f ? -448.0f : v[i]);
          s[kps + i] = orc_f32_to_e4m3(x);
        }
        continue;
      }
      float mn = INFINITY, mx = -INFINITY;
      for (int i = 0; i < d; ++i) {
        if (v[i] < mn) mn = v[i];
        if (v[i] > mx) mx = v[i];
      }
      /* a zero minimum is stored as +0 whatever the signs of the zeros in
       * the row, so the bytes do not depend on the order of the reduction */
      mn = mn + 0.0f;
      float levels = (float)((1 << vb) - 1);
      float sc = (mx - mn) / levels;
      if (!(sc > 1e-6f)) sc = 1e-6f;
      uint16_t sc16 = orc_f32_to_f16(sc), z16 = orc_f32_to_f16(mn);
      float scr = orc_f16_to_f32(sc16), zr = orc_f16_to_f32(z16);
      uint8_t* vd = s + kps;
      for (int i = 0; i < d; ++i) {
        float idx = nearbyintf((v[i] - zr) / scr);
        if (idx < 0.0f) idx = 0.0f;
        if (idx > levels) idx = levels;
        put_bits(vd, i, vb, (unsigned)idx);
      }
      vd[vdb + 0] = (uint8_t)(sc16 & 0xFF);
      vd[vdb + 1] = (uint8_t)(sc16 >> 8);
      vd[vdb + 2] = (uint8_t)(z16 & 0xFF);
      vd[vdb + 3] = (uint8_t)(z16 >> 8);
    }
  }
  return 0;
}

typedef struct {
  const uint8_t* cache;
  const int32_t* bt_row;
  const float* centroids;
  int block_size, hk, kvh, d, slot_bytes, key_fmt, val_fmt, norm_correction;
  const double* qv;  /* FP8 keys: the query; centroid keys: Pi q */
  double sm_scale;
} tq_ctx;

static const uint8_t* tq_slot(const tq_ctx* c, int64_t t) {
  int64_t page = page_of(c->bt_row, t, c->block_size);
  return c->cache + ((page * c->block_size + t % c->block_size) * c->hk + c->kvh) *
                        (int64_t)c->slot_bytes;
}

/* [tq] _tq_decode_stage1, score: FP8 keys -> ATTN_SCALE * q . e4m3(k);
 * centroid keys -> ATTN_SCALE * norm16 * (q_rot . c[idx]), with the
 * centroid vector optionally renormalized by 1/sqrt(sum c^2 + 1e-16)
 * (NORM_CORRECTION). */
static double tq_score(void* p, int64_t t) {
  tq_ctx* c = p;
  const uint8_t* s = tq_slot(c, t);
  double dot = 0.0;
  if (c->key_fmt == 1) {
    for (int i = 0; i < c->d; ++i) dot += c->qv[i] * (double)orc_e4m3_to_f32(s[i]);
    return c->sm_scale * dot;
  }
  int kb = key_bits(c->key_fmt);
  int mse_bytes = (c->d * kb + 7) / 8;
  double cs = 0.0;
  for (int i = 0; i < c->d; ++i) {
    double cv = (double)c->centroids[get_bits(s, i, kb)];
    dot += c->qv[i] * cv;
    cs += cv * cv;
  }
  if (c->norm_correction) dot /= sqrt(cs + 1e-16);
  double nrm = (double)orc_f16_to_f32((uint16_t)(s[mse_bytes] | (s[mse_bytes + 1] << 8)));
  return c->sm_scale * nrm * dot;
}

/* [tq] _tq_decode_stage1, value: idx * scale16 + zero16 (3- or 4-bit);
 * FP8 values: e4m3(byte). */
static void tq_value(void* p, int64_t t, double* v) {
  tq_ctx* c = p;
  const uint8_t* vd = tq_slot(c, t) + key_region(c->d, c->key_fmt);
  if (c->val_fmt == 3) {
    for (int i = 0; i < c->d; ++i) v[i] = (double)orc_e4m3_to_f32(vd[i]);
    return;
  }
  int vb = val_bits(c->val_fmt);
  int vdb = val_data_bytes(c->d, c->val_fmt);
  double sc = (double)orc_f16_to_f32((uint16_t)(vd[vdb] | (vd[vdb + 1] << 8)));
  double z = (double)orc_f16_to_f32((uint16_t)(vd[vdb + 2] | (vd[vdb + 3] << 8)));
  for (int i = 0; i < c->d; ++i) v[i] = (double)get_bits(vd, i, vb) * sc + z;
}

/* [tq] triton_turboquant_decode_attention: q_rot = q @ Pi^T for centroid
 * keys (the query itself for FP8 keys); stage 1 + stage 2 as in
 * attend_row; the output is in the original (unrotated) value space. */
int orc_tq_decode(const float* q, const uint8_t* kv_cache,
                  const int32_t* block_table, int max_blocks,
                  const int32_t* seq_lens, const float* centroids,
                  const float* rot_signs, int B, int hq, int hk, int d,
                  int block_size, int slot_bytes, int key_fmt, int val_fmt,
                  int norm_correction, int num_splits, double sm_scale,
                  const int32_t* rows, int n_rows, double* out, double* lse) {
  if (d <= 0 || d > 1024 || (d & (d - 1)) != 0 || hk <= 0 || hq % hk != 0)
    return -1;
  if (orc_tq_slot_bytes(d, key_fmt, val_fmt) < 0) return -1;
  int total = rows ? n_rows : B * hq;
  double qv[1024];
  for (int r = 0; r < total; ++r) {
    int flat = rows ? rows[r] : r;
    int b = flat / hq, h = flat % hq;
    if (key_fmt == 1)
      for (int i = 0; i < d; ++i) qv[i] = (double)q[(size_t)flat * d + i];
    else
      rotate_f64(q + (size_t)flat * d, rot_signs, d, qv);
    tq_ctx c = {kv_cache, block_table + (size_t)b * max_blocks, centroids,
                block_size, hk, h / (hq / hk), d, slot_bytes, key_fmt, val_fmt,
                norm_correction, qv, sm_scale};
    token_src src = {tq_score, tq_value, &c, d};
    attend_row(&src, seq_lens[b], num_splits, out + (size_t)r * d, lse + r);
  }
  return 0;
}

/* [tq] _tq_full_dequant_kv: every position pos < max_seq of every (b, kv
 * head), read through the block table (page = block_table[b, pos / bs]),
 * rebuilt as fp16 rows of k_out / v_out [B, hk, max_seq, d]. The page takes
 * no sequence lengths; positions whose page lies outside [0, num_blocks)
 * are written as zeros here (reading: the page would read outside the
 * cache). Keys: FP8 -> fp32 -> fp16; centroid keys c[idx] (LSB-first b-bit
 * indices), with norm correction c * (1 / sqrt(sum_d c^2 + 1e-16)) (the sum
 * in dimension order), then fl32(norm16 * c) -> fp16. Values: 3/4-bit
 * uniform fma(idx, scale16, zero16) in fp32 -> fp16 (one rounding, the
 * page compiler's contraction); other value widths (FP8 values) give zeros,
 * as the page's kernel does. All fp16 roundings are to nearest even. */
int orc_tq_full_dequant(const uint8_t* kv_cache, const int32_t* block_table,
                        int max_blocks, const float* centroids, int B, int hk,
                        int d, int block_size, int64_t num_blocks,
                        int slot_bytes, int key_fmt, int val_fmt,
                        int norm_correction, int max_seq, uint16_t* k_out,
                        uint16_t* v_out) {
  if (d <= 0 || d > 1024 || (d & (d - 1)) != 0) return -1;
  if (key_fmt < 1 || key_fmt > 3 || val_fmt < 1 || val_fmt > 3) return -1;
  if (slot_bytes < orc_tq_slot_bytes(d, key_fmt, val_fmt)) return -1;
  if (max_seq < 0 || (int64_t)max_seq > (int64_t)max_blocks * block_size) return -1;
  const int kb = key_bits(key_fmt), vb = val_bits(val_fmt);
  const int mse_bytes = (d * kb + 7) / 8, kps = key_region(d, key_fmt);
  const int vdb = val_data_bytes(d, val_fmt);
  float c[1024];
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < hk; ++h)
      for (int pos = 0; pos < max_seq; ++pos) {
        size_t o = (((size_t)b * hk + h) * max_seq + pos) * d;
        int64_t page = block_table[(size_t)b * max_blocks + pos / block_size];
        if (page < 0 || page >= num_blocks) {
          for (int i = 0; i < d; ++i) k_out[o + i] = v_out[o + i] = 0;
          continue;
        }
        const uint8_t* slot = kv_cache +
            ((page * block_size + pos % block_size) * hk + h) * (int64_t)slot_bytes;
        if (key_fmt == 1) {
          for (int i = 0; i < d; ++i) k_out[o + i] = orc_f32_to_f16(orc_e4m3_to_f32(slot[i]));
        } else {
          for (int i = 0; i < d; ++i) c[i] = centroids[get_bits(slot, i, kb)];
          if (norm_correction) {
            float ss = 0.0f;
            for (int i = 0; i < d; ++i) ss = ss + c[i] * c[i];
            float inv = 1.0f / sqrtf(ss + 1e-16f);
            for (int i = 0; i < d; ++i) c[i] = c[i] * inv;
          }
          float nrm = orc_f16_to_f32((uint16_t)(slot[mse_bytes] | (slot[mse_bytes + 1] << 8)));
          for (int i = 0; i < d; ++i) k_out[o + i] = orc_f32_to_f16(nrm * c[i]);
        }
        if (val_fmt == 3) {
          for (int i = 0; i < d; ++i) v_out[o + i] = 0;
        } else {
          const uint8_t* vs = slot + kps;
          float sc = orc_f16_to_f32((uint16_t)(vs[vdb] | (vs[vdb + 1] << 8)));
          float zr = orc_f16_to_f32((uint16_t)(vs[vdb + 2] | (vs[vdb + 3] << 8)));
          for (int i = 0; i < d; ++i)
            v_out[o + i] = orc_f32_to_f16(fmaf((float)get_bits(vs, i, vb), sc, zr));
        }
      }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* [kpool] _fwht_quant_kernel / fwht128_quant_fp8, per 128-wide bf16 row:   */
/*   x = fp32(row); seven butterfly stages (strides 1..64) in fp32;         */
/*   x = x * fl32(0.08838834764831845); x = fp32(bf16(x));                   */
/*   absmax = max(max |x|, 1e-4); scale = exp2(ceil(log2(absmax * fl32(1/448)))); */
/*   y = e4m3(clamp(x / scale, -448, 448)).                                  */
/* ------------------------------------------------------------------------ */
/* absmax -> max(absmax, 1e-4) -> exp2(ceil(log2(absmax * fl32(1/448)))). */
float orc_fp8_pow2_scale(float amax) {
  const float inv_448 = (float)(1.0 / 448.0);
  if (!(amax > 1e-4f)) amax = 1e-4f;
  return exp2f(ceilf(log2f(amax * inv_448)));
}

void orc_fwht128_quant_fp8(const uint16_t* x_bf16, int64_t rows, uint8_t* y,
                           float* scale) {
  const float inv_sqrt128 = 0.08838834764831845f;
  float x[128];
  for (int64_t r = 0; r < rows; ++r) {
    for (int i = 0; i < 128; ++i) x[i] = orc_bf16_to_f32(x_bf16[r * 128 + i]);
    orc_fwht_f32(x, 128);
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) {
      x[i] = orc_bf16_to_f32(orc_f32_to_bf16(x[i] * inv_sqrt128));
      if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    }
    float s = orc_fp8_pow2_scale(amax);
    scale[r] = s;
    for (int i = 0; i < 128; ++i) {
      float v = x[i] / s;
      if (v < -448.0f) v = -448.0f;
      if (v > 448.0f) v = 448.0f;
      y[r * 128 + i] = orc_f32_to_e4m3(v);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* [kpool] _kpool_softmax_rotate_write_cache_kernel and its host wrapper     */
/* kpool_compress_and_write_cache: one pool of P tokens -> one indexer entry. */
/*   per dimension d: m_d = max_s (score[s,d] + ape[s,d]);                   */
/*   p[s,d] = e^(score[s,d] + ape[s,d] - m_d); den_d = sum_s p[s,d];          */
/*   acc_d = sum_s k[s,d] p[s,d]; x_d = fp32(bf16(acc_d / den_d));            */
/*   then the Hadamard-128 path of fwht128_quant_fp8 (fp32 butterflies,      */
/*   x fl32(1/sqrt(128)), bf16 round), absmax with a 1e-4 floor, and either  */
/*   the power-of-two scale (round_scale) or absmax * fl32(1/448); codes are */
/*   e4m3(clamp(x / scale, +-448)). Everything is fp32 with one rounding per */
/*   operation, slots in order 0 .. P-1.                                     */
/* Readings: the exponential is e^x rounded once to fp32 (orc_exp_f32); the  */
/* per-slot accumulation acc += k * p is one fused multiply-add (the pages'  */
/* compiler fuses that multiply-add by default); den += p is a plain add.    */
/* ------------------------------------------------------------------------ */

/* e^x rounded to the nearest fp32. The double exp is accurate to about one
 * double ulp, far inside half an fp32 ulp, so one rounding to fp32 gives
 * the correctly rounded value except when e^x lies within ~2^-52 relative
 * of an fp32 rounding midpoint. */
float orc_exp_f32(float x) { return (float)exp((double)x); }

/* Indexer page of [kpool] kpool_compress_and_write_cache: a page of
 * block_size entries is block_size * (head_dim + 4) bytes; entry t's head_dim
 * E4M3 codes start at byte t * head_dim and its fp32 scale at byte
 * block_size * head_dim + 4 t. Masked pools (write_mask[i] == 0) produce
 * nothing; locations outside [0, num_blocks * block_size) are not written
 * (reading, as for the other writers). Inputs: slot_k [n, P, 128] bf16 bits,
 * slot_score [n, P, 128] in score_dtype (0 f32, 1 f16, 2 bf16), ape [P, 128]
 * f32. Either output may be absent, not both; the compressed output is not
 * taken together with a write mask (the pages refuse that pairing). */
int orc_kpool_compress_and_write(const uint16_t* slot_k, const void* slot_score,
                                 int score_dtype, const float* ape,
                                 const int64_t* loc, const uint8_t* write_mask,
                                 int64_t n_pools, int pool_size, int head_dim,
                                 uint8_t* kv_cache, int64_t num_blocks,
                                 int block_size, int round_scale,
                                 uint8_t* compressed_k, float* compressed_scale) {
  const float inv_sqrt128 = 0.08838834764831845f;
  const float inv_448 = (float)(1.0 / 448.0);
  if (head_dim != 128 || pool_size < 1 || n_pools < 0) return -1;
  if (!kv_cache && !compressed_k) return -1;
  if (write_mask && compressed_k) return -1;
  if ((compressed_k == NULL) != (compressed_scale == NULL)) return -1;
  if (kv_cache && (!loc || num_blocks < 0 || block_size < 1)) return -1;
  const int64_t page_bytes = (int64_t)block_size * (head_dim + 4);
  float x[128];
  uint8_t q[128];
  for (int64_t i = 0; i < n_pools; ++i) {
    if (write_mask && !write_mask[i]) continue;
    for (int d = 0; d < 128; ++d) {
      float m = -INFINITY;
      for (int s = 0; s < pool_size; ++s) {
        int64_t e = (i * pool_size + s) * 128 + d;
        float v = load_elem(slot_score, score_dtype, e) + ape[s * 128 + d];
        if (v > m) m = v;
      }
      float acc = 0.0f, den = 0.0f;
      for (int s = 0; s < pool_size; ++s) {
        int64_t e = (i * pool_size + s) * 128 + d;
        float v = load_elem(slot_score, score_dtype, e) + ape[s * 128 + d];
        float p = orc_exp_f32(v - m);
        den = den + p;
        acc = fmaf(orc_bf16_to_f32(slot_k[e]), p, acc);
      }
      x[d] = orc_bf16_to_f32(orc_f32_to_bf16(acc / den));
    }
    orc_fwht_f32(x, 128);
    float amax = 0.0f;
    for (int d = 0; d < 128; ++d) {
      x[d] = orc_bf16_to_f32(orc_f32_to_bf16(x[d] * inv_sqrt128));
      if (fabsf(x[d]) > amax) amax = fabsf(x[d]);
    }
    float sc;
    if (round_scale) {
      sc = orc_fp8_pow2_scale(amax);
    } else {
      if (!(amax > 1e-4f)) amax = 1e-4f;
      sc = amax * inv_448;
    }
    for (int d = 0; d < 128; ++d) {
      float v = x[d] / sc;
      if (v < -448.0f) v = -448.0f;
      if (v > 448.0f) v = 448.0f;
      q[d] = orc_f32_to_e4m3(v);
    }
    if (kv_cache) {
      int64_t l = loc[i];
      if (l >= 0 && l < num_blocks * (int64_t)block_size) {
        int64_t pg = l / block_size, off = l % block_size;
        uint8_t* page = kv_cache + pg * page_bytes;
        memcpy(page + off * 128, q, 128);
        memcpy(page + (int64_t)block_size * 128 + off * 4, &sc, 4);
      }
    }
    if (compressed_k) {
      memcpy(compressed_k + i * 128, q, 128);
      compressed_scale[i] = sc;
    }
  }
  return 0;
}

/* Element-wise array forms of the scalar converters (kind: 0 f32->bf16,
 * 1 bf16->f32, 2 f32->f16, 3 f16->f32, 4 f32->e4m3, 5 e4m3->f32). */
void orc_convert(int kind, const void* in, void* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    switch (kind) {
      case 0: ((uint16_t*)out)[i] = orc_f32_to_bf16(((const float*)in)[i]); break;
      case 1: ((float*)out)[i] = orc_bf16_to_f32(((const uint16_t*)in)[i]); break;
      case 2: ((uint16_t*)out)[i] = orc_f32_to_f16(((const float*)in)[i]); break;
      case 3: ((float*)out)[i] = orc_f16_to_f32(((const uint16_t*)in)[i]); break;
      case 4: ((uint8_t*)out)[i] = orc_f32_to_e4m3(((const float*)in)[i]); break;
      case 5: ((float*)out)[i] = orc_e4m3_to_f32(((const uint8_t*)in)[i]); break;
      default: break;
    }
  }
}
