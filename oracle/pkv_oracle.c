/*
 * pkv_oracle.c -- slow, plain, fp64 CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it (through oracle/oracle.py).  It shares
 * no header, table or helper with the HIP path.
 *
 * What it computes, and where the pages define it:
 *  - Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V, evaluated for the single
 *    query of a decode step over the prefix plus the new token
 *    ("KV Cache 与 PageAttention深度实战", section 1.2, the attention formula and
 *    Output_t = Attention(Q_t, [K_prefix, K_t], [V_prefix, V_t])).  The scale is
 *    an explicit argument; callers pass 1/sqrt(d).
 *  - K/V are reached through a per-sequence block table that maps logical
 *    block j to a physical block ("Transformer 推理优化：KV Cache、PagedAttention
 *    与 vLLM", section 3.3 Block Table; "KV Cache 与 PageAttention深度实战",
 *    section 3.2: attention addresses K/V indirectly through the block table).
 *    The oracle walks the table in logical order, token by token.
 *  - Physical layout (a reading; the pages only say a block holds the KV of
 *    16 tokens): cache[block][kv_head][offset][dim], one (block, head) tile
 *    contiguous.  Element index = ((blk*H_kv + h)*bs + off)*d + i.
 *  - Grouped-query attention: q-head h reads kv-head h / (H_q/H_kv) (a reading;
 *    the pages name GQA for Qwen3-8B and Llama-3-70B without the mapping).
 *  - FP8 E4M3 KV (range +-448, "大语言模型推理引擎深度剖析", section 4.2): OCP
 *    E4M3FN, per-tensor scale, real value = decode(code) * scale.
 *  - Per-channel scales ("大语言模型推理引擎深度剖析", section 4.3: each head
 *    dimension of the K and V tensors is quantised on its own, stored as FP8
 *    and dequantised for compute): one scale per (kv-head, dim) channel, for
 *    K and V separately, for E4M3 and INT8 codes alike; real value = code *
 *    scale[kv_head][dim].
 *  - INT8 KV ("推理加速三板斧", section 2.3, which lists INT8 KV caches
 *    next to FP8 without the encoding; reading: symmetric, one scale per
 *    tensor like FP8): code = the integer nearest to the binary32 product
 *    x * (1/scale), ties to even, saturated to +-127, NaN -> 0; real value =
 *    code * scale.
 *  - Cache append: only the new token's K and V are written ("Transformer 推理
 *    优化", section 2.2), at slot = physical_block*bs + offset.
 *  - Several queries per sequence in one pass: a chunk of a long prompt
 *    ("vLLM推理引擎深度解析" section 3.3; "推理加速三板斧" section 4.5, chunks
 *    of about 512 tokens scheduled alongside decode requests) or the draft
 *    tokens a target model checks in one parallel pass
 *    ("大语言模型推理引擎深度剖析" section 4.1, typically 3-8 of them).  The
 *    chunk's K/V are in the cache first; query i of a chunk of n at the end
 *    of a context of ctx tokens sits at position ctx - n + i and attends to
 *    positions 0 .. that position (each token sees its prefix, as in the
 *    prefix-plus-current form of section 1.2 of "KV Cache 与
 *    PageAttention深度实战").
 *
 * Everything is evaluated in double precision with plain loops.  Compile
 * without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8_E4M3 = 3, ORC_INT8 = 4 };

/* Caches whose codes carry a per-tensor scale. */
static int scaled_dtype(int dt) { return dt == ORC_FP8_E4M3 || dt == ORC_INT8; }

/* ---------------------------------------------------------------- decoders */

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-10 * 2^-14 */
  else if (e == 31)
    v = (m == 0) ? INFINITY : NAN;
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -v : v;
}

/* bfloat16 is the top half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double orc_f32_bits_to_f64(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite magnitude 1.75 * 2^8 = 448. */
double orc_e4m3_to_f64(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6); /* subnormal */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* The values of the 127 non-negative finite codes, from the decoder above,
 * filled once when the library is loaded. */
static double e4m3_value[127];
__attribute__((constructor)) static void fill_e4m3_values(void) {
  for (int c = 0; c <= 126; ++c) e4m3_value[c] = orc_e4m3_to_f64((uint8_t)c);
}

/* Encode a binary32 value as E4M3FN: the nearest finite code, ties to the
 * code with an even mantissa, magnitudes beyond 448 (and infinities)
 * saturate to +-448, NaN gives 0x7F.  Written as a search over the 127
 * non-negative finite codes so that it is the definition itself. */
uint8_t orc_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  uint32_t u;
  memcpy(&u, &x, 4);
  int neg = (u >> 31) & 1;
  double ax = fabs((double)x);
  /* Beyond the largest code every magnitude saturates (infinities
   * included).  The search below could not show it for huge values: there
   * ax - code rounds to ax in double for every code and the distances tie. */
  if (ax >= 448.0) return (uint8_t)(neg ? 0xFE : 0x7E);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 126; ++c) {
    double d = fabs(ax - e4m3_value[c]);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (neg ? 0x80 : 0));
}

/* INT8 code of a binary32 value: nearest integer, ties to even (the default
 * rounding of nearbyint), saturated to +-127; NaN -> 0. */
uint8_t orc_int8_encode(float x) {
  if (isnan(x)) return 0;
  double r = nearbyint((double)x);
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (uint8_t)(int8_t)r;
}

/* Every f16 and E4M3 bit pattern's value, from the decoders above, filled
 * once when the library is loaded (the decoders are the definition; the
 * tables only save recomputing them per element). */
static double f16_value[65536];
static double e4m3_code_value[256];
__attribute__((constructor)) static void fill_decode_tables(void) {
  for (int b = 0; b < 65536; ++b) f16_value[b] = orc_f16_to_f64((uint16_t)b);
  for (int c = 0; c < 256; ++c) e4m3_code_value[c] = orc_e4m3_to_f64((uint8_t)c);
}

static double load_elem(const void* base, int64_t idx, int dtype) {
  switch (dtype) {
    case ORC_F32: return orc_f32_bits_to_f64(((const uint32_t*)base)[idx]);
    case ORC_F16: return f16_value[((const uint16_t*)base)[idx]];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t*)base)[idx]);
    case ORC_FP8_E4M3: return e4m3_code_value[((const uint8_t*)base)[idx]];
    case ORC_INT8: return (double)((const int8_t*)base)[idx];
  }
  return NAN;
}

/* The new-token value as binary32 (every f16/bf16 value is exact in f32). */
static float load_as_f32(const void* base, int64_t idx, int dtype) {
  return (float)load_elem(base, idx, dtype);
}

void orc_bits_to_f64(const void* src, int dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, i, dtype);
}

void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

void orc_int8_encode_array(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_int8_encode(x[i]);
}

/* --------------------------------------------------------------- KV bytes */

/* Per-token KV bytes over the whole model: 2 (K and V) x layers x kv_heads x
 * head_dim x element bytes ("Transformer 推理优化", section 2.5). */
uint64_t orc_kv_bytes_per_token(int layers, int kv_heads, int head_dim,
                                int elem_bytes) {
  return 2ull * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim *
         (uint64_t)elem_bytes;
}

/* ------------------------------------------------------------ cache append */

static int elem_bytes(int dtype) {
  return dtype == ORC_F32 ? 4 : (dtype == ORC_FP8_E4M3 || dtype == ORC_INT8 ? 1 : 2);
}

/* Write the new tokens' K and V rows into the paged caches.
 * k_new/v_new: [T][H_kv][d] in new_dtype.  slot_mapping[t] < 0 skips token t.
 * Bit copy when kv_dtype == new_dtype; for an E4M3 cache each element is
 * encoded from the f32 value x * (1/scale), with 1/scale and the product
 * both rounded to binary32.  Returns -1 on an out-of-range slot, else 0. */
int orc_cache_append(void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const int64_t* slot_mapping,
                     int num_tokens, int num_kv_heads, int head_dim,
                     int block_size, int num_blocks, int new_dtype,
                     int kv_dtype, float k_scale, float v_scale) {
  const int eb_new = elem_bytes(new_dtype), eb_kv = elem_bytes(kv_dtype);
  for (int t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= (int64_t)num_blocks * block_size) return -1;
    int64_t blk = slot / block_size, off = slot % block_size;
    int bad = 0;
    /* a token's elements are written once each: they may be shared among
     * threads */
#pragma omp parallel for collapse(2) schedule(static) if (num_kv_heads * head_dim >= 512)
    for (int h = 0; h < num_kv_heads; ++h) {
      for (int i = 0; i < head_dim; ++i) {
        int64_t src = ((int64_t)t * num_kv_heads + h) * head_dim + i;
        int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + i;
        for (int which = 0; which < 2; ++which) {
          const void* nb = which ? v_new : k_new;
          void* cb = which ? v_cache : k_cache;
          if (scaled_dtype(kv_dtype)) {
            float scale = which ? v_scale : k_scale;
            float inv = 1.0f / scale;
            float y = load_as_f32(nb, src, new_dtype) * inv;
            ((uint8_t*)cb)[dst] =
                kv_dtype == ORC_FP8_E4M3 ? orc_e4m3_encode(y) : orc_int8_encode(y);
          } else if (eb_new != eb_kv) {
#pragma omp atomic write
            bad = 1;
          } else {
            memcpy((char*)cb + dst * eb_kv, (const char*)nb + src * eb_new, eb_kv);
          }
        }
      }
    }
    if (bad) return -2;
  }
  return 0;
}

/* The same append with one scale per (kv-head, dim) channel: element i of
 * kv-head h is encoded from the binary32 product x * fp32(1/scale[h*d+i]).
 * Caches must hold one-byte codes (E4M3 or INT8). */
int orc_cache_append_channel(void* k_cache, void* v_cache, const void* k_new,
                             const void* v_new, const int64_t* slot_mapping,
                             int num_tokens, int num_kv_heads, int head_dim,
                             int block_size, int num_blocks, int new_dtype,
                             int kv_dtype, const float* k_scales, const float* v_scales) {
  if (!scaled_dtype(kv_dtype)) return -2;
  for (int t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= (int64_t)num_blocks * block_size) return -1;
    int64_t blk = slot / block_size, off = slot % block_size;
#pragma omp parallel for collapse(2) schedule(static) if (num_kv_heads * head_dim >= 512)
    for (int h = 0; h < num_kv_heads; ++h) {
      for (int i = 0; i < head_dim; ++i) {
        int64_t src = ((int64_t)t * num_kv_heads + h) * head_dim + i;
        int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + i;
        for (int which = 0; which < 2; ++which) {
          float scale = (which ? v_scales : k_scales)[h * head_dim + i];
          float inv = 1.0f / scale;
          float y = load_as_f32(which ? v_new : k_new, src, new_dtype) * inv;
          ((uint8_t*)(which ? v_cache : k_cache))[dst] =
              kv_dtype == ORC_FP8_E4M3 ? orc_e4m3_encode(y) : orc_int8_encode(y);
        }
      }
    }
  }
  return 0;
}

/* Decode attention over a cache with per-channel scales: the K element of
 * (token t, kv-head h, dim i) is code * k_scales[h*d+i], likewise V.  Plain
 * loops over the block table; out[S][H_q][d]. */
int orc_paged_decode_channel(double* out, const void* q, int q_dtype, const void* k_cache,
                             const void* v_cache, int kv_dtype, const int32_t* block_tables,
                             const int32_t* context_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size,
                             int max_blocks_per_seq, double scale, const double* k_scales,
                             const double* v_scales) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || !scaled_dtype(kv_dtype))
    return -1;
  const int g = num_q_heads / num_kv_heads;
  const int max_ctx = max_blocks_per_seq * block_size;
  double* z = (double*)malloc(sizeof(double) * (max_ctx > 0 ? max_ctx : 1));
  if (!z) return -3;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = context_lens[s];
    if (n > max_ctx) { free(z); return -2; }
    for (int hq = 0; hq < num_q_heads; ++hq) {
      const int hk = hq / g;
      double* o = out + ((int64_t)s * num_q_heads + hq) * head_dim;
      for (int i = 0; i < head_dim; ++i) o[i] = 0.0;
      if (n <= 0) continue;
      double m = -INFINITY;
      for (int t = 0; t < n; ++t) {
        const int32_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
        const int64_t base = (((int64_t)phys * num_kv_heads + hk) * block_size +
                              t % block_size) * head_dim;
        double dot = 0.0;
        for (int i = 0; i < head_dim; ++i)
          dot += load_elem(q, ((int64_t)s * num_q_heads + hq) * head_dim + i, q_dtype) *
                 (load_elem(k_cache, base + i, kv_dtype) * k_scales[hk * head_dim + i]);
        z[t] = scale * dot;
        if (z[t] > m) m = z[t];
      }
      double l = 0.0;
      for (int t = 0; t < n; ++t) {
        z[t] = exp(z[t] - m);
        l += z[t];
      }
      for (int t = 0; t < n; ++t) {
        const int32_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
        const int64_t base = (((int64_t)phys * num_kv_heads + hk) * block_size +
                              t % block_size) * head_dim;
        const double wt = z[t] / l;
        for (int i = 0; i < head_dim; ++i)
          o[i] += wt * (load_elem(v_cache, base + i, kv_dtype) * v_scales[hk * head_dim + i]);
      }
    }
  }
  free(z);
  return 0;
}

/* --------------------------------------------------------- decode attention */

typedef struct {
  const void* q;
  int q_dtype;
  const void* k_cache;
  const void* v_cache;
  int kv_dtype;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int max_blocks_per_seq;
  double scale, k_scale, v_scale;
} orc_args;

/* Element i of token t of sequence s, kv-head h, found through the block
 * table: logical block t / bs, slot t % bs inside the physical block. */
static double cache_elem(const orc_args* a, const void* cache, double cscale,
                         int s, int h, int t, int i) {
  int32_t phys = a->block_tables[(int64_t)s * a->max_blocks_per_seq + t / a->block_size];
  int64_t idx = (((int64_t)phys * a->num_kv_heads + h) * a->block_size +
                 t % a->block_size) * a->head_dim + i;
  return load_elem(cache, idx, a->kv_dtype) * cscale;
}

static double logit(const orc_args* a, int s, int hq, int t) {
  int g = a->num_q_heads / a->num_kv_heads;
  int hk = hq / g;
  double dot = 0.0;
  for (int i = 0; i < a->head_dim; ++i) {
    double qi = load_elem(a->q, ((int64_t)s * a->num_q_heads + hq) * a->head_dim + i, a->q_dtype);
    dot += qi * cache_elem(a, a->k_cache, a->k_scale, s, hk, t, i);
  }
  return a->scale * dot;
}

/* softmax weights of one (sequence, q-head) over its context, w[ctx]. */
static void weights(const orc_args* a, int s, int hq, int t0, int t1, double* z,
                    double* m_out, double* l_out) {
  double m = -INFINITY;
  for (int t = t0; t < t1; ++t) {
    z[t - t0] = logit(a, s, hq, t);
    if (z[t - t0] > m) m = z[t - t0];
  }
  double l = 0.0;
  for (int t = t0; t < t1; ++t) {
    z[t - t0] = exp(z[t - t0] - m);
    l += z[t - t0];
  }
  *m_out = m;
  *l_out = l;
}

/* One output row, out[s][hq][:], over the sequence's n = context_lens[s]
 * tokens: the softmax weights of the row's logits, then the weighted sum of
 * its V rows.  w holds at least n doubles of scratch.  n <= 0 gives zeros. */
static void decode_row(const orc_args* a, int s, int hq, double* w, double* o) {
  const int g = a->num_q_heads / a->num_kv_heads;
  const int n = a->context_lens[s];
  for (int i = 0; i < a->head_dim; ++i) o[i] = 0.0;
  if (n <= 0) return;
  double m, l;
  weights(a, s, hq, 0, n, w, &m, &l);
  for (int t = 0; t < n; ++t) {
    double wt = w[t] / l;
    for (int i = 0; i < a->head_dim; ++i)
      o[i] += wt * cache_elem(a, a->v_cache, a->v_scale, s, hq / g, t, i);
  }
}

/* Every (sequence, q-head) row is independent of the others, so the rows may
 * be shared among threads: each row is still computed by one thread with the
 * same loops in the same order, and the result does not depend on the thread
 * count, bit for bit.  num_threads <= 1 runs serially. */
static int decode_rows(const orc_args* a, double* out, int num_threads) {
  const int max_ctx = a->max_blocks_per_seq * a->block_size;
  for (int s = 0; s < a->num_seqs; ++s)
    if (a->context_lens[s] > max_ctx) return -2;
  const int64_t nrows = (int64_t)a->num_seqs * a->num_q_heads;
  int failed = 0;
#pragma omp parallel num_threads(num_threads > 1 ? num_threads : 1) if (num_threads > 1)
  {
    double* w = (double*)malloc(sizeof(double) * (max_ctx > 0 ? max_ctx : 1));
    if (!w) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!w) continue;
      const int s = (int)(r / a->num_q_heads), hq = (int)(r % a->num_q_heads);
      decode_row(a, s, hq, w, out + r * a->head_dim);
    }
    free(w);
  }
  return failed ? -3 : 0;
}

static orc_args decode_args(const void* q, int q_dtype, const void* k_cache,
                            const void* v_cache, int kv_dtype, const int32_t* block_tables,
                            const int32_t* context_lens, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size,
                            int max_blocks_per_seq, double scale, double k_scale,
                            double v_scale) {
  orc_args a = {q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                block_size, max_blocks_per_seq, scale,
                scaled_dtype(kv_dtype) ? k_scale : 1.0,
                scaled_dtype(kv_dtype) ? v_scale : 1.0};
  return a;
}

/* out[S][H_q][d] (double).  A sequence with context length 0 yields zeros. */
int orc_paged_decode(double* out, const void* q, int q_dtype, const void* k_cache,
                     const void* v_cache, int kv_dtype,
                     const int32_t* block_tables, const int32_t* context_lens,
                     int num_seqs, int num_q_heads, int num_kv_heads,
                     int head_dim, int block_size, int max_blocks_per_seq,
                     double scale, double k_scale, double v_scale) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  const orc_args a = decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                 context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, scale, k_scale, v_scale);
  return decode_rows(&a, out, 1);
}

/* The same result with the rows shared among num_threads threads. */
int orc_paged_decode_mt(double* out, const void* q, int q_dtype, const void* k_cache,
                        const void* v_cache, int kv_dtype,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int num_seqs, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int max_blocks_per_seq,
                        double scale, double k_scale, double v_scale, int num_threads) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  const orc_args a = decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                 context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, scale, k_scale, v_scale);
  return decode_rows(&a, out, num_threads);
}

/* One output row of a multi-query call: q row `row` of sequence s, q-head hq,
 * sitting at position p, over tokens 0..p.  z holds at least p + 1 doubles. */
static void mq_row(const orc_args* a, int s, int64_t row, int hq, int p, double* z,
                   double* o) {
  const int g = a->num_q_heads / a->num_kv_heads, hk = hq / g, d = a->head_dim;
  double m = -INFINITY;
  for (int t = 0; t <= p; ++t) {
    double dot = 0.0;
    for (int e = 0; e < d; ++e) {
      const double qe = load_elem(a->q, (row * a->num_q_heads + hq) * d + e, a->q_dtype);
      dot += qe * cache_elem(a, a->k_cache, a->k_scale, s, hk, t, e);
    }
    z[t] = a->scale * dot;
    if (z[t] > m) m = z[t];
  }
  double l = 0.0;
  for (int t = 0; t <= p; ++t) {
    z[t] = exp(z[t] - m);
    l += z[t];
  }
  for (int t = 0; t <= p; ++t) {
    const double wt = z[t] / l;
    for (int e = 0; e < d; ++e) o[e] += wt * cache_elem(a, a->v_cache, a->v_scale, s, hk, t, e);
  }
}

/* Every (row, q-head) is independent; with num_threads > 1 they are shared
 * among threads, each computed by one thread exactly as serially. */
static int multiquery_rows(const orc_args* a, double* out, const int32_t* query_start,
                           int num_rows, int num_threads) {
  const int max_ctx = a->max_blocks_per_seq * a->block_size;
  const int hq_n = a->num_q_heads, d = a->head_dim;
  for (int64_t i = 0; i < (int64_t)num_rows * hq_n * d; ++i) out[i] = 0.0;
  /* the placed rows: (sequence, row, position) of every row with p >= 0 */
  int64_t placed = 0;
  for (int s = 0; s < a->num_seqs; ++s) {
    const int ctx = a->context_lens[s];
    const int r0 = query_start[s], n = query_start[s + 1] - r0;
    if (ctx > max_ctx || n < 0 || r0 < 0 || r0 + n > num_rows) return -2;
    for (int i = 0; i < n; ++i)
      if (ctx - n + i >= 0) ++placed;
  }
  int32_t* rs = (int32_t*)malloc(sizeof(int32_t) * (placed > 0 ? placed : 1) * 3);
  if (!rs) return -3;
  int64_t k = 0;
  for (int s = 0; s < a->num_seqs; ++s) {
    const int ctx = a->context_lens[s];
    const int r0 = query_start[s], n = query_start[s + 1] - r0;
    for (int i = 0; i < n; ++i) {
      const int p = ctx - n + i;   /* position of this query */
      if (p < 0) continue;
      rs[3 * k] = s;
      rs[3 * k + 1] = r0 + i;
      rs[3 * k + 2] = p;
      ++k;
    }
  }
  int failed = 0;
  const int64_t items = placed * hq_n;
#pragma omp parallel num_threads(num_threads > 1 ? num_threads : 1) if (num_threads > 1)
  {
    double* z = (double*)malloc(sizeof(double) * (max_ctx > 0 ? max_ctx : 1));
    if (!z) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
      if (!z) continue;
      const int64_t j = it / hq_n;
      const int hq = (int)(it % hq_n);
      const int64_t row = rs[3 * j + 1];
      mq_row(a, rs[3 * j], row, hq, rs[3 * j + 2], z, out + (row * hq_n + hq) * d);
    }
    free(z);
  }
  free(rs);
  return failed ? -3 : 0;
}

/* Multi-query attention through the block table.  Sequence s owns the
 * query rows query_start[s] .. query_start[s+1]-1 of q and out ([rows][H_q]
 * [d]); with n = that count and ctx = context_lens[s], row query_start[s]+i
 * is position p = ctx - n + i and attends to tokens 0..p.  A row with p < 0
 * (n > ctx) and every row no sequence owns yields zeros.  With n = 1 a row is
 * the decode output of its sequence. */
int orc_paged_multiquery(double* out, const void* q, int q_dtype, const void* k_cache,
                         const void* v_cache, int kv_dtype, const int32_t* block_tables,
                         const int32_t* context_lens, const int32_t* query_start,
                         int num_seqs, int num_rows, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int max_blocks_per_seq, double scale,
                         double k_scale, double v_scale) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  const orc_args a = decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                 context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, scale, k_scale, v_scale);
  return multiquery_rows(&a, out, query_start, num_rows, 1);
}

/* The same result with the (row, q-head) pairs shared among num_threads
 * threads. */
int orc_paged_multiquery_mt(double* out, const void* q, int q_dtype, const void* k_cache,
                            const void* v_cache, int kv_dtype, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start,
                            int num_seqs, int num_rows, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int max_blocks_per_seq, double scale,
                            double k_scale, double v_scale, int num_threads) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  const orc_args a = decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                 context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, scale, k_scale, v_scale);
  return multiquery_rows(&a, out, query_start, num_rows, num_threads);
}

/* Normalised softmax weights of one (sequence, q-head): w[ctx]. */
int orc_softmax_weights(double* w, int s, int hq, const void* q, int q_dtype,
                        const void* k_cache, int kv_dtype,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int num_seqs, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int max_blocks_per_seq,
                        double scale, double k_scale) {
  orc_args a = {q, q_dtype, k_cache, NULL, kv_dtype, block_tables,
                context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                block_size, max_blocks_per_seq, scale,
                scaled_dtype(kv_dtype) ? k_scale : 1.0, 1.0};
  int n = context_lens[s];
  if (n <= 0) return 0;
  double m, l;
  weights(&a, s, hq, 0, n, w, &m, &l);
  for (int t = 0; t < n; ++t) w[t] /= l;
  return n;
}

/* Statistics of one partition [t0, t1) of one (sequence, q-head):
 *   m = max_t z_t,  l = sum_t exp(z_t - m),  acc = sum_t exp(z_t - m) v_t.
 * These are the quantities a partitioned evaluation keeps; merging them with
 * orc_lse_merge must give the direct result. */
int orc_partition_stats(double* m_out, double* l_out, double* acc, int s, int hq,
                        int t0, int t1, const void* q, int q_dtype,
                        const void* k_cache, const void* v_cache, int kv_dtype,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int num_seqs, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int max_blocks_per_seq,
                        double scale, double k_scale, double v_scale) {
  orc_args a = {q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                block_size, max_blocks_per_seq, scale,
                scaled_dtype(kv_dtype) ? k_scale : 1.0,
                scaled_dtype(kv_dtype) ? v_scale : 1.0};
  int g = num_q_heads / num_kv_heads;
  for (int i = 0; i < head_dim; ++i) acc[i] = 0.0;
  if (t1 <= t0) { *m_out = -INFINITY; *l_out = 0.0; return 0; }
  double* w = (double*)malloc(sizeof(double) * (t1 - t0));
  if (!w) return -3;
  weights(&a, s, hq, t0, t1, w, m_out, l_out);
  for (int t = t0; t < t1; ++t)
    for (int i = 0; i < head_dim; ++i)
      acc[i] += w[t - t0] * cache_elem(&a, v_cache, a.v_scale, s, hq / g, t, i);
  free(w);
  return 0;
}

/* Log-sum-exp merge of P partition statistics into one output row:
 *   M = max_p m_p,  L = sum_p l_p e^(m_p - M),  out = sum_p acc_p e^(m_p - M) / L.
 * Partitions with l_p == 0 (empty) contribute nothing; all empty gives zeros. */
void orc_lse_merge(double* out, const double* m, const double* l,
                   const double* acc, int num_parts, int head_dim) {
  double M = -INFINITY;
  for (int p = 0; p < num_parts; ++p)
    if (l[p] > 0.0 && m[p] > M) M = m[p];
  for (int i = 0; i < head_dim; ++i) out[i] = 0.0;
  if (M == -INFINITY) return;
  double L = 0.0;
  for (int p = 0; p < num_parts; ++p)
    if (l[p] > 0.0) L += l[p] * exp(m[p] - M);
  for (int p = 0; p < num_parts; ++p) {
    if (l[p] <= 0.0) continue;
    double f = exp(m[p] - M) / L;
    for (int i = 0; i < head_dim; ++i) out[i] += f * acc[(int64_t)p * head_dim + i];
  }
}
