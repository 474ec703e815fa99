/*
 * pkv.h -- C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * The library implements the decode-side hot path of PagedAttention: the KV
 * cache lives in a pool of fixed 16-token blocks, each sequence reaches its
 * blocks through a block table that maps logical block j to any physical
 * block, and one decode step appends the new token's K/V rows and then runs
 * single-query attention over the whole context.
 *
 * Sources for the operations (page title, section):
 *   - "Transformer 推理优化：KV Cache、PagedAttention 与 vLLM": 2.2 (only the
 *     new token's K and V are computed and appended), 2.5 (KV bytes per
 *     token), 3.2-3.3 (16-token blocks, block table, non-contiguous blocks),
 *     3.5 (copy-on-write of shared blocks).
 *   - "KV Cache 与 PageAttention深度实战": 1.2 (Attention(Q,K,V) =
 *     softmax(QK^T/sqrt(d_k))V; the decode output attends over
 *     [K_prefix, K_t], [V_prefix, V_t]), 3.2 (attention gathers K/V through
 *     the block table), 4.1 (blocks swapped out to CPU memory when space is
 *     short).
 *   - "大语言模型推理引擎深度剖析": 2.2 (O(1) block allocation and release),
 *     2.3 (shared prefix blocks, reference counts, copy before write),
 *     3.3 (preemption by swapping blocks to host DRAM), 4.1 (draft tokens
 *     verified in one parallel pass), 4.2 (FP8 E4M3 with range +-448), 4.3
 *     (FP8 KV cache, dequantised for compute).
 *   - "vLLM推理引擎深度解析": 2.2 (block pool, block tables, free-block queue,
 *     a new block every 16 generated tokens), 3.3 (chunked prefill).
 *   - "推理加速三板斧": 4.5 (prompts cut into chunks of about 512 tokens and
 *     scheduled with decode requests).
 *
 * Conventions shared by every entry point:
 *   - Every call returns a pkv_status; nothing throws across the ABI.  On an
 *     error, pkv_last_error() returns a message for the calling thread.
 *   - Device pointers are caller-owned device memory (for example torch
 *     tensors).  The library never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     GPU calls are asynchronous on that stream; argument errors are reported
 *     synchronously before anything is launched.
 *   - Cache layout: k_cache and v_cache are separate arrays
 *       [num_blocks][num_kv_heads][block_size][head_dim]
 *     so that the 16 x head_dim tile of one (block, kv-head) is contiguous.
 *     Token t of a sequence lives in physical block block_tables[s][t / 16]
 *     at offset t % 16.  slot = physical_block * 16 + offset.
 *   - q-head h attends with kv-head h / (num_q_heads / num_kv_heads).
 *   - FP8 caches hold OCP E4M3FN codes with one scale per tensor (k_scale for
 *     K, v_scale for V): real value = decode(code) * scale.
 *   - INT8 caches ("推理加速三板斧", section 2.3 lists INT8 KV beside FP8) hold
 *     symmetric signed codes in [-127, 127] with one scale per tensor: real
 *     value = code * scale.  Everything said of FP8 caches below (16-bit q,
 *     scales, the kernels that serve them) holds for INT8 caches as well.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* bad pointer, size, shape or id */
  PKV_ERR_UNSUPPORTED = 2,   /* valid but not implemented (block size, head dim, dtype mix) */
  PKV_ERR_OUT_OF_BLOCKS = 3, /* the pool cannot satisfy the request; nothing changed */
  PKV_ERR_REFCOUNT = 4,      /* reference-count misuse (decref of a free block, ...) */
  PKV_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed */
  PKV_ERR_WORKSPACE = 6      /* workspace missing or smaller than pkv_decode_workspace_size */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3, PKV_INT8 = 4 } pkv_dtype;

/* Which decode kernel family runs.  AUTO picks per shape (see
 * pkv_decode_algo_for): MFMA when the q-head group g > 1 and the dtypes
 * allow it, else VECTOR.  VECTOR: per-lane fp32 arithmetic with wavefront
 * reductions.  MFMA: QK^T and PV on the matrix cores (16-bit or FP8 caches,
 * 16-bit q). */
typedef enum { PKV_ALGO_AUTO = 0, PKV_ALGO_VECTOR = 1, PKV_ALGO_MFMA = 2 } pkv_algo;

/* Message describing the last error on the calling thread ("" if none). */
const char* pkv_last_error(void);
const char* pkv_status_string(int32_t status);
/* Library version: major*10000 + minor*100 + patch. */
int32_t pkv_version(void);

/* --------------------------------------------------------------- sizes -- */

/* KV-cache bytes per token of a whole model: 2 x layers x kv_heads x head_dim
 * x element bytes ("Transformer 推理优化", section 2.5; e.g. 147,456 for 36
 * layers, 8 KV heads, head_dim 128, fp16).  Returns 0 on a bad dtype. */
uint64_t pkv_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                int32_t dtype);

/* --------------------------------------------------------- cache append -- */

/* Write the K/V rows of num_tokens new tokens into the paged caches: a
 * decode step computes K and V for its new token only and adds them to the
 * cache ("Transformer 推理优化：KV Cache、PagedAttention 与 vLLM", section
 * 2.2), in the slot its sequence's block table gives it (same page, section
 * 3.3: logical block t / 16 maps to a physical block, offset t % 16; a new
 * block is taken every 16 tokens, "vLLM推理引擎深度解析", section 2.2).
 *   k_new, v_new : device, [num_tokens][num_kv_heads][head_dim] of new_dtype,
 *                  contiguous.
 *   slot_mapping : device int64[num_tokens]; slot = block * block_size + offset.
 *                  A negative slot skips that token (padding).  Slots at or
 *                  beyond num_blocks * block_size are also skipped (the kernel
 *                  never writes out of bounds).  Slots must be distinct within
 *                  one call; the block pool guarantees this.
 *   dtypes       : kv_dtype == new_dtype (bit copy), or kv_dtype == FP8_E4M3
 *                  with new_dtype in {F32, F16, BF16}: each element becomes the
 *                  E4M3 code nearest to the binary32 product x * (1/scale),
 *                  ties to even, saturating at +-448, NaN -> 0x7F; 1/scale is
 *                  rounded to binary32 first.  kv_dtype == INT8: the integer
 *                  nearest to the same product, ties to even, saturating at
 *                  +-127, NaN -> 0.  k_scale/v_scale must be > 0 and finite
 *                  for FP8 and INT8 and are ignored otherwise.
 *   block_size must be 16; head_dim a multiple of 8 in [8, 256]. */
pkv_status pkv_paged_cache_append(void* k_cache, void* v_cache, const void* k_new,
                                  const void* v_new, const int64_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t new_dtype,
                                  int32_t kv_dtype, float k_scale, float v_scale, void* stream);

/* The same append into an FP8 or INT8 cache with per-channel scales
 * ("大语言模型推理引擎深度剖析", section 4.3: each head dimension of the K and V
 * tensors quantised on its own): element i of kv-head h is encoded from the
 * binary32 product x * (1/k_scales[h*head_dim + i]) (likewise V), the
 * reciprocal rounded to binary32.
 *   k_scales, v_scales : device float[num_kv_heads][head_dim]; every scale
 *                        must be finite and > 0 (read on the device, not
 *                        checked).
 * PKV_ERR_UNSUPPORTED for a 16-bit or f32 cache. */
pkv_status pkv_paged_cache_append_per_channel(void* k_cache, void* v_cache, const void* k_new,
                                              const void* v_new, const int64_t* slot_mapping,
                                              int32_t num_tokens, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, int32_t new_dtype,
                                              int32_t kv_dtype, const float* k_scales,
                                              const float* v_scales, void* stream);

/* ------------------------------------------------------ decode attention -- */

/* Effective partition size (tokens) an AUTO decode call with these arguments
 * will use: partition_size itself if > 0 (it must be a multiple of 16); for
 * partition_size 0, 0 when the call runs the balanced schedule (q-head group
 * g > 1 with a 16-bit or FP8 cache, at most 2048 sequences: the work is cut
 * into equal shares of 16-token blocks instead of fixed partitions), else
 * the library's choice of fixed partition (a single pass when the sequences
 * times kv-heads reach 2048).  A fixed-partition call whose
 * max_blocks_per_seq * 16 fits in one partition runs single-pass.  Returns -1
 * on bad arguments. */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq, int32_t kv_dtype,
                                  int32_t partition_size);

/* The partition_size to pass for a batch whose context lengths the caller
 * holds on the host (a serving loop has them after its block bookkeeping).
 * Where AUTO would run the balanced schedule, this weighs it against one
 * fixed partition of max_blocks_per_seq * 16 tokens per (sequence, kv-head
 * chunk), run single-pass: no partials and no merge kernel, but only as even
 * as the lengths are.  Returns 0 (balanced) or max_blocks_per_seq * 16; in
 * every other case the same as pkv_decode_partition_size(..., 0).  Both
 * choices compute the same attention.
 *   context_lens : host int32[num_seqs], the lengths the decode call will see
 *                  (clamped to [0, max_blocks_per_seq * 16] as it does).
 * Pure host function, O(num_seqs * kv-head chunks * log 256).  Returns -1 on
 * bad arguments. */
int32_t pkv_decode_partition_size_for_lengths(const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_blocks_per_seq,
                                              int32_t kv_dtype);

/* Bytes of device workspace a decode call with these arguments needs (0 for a
 * single-pass fixed partition).  Fixed partitions: float m[S][H_q][P],
 * float l[S][H_q][P], float acc[S][H_q][P][head_dim] (each part 256-byte
 * aligned), P = ceil(max_blocks_per_seq * 16 / partition).  Balanced
 * schedule: two partial slots (m, l and acc of up to 16 q-heads) per wave of
 * its grid.  For partition_size 0 the size covers both schedules.  Returns
 * SIZE_MAX on bad arguments. */
size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t kv_dtype,
                                 int32_t partition_size);

/* Kernel family AUTO resolves to for these arguments (PKV_ALGO_VECTOR or
 * PKV_ALGO_MFMA), or -1 if the combination is unsupported. */
int32_t pkv_decode_algo_for(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t q_dtype, int32_t kv_dtype);

/* Single-query paged attention for one decode step ("KV Cache 与
 * PageAttention深度实战", sections 1.2 and 3.2):
 *   out[s][h][:] = sum_t softmax_t(scale * q[s][h] . K_s[t]) * V_s[t]
 * over t < context_lens[s], K_s[t] and V_s[t] read through block_tables.
 *   out          : device, [num_seqs][num_q_heads][head_dim] of q_dtype,
 *                  rounded to nearest even.  A sequence with context length
 *                  <= 0 gets zeros.
 *   q            : device, [num_seqs][num_q_heads][head_dim] of q_dtype.
 *   block_tables : device int32[num_seqs][max_blocks_per_seq]; only the first
 *                  ceil(context_lens[s] / 16) entries of a row are read.  An
 *                  entry outside [0, num_blocks) is skipped (its tokens get no
 *                  weight) instead of being read.
 *   context_lens : device int32[num_seqs], tokens per sequence after this
 *                  step's append; values above max_blocks_per_seq * 16 are
 *                  clamped to it.
 *   dtypes       : (q, kv) in {(F32,F32), (F16,F16), (BF16,BF16),
 *                  (F16,FP8_E4M3), (BF16,FP8_E4M3)}; k_scale/v_scale apply to
 *                  FP8 caches only.
 *   shape limits : block_size 16; head_dim 64 or 128; num_q_heads a multiple
 *                  of num_kv_heads.
 *   partition_size: 0 = library's schedule (balanced shares on the matrix
 *                  cores, then a merge kernel for the segments split between
 *                  waves, when the algo resolves to MFMA and the cache is
 *                  16-bit or FP8; else fixed partitions of its choice), else
 *                  a multiple of 16 in [16, 2^20] (fixed partitions plus the
 *                  reduction kernel when a context spans several).  On the
 *                  matrix cores, with several partitions, a persistent grid
 *                  computes the partitions (each one whole in one wave, the
 *                  waves' shares cut at partition boundaries); the result
 *                  does not depend on the grid size.
 *   workspace    : device memory of at least pkv_decode_workspace_size(...)
 *                  bytes (may be NULL when that is 0).  Its contents on entry
 *                  do not matter; calls sharing one workspace must not
 *                  overlap in time. */
pkv_status pkv_paged_decode_attention(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
                                      int32_t kv_dtype, float k_scale, float v_scale,
                                      int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Same as pkv_paged_decode_attention with an explicit kernel family. */
pkv_status pkv_paged_decode_attention_algo(void* out, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_blocks_per_seq,
                                           float scale, int32_t q_dtype, int32_t kv_dtype,
                                           float k_scale, float v_scale, int32_t partition_size,
                                           void* workspace, size_t workspace_bytes,
                                           int32_t algo, void* stream);

/* Same as pkv_paged_decode_attention_algo, and stamps caller-created HIP
 * events (hipEvent_t passed as void*, NULL = skip) for timing the kernels
 * from outside the library.  ev_begin and ev_mid are stamped by the decode
 * kernel's own dispatch (hipExtLaunchKernel) at its start and end, so they
 * bracket that kernel alone; ev_end by the end of the merge or reduction
 * kernel, or recorded on `stream` right after the decode kernel when the
 * call runs a single pass. */
pkv_status pkv_paged_decode_attention_profiled(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, float k_scale, float v_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, int32_t algo, void* stream, void* ev_begin, void* ev_mid,
    void* ev_end);

/* The decode step's append and its attention in one call: the result is that
 * of pkv_paged_cache_append(k_cache, v_cache, k_new, v_new, slot_mapping,
 * num_tokens = num_seqs, ..., new_dtype = q_dtype, kv_dtype, k_scale,
 * v_scale) followed by pkv_paged_decode_attention_profiled with the other
 * arguments ("Transformer 推理优化：KV Cache、PagedAttention 与 vLLM",
 * sections 2.2 and 3.3: a decode step stores the new token's K and V at its
 * slot, then attends over the whole context).  On the MFMA paths (fixed
 * partitions, the balanced grid, partitions on the persistent grid) the
 * decode kernel writes the rows itself, with no append launch before it:
 * every wave that consumes the slot's block puts the encoded row into the
 * loaded tile, so no read waits for the write.  The vector kernel
 * (algo = vector, f32 caches, MHA under AUTO) runs the append kernel first.
 *   k_new, v_new : device [num_seqs][num_kv_heads][head_dim] in q_dtype,
 *                  16-byte aligned: sequence s's new row.
 *   slot_mapping : device int64[num_seqs].  Negative: sequence s appends
 *                  nothing.  Otherwise a slot in a block that no other
 *                  sequence's context reads (a block being written is
 *                  private: copy-on-write, same page, section 3.5), distinct
 *                  across sequences; normally the slot of the context's last
 *                  token, block_tables[s][(L-1)/16] * 16 + (L-1) % 16 with
 *                  L = context_lens[s].  A slot in a block that another
 *                  sequence reads is still written, but that sequence's
 *                  output is then unspecified.
 *   events       : as for pkv_paged_decode_attention_profiled (they stamp
 *                  the decode kernel, not an append launched before it).
 * FP8/INT8 scales must be finite and > 0 (the append's rule); other errors as
 * for pkv_paged_decode_attention_profiled. */
pkv_status pkv_paged_decode_attention_appending(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int64_t* slot_mapping, void* k_cache, void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    float scale, int32_t q_dtype, int32_t kv_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t algo, void* stream,
    void* ev_begin, void* ev_mid, void* ev_end);

/* Decode over an FP8 or INT8 cache with per-channel scales (see
 * pkv_paged_cache_append_per_channel): the K element of (token, kv-head h,
 * dim i) is code * k_scales[h*head_dim + i], likewise V.  The K scales are
 * folded into q (q_i * k_scales_i in binary32, entering the matrix cores as a
 * 16-bit head plus remainder, about 16 mantissa bits); the V scales multiply
 * each output dim.  Arguments, schedules, workspace, algo and events as for
 * pkv_paged_decode_attention_profiled.  PKV_ERR_UNSUPPORTED for a 16-bit or
 * f32 cache; multi-query calls take per-tensor scales only. */
pkv_status pkv_paged_decode_attention_per_channel(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, const float* k_scales, const float* v_scales, int32_t partition_size,
    void* workspace, size_t workspace_bytes, int32_t algo, void* stream, void* ev_begin,
    void* ev_mid, void* ev_end);

/* Bytes of the static device scratch array of pkv_paged_decode_attention_noalloc
 * (one per GPU, held until the process ends): 32 MiB. */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * call as pkv_paged_decode_attention_algo (same arguments, schedules, kernels
 * and results, bit for bit) without the workspace: the partial results of
 * split contexts go to a static device array of the library, one per GPU, of
 * PKV_NOALLOC_SCRATCH_BYTES.  The call allocates nothing: the first call on a
 * device only looks the array's address up (hipGetSymbolAddress) and keeps it.
 *   - A call whose schedule needs more than PKV_NOALLOC_SCRATCH_BYTES (compare
 *     pkv_decode_workspace_size) returns PKV_ERR_WORKSPACE before anything is
 *     launched; a larger partition_size needs less.
 *   - Every call on one GPU shares that GPU's array.  Its contents on entry do
 *     not matter (a call writes every partial it reads), but calls that
 *     overlap in time on one GPU (other streams, other threads) race on it and
 *     may corrupt each other's results: serialise them.
 * Errors as for pkv_paged_decode_attention; PKV_ERR_HIP if the array's
 * address cannot be looked up. */
pkv_status pkv_paged_decode_attention_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, float k_scale, float v_scale, int32_t partition_size, int32_t algo,
    void* stream);

/* ------------------------------------------- multi-query attention -- */

/* Several query rows per sequence in one pass: a chunk of a long prompt
 * ("vLLM推理引擎深度解析", section 3.3; "推理加速三板斧", section 4.5: prompts
 * cut into chunks of about 512 tokens and scheduled with decode requests) or
 * the draft tokens a target model verifies at once ("大语言模型推理引擎深度剖析",
 * section 4.1).  Sequence s owns rows query_start[s] .. query_start[s+1]-1 of
 * q and out; they are its last n positions, appended to the cache before the
 * call (pkv_paged_cache_append), so row i sits at position
 * context_lens[s] - n + i and attends to positions 0 .. that position
 * through the block table (each token sees its prefix,
 * "KV Cache 与 PageAttention深度实战", section 1.2).  One row per sequence is
 * exactly pkv_paged_decode_attention.
 *   q, out       : device [num_rows][num_q_heads][head_dim], q dtype (F16 or
 *                  BF16); rows no sequence owns are not written.
 *   query_start  : device int32[num_seqs + 1], non-decreasing; rows are
 *                  clamped to [0, num_rows).  A sequence's rows past
 *                  max_query_len are not computed (with partitions their
 *                  output is unspecified): pass the largest row count.
 *   caches       : the q dtype or FP8_E4M3, as for decode; block_tables,
 *                  context_lens, block_size, num_blocks, scale, k_scale,
 *                  v_scale as for decode.  Rows with n > context_lens[s]
 *                  whose position is negative get zeros.
 *   partition_size: 0 = pkv_multiquery_partition_size's choice, else a
 *                  multiple of 16 (fixed partitions).  With more than one
 *                  partition, or with the balanced schedule, the call needs
 *                  a 256-byte-aligned workspace of
 *                  pkv_multiquery_workspace_size bytes and runs a second,
 *                  merging kernel.
 * Runs on the matrix cores: 16 MFMA columns are 16 / min(g, 16) rows times
 * min(g, 16) q-heads of one kv-head.  The balanced schedule splits the
 * blocks that every (sequence, row tile, kv-head) must read into equal
 * shares of a persistent grid, as the balanced decode schedule does, so
 * ragged contexts leave no CU idle.  partition_size 0 takes it when one
 * workgroup per (sequence, kv-head chunk, row tile) would give fewer than
 * 2048 workgroups, num_seqs <= 2048 and num_seqs x ceil(max_query_len /
 * rows per tile) <= 4096 (draft verification of a few rows); otherwise the
 * fixed grid runs.  Errors as for decode; PKV_ERR_UNSUPPORTED
 * for f32 q, head_dim not in {64, 128}, or a grid beyond 65535 sequences,
 * 65535 kv-heads x row tiles or 2^31 rows x q-heads. */
pkv_status pkv_paged_multiquery_attention(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_rows, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, float scale, int32_t q_dtype, int32_t kv_dtype, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    void* stream);
/* The same, with events as for pkv_paged_decode_attention_profiled:
 * ev_begin and ev_mid stamped by the attention kernel's own dispatch,
 * ev_end by the end of the merging kernel (or recorded after a single pass);
 * any may be NULL. */
pkv_status pkv_paged_multiquery_attention_profiled(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_rows, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, float scale, int32_t q_dtype, int32_t kv_dtype, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    void* stream, void* ev_begin, void* ev_mid, void* ev_end);
/* Partition (tokens) a multi-query call with partition_size 0 uses: 0 for
 * the balanced schedule (see pkv_paged_multiquery_attention); otherwise one
 * pass over max_blocks_per_seq * 16 tokens when the sequences x kv-heads x
 * row tiles reach 2048 workgroups, else 512 to 128 tokens.  partition_size
 * > 0 is returned as is.  -1 on bad arguments. */
int32_t pkv_multiquery_partition_size(int32_t num_seqs, int32_t max_query_len,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t max_blocks_per_seq, int32_t partition_size);
/* The partition_size to pass for a multi-query batch whose context lengths
 * the caller holds on the host (context_lens, host int32[num_seqs]).  Where
 * pkv_multiquery_partition_size(..., 0) picks the balanced schedule, this
 * weighs it against one fixed pass of max_blocks_per_seq * 16 tokens, which
 * then runs four column tiles per wave: the single pass when its workgroups
 * (at most two per CU) finish no later than the balanced shares plus their
 * merge, as with uniform draft verification.  Returns 0 or
 * max_blocks_per_seq * 16 then; otherwise what pkv_multiquery_partition_size
 * returns.  -1 on bad arguments (context_lens NULL with num_seqs > 0). */
int32_t pkv_multiquery_partition_size_for_lengths(const int32_t* context_lens, int32_t num_seqs,
                                                  int32_t max_query_len, int32_t num_q_heads,
                                                  int32_t num_kv_heads, int32_t max_blocks_per_seq,
                                                  int32_t kv_dtype);
/* Workspace bytes of a multi-query call.  Balanced schedule: float
 * (m, l)[2 W][16][2] and acc[2 W][16][head_dim] for the W = 4 x
 * (compute units of the current device) waves of its grid (two partial
 * slots per wave),
 * each part 256-byte aligned.  Fixed partitions: 0 for one partition, else
 * float m[rows][H_q][P], l[rows][H_q][P], acc[rows][H_q][P][head_dim], each
 * part 256-byte aligned.  SIZE_MAX on bad arguments. */
size_t pkv_multiquery_workspace_size(int32_t num_rows, int32_t num_seqs, int32_t max_query_len,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_blocks_per_seq,
                                     int32_t partition_size);

/* ------------------------------------------------------------ swapping -- */

/* Copy whole blocks between two caches of the same layout ([blocks][H_kv]
 * [16][d], block_bytes per block of one cache), K and V: for i < num_pairs,
 * block src_dst_pairs[2i] of (src_k, src_v) goes to block src_dst_pairs[2i+1]
 * of (dst_k, dst_v).  Either side may be pinned host memory
 * (hipHostMalloc), which the kernel reads or writes through its mapping:
 * swapping a preempted request's blocks to host DRAM and back
 * ("大语言模型推理引擎深度剖析", section 3.3, bounded by the host link).
 *   src_dst_pairs : int32[num_pairs][2] readable by the device; a pair with
 *                   an id outside [0, src_num_blocks) or [0, dst_num_blocks)
 *                   is skipped.  When src and dst are the same cache, no
 *                   destination may also be a source of the call.
 *   block_bytes   : a multiple of 16; caches 16-byte aligned.
 * Every buffer must be device memory or pinned host memory: the call looks
 * each one up (hipPointerGetAttributes) and returns PKV_ERR_INVALID_ARG for
 * memory a kernel cannot reach, such as pageable host memory.
 * Asynchronous on stream. */
pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                           const void* src_v, int32_t src_num_blocks,
                           const int32_t* src_dst_pairs, int32_t num_pairs, int64_t block_bytes,
                           void* stream);

/* ---------------------------------------------------- copy-on-write copy -- */

/* Copy whole physical blocks, K and V: for i < num_pairs, block
 * src_dst_pairs[2i] is copied into block src_dst_pairs[2i+1] ("大语言模型推理
 * 引擎深度剖析", section 2.3: a shared block is copied before it is written).
 *   src_dst_pairs : device int32[num_pairs][2]; pairs with an id outside
 *                   [0, num_blocks) are skipped.  Destinations must be
 *                   distinct and no destination may be a source.
 *   block_bytes   : bytes of one physical block of one cache
 *                   (num_kv_heads * block_size * head_dim * element bytes),
 *                   a multiple of 16.
 * The caches and the pairs must be device memory or pinned host memory: the
 * call looks each pointer up (hipPointerGetAttributes) and returns
 * PKV_ERR_INVALID_ARG for memory no kernel can reach (pageable host memory)
 * before launching anything. */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                           int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                           void* stream);

/* ------------------------------------------------------ host block pool -- */

/* Host-side pool of physical block ids with reference counts ("vLLM推理引擎
 * 深度解析", section 2.2; "大语言模型推理引擎深度剖析", sections 2.2-2.3).
 * Free ids wait in a FIFO queue (initially free_order, or 0..num_blocks-1
 * when free_order is NULL); a block whose count falls to 0 joins its tail.
 * Every operation is O(1) per block touched.  A pool is not thread-safe:
 * one owner at a time.  Block tables are caller-owned host int32 arrays. */
typedef struct pkv_pool pkv_pool;

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);
/* Take the block at the head of the free queue (count becomes 1). */
pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t* block_out);
/* Count += 1 for a block in use; PKV_ERR_REFCOUNT for a free block. */
pkv_status pkv_pool_incref(pkv_pool* pool, int32_t block);
/* Count -= 1; at 0 the block joins the free queue.  PKV_ERR_REFCOUNT for a
 * free block. */
pkv_status pkv_pool_decref(pkv_pool* pool, int32_t block);
/* Count of a block (0 = free), or -1 for an id out of range. */
int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t block);
int32_t pkv_pool_num_free(const pkv_pool* pool);
int32_t pkv_pool_num_blocks(const pkv_pool* pool);
int32_t pkv_pool_block_size(const pkv_pool* pool);
/* Copy the free queue, head first, into out[0..cap); *n receives its length.
 * PKV_ERR_INVALID_ARG if cap is too small (nothing written then). */
pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* A new table holding ceil(prompt_len / block_size) freshly allocated blocks.
 * table: host int32[cap]; *nblocks receives the count. */
pkv_status pkv_seq_create(pkv_pool* pool, int32_t prompt_len, int32_t* table, int32_t cap,
                          int32_t* nblocks);
/* Share every block of a table with a new sequence: each count += 1.  The
 * caller copies the table itself. */
pkv_status pkv_seq_fork(pkv_pool* pool, const int32_t* table, int32_t nblocks);
/* Slots for the n_new positions cur_len .. cur_len+n_new-1 of a sequence whose
 * table is table[0..*nblocks).  A position past the table takes a new block
 * (a new block every block_size tokens); a position in an existing block whose
 * count is above 1 first gets a private copy: a new block replaces it in the
 * table, the old count drops by one and (src, dst) is appended to
 * cow_pairs[2*k], cow_pairs[2*k+1] for the caller to copy on the device with
 * pkv_copy_blocks.  slots_out: host int64[n_new].  cow_pairs: host
 * int32[2*cow_cap] (may be NULL if cow_cap is 0); *n_cow receives the count.
 * All-or-nothing: PKV_ERR_OUT_OF_BLOCKS (pool too small),
 * PKV_ERR_INVALID_ARG (gap after the table, table capacity or cow_cap too
 * small) leave the pool and the table unchanged. */
pkv_status pkv_seq_append_slots(pkv_pool* pool, int32_t* table, int32_t* nblocks, int32_t cap,
                                int32_t cur_len, int32_t n_new, int64_t* slots_out,
                                int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow);
/* One decode step's bookkeeping for a whole batch in one call ("vLLM推理引擎
 * 深度解析", section 2.2: a new block each time 16 more tokens are produced;
 * "大语言模型推理引擎深度剖析", section 2.3: a shared block is copied before it
 * is written).  The same as pkv_seq_append_slots applied to sequences
 * 0 .. num_seqs-1 in that order, on the decode layout directly:
 *   block_tables : host int32[num_seqs][max_blocks_per_seq], row s is sequence
 *                  s's table; entries past nblocks[s] are free to overwrite.
 *   nblocks      : host int32[num_seqs], blocks in each row (in/out).
 *   context_lens : host int32[num_seqs], tokens already held (in); on return
 *                  each has grown by its n_new, as the decode call expects.
 *   n_new        : host int32[num_seqs] positions to add per sequence, or NULL
 *                  for one each (a decode step).
 *   slot_mapping : host int64[sum of n_new], slots of the new positions,
 *                  sequence by sequence, as pkv_paged_cache_append takes them.
 *   cow_pairs    : host int32[2*cow_cap]: (src, dst) for pkv_copy_blocks, in
 *                  the order the copies are made; *n_cow receives their count
 *                  and *n_slots (may be NULL) the length of slot_mapping.
 * A shared block written by several sequences of the batch is copied by all
 * but the last of its holders when every holder writes it.  All-or-nothing:
 * any error (PKV_ERR_OUT_OF_BLOCKS, or PKV_ERR_INVALID_ARG for a gap, a full
 * row, a bad block, cow_cap too small) leaves the pool, the tables, nblocks
 * and context_lens unchanged. */
pkv_status pkv_batch_append_slots(pkv_pool* pool, int32_t* block_tables,
                                  int32_t max_blocks_per_seq, int32_t* nblocks,
                                  int32_t* context_lens, const int32_t* n_new, int32_t num_seqs,
                                  int64_t* slot_mapping, int32_t* cow_pairs, int32_t cow_cap,
                                  int32_t* n_cow, int32_t* n_slots);
/* Prefix caching ("vLLM推理引擎深度解析", section 4.1: computed KV blocks of
 * shared prompts are cached and reused; "KV Cache 与 PageAttention深度实战",
 * section 4.2: an LRU cache of computed prefix blocks that a request with the
 * same prefix reuses directly).  A full block is known by the exact key
 * (parent block, the parent's allocation generation, its block_size token
 * ids), the first block's parent being -1.  Registered blocks stay findable
 * while in use and after release, at the tail of the free queue, until
 * allocation reaches them at the head (least recently freed first) and
 * evicts them; a block's generation advances at every hand-out, so a chain
 * whose parent was reused never matches.  Blocks never registered behave as
 * before; a pool that is never asked to register behaves exactly as without
 * caching.
 *
 * A table for a prompt of token ids: its longest run of cached full blocks
 * from the start is reused (one more reference each; a free one leaves the
 * queue), the rest are new blocks.  table: host int32[cap]; *nblocks receives
 * ceil(prompt_len / block_size), *cached_tokens the tokens whose K/V are
 * already in the reused blocks (a multiple of block_size).  All-or-nothing:
 * PKV_ERR_OUT_OF_BLOCKS or PKV_ERR_INVALID_ARG (cap too small) change
 * nothing. */
pkv_status pkv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int32_t prompt_len,
                                int32_t* table, int32_t cap, int32_t* nblocks,
                                int32_t* cached_tokens);
/* Declare the full blocks among the first num_tokens tokens of a sequence
 * (table[0..nblocks), tokens[0..num_tokens)) computed: each becomes findable
 * under its key, unless another block already holds that key (it then stays
 * unregistered).  Call it once the K/V of those tokens are in the cache.
 * PKV_ERR_INVALID_ARG if a block is registered under another key,
 * PKV_ERR_REFCOUNT for a free block; nothing changes on an error. */
pkv_status pkv_pool_register_blocks(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                                    const int32_t* table, int32_t nblocks);
/* Blocks currently findable in the prefix cache (-1 for NULL). */
int32_t pkv_pool_cached_blocks(const pkv_pool* pool);
/* Swap a sequence to another pool: the pools stand for device blocks and
 * host-memory blocks ("大语言模型推理引擎深度剖析", section 3.3: under memory
 * pressure a request's blocks move from HBM to host DRAM and come back
 * without recomputation; "KV Cache 与 PageAttention深度实战", section 4.1).
 * Takes nblocks blocks of `to` in free-queue order into table_out, writes
 * (table[i], table_out[i]) to pairs_out[2i], pairs_out[2i+1] for
 * pkv_swap_blocks, then releases `table` in `from` as pkv_seq_free does
 * (blocks shared with other sequences stay).  from == to is allowed (every
 * new block is taken before any is released).  table_out: host int32[nblocks];
 * pairs_out: host int32[2*nblocks].  All-or-nothing: PKV_ERR_OUT_OF_BLOCKS,
 * PKV_ERR_REFCOUNT or PKV_ERR_INVALID_ARG (bad id, block sizes differ) change
 * neither pool. */
pkv_status pkv_seq_swap(pkv_pool* from, pkv_pool* to, const int32_t* table, int32_t nblocks,
                        int32_t* table_out, int32_t* pairs_out);
/* Release a sequence: decref its blocks from the last to the first. */
pkv_status pkv_seq_free(pkv_pool* pool, const int32_t* table, int32_t nblocks);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
