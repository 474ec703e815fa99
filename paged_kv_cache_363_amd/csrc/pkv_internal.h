// Internal declarations shared by the library's translation units.
#pragma once
#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Record a message for pkv_last_error() on this thread and return `st`.
pkv_status fail(pkv_status st, const char* fmt, ...);
void clear_error();

inline int elem_bytes(int32_t dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    case PKV_INT8: return 1;
  }
  return 0;
}

// Caches of one-byte codes with a per-tensor scale (E4M3 or INT8): the
// kernels widen the codes in registers and fold the scales in.
inline constexpr bool byte_codes(int32_t dt) { return dt == PKV_FP8_E4M3 || dt == PKV_INT8; }

constexpr int kBlockSize = 16;   // tokens per physical block
constexpr int kWaves = 4;        // waves per decode workgroup
constexpr int kMaxPartition = 1 << 20;
constexpr int kMaxStreamSeqs = 2048;        // sequences the balanced schedule handles per call
constexpr int kDefaultCUs = 256;            // an MI355X, when no device answers
// Compute units of the calling thread's current HIP device, read once per
// device; kDefaultCUs when no device is visible (the host planners still
// answer on a machine without one).
int32_t device_cus();
// XCDs (compute dies, each with its own L2) of the current device, read once
// per device; 8 (an MI355X) when no device answers.
int32_t device_xccs();
// Workgroups of 4 waves the balanced schedules launch for calls made by the
// calling thread: the device's CU count (one wave per SIMD) unless the
// thread set an override (pkv_set_stream_workgroups).
int32_t stream_workgroups();
constexpr int kMaxStreamTiles = 4096;        // (sequence, row tile) pairs of a balanced multi-query call

// Units a schedule charges for starting a piece of a segment, in blocks.
// Where a piece starts with its own load pipeline (the one-workgroup-per-
// partition kernels, the multi-query kernels) a start costs about two loaded
// HBM round trips (q rows and block ids, then the first K/V tiles), ~2 us,
// against ~1.3 us per 16-bit block and ~0.7 us per E4M3 block per wave at one
// wave per SIMD: 4 and 3 units.  The balanced decode kernel keeps one load
// pipeline through a wave's whole share, so a new piece costs only the close
// of the previous one and the q rows staged in LDS; 2 units measured best on
// a ragged batch (Qwen3-8B-shaped, 64 sequences of 256..4096 tokens: 88.8 us
// at 1 unit, 88.5 at 2, 89.0 at 4) and on 32K contexts.
#ifndef PKV_RESTART_UNITS_16
#define PKV_RESTART_UNITS_16 4
#endif
#ifndef PKV_RESTART_UNITS_FP8
#define PKV_RESTART_UNITS_FP8 3
#endif
#ifndef PKV_STREAM_RESTART_UNITS
#define PKV_STREAM_RESTART_UNITS 2
#endif
inline int kv_restart_units(int32_t kv_dtype) {
  return byte_codes(kv_dtype) ? PKV_RESTART_UNITS_FP8 : PKV_RESTART_UNITS_16;
}
inline int stream_restart_units(int32_t) { return PKV_STREAM_RESTART_UNITS; }

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq;
  int32_t q_dtype, kv_dtype;
  float scale, k_scale, v_scale;
  int32_t partition;   // tokens per partition
  int32_t num_parts;   // max partitions per sequence (1 = single pass)
  float* ws_m;         // [S][Hq][P]
  float* ws_l;         // [S][Hq][P]
  float* ws_acc;       // [S][Hq][P][D]
  void* stream;
  // events the next launch's dispatch timestamps itself (launch_kernel)
  void* ev_start = nullptr;
  void* ev_stop = nullptr;
  // per-channel scales of a one-byte-code cache, device float[H_kv][D] each;
  // nullptr: k_scale / v_scale apply to the whole tensor
  const float* k_scales = nullptr;
  const float* v_scales = nullptr;
  // the step's new K/V rows [S][H_kv][D] (q dtype) and their slots, appended
  // by the decode kernel (nullptr: the caches already hold them)
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int64_t* slots = nullptr;
  float k_inv = 1.0f, v_inv = 1.0f;
};

// Multi-query call: rows query_start[s] .. query_start[s+1]-1 belong to
// sequence s (at most max_query_len of them are computed).
struct MQArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t num_seqs, num_rows, max_query_len;
  int32_t num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq;
  int32_t q_dtype, kv_dtype;
  float scale, k_scale, v_scale;
  int32_t partition;   // tokens per partition
  int32_t num_parts;   // partitions in the grid (1 = single pass)
  float* ws_m;         // [rows][Hq][P]
  float* ws_l;         // [rows][Hq][P]
  float* ws_acc;       // [rows][Hq][P][D]
  int32_t max_ntl;      // column tiles per wave at most (the plan's choice)
  // balanced schedule (launch_multiquery_stream): workers and partial slots
  int32_t stream_grid;  // workgroups of 4 waves
  float* st_ml;         // [2 W][16][2]
  float* st_part;       // [2 W][16][D]
  void* stream;
  // events the next launch's dispatch timestamps itself (launch_kernel)
  void* ev_start = nullptr;
  void* ev_stop = nullptr;
};

// Column layout of a multi-query MFMA tile: 16 columns = qpt query rows x
// chunk q-heads of one kv-head; hchunks head groups per kv-head.  One wave
// carries ntl such column tiles (ntl * qpt consecutive rows, a row tile)
// against each K/V load, at most max_ntl (1, 2 or 4) and no more than the
// rows need; qtiles row tiles cover max_query_len rows.
struct MQTiles {
  int chunk, hchunks, qpt, ntl, qtiles;
};
inline MQTiles mq_tiles(int g, int max_query_len, int max_ntl) {
  MQTiles t;
  t.chunk = g < 16 ? g : 16;
  t.hchunks = (g + t.chunk - 1) / t.chunk;
  t.qpt = 16 / t.chunk;
  const int col_tiles = (max_query_len + t.qpt - 1) / t.qpt;
  t.ntl = col_tiles >= 4 ? 4 : (col_tiles >= 2 ? 2 : 1);
  if (t.ntl > max_ntl) t.ntl = max_ntl;
  t.qtiles = (max_query_len + t.qpt * t.ntl - 1) / (t.qpt * t.ntl);
  return t;
}

// Argument checks, schedule choice and launches of every decode entry point
// (pkv_capi.cpp); k_scales / v_scales: per-channel scales or nullptr.
pkv_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
                       int32_t kv_dtype, float k_scale, float v_scale, const float* k_scales,
                       const float* v_scales, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, int32_t algo, void* stream, void* ev_begin,
                       void* ev_mid, void* ev_end, const void* k_new = nullptr,
                       const void* v_new = nullptr, const int64_t* slot_mapping = nullptr,
                       float k_inv = 1.0f, float v_inv = 1.0f);

// Kernel launchers (return hipError_t as int).
int launch_multiquery(const MQArgs& a);
int launch_multiquery_reduce(const MQArgs& a);
int launch_multiquery_stream(const MQArgs& a);
int launch_multiquery_split_merge(const MQArgs& a);
int launch_decode_vector(const DecodeArgs& a);
int launch_decode_mfma(const DecodeArgs& a);
int launch_decode_reduce(const DecodeArgs& a);
int launch_decode_stream(const DecodeArgs& a, int grid, void* ws, size_t off_ml, size_t off_part);
// fixed partitions on the persistent grid: partials into a.ws_m / ws_l / ws_acc
int launch_decode_stream_parts(const DecodeArgs& a, int grid);
int launch_decode_split_merge(const DecodeArgs& a, int grid, void* ws, size_t off_ml,
                              size_t off_part);
int launch_cache_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                        const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int32_t num_blocks, int32_t new_dtype, int32_t kv_dtype,
                        float k_inv_scale, float v_inv_scale, void* stream,
                        const float* k_scales = nullptr, const float* v_scales = nullptr);
int launch_swap_blocks(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k,
                       const void* src_v, int32_t src_blocks, const int32_t* pairs,
                       int32_t num_pairs, int64_t block_bytes, void* stream);
int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                       int32_t num_blocks, int64_t block_bytes, void* stream);

}  // namespace pkv
