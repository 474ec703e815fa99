// C ABI entry points: argument checks, partition and workspace sizing,
// kernel-family choice and launches.  Nothing here computes attention; every
// step of the decode path runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <functional>
#include <queue>
#include <vector>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "pkv.h"
#include "pkv_internal.h"
#include "pkv_probe.h"

namespace pkv {

static thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bool valid_dtype(int32_t dt) { return dt >= PKV_F32 && dt <= PKV_INT8; }

// (q, kv) dtype pairs the decode kernels implement.
static bool decode_pair_ok(int32_t q, int32_t kv) {
  if (q == PKV_F32) return kv == PKV_F32;
  if (q == PKV_F16) return kv == PKV_F16 || byte_codes(kv);
  if (q == PKV_BF16) return kv == PKV_BF16 || byte_codes(kv);
  return false;
}

static int32_t choose_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx) {
  // One workgroup per (sequence, kv-head) already gives 8 workgroups per CU
  // of a 256-CU MI355X: run single-pass, with no partials and no reduction.
  if ((int64_t)num_seqs * num_kv_heads >= 2048) return max_ctx > kBlockSize ? max_ctx : kBlockSize;
  // Otherwise enough partitions to cover the CUs several times over, without
  // cutting contexts into slivers whose partials cost more than they save.
  int32_t ps = 512;
  while (ps > 128) {
    const int64_t units = (int64_t)num_seqs * num_kv_heads * ((max_ctx + ps - 1) / ps);
    if (units >= 2048) break;
    ps /= 2;
  }
  return ps;
}

// AUTO: the matrix cores when the q-head group makes QK^T and PV real
// contractions (g > 1) and the dtypes allow it; for g = 1 an MFMA tile would
// use one of its 16 columns, so the vector kernel serves.
static int32_t resolve_algo(int32_t g, int32_t q, int32_t kv) {
  const bool mfma_ok = (q == PKV_F16 || q == PKV_BF16) && (kv == q || byte_codes(kv));
  return mfma_ok && g > 1 ? PKV_ALGO_MFMA : PKV_ALGO_VECTOR;
}

int32_t device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  if (dev < kMaxDevices) {
    const int32_t v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = kDefaultCUs;
  }
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int32_t device_xccs() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 8;
  }
  if (dev < kMaxDevices) {
    const int32_t v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 8;
  }
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// 0: no override (the device's CU count)
static thread_local int32_t t_stream_workgroups = 0;

int32_t stream_workgroups() {
  return t_stream_workgroups > 0 ? t_stream_workgroups : device_cus();
}

#ifndef PKV_PARTS_ON_STREAM_GRID
#define PKV_PARTS_ON_STREAM_GRID 1
#endif
// MFMA calls with fixed partitions run on the persistent grid (one pipelined
// pass per wave through whole partitions) rather than one workgroup per
// partition.
constexpr bool kPartsOnStreamGrid = PKV_PARTS_ON_STREAM_GRID != 0;

struct Plan {
  // fixed partitions (the partition kernels plus the reduction kernel)
  int32_t partition;
  int32_t num_parts;
  size_t ws_bytes;   // max over the schedules this call may use
  size_t off_l, off_acc;
  // balanced schedule (partition_size == 0, MFMA-capable caches)
  bool stream_ok;
  // the fixed partitions on the balanced schedule's persistent grid
  // (partition_size > 0 with more than one partition, MFMA-capable caches)
  bool parts_stream_ok;
  int32_t stream_grid;
  size_t stream_off_ml, stream_off_part, stream_bytes;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool stream_capable_kv(int32_t kv_dtype) {
  return kv_dtype == PKV_F16 || kv_dtype == PKV_BF16 || byte_codes(kv_dtype);
}

static bool make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t kv_dtype,
                      int32_t partition_size, Plan* plan) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq < 0 || partition_size < 0 || num_q_heads % num_kv_heads != 0)
    return false;
  if (partition_size > 0 && (partition_size % kBlockSize != 0 || partition_size > kMaxPartition))
    return false;
  const int32_t max_ctx = max_blocks_per_seq * kBlockSize;
  const int32_t ps = partition_size > 0 ? partition_size
                                        : choose_partition(num_seqs, num_kv_heads, max_ctx);
  plan->partition = ps;
  plan->num_parts = max_ctx <= ps ? 1 : (max_ctx + ps - 1) / ps;
  plan->off_l = plan->off_acc = 0;
  size_t fixed_bytes = 0;
  if (plan->num_parts > 1) {
    const size_t rows = (size_t)num_seqs * num_q_heads * plan->num_parts;
    const size_t bm = align256(rows * sizeof(float));
    plan->off_l = bm;
    plan->off_acc = 2 * bm;
    fixed_bytes = 2 * bm + align256(rows * head_dim * sizeof(float));
  }
  // balanced schedule: every sequence's block count fits the in-LDS prefix
  // and the unit count stays below 2^31
  const int32_t g = num_q_heads / num_kv_heads;
  const int32_t chunk = g < 16 ? g : 16;
  const int64_t Y = (int64_t)num_kv_heads * ((g + chunk - 1) / chunk);
  const bool grid_ok = stream_capable_kv(kv_dtype) && num_seqs <= kMaxStreamSeqs &&
                       (int64_t)num_seqs * (max_blocks_per_seq + stream_restart_units(kv_dtype)) * Y <
                           ((int64_t)1 << 31);
  plan->stream_ok = partition_size == 0 && grid_ok;
  plan->parts_stream_ok = kPartsOnStreamGrid && partition_size > 0 && plan->num_parts > 1 && grid_ok;
  plan->stream_grid = stream_workgroups();
  plan->stream_off_ml = plan->stream_off_part = plan->stream_bytes = 0;
  if (plan->stream_ok) {
    const size_t workers = (size_t)plan->stream_grid * 4;
    const size_t ml = align256(2 * workers * chunk * 2 * sizeof(float));
    plan->stream_off_ml = 0;
    plan->stream_off_part = ml;
    plan->stream_bytes = ml + align256(2 * workers * chunk * head_dim * sizeof(float));
  }
  plan->ws_bytes = fixed_bytes > plan->stream_bytes ? fixed_bytes : plan->stream_bytes;
  return true;
}

// Multi-query calls

struct MQPlan {
  int32_t partition, num_parts;   // partition 0: the balanced schedule
  int32_t max_ntl;                 // column tiles per wave at most
  size_t off_l, off_acc, ws_bytes;
  bool stream;                     // balanced schedule (partition_size 0)
  int32_t stream_grid;
  size_t st_off_part;              // the (m, l) slots start the workspace
};

// The fixed grid with four column tiles per wave has at most two workgroups
// per CU.
static bool mq_small_grid(int32_t num_seqs, int32_t num_kv_heads, int32_t g, int32_t mq) {
  const MQTiles t4 = mq_tiles(g, mq, 4);
  return (int64_t)num_seqs * num_kv_heads * t4.hchunks * t4.qtiles <= 2 * device_cus();
}

// Partition and workspace of a multi-query call; false on bad arguments.
bool mq_plan(int32_t num_rows, int32_t num_seqs, int32_t max_query_len, int32_t num_q_heads,
             int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
             int32_t partition_size, MQPlan* plan) {
  if (num_rows < 0 || num_seqs < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || max_blocks_per_seq < 0 || partition_size < 0 ||
      num_q_heads % num_kv_heads != 0)
    return false;
  if (partition_size > 0 && (partition_size % kBlockSize != 0 || partition_size > kMaxPartition))
    return false;
  const int32_t max_ctx = max_blocks_per_seq * kBlockSize;
  const int32_t g = num_q_heads / num_kv_heads;
  const int32_t mq = max_query_len > 0 ? max_query_len : 1;
  // Balanced schedule, with up to four column tiles per wave: partition_size
  // 0 and a fixed grid of one workgroup per (sequence, kv-head chunk, row
  // tile) too small to fill the chip (the same 2048 as choose_partition:
  // below it the fixed path would cut the contexts into partitions), while
  // the sequences and their row tiles fit the in-LDS prefix sums and the
  // unit count stays below 2^31 (at the largest restart count).  Measured:
  // draft verification and mixed batches of a few rows gain; long prompt
  // chunks, whose fixed grid is large and whose tiles are compute-bound, run
  // faster on the fixed grid.
  {
    const MQTiles t = mq_tiles(g, mq, 4);
    const int64_t Y = (int64_t)num_kv_heads * t.hchunks;
    const int64_t tiles = (int64_t)num_seqs * t.qtiles;
    const int64_t r_max = kv_restart_units(PKV_BF16) > kv_restart_units(PKV_FP8_E4M3)
                              ? kv_restart_units(PKV_BF16)
                              : kv_restart_units(PKV_FP8_E4M3);
    plan->stream = partition_size == 0 && tiles * Y < 2048 && num_seqs <= kMaxStreamSeqs &&
                   tiles <= kMaxStreamTiles &&
                   tiles * (max_blocks_per_seq + r_max) * Y < ((int64_t)1 << 31);
    plan->stream_grid = stream_workgroups();
    plan->st_off_part = 0;
    if (plan->stream) {
      const size_t workers = (size_t)plan->stream_grid * kWaves;
      const size_t cols = (size_t)16 * t.ntl;   // columns of a row tile
      plan->max_ntl = 4;
      plan->partition = 0;
      plan->num_parts = 1;
      plan->off_l = plan->off_acc = 0;
      plan->st_off_part = align256(2 * workers * cols * 2 * sizeof(float));
      plan->ws_bytes = plan->st_off_part + align256(2 * workers * cols * head_dim * sizeof(float));
      return true;
    }
  }
  // Fixed grid: four column tiles per wave.  Each K/V load and its widening
  // serve four times the columns of one tile, and a (sequence, kv-head) is
  // read once instead of once per pair of tiles.  Four tiles' accumulators
  // leave one wave per SIMD; since the tile update takes its logits against
  // the running references (no cross-lane maximum per block), that wave
  // keeps the matrix cores busier than two waves of two tiles.  Measured on
  // the fixed grid with 2 / 4 tiles: 8-row verification on the 70B-shaped
  // E4M3 cache 47.2 / 43.2 us, on its INT8 cache 48.4 / 46.4 us, 512-row
  // chunks at 32K tokens 9.19 / 7.86 ms, 64-row MHA chunks 401 / 404 us.
  plan->max_ntl = 4;
#ifdef PKV_MQ_FORCE_NTL
  plan->max_ntl = PKV_MQ_FORCE_NTL;
#endif
  const MQTiles t = mq_tiles(g, mq, plan->max_ntl);
  // workgroups per sequence and partition: kv-heads x head chunks x row tiles
  const int64_t per_seq = (int64_t)num_kv_heads * t.hchunks * t.qtiles;
  const int32_t ps = partition_size > 0
                         ? partition_size
                         : choose_partition(num_seqs, per_seq > INT32_MAX ? INT32_MAX
                                                                          : (int32_t)per_seq,
                                            max_ctx);
  plan->partition = ps;
  plan->num_parts = max_ctx <= ps ? 1 : (max_ctx + ps - 1) / ps;
  plan->off_l = plan->off_acc = plan->ws_bytes = 0;
  if (plan->num_parts > 1) {
    const size_t rows = (size_t)num_rows * num_q_heads * plan->num_parts;
    const size_t bm = align256(rows * sizeof(float));
    plan->off_l = bm;
    plan->off_acc = 2 * bm;
    plan->ws_bytes = 2 * bm + align256(rows * head_dim * sizeof(float));
  }
  return true;
}

}  // namespace pkv

using namespace pkv;

// Body of both append entry points; k_scales / v_scales: per-channel scales
// (device [H_kv][d]) of a one-byte-code cache, or nullptr for k_scale/v_scale.
static pkv_status append_impl(void* k_cache, void* v_cache, const void* k_new,
                              const void* v_new, const int64_t* slot_mapping,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t new_dtype,
                              int32_t kv_dtype, float k_scale, float v_scale,
                              const float* k_scales, const float* v_scales, void* stream) {
  clear_error();
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(PKV_ERR_INVALID_ARG, "cache_append: bad sizes");
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "cache_append: block_size must be 16 (got %d)", block_size);
  if (head_dim < 8 || head_dim > 256 || head_dim % 8 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "cache_append: head_dim must be a multiple of 8 in [8,256]");
  if (!valid_dtype(new_dtype) || !valid_dtype(kv_dtype))
    return fail(PKV_ERR_INVALID_ARG, "cache_append: bad dtype");
  if (byte_codes(new_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "cache_append: new rows must be f32, f16 or bf16");
  if (kv_dtype != new_dtype && !byte_codes(kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED,
                "cache_append: kv dtype must equal the new rows' dtype or be FP8/INT8");
  float k_inv = 1.0f, v_inv = 1.0f;
  if (byte_codes(kv_dtype)) {
    if (!(k_scale > 0.0f) || !std::isfinite(k_scale) || !(v_scale > 0.0f) ||
        !std::isfinite(v_scale))
      return fail(PKV_ERR_INVALID_ARG, "cache_append: FP8/INT8 scales must be finite and > 0");
    k_inv = 1.0f / k_scale;
    v_inv = 1.0f / v_scale;
  }
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "cache_append: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID_ARG, "cache_append: caches and new rows must be 16-byte aligned");
  int rc = launch_cache_append(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                               num_kv_heads, head_dim, num_blocks, new_dtype, kv_dtype, k_inv,
                               v_inv, stream, k_scales, v_scales);
  if (rc != 0) return fail(PKV_ERR_HIP, "cache_append: launch failed: %s",
                           hipGetErrorString((hipError_t)rc));
  return PKV_OK;
}

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_status_string(int32_t st) {
  switch (st) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PKV_ERR_REFCOUNT: return "reference count error";
    case PKV_ERR_HIP: return "HIP error";
    case PKV_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

int32_t pkv_version(void) { return 100; }

pkv_status pkv_set_stream_workgroups(int32_t n) {
  clear_error();
  if (n < 0 || n > 65535) return fail(PKV_ERR_INVALID_ARG, "set_stream_workgroups: bad count");
  t_stream_workgroups = n;
  return PKV_OK;
}

uint64_t pkv_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                int32_t dtype) {
  if (!valid_dtype(dtype) || layers < 0 || kv_heads < 0 || head_dim < 0) return 0;
  return 2ull * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim *
         (uint64_t)elem_bytes(dtype);
}

pkv_status pkv_paged_cache_append(void* k_cache, void* v_cache, const void* k_new,
                                  const void* v_new, const int64_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t new_dtype,
                                  int32_t kv_dtype, float k_scale, float v_scale, void* stream) {
  return append_impl(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens, num_kv_heads,
                     head_dim, block_size, num_blocks, new_dtype, kv_dtype, k_scale, v_scale,
                     nullptr, nullptr, stream);
}

pkv_status pkv_paged_cache_append_per_channel(void* k_cache, void* v_cache, const void* k_new,
                                              const void* v_new, const int64_t* slot_mapping,
                                              int32_t num_tokens, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, int32_t new_dtype,
                                              int32_t kv_dtype, const float* k_scales,
                                              const float* v_scales, void* stream) {
  clear_error();
  if (!byte_codes(kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "cache_append_per_channel: the cache must hold FP8 or INT8 codes");
  if (num_tokens > 0 && (!k_scales || !v_scales))
    return fail(PKV_ERR_INVALID_ARG, "cache_append_per_channel: NULL scale array");
  // the per-tensor scale checks see 1.0; each channel's scale is the caller's
  // contract (finite, > 0), read on the device
  return append_impl(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens, num_kv_heads,
                     head_dim, block_size, num_blocks, new_dtype, kv_dtype, 1.0f, 1.0f, k_scales,
                     v_scales, stream);
}

int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq, int32_t kv_dtype,
                                  int32_t partition_size) {
  Plan plan;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, kv_dtype,
                 partition_size, &plan))
    return -1;
  // AUTO runs the balanced schedule for a q-head group g > 1 (see resolve_algo)
  return plan.stream_ok && num_q_heads / num_kv_heads > 1 ? 0 : plan.partition;
}

int32_t pkv_decode_partition_size_for_lengths(const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_blocks_per_seq,
                                              int32_t kv_dtype) {
  const int32_t auto_ps = pkv_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                    max_blocks_per_seq, kv_dtype, 0);
  if (auto_ps != 0) return auto_ps;   // no balanced schedule to weigh (or bad arguments)
  if (num_seqs > 0 && !context_lens) return -1;
  const int64_t max_ctx = (int64_t)max_blocks_per_seq * kBlockSize;
  if (max_ctx == 0 || max_ctx > kMaxPartition) return 0;
  const int32_t g = num_q_heads / num_kv_heads;
  const int32_t chunk = g < 16 ? g : 16;
  const int64_t Y = (int64_t)num_kv_heads * ((g + chunk - 1) / chunk);
  const int64_t R = stream_restart_units(kv_dtype);   // a piece of the balanced schedule
  const int64_t Rf = kv_restart_units(kv_dtype);      // a wave's start in a fixed partition
  // Costs in block loads of one wave (both schedules stream at the same
  // per-wave rate; only the split differs).
  //  balanced: the grid's waves share all units equally, then the merge
  //            kernel runs (worth about kMergeUnits block loads);
  //  one fixed partition per (sequence, kv-head chunk): a workgroup's four
  //            waves take a quarter of the sequence each (plus one restart)
  //            and the workgroups start, in grid order, on whichever CU frees
  //            up first.
  constexpr int64_t kMergeUnits = 4;
  int64_t units = 0;
  std::vector<int64_t> work(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t len = context_lens[s] < 0 ? 0 : (context_lens[s] > max_ctx ? max_ctx : context_lens[s]);
    const int64_t nbk = (len + kBlockSize - 1) / kBlockSize;
    units += nbk > 0 ? nbk + R : 0;
    work[s] = nbk > 0 ? (nbk + kWaves - 1) / kWaves + Rf : 0;
  }
  if (units == 0) return 0;
  const int64_t W = (int64_t)stream_workgroups() * kWaves;
  const int64_t t_bal = (Y * units + W - 1) / W + kMergeUnits;
  // list scheduling of the fixed grid (kv-head chunk fastest, then sequence)
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int32_t i = 0, n = device_cus(); i < n; ++i) free_at.push(0);
  int64_t t_fix = 0;
  for (int32_t s = 0; s < num_seqs && t_fix <= t_bal; ++s) {
    for (int64_t y = 0; y < Y; ++y) {
      const int64_t t = free_at.top() + work[s];
      free_at.pop();
      free_at.push(t);
      if (t > t_fix) t_fix = t;
    }
  }
  return t_fix <= t_bal ? (int32_t)max_ctx : 0;
}

}  // extern "C"

namespace pkv {
int launch_stream_read_probe(const void* buf, int64_t buf_bytes, const int32_t* tile_ids,
                             int32_t num_tiles, uint32_t* sink, int32_t workgroups, void* stream,
                             void* ev_start, void* ev_stop);
}

extern "C" {

pkv_status pkv_stream_read_probe(const void* buf, int64_t buf_bytes, const int32_t* tile_ids,
                                 int32_t num_tiles, uint32_t* sink, int32_t workgroups,
                                 void* stream, void* ev_start, void* ev_stop) {
  clear_error();
  if (buf_bytes < 0 || num_tiles < 0 || workgroups < 1 || workgroups > 65535)
    return fail(PKV_ERR_INVALID_ARG, "stream_read_probe: bad sizes");
  if (!buf || !tile_ids || !sink)
    return fail(PKV_ERR_INVALID_ARG, "stream_read_probe: NULL pointer");
  if (!aligned16(buf))
    return fail(PKV_ERR_INVALID_ARG, "stream_read_probe: buf must be 16-byte aligned");
  const int rc = launch_stream_read_probe(buf, buf_bytes, tile_ids, num_tiles, sink, workgroups,
                                          stream, ev_start, ev_stop);
  if (rc != 0)
    return fail(PKV_ERR_HIP, "stream_read_probe: launch failed: %s",
                hipGetErrorString((hipError_t)rc));
  return PKV_OK;
}

size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t kv_dtype,
                                 int32_t partition_size) {
  Plan plan;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, kv_dtype,
                 partition_size, &plan))
    return SIZE_MAX;
  return plan.ws_bytes;
}

int32_t pkv_decode_algo_for(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t q_dtype, int32_t kv_dtype) {
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  if (head_dim != 64 && head_dim != 128) return -1;
  if (!decode_pair_ok(q_dtype, kv_dtype)) return -1;
  return resolve_algo(num_q_heads / num_kv_heads, q_dtype, kv_dtype);
}

}  // extern "C"

// Body of every decode entry point; k_scales / v_scales (device [H_kv][d]) are
// per-channel scales of a one-byte-code cache, or nullptr.
pkv_status pkv::decode_impl(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, float k_scale, float v_scale, const float* k_scales,
    const float* v_scales, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t algo, void* stream, void* ev_begin, void* ev_mid, void* ev_end, const void* k_new,
    const void* v_new, const int64_t* slot_mapping, float k_inv, float v_inv) {
  clear_error();
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0)
    return fail(PKV_ERR_INVALID_ARG, "decode: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "decode: num_q_heads %% num_kv_heads != 0");
  if (num_seqs > 65535 || num_q_heads > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "decode: at most 65535 sequences and q-heads per call");
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "decode: block_size must be 16 (got %d)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "decode: head_dim must be 64 or 128 (got %d)", head_dim);
  if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return fail(PKV_ERR_INVALID_ARG, "decode: bad dtype");
  if (!decode_pair_ok(q_dtype, kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "decode: unsupported (q, kv) dtype pair (%d, %d)", q_dtype,
                kv_dtype);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "decode: scale must be finite");
  if (byte_codes(kv_dtype) && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return fail(PKV_ERR_INVALID_ARG, "decode: FP8/INT8 scales must be finite");
  if (partition_size < 0 || (partition_size > 0 && (partition_size % kBlockSize != 0 ||
                                                     partition_size > kMaxPartition)))
    return fail(PKV_ERR_INVALID_ARG, "decode: partition_size must be 0 or a multiple of 16 <= %d",
                kMaxPartition);
  if (algo < PKV_ALGO_AUTO || algo > PKV_ALGO_MFMA)
    return fail(PKV_ERR_INVALID_ARG, "decode: bad algo %d", algo);
  const int32_t g = num_q_heads / num_kv_heads;
  const bool mfma_ok =
      (q_dtype == PKV_F16 || q_dtype == PKV_BF16) && (kv_dtype == q_dtype || byte_codes(kv_dtype));
  if (algo == PKV_ALGO_MFMA && !mfma_ok)
    return fail(PKV_ERR_UNSUPPORTED, "decode: the MFMA path needs 16-bit q and a 16-bit/FP8 cache");
  if (algo == PKV_ALGO_AUTO) algo = resolve_algo(g, q_dtype, kv_dtype);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "decode: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "decode: out, q and the caches must be 16-byte aligned");
  Plan plan;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, kv_dtype,
                 partition_size, &plan))
    return fail(PKV_ERR_INVALID_ARG, "decode: bad partition arguments");
  // the balanced kernels address a block's tile of one kv-head by the 31-bit
  // index id * num_kv_heads + head
  const bool tiles_fit = (int64_t)num_blocks * num_kv_heads < ((int64_t)1 << 31);
  const bool use_stream = plan.stream_ok && tiles_fit && algo == PKV_ALGO_MFMA;
  const size_t need = use_stream ? plan.stream_bytes : (plan.num_parts > 1 ? plan.ws_bytes : 0);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "decode: workspace needs %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(PKV_ERR_INVALID_ARG, "decode: workspace must be 256-byte aligned");
  }
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.scale = scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.partition = plan.partition;
  a.num_parts = plan.num_parts;
  char* ws = static_cast<char*>(workspace);
  a.ws_m = plan.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_l = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.off_l) : nullptr;
  a.ws_acc = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.off_acc) : nullptr;
  a.stream = stream;
  // ev_begin / ev_mid: stamped by the decode kernel's own dispatch (its start
  // and end); ev_end: by the merge or reduction kernel's end, else recorded
  // right after the decode kernel
  a.ev_start = ev_begin;
  a.ev_stop = ev_mid;
  if (k_new) {
    // the step's new rows: appended by the MFMA decode kernels themselves,
    // else (vector kernel, per-channel scales) by the append kernel first
    const bool fused = algo == PKV_ALGO_MFMA && !k_scales;
    if (fused) {
      a.k_new = k_new;
      a.v_new = v_new;
      a.slots = slot_mapping;
      a.k_inv = k_inv;
      a.v_inv = v_inv;
    } else {
      const int rc = launch_cache_append(const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                                         k_new, v_new, slot_mapping, num_seqs, num_kv_heads,
                                         head_dim, num_blocks, q_dtype, kv_dtype, k_inv, v_inv,
                                         stream, nullptr, nullptr);
      if (rc != 0)
        return fail(PKV_ERR_HIP, "decode: append launch failed: %s",
                    hipGetErrorString((hipError_t)rc));
    }
  }
  if (use_stream) {
    int rc = launch_decode_stream(a, plan.stream_grid, workspace, plan.stream_off_ml,
                                  plan.stream_off_part);
    if (rc != 0)
      return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString((hipError_t)rc));
    a.ev_start = nullptr;
    a.ev_stop = ev_end;
    rc = launch_decode_split_merge(a, plan.stream_grid, workspace, plan.stream_off_ml,
                                   plan.stream_off_part);
    if (rc != 0)
      return fail(PKV_ERR_HIP, "decode: merge launch failed: %s",
                  hipGetErrorString((hipError_t)rc));
    return PKV_OK;
  }
  int rc = (algo == PKV_ALGO_MFMA)
               ? (plan.parts_stream_ok && tiles_fit ? launch_decode_stream_parts(a, plan.stream_grid)
                                       : launch_decode_mfma(a))
               : launch_decode_vector(a);
  if (rc != 0)
    return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString((hipError_t)rc));
  if (plan.num_parts > 1) {
    a.ev_start = nullptr;
    a.ev_stop = ev_end;
    rc = launch_decode_reduce(a);
    if (rc != 0)
      return fail(PKV_ERR_HIP, "decode: reduce launch failed: %s",
                  hipGetErrorString((hipError_t)rc));
  } else if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end),
                                      static_cast<hipStream_t>(stream)) != hipSuccess) {
    return fail(PKV_ERR_HIP, "decode: hipEventRecord failed");
  }
  return PKV_OK;
}

extern "C" {

pkv_status pkv_paged_decode_attention_profiled(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, float k_scale, float v_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, int32_t algo, void* stream, void* ev_begin, void* ev_mid,
    void* ev_end) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                     q_dtype, kv_dtype, k_scale, v_scale, nullptr, nullptr, partition_size,
                     workspace, workspace_bytes, algo, stream, ev_begin, ev_mid, ev_end);
}

pkv_status pkv_paged_decode_attention_appending(
    void* out, const void* q, const void* k_new, const void* v_new,
    const int64_t* slot_mapping, void* k_cache, void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    float scale, int32_t q_dtype, int32_t kv_dtype, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t algo, void* stream,
    void* ev_begin, void* ev_mid, void* ev_end) {
  clear_error();
  // the append's own checks (pkv_paged_cache_append with num_tokens = num_seqs)
  float k_inv = 1.0f, v_inv = 1.0f;
  if (byte_codes(kv_dtype)) {
    if (!(k_scale > 0.0f) || !std::isfinite(k_scale) || !(v_scale > 0.0f) ||
        !std::isfinite(v_scale))
      return fail(PKV_ERR_INVALID_ARG, "decode_appending: FP8/INT8 scales must be finite and > 0");
    k_inv = 1.0f / k_scale;
    v_inv = 1.0f / v_scale;
  }
  if (num_seqs > 0) {
    if (!k_new || !v_new || !slot_mapping)
      return fail(PKV_ERR_INVALID_ARG, "decode_appending: NULL pointer");
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(PKV_ERR_INVALID_ARG, "decode_appending: new rows must be 16-byte aligned");
  }
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                     q_dtype, kv_dtype, k_scale, v_scale, nullptr, nullptr, partition_size,
                     workspace, workspace_bytes, algo, stream, ev_begin, ev_mid, ev_end,
                     num_seqs > 0 ? k_new : nullptr, v_new, slot_mapping, k_inv, v_inv);
}

pkv_status pkv_paged_decode_attention_per_channel(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, const float* k_scales, const float* v_scales, int32_t partition_size,
    void* workspace, size_t workspace_bytes, int32_t algo, void* stream, void* ev_begin,
    void* ev_mid, void* ev_end) {
  clear_error();
  if (!byte_codes(kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "decode_per_channel: the cache must hold FP8 or INT8 codes");
  if (num_seqs > 0 && (!k_scales || !v_scales))
    return fail(PKV_ERR_INVALID_ARG, "decode_per_channel: NULL scale array");
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                     q_dtype, kv_dtype, 1.0f, 1.0f, k_scales, v_scales, partition_size,
                     workspace, workspace_bytes, algo, stream, ev_begin, ev_mid, ev_end);
}

pkv_status pkv_paged_decode_attention_algo(void* out, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_blocks_per_seq,
                                           float scale, int32_t q_dtype, int32_t kv_dtype,
                                           float k_scale, float v_scale, int32_t partition_size,
                                           void* workspace, size_t workspace_bytes,
                                           int32_t algo, void* stream) {
  return pkv_paged_decode_attention_profiled(
      out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
      head_dim, block_size, num_blocks, max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale,
      v_scale, partition_size, workspace, workspace_bytes, algo, stream, nullptr, nullptr,
      nullptr);
}

pkv_status pkv_paged_decode_attention(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
                                      int32_t kv_dtype, float k_scale, float v_scale,
                                      int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return pkv_paged_decode_attention_algo(
      out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
      head_dim, block_size, num_blocks, max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale,
      v_scale, partition_size, workspace, workspace_bytes, PKV_ALGO_AUTO, stream);
}

/* ---------------------------------------------------- multi-query -- */

int32_t pkv_multiquery_partition_size(int32_t num_seqs, int32_t max_query_len,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t max_blocks_per_seq, int32_t partition_size) {
  MQPlan plan;
  if (!mq_plan(0, num_seqs, max_query_len, num_q_heads, num_kv_heads, 128, max_blocks_per_seq,
               partition_size, &plan))
    return -1;
  return plan.partition;
}

int32_t pkv_multiquery_partition_size_for_lengths(const int32_t* context_lens, int32_t num_seqs,
                                                  int32_t max_query_len, int32_t num_q_heads,
                                                  int32_t num_kv_heads, int32_t max_blocks_per_seq,
                                                  int32_t kv_dtype) {
  const int32_t auto_ps = pkv_multiquery_partition_size(num_seqs, max_query_len, num_q_heads,
                                                        num_kv_heads, max_blocks_per_seq, 0);
  if (auto_ps != 0) return auto_ps;   // no balanced schedule to weigh (or bad arguments)
  if (num_seqs > 0 && !context_lens) return -1;
  const int64_t max_ctx = (int64_t)max_blocks_per_seq * kBlockSize;
  const int32_t g = num_q_heads / num_kv_heads;
  const int32_t mq = max_query_len > 0 ? max_query_len : 1;
  if (max_ctx == 0 || max_ctx > kMaxPartition || !mq_small_grid(num_seqs, num_kv_heads, g, mq))
    return 0;
  const MQTiles t = mq_tiles(g, mq, 4);
  const int64_t Y = (int64_t)num_kv_heads * t.hchunks;
  const int64_t R = kv_restart_units(kv_dtype);
  // Costs in block loads of one wave, as for decode (both schedules run four
  // column tiles per wave here):
  //  balanced: the grid's waves share every row tile's units equally, then
  //            the merge kernel runs (its 16-column partials weigh about
  //            kMergeUnits block loads);
  //  one pass: a workgroup's four waves take a quarter of the sequence each
  //            (plus one restart), list-scheduled over the CUs.
  constexpr int64_t kMergeUnits = 8;
  int64_t units = 0;
  std::vector<int64_t> work(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t len = context_lens[s] < 0 ? 0 : (context_lens[s] > max_ctx ? max_ctx : context_lens[s]);
    const int64_t nbk = (len + kBlockSize - 1) / kBlockSize;
    units += nbk > 0 ? nbk + R : 0;
    work[s] = nbk > 0 ? (nbk + kWaves - 1) / kWaves + R : 0;
  }
  if (units == 0) return 0;
  const int64_t W = (int64_t)stream_workgroups() * kWaves;
  const int64_t t_bal = (Y * t.qtiles * units + W - 1) / W + kMergeUnits;
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
  for (int32_t i = 0, n = device_cus(); i < n; ++i) free_at.push(0);
  int64_t t_fix = 0;
  for (int32_t s = 0; s < num_seqs && t_fix <= t_bal; ++s) {
    for (int64_t y = 0; y < Y * t.qtiles; ++y) {
      const int64_t tt = free_at.top() + work[s];
      free_at.pop();
      free_at.push(tt);
      if (tt > t_fix) t_fix = tt;
    }
  }
  return t_fix <= t_bal ? (int32_t)max_ctx : 0;
}

size_t pkv_multiquery_workspace_size(int32_t num_rows, int32_t num_seqs, int32_t max_query_len,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_blocks_per_seq,
                                     int32_t partition_size) {
  MQPlan plan;
  if (!mq_plan(num_rows, num_seqs, max_query_len, num_q_heads, num_kv_heads, head_dim,
               max_blocks_per_seq, partition_size, &plan))
    return SIZE_MAX;
  return plan.ws_bytes;
}

pkv_status pkv_paged_multiquery_attention_profiled(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_rows, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, float scale, int32_t q_dtype, int32_t kv_dtype, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    void* stream, void* ev_begin, void* ev_mid, void* ev_end) {
  clear_error();
  if (num_seqs < 0 || num_rows < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(PKV_ERR_INVALID_ARG, "multiquery: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "multiquery: num_q_heads %% num_kv_heads != 0");
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "multiquery: block_size must be 16 (got %d)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "multiquery: head_dim must be 64 or 128 (got %d)",
                head_dim);
  if (!valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return fail(PKV_ERR_INVALID_ARG, "multiquery: bad dtype");
  if (!((q_dtype == PKV_F16 || q_dtype == PKV_BF16) &&
        (kv_dtype == q_dtype || byte_codes(kv_dtype))))
    return fail(PKV_ERR_UNSUPPORTED,
                "multiquery: needs 16-bit q and a cache of the same dtype or E4M3 (%d, %d)",
                q_dtype, kv_dtype);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "multiquery: scale must be finite");
  if (byte_codes(kv_dtype) && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return fail(PKV_ERR_INVALID_ARG, "multiquery: FP8/INT8 scales must be finite");
  MQPlan plan;
  if (!mq_plan(num_rows, num_seqs, max_query_len, num_q_heads, num_kv_heads, head_dim,
               max_blocks_per_seq, partition_size, &plan))
    return fail(PKV_ERR_INVALID_ARG,
                "multiquery: partition_size must be 0 or a multiple of 16 <= %d", kMaxPartition);
  const MQTiles t = mq_tiles(num_q_heads / num_kv_heads, max_query_len > 0 ? max_query_len : 1,
                            plan.max_ntl);
  if (!plan.stream && (num_seqs > 65535 || (int64_t)num_kv_heads * t.hchunks * t.qtiles > 65535 ||
                      plan.num_parts > 65535))
    return fail(PKV_ERR_UNSUPPORTED,
                "multiquery: grid too large (sequences, kv-heads x row tiles, rows x q-heads)");
  if ((int64_t)num_rows * num_q_heads > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED,
                "multiquery: grid too large (sequences, kv-heads x row tiles, rows x q-heads)");
  if (num_seqs == 0 || num_rows == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return fail(PKV_ERR_INVALID_ARG, "multiquery: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "multiquery: out, q and the caches must be 16-byte aligned");
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(PKV_ERR_WORKSPACE, "multiquery: workspace needs %zu bytes, got %zu",
                  plan.ws_bytes, workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(PKV_ERR_INVALID_ARG, "multiquery: workspace must be 256-byte aligned");
  }
  MQArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_rows = num_rows;
  a.max_query_len = max_query_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.scale = scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.partition = plan.partition;
  a.num_parts = plan.num_parts;
  char* ws = static_cast<char*>(workspace);
  a.ws_m = plan.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_l = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.off_l) : nullptr;
  a.ws_acc = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.off_acc) : nullptr;
  a.max_ntl = plan.max_ntl;
  a.stream_grid = plan.stream_grid;
  a.st_ml = plan.stream ? reinterpret_cast<float*>(ws) : nullptr;
  a.st_part = plan.stream ? reinterpret_cast<float*>(ws + plan.st_off_part) : nullptr;
  a.stream = stream;
  // events as for decode: stamped by the attention kernel's dispatch, ev_end
  // by the merging kernel's end or recorded after a single pass
  a.ev_start = ev_begin;
  a.ev_stop = ev_mid;
  if (plan.stream) {
    int rc = launch_multiquery_stream(a);
    if (rc != 0)
      return fail(PKV_ERR_HIP, "multiquery: launch failed: %s", hipGetErrorString((hipError_t)rc));
    a.ev_start = nullptr;
    a.ev_stop = ev_end;
    rc = launch_multiquery_split_merge(a);
    if (rc != 0)
      return fail(PKV_ERR_HIP, "multiquery: merge launch failed: %s",
                  hipGetErrorString((hipError_t)rc));
    return PKV_OK;
  }
  int rc = launch_multiquery(a);
  if (rc != 0)
    return fail(PKV_ERR_HIP, "multiquery: launch failed: %s", hipGetErrorString((hipError_t)rc));
  if (plan.num_parts > 1) {
    a.ev_start = nullptr;
    a.ev_stop = ev_end;
    rc = launch_multiquery_reduce(a);
    if (rc != 0)
      return fail(PKV_ERR_HIP, "multiquery: reduce launch failed: %s",
                  hipGetErrorString((hipError_t)rc));
  } else if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end),
                                      static_cast<hipStream_t>(stream)) != hipSuccess) {
    return fail(PKV_ERR_HIP, "multiquery: hipEventRecord failed");
  }
  return PKV_OK;
}

pkv_status pkv_paged_multiquery_attention(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_rows, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, float scale, int32_t q_dtype, int32_t kv_dtype, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    void* stream) {
  return pkv_paged_multiquery_attention_profiled(
      out, q, k_cache, v_cache, block_tables, context_lens, query_start, num_seqs, num_rows,
      max_query_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
      max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale, partition_size, workspace,
      workspace_bytes, stream, nullptr, nullptr, nullptr);
}

// Address through which a kernel reaches p: device memory as is, pinned host
// memory through its device mapping; nullptr for memory no kernel can touch
// (pageable host memory), so that such a call fails instead of faulting.
static const void* kernel_view(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky "not registered" error
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return p;
  if (at.type == hipMemoryTypeHost) return at.devicePointer;
  return nullptr;
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                           int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                           void* stream) {
  clear_error();
  if (num_pairs < 0 || num_blocks < 0 || block_bytes <= 0 || block_bytes % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: bad sizes");
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst_pairs)
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: caches must be 16-byte aligned");
  // every buffer is read or written by the kernel: memory it cannot reach
  // (pageable host memory) is refused here instead of faulting the GPU
  void* kc = const_cast<void*>(kernel_view(k_cache));
  void* vc = const_cast<void*>(kernel_view(v_cache));
  const int32_t* pp = static_cast<const int32_t*>(kernel_view(src_dst_pairs));
  if (!kc || !vc || !pp)
    return fail(PKV_ERR_INVALID_ARG,
                "copy_blocks: the caches and the pairs must be device or pinned host memory");
  if (!aligned16(kc) || !aligned16(vc))
    return fail(PKV_ERR_INVALID_ARG, "copy_blocks: caches must be 16-byte aligned");
  int rc = launch_copy_blocks(kc, vc, pp, num_pairs, num_blocks, block_bytes, stream);
  if (rc != 0)
    return fail(PKV_ERR_HIP, "copy_blocks: launch failed: %s", hipGetErrorString((hipError_t)rc));
  return PKV_OK;
}

pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                           const void* src_v, int32_t src_num_blocks,
                           const int32_t* src_dst_pairs, int32_t num_pairs, int64_t block_bytes,
                           void* stream) {
  clear_error();
  if (num_pairs < 0 || dst_num_blocks < 0 || src_num_blocks < 0 || block_bytes <= 0 ||
      block_bytes % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: bad sizes");
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !src_dst_pairs)
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: NULL pointer");
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: caches must be 16-byte aligned");
  void* dk = const_cast<void*>(kernel_view(dst_k));
  void* dv = const_cast<void*>(kernel_view(dst_v));
  const void* sk = kernel_view(src_k);
  const void* sv = kernel_view(src_v);
  const int32_t* pp = static_cast<const int32_t*>(kernel_view(src_dst_pairs));
  if (!dk || !dv || !sk || !sv || !pp)
    return fail(PKV_ERR_INVALID_ARG,
                "swap_blocks: every buffer must be device memory or pinned host memory");
  if (!aligned16(dk) || !aligned16(dv) || !aligned16(sk) || !aligned16(sv))
    return fail(PKV_ERR_INVALID_ARG, "swap_blocks: caches must be 16-byte aligned");
  int rc = launch_swap_blocks(dk, dv, dst_num_blocks, sk, sv, src_num_blocks, pp, num_pairs,
                              block_bytes, stream);
  if (rc != 0)
    return fail(PKV_ERR_HIP, "swap_blocks: launch failed: %s", hipGetErrorString((hipError_t)rc));
  return PKV_OK;
}

}  // extern "C"
