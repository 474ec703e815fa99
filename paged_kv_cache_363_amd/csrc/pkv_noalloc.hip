// Decode attention that allocates nothing: the partial results of split
// contexts (the balanced schedule's pieces, fixed partitions) go to a
// static device array of the library instead of a caller workspace, for
// callers that cannot allocate device memory.  The attention itself runs in
// the same kernels as every other decode entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "pkv.h"
#include "pkv_internal.h"

// One copy per GPU, loaded with the library's code object and held until
// the process ends.  Host code never uses this name as an address (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up on the
// first call on that device (with the device current) and kept.
pkv_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return pkv::fail(PKV_ERR_HIP, "decode_noalloc: hipGetDevice failed: %s",
                     hipGetErrorString(e));
  }
  if (dev >= kMaxDevices)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "decode_noalloc: device index %d beyond %d", dev,
                     kMaxDevices - 1);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return pkv::fail(PKV_ERR_HIP,
                         "decode_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
                         hipGetErrorString(e));
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_decode_attention_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, int32_t q_dtype,
    int32_t kv_dtype, float k_scale, float v_scale, int32_t partition_size, int32_t algo,
    void* stream) {
  pkv::clear_error();
  void* ws = nullptr;
  const pkv_status st = scratch_of_current_device(&ws);
  if (st != PKV_OK) return st;
  const pkv_status rc = pkv::decode_impl(
      out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
      head_dim, block_size, num_blocks, max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale,
      v_scale, nullptr, nullptr, partition_size, ws, (size_t)PKV_NOALLOC_SCRATCH_BYTES, algo,
      stream, nullptr, nullptr, nullptr);
  if (rc == PKV_ERR_WORKSPACE) {
    const std::string why = pkv_last_error();
    return pkv::fail(PKV_ERR_WORKSPACE,
                     "decode_noalloc: %s; the static scratch holds %zu bytes "
                     "(PKV_NOALLOC_SCRATCH_BYTES): use pkv_paged_decode_attention with a "
                     "caller workspace, or a larger partition_size",
                     why.c_str(), (size_t)PKV_NOALLOC_SCRATCH_BYTES);
  }
  return rc;
}
