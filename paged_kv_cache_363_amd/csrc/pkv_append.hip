// Cache append (slot_mapping write) and whole-block copy kernels.
//
// Append: each decode step computes K and V for the new token only and stores
// them next to the earlier ones ("Transformer 推理优化：KV Cache、
// PagedAttention 与 vLLM", section 2.2); the destination is the slot the block
// pool handed out, slot = physical_block * 16 + offset (same page, 3.3).
// Copy: a block shared by several tables is duplicated before one of them
// writes into it ("大语言模型推理引擎深度剖析", section 2.3).
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

using namespace pkvd;

constexpr int kAppendThreads = 256;
constexpr int kElemsPerThread = 8;

// One thread moves 8 consecutive elements of one (token, kv-head) row.
template <int NEW_DT, int KV_DT>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, const uint8_t* __restrict__ kn,
    const uint8_t* __restrict__ vn, const int64_t* __restrict__ slots, int num_tokens, int H,
    int D, int num_blocks, float k_inv, float v_inv, const float* __restrict__ k_sc,
    const float* __restrict__ v_sc) {
  const int chunks = D / kElemsPerThread;
  const int64_t gid = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * H * chunks;
  if (gid >= total) return;
  const int c = (int)(gid % chunks);
  const int64_t th = gid / chunks;
  const int h = (int)(th % H);
  const int64_t t = th / H;
  const int64_t src = (t * H + h) * D + (int64_t)c * kElemsPerThread;
  constexpr int nb_in = DType<NEW_DT>::bytes * kElemsPerThread;
  constexpr int NI = nb_in / 16;
  // The new rows do not depend on the slot: their loads go out with the
  // slot's, so that the two round trips overlap.
  uint4 raw[2][NI];
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int i = 0; i < NI; ++i)
      raw[which][i] = reinterpret_cast<const uint4*>((which ? vn : kn) + src * DType<NEW_DT>::bytes)[i];
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= (int64_t)num_blocks * pkv::kBlockSize) {
    // the rows are used on this path too, so the compiler keeps their loads
    // above the branch
#pragma unroll
    for (int which = 0; which < 2; ++which)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        asm volatile("" ::"v"(raw[which][i].x), "v"(raw[which][i].y), "v"(raw[which][i].z),
                     "v"(raw[which][i].w));
    return;
  }
  const int64_t blk = slot / pkv::kBlockSize, off = slot % pkv::kBlockSize;
  const int64_t dst = ((blk * H + h) * pkv::kBlockSize + off) * D + (int64_t)c * kElemsPerThread;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    uint8_t* outp = (which ? vc : kc) + dst * DType<KV_DT>::bytes;
    if constexpr (KV_DT == NEW_DT) {
#pragma unroll
      for (int i = 0; i < NI; ++i) reinterpret_cast<uint4*>(outp)[i] = raw[which][i];
    } else {
      static_assert(KV_DT == PKV_FP8_E4M3 || KV_DT == PKV_INT8,
                    "only E4M3 and INT8 caches convert");
      const float inv = which ? v_inv : k_inv;
      // per-channel scales (a scale per (kv-head, dim)): the element's own
      // reciprocal, rounded to binary32 like the per-tensor one
      const float* sc = which ? v_sc : k_sc;
      float invs[kElemsPerThread];
#pragma unroll
      for (int i = 0; i < kElemsPerThread; ++i)
        invs[i] = sc ? __fdiv_rn(1.0f, sc[(int64_t)h * D + c * kElemsPerThread + i]) : inv;
      float f[kElemsPerThread];
      if constexpr (NEW_DT == PKV_F32) {
        chunk_to_f32<PKV_F32>(raw[which][0], f);
        chunk_to_f32<PKV_F32>(raw[which][1], f + 4);
      } else {
        chunk_to_f32<NEW_DT>(raw[which][0], f);
      }
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KV_DT == PKV_FP8_E4M3) {
          lo |= f32_to_e4m3(f[i] * invs[i]) << (8 * i);
          hi |= f32_to_e4m3(f[4 + i] * invs[4 + i]) << (8 * i);
        } else {
          lo |= f32_to_i8(f[i] * invs[i]) << (8 * i);
          hi |= f32_to_i8(f[4 + i] * invs[4 + i]) << (8 * i);
        }
      }
      *reinterpret_cast<uint2*>(outp) = make_uint2(lo, hi);
    }
  }
}

// One workgroup copies one physical block of K (blockIdx.y == 0) or V.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ kc,
                                                          uint8_t* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t block_bytes) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* base = blockIdx.y ? vc : kc;
  const uint4* s = reinterpret_cast<const uint4*>(base + (int64_t)src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(base + (int64_t)dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += 256) d[i] = s[i];
}

// One workgroup copies one block of K (blockIdx.y == 0) or V between two
// caches of the same block layout; either may be pinned host memory mapped
// into the device's address space (swapping blocks out and back in).
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    uint8_t* __restrict__ dk, uint8_t* __restrict__ dv, int dst_blocks,
    const uint8_t* __restrict__ sk, const uint8_t* __restrict__ sv, int src_blocks,
    const int32_t* __restrict__ pairs, int64_t block_bytes) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s =
      reinterpret_cast<const uint4*>((blockIdx.y ? sv : sk) + (int64_t)src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>((blockIdx.y ? dv : dk) + (int64_t)dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += 256) d[i] = s[i];
}

template <int NEW_DT, int KV_DT>
int launch_append_t(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int64_t* slots, int32_t T, int32_t H, int32_t D, int32_t nb,
                    float k_inv, float v_inv, hipStream_t stream, const float* k_sc,
                    const float* v_sc) {
  const int64_t total = (int64_t)T * H * (D / kElemsPerThread);
  const int64_t grid = (total + kAppendThreads - 1) / kAppendThreads;
  cache_append_kernel<NEW_DT, KV_DT><<<dim3((unsigned)grid), dim3(kAppendThreads), 0, stream>>>(
      (uint8_t*)k_cache, (uint8_t*)v_cache, (const uint8_t*)k_new, (const uint8_t*)v_new, slots,
      T, H, D, nb, k_inv, v_inv, k_sc, v_sc);
  return (int)hipGetLastError();
}

}  // namespace

namespace pkv {

int launch_cache_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                        const int64_t* slots, int32_t T, int32_t H, int32_t D, int32_t nb,
                        int32_t new_dt, int32_t kv_dt, float k_inv, float v_inv, void* stream,
                        const float* k_sc, const float* v_sc) {
  hipStream_t st = (hipStream_t)stream;
  if (kv_dt == new_dt) {
    switch (kv_dt) {
      case PKV_F32:
        return launch_append_t<PKV_F32, PKV_F32>(k_cache, v_cache, k_new, v_new, slots, T, H, D,
                                                 nb, k_inv, v_inv, st, k_sc, v_sc);
      case PKV_F16:
        return launch_append_t<PKV_F16, PKV_F16>(k_cache, v_cache, k_new, v_new, slots, T, H, D,
                                                 nb, k_inv, v_inv, st, k_sc, v_sc);
      case PKV_BF16:
        return launch_append_t<PKV_BF16, PKV_BF16>(k_cache, v_cache, k_new, v_new, slots, T, H,
                                                   D, nb, k_inv, v_inv, st, k_sc, v_sc);
    }
  } else if (kv_dt == PKV_FP8_E4M3) {
    switch (new_dt) {
      case PKV_F32:
        return launch_append_t<PKV_F32, PKV_FP8_E4M3>(k_cache, v_cache, k_new, v_new, slots, T,
                                                      H, D, nb, k_inv, v_inv, st, k_sc, v_sc);
      case PKV_F16:
        return launch_append_t<PKV_F16, PKV_FP8_E4M3>(k_cache, v_cache, k_new, v_new, slots, T,
                                                      H, D, nb, k_inv, v_inv, st, k_sc, v_sc);
      case PKV_BF16:
        return launch_append_t<PKV_BF16, PKV_FP8_E4M3>(k_cache, v_cache, k_new, v_new, slots, T,
                                                       H, D, nb, k_inv, v_inv, st, k_sc, v_sc);
    }
  } else if (kv_dt == PKV_INT8) {
    switch (new_dt) {
      case PKV_F32:
        return launch_append_t<PKV_F32, PKV_INT8>(k_cache, v_cache, k_new, v_new, slots, T, H, D,
                                                  nb, k_inv, v_inv, st, k_sc, v_sc);
      case PKV_F16:
        return launch_append_t<PKV_F16, PKV_INT8>(k_cache, v_cache, k_new, v_new, slots, T, H, D,
                                                  nb, k_inv, v_inv, st, k_sc, v_sc);
      case PKV_BF16:
        return launch_append_t<PKV_BF16, PKV_INT8>(k_cache, v_cache, k_new, v_new, slots, T, H,
                                                   D, nb, k_inv, v_inv, st, k_sc, v_sc);
    }
  }
  return (int)hipErrorInvalidValue;
}

int launch_swap_blocks(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k,
                       const void* src_v, int32_t src_blocks, const int32_t* pairs,
                       int32_t num_pairs, int64_t block_bytes, void* stream) {
  if (num_pairs <= 0) return 0;
  swap_blocks_kernel<<<dim3(num_pairs, 2), dim3(256), 0, (hipStream_t)stream>>>(
      (uint8_t*)dst_k, (uint8_t*)dst_v, dst_blocks, (const uint8_t*)src_k,
      (const uint8_t*)src_v, src_blocks, pairs, block_bytes);
  return (int)hipGetLastError();
}

int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                       int32_t num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs <= 0) return 0;
  copy_blocks_kernel<<<dim3(num_pairs, 2), dim3(256), 0, (hipStream_t)stream>>>(
      (uint8_t*)k_cache, (uint8_t*)v_cache, pairs, num_blocks, block_bytes);
  return (int)hipGetLastError();
}

}  // namespace pkv
