// Streaming-read probe: the HBM read rate this GPU achieves for the access
// pattern of paged decode, measured beside the 8 TB/s spec figure.  Paged
// decode reads whole (block, kv-head) tiles of a few KiB each, scattered over
// the pool in table order; here 4 KiB tiles are read in a caller-given
// (shuffled) order, each wave streaming one contiguous share of the list
// with four tiles in flight, on a persistent grid like the balanced decode
// kernel's.  The loads are non-temporal, as the decode kernels' 16-bit paths
// use.  The tile list is read through the scalar path (its index is uniform
// per wave), so no tile load waits on an id load.  Nothing is computed but
// an XOR of the bytes, stored once per thread so the loads cannot be
// dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_launch.h"


namespace {

// The tiles stay in the load's own vector type: converted to uint4, some of
// their words were given other registers across the loop's back edge, and
// the copies there waited for every load in flight.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

constexpr int kTileBytes = 4096;
constexpr int kDepth = 4;   // tiles in flight per wave

struct ProbeParams {
  const u32x4* buf;
  int64_t buf_tiles;
  const int32_t* ids;
  int32_t ntiles;
  uint32_t* sink;
};

__global__ __launch_bounds__(256) void stream_read_probe_kernel(ProbeParams pp) {
  const u32x4* __restrict__ buf = pp.buf;
  const int32_t* __restrict__ ids = pp.ids;
  const int64_t buf_tiles = pp.buf_tiles;
  const int32_t ntiles = pp.ntiles;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = gridDim.x * 4;
  const int64_t t0 = (int64_t)ntiles * w / W, t1 = (int64_t)ntiles * (w + 1) / W;
  uint32_t acc = 0;
  if (t1 > t0) {
    // tile t of the share (clamped to its last tile), an id outside the
    // buffer reading tile 0
    auto tile = [&](int64_t t) {
      const int32_t id = ids[t < t1 ? t : t1 - 1];
      const int64_t i = (uint32_t)id < (uint64_t)buf_tiles ? id : 0;
      return buf + i * (kTileBytes / 16);
    };
    u32x4 b[kDepth][4];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const u32x4* p = tile(t0 + d);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[d][j] = ld_nt(p + j * 64 + lane);
      __builtin_amdgcn_sched_barrier(0);   // tiles issue in order, oldest first
    }
    for (int64_t t = t0; t < t1; t += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        // fold unconditionally (tiles past the share repeat its last one), so
        // the wait covers one tile, not the pipeline; the rotation keeps the
        // folds of different tiles from being merged into one wait
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) x ^= b[d][j][0] ^ b[d][j][1] ^ b[d][j][2] ^ b[d][j][3];
        acc = ((acc << 1) | (acc >> 31)) ^ x;
        const u32x4* p = tile(t + d + kDepth);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[d][j] = ld_nt(p + j * 64 + lane);
        // keep the next tile's reads below this tile's reload: hoisted, they
        // would make the loop top wait for every tile in flight
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  pp.sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

namespace pkv {

int launch_stream_read_probe(const void* buf, int64_t buf_bytes, const int32_t* tile_ids,
                             int32_t num_tiles, uint32_t* sink, int32_t workgroups,
                             void* stream, void* ev_start, void* ev_stop) {
  ProbeParams pp;
  pp.buf = static_cast<const u32x4*>(buf);
  pp.buf_tiles = buf_bytes / kTileBytes;
  pp.ids = tile_ids;
  pp.ntiles = num_tiles;
  pp.sink = sink;
  return launch_kernel(stream_read_probe_kernel, dim3(workgroups), dim3(256), stream, pp,
                       ev_start, ev_stop);
}

}  // namespace pkv
