// Pieces shared by the decode kernels: kernel parameters, the partition
// bookkeeping and the epilogue that merges the waves of a workgroup.
//
// Every decode workgroup owns one (partition, kv-head, head chunk, sequence).
// Its waves take the partition's 16-token blocks round-robin and each keeps
// an online softmax: a running maximum m of the logits (base-2 units), the
// running sum l of 2^(z - m) and the running output sum acc of 2^(z - m) v.
// Rescaling by 2^(m_old - m_new) whenever m grows keeps the three consistent,
// which is exact in real arithmetic.  The epilogue merges the waves with the
// same log-sum-exp rule and either writes the normalised output (one
// partition per sequence) or the partition's (m, l, acc) for the reduction
// kernel.
#pragma once
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkvd {

struct DecodeParams {
  void* out;
  const void* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  const int32_t* cl;
  int Hq, Hkv, g, nb, mb;
  int part_blocks;   // 16-token blocks per partition
  int num_parts;     // partitions per sequence in the grid (1 = single pass)
  int hchunks;       // head chunks per kv-head
  int chunk_heads;   // q-heads per chunk
  float sl2;         // scale * log2(e) * k_scale
  float vsc;         // v_scale (1 unless FP8)
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  const float* ks;   // per-channel K scales [Hkv][D] (nullptr: per tensor)
  const float* vs;   // per-channel V scales [Hkv][D] (nullptr: vsc)
  // The step's new rows, appended by the decode kernel itself (nullptr: none):
  // kn, vn [S][Hkv][D] in the q dtype, slot of sequence s in slots[s],
  // encoded with k_inv / v_inv (1 / scale in binary32, as the cache append)
  const uint8_t* kn;
  const uint8_t* vn;
  const int64_t* slots;
  float k_inv, v_inv;
};

// Output store in the q dtype.
template <int QT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (QT == PKV_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (QT == PKV_F16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16(v);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  }
}

// Four consecutive outputs in the q dtype, at an element index that is a
// multiple of 4 (out is 16-byte aligned): one 16- or 8-byte store.
template <int QT>
__device__ __forceinline__ void store_out4(void* out, int64_t idx, float a, float b, float c,
                                           float d) {
  if constexpr (QT == PKV_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = make_float4(a, b, c, d);
  } else {
    uint32_t lo, hi;
    if constexpr (QT == PKV_F16) {
      lo = (uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16);
      hi = (uint32_t)f32_to_f16(c) | ((uint32_t)f32_to_f16(d) << 16);
    } else {
      lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
      hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
    }
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = make_uint2(lo, hi);
  }
}

// N consecutive outputs (N = 4 or 8) in the q dtype at an element index that
// is a multiple of N: one store of 2N bytes for a 16-bit dtype.
template <int QT, int N>
__device__ __forceinline__ void store_out_n(void* out, int64_t idx, const float* v) {
  static_assert(N == 4 || N == 8, "4 or 8 outputs");
  if constexpr (QT == PKV_F32 || N == 4) {
#pragma unroll
    for (int k = 0; k < N; k += 4) store_out4<QT>(out, idx + k, v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (QT == PKV_F16)
        w[k] = (uint32_t)f32_to_f16(v[2 * k]) | ((uint32_t)f32_to_f16(v[2 * k + 1]) << 16);
      else
        w[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
    }
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + idx) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Merge the NWV waves' (m, l, acc) held in LDS and write the result.
//   sm_m, sm_l : [NWV][HP]      sm_o : [NWV][HP][D + 4], 16-byte aligned
// Each thread takes whole quads of 4 consecutive dims of one head, a number
// of them known at compile time, and writes each with one store: a loop
// with a store per element made every iteration wait for the previous
// store (loads and stores share one counter) and the first one for the K/V
// loads still in flight.
template <int QT, int D, int HP, int NWV = pkv::kWaves>
__device__ __forceinline__ void merge_waves_and_store(const DecodeParams& p, const float* sm_m,
                                                      const float* sm_l, const float* sm_o,
                                                      int nh, int s, int h_first, int part) {
  constexpr int LD = D + 4;
  constexpr int QD = D / 4;                                   // quads per head row
  constexpr int ITER = (HP * QD + 64 * NWV - 1) / (64 * NWV);
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int qi = threadIdx.x + it * 64 * NWV;
    const int h = qi / QD, d = (qi % QD) * 4;
    if (h >= nh) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, sm_m[w * HP + h]);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float mw = sm_m[w * HP + h];
        const float f = (mw == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += f * sm_l[w * HP + h];
        const float4 x = *reinterpret_cast<const float4*>(sm_o + (w * HP + h) * LD + d);
        acc.x += f * x.x;
        acc.y += f * x.y;
        acc.z += f * x.z;
        acc.w += f * x.w;
      }
    }
    const int64_t row = (int64_t)s * p.Hq + h_first + h;
    float4 vsc = make_float4(p.vsc, p.vsc, p.vsc, p.vsc);
    if (p.vs) {   // the caller's scale array: no alignment beyond 4 bytes
      const float* v = p.vs + (int64_t)((h_first + h) / p.g) * D + d;
      vsc = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (p.num_parts == 1) {
      store_out4<QT>(p.out, row * D + d, L > 0.f ? acc.x * vsc.x / L : 0.f,
                     L > 0.f ? acc.y * vsc.y / L : 0.f, L > 0.f ? acc.z * vsc.z / L : 0.f,
                     L > 0.f ? acc.w * vsc.w / L : 0.f);
    } else {
      const int64_t pr = row * p.num_parts + part;
      *reinterpret_cast<float4*>(p.ws_acc + pr * D + d) =
          make_float4(acc.x * vsc.x, acc.y * vsc.y, acc.z * vsc.z, acc.w * vsc.w);
      if (d == 0) {
        p.ws_m[pr] = M;
        p.ws_l[pr] = L;
      }
    }
  }
}

// Kernel parameters for a launch whose workgroups each serve up to
// `chunk_heads` q-heads of one kv-head.
inline DecodeParams make_params(const pkv::DecodeArgs& a, int chunk_heads) {
  DecodeParams p;
  p.out = a.out;
  p.q = a.q;
  p.kc = static_cast<const uint8_t*>(a.k_cache);
  p.vc = static_cast<const uint8_t*>(a.v_cache);
  p.bt = a.block_tables;
  p.cl = a.context_lens;
  p.Hq = a.num_q_heads;
  p.Hkv = a.num_kv_heads;
  p.g = a.num_q_heads / a.num_kv_heads;
  p.nb = a.num_blocks;
  p.mb = a.max_blocks_per_seq;
  p.part_blocks = a.partition / pkv::kBlockSize;
  p.num_parts = a.num_parts;
  p.chunk_heads = p.g < chunk_heads ? p.g : chunk_heads;
  p.hchunks = (p.g + p.chunk_heads - 1) / p.chunk_heads;
  const bool fp8 = pkv::byte_codes(a.kv_dtype);   // scaled one-byte codes
  p.sl2 = a.scale * kLog2e * (fp8 ? a.k_scale : 1.0f);
  p.vsc = fp8 ? a.v_scale : 1.0f;
  p.ws_m = a.ws_m;
  p.ws_l = a.ws_l;
  p.ws_acc = a.ws_acc;
  p.ks = a.k_scales;
  p.vs = a.v_scales;
  p.kn = static_cast<const uint8_t*>(a.k_new);
  p.vn = static_cast<const uint8_t*>(a.v_new);
  p.slots = a.slots;
  p.k_inv = a.k_inv;
  p.v_inv = a.v_inv;
  if (p.ks) p.sl2 = a.scale * kLog2e;   // the K scales go into q instead
  return p;
}

// Context length of sequence s, clamped to what the table can hold.
__device__ __forceinline__ int clamped_ctx(const DecodeParams& p, int s) {
  int n = p.cl[s];
  const int cap = p.mb * pkv::kBlockSize;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace pkvd
