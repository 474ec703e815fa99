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

// Merge the NWV waves' (m, l, acc) held in LDS and write the result.
//   sm_m, sm_l : [NWV][HP]      sm_o : [NWV][HP][D + 4]
template <int QT, int D, int HP, int NWV = pkv::kWaves>
__device__ __forceinline__ void merge_waves_and_store(const DecodeParams& p, const float* sm_m,
                                                      const float* sm_l, const float* sm_o,
                                                      int nh, int s, int h_first, int part) {
  constexpr int LD = D + 4;
  for (int idx = threadIdx.x; idx < nh * D; idx += 64 * NWV) {
    const int h = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, sm_m[w * HP + h]);
    float L = 0.f, acc = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float mw = sm_m[w * HP + h];
        const float f = (mw == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += f * sm_l[w * HP + h];
        acc += f * sm_o[(w * HP + h) * LD + d];
      }
    }
    const int64_t row = (int64_t)s * p.Hq + h_first + h;
    const float vsc = p.vs ? p.vs[(int64_t)((h_first + h) / p.g) * D + d] : p.vsc;
    if (p.num_parts == 1) {
      store_out<QT>(p.out, row * D + d, L > 0.f ? acc * vsc / L : 0.f);
    } else {
      const int64_t pr = row * p.num_parts + part;
      p.ws_acc[pr * D + d] = acc * vsc;
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
