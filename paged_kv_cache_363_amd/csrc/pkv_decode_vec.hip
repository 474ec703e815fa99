// Paged decode attention on the vector ALUs, plus the split-K reduction.
//
// Every lane owns 16-byte chunks of the 16-token K and V tiles (chunk j*64+l
// of a tile goes to lane l, so each load instruction of a wave reads 1 KiB of
// contiguous memory).  A token's row spans CPT consecutive lanes; the partial
// dot products of those lanes are summed with butterfly shuffles, after which
// every lane holding part of a token knows its logit for all the q-heads of
// the group, so the PV update needs no further exchange: each lane scales its
// own V chunk.  This path serves every dtype pair (it is the only one for f32
// and for MHA, g = 1); see pkv_decode_mfma.hip for the matrix-core path.
//
// Math: softmax(q K^T * scale) V through the block table ("KV Cache 与
// PageAttention深度实战", sections 1.2 and 3.2) with an online softmax in base
// 2; partitions of a long context are merged by the log-sum-exp rule.
#include <hip/hip_runtime.h>

#include "pkv_decode_common.h"
#include "pkv_launch.h"

namespace {

using namespace pkvd;

template <int QT>
__device__ __forceinline__ void load_q(const void* q, int64_t off, int n, float* f) {
  // n consecutive q elements (n = 4, 8 or 16) starting at element `off`
  if constexpr (QT == PKV_F32) {
    const float* p = reinterpret_cast<const float*>(q) + off;
    for (int i = 0; i < n; ++i) f[i] = p[i];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(q) + off;
    for (int i = 0; i < n; ++i)
      f[i] = QT == PKV_F16 ? f16_lo(p[i]) : bf16_lo(p[i]);
  }
}

// Waves per workgroup of the vector kernel, which take the partition's
// blocks round robin.  Eight: two waves share each SIMD, so one wave's
// dot products and exps overlap another's loads (measured on the
// Llama-2-7B-shaped MHA workload: 195.8 -> 186.6 us against four).  The
// MFMA kernels keep pkv::kWaves.
constexpr int kVecWaves = 8;

template <int QT, int KVT, int D, int GMAX>
__global__ __launch_bounds__(64 * kVecWaves) void decode_vec_kernel(DecodeParams p) {
  constexpr int EB = DType<KVT>::bytes;
  constexpr int EPC = 16 / EB;          // elements per 16-byte chunk
  constexpr int CPT = D / EPC;          // chunks (lanes) per token row
  constexpr int NJ = D * EB / 64;       // chunks per lane per tile
  constexpr int64_t TILE = 16 * D * EB;
  constexpr int LD = D + 4;
  static_assert(CPT >= 1 && CPT <= 64 && NJ >= 1, "tile shape");

  __shared__ float sm_m[kVecWaves * GMAX];
  __shared__ float sm_l[kVecWaves * GMAX];
  __shared__ __align__(16) float sm_o[kVecWaves * GMAX * LD];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int part = blockIdx.x, s = blockIdx.z;
  const int hk = blockIdx.y / p.hchunks, hc = blockIdx.y % p.hchunks;
  const int h_first = hk * p.g + hc * p.chunk_heads;
  const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
  const int ctx = clamped_ctx(p, s);
  const int nblk = (ctx + 15) >> 4;
  const int b_begin = part * p.part_blocks;
  if (part > 0 && b_begin >= nblk) return;
  const int b_end = min(b_begin + p.part_blocks, nblk);

  const int dim0 = (lane % CPT) * EPC;  // the lane's dims, the same for every chunk j
  float qf[GMAX][EPC];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < nh) {
      load_q<QT>(p.q, ((int64_t)s * p.Hq + h_first + h) * D + dim0, EPC, qf[h]);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) qf[h][e] = 0.f;
    }
  }
  if (p.ks) {   // per-channel K scales: q_i * ks_i, so the codes enter as they are
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float ke = p.ks[(int64_t)hk * D + dim0 + e];
#pragma unroll
      for (int h = 0; h < GMAX; ++h) qf[h][e] *= ke;
    }
  }

  float acc[GMAX][EPC];
  float m_run[GMAX], l_run[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
  }

  const int64_t blk_stride = (int64_t)p.Hkv * TILE;
  const int64_t head_off = (int64_t)hk * TILE;
  const int32_t* btrow = p.bt + (int64_t)s * p.mb;

  for (int b = b_begin + w; b < b_end; b += kVecWaves) {
    const int phys = btrow[b];
    if ((unsigned)phys >= (unsigned)p.nb) continue;   // bad table entry: no weight
    const int valid = min(16, ctx - b * 16);
    const uint4* kt = reinterpret_cast<const uint4*>(p.kc + phys * blk_stride + head_off);
    const uint4* vt = reinterpret_cast<const uint4*>(p.vc + phys * blk_stride + head_off);
    uint4 kr[NJ], vr[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) kr[j] = ld_tile16<true>(kt + j * 64 + lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j) vr[j] = ld_tile16<true>(vt + j * 64 + lane);

    float z[NJ][GMAX];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float kf[EPC];
      chunk_to_f32<KVT>(kr[j], kf);
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) a = fmaf(qf[h][e], kf[e], a);
        z[j][h] = a;
      }
    }
    // sum the partial dots of the CPT lanes sharing a token
#pragma unroll
    for (int off = 1; off < CPT; off <<= 1)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int h = 0; h < GMAX; ++h) z[j][h] += __shfl_xor(z[j][h], off);

    float bm[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) bm[h] = kNegInf;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int tok = (j * 64 + lane) / CPT;
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        z[j][h] = tok < valid ? z[j][h] * p.sl2 : kNegInf;
        bm[h] = fmaxf(bm[h], z[j][h]);
      }
    }
    // block maximum over the lanes holding other tokens
#pragma unroll
    for (int off = CPT; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < GMAX; ++h) bm[h] = fmaxf(bm[h], __shfl_xor(bm[h], off));

    float alpha[GMAX];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      const float m_new = fmaxf(m_run[h], bm[h]);
      alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - m_new);
      moved |= alpha[h] != 1.0f;
      m_run[h] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        z[j][h] = __builtin_amdgcn_exp2f(z[j][h] - m_new);
        ps += z[j][h];
      }
      // each token's weight is replicated over its CPT lanes: count it once
      l_run[h] = l_run[h] * alpha[h] + ((lane % CPT) == 0 ? ps : 0.f);
    }
    if (__any(moved)) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha[h];
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float vf[EPC];
      chunk_to_f32<KVT>(vr[j], vf);
      if ((j * 64 + lane) / CPT >= valid) {
        // stale slot past the context (possibly NaN): contributes nothing
#pragma unroll
        for (int e = 0; e < EPC; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(z[j][h], vf[e], acc[h][e]);
    }
  }

  // l: every lane holds part of it; acc: lanes with equal dims hold parts
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l_run[h] += __shfl_xor(l_run[h], off);
#pragma unroll
    for (int off = CPT; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
  }
  if (lane < CPT) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < nh) {
        if (lane == 0) {
          sm_m[w * GMAX + h] = m_run[h];
          sm_l[w * GMAX + h] = l_run[h];
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm_o[(w * GMAX + h) * LD + dim0 + e] = acc[h][e];
      }
    }
  }
  __syncthreads();
  merge_waves_and_store<QT, D, GMAX, kVecWaves>(p, sm_m, sm_l, sm_o, nh, s, h_first, part);
}

// Split-K reduction: one workgroup of NW waves per (sequence, q-head)
// merges the partitions that cover the sequence's context,
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p acc_p 2^(m_p - M) / L.
// Wave w merges a contiguous 1/NW of the row's partitions the same way (lane
// p holds partition p's weight, and the accumulator rows are read with
// independent loads); the waves' (M_w, L_w, acc_w) are then combined in LDS
// by the same rule.  With many partitions one wave per row keeps too few
// loads in flight (64 partitions take eight dependent rounds); with few, the
// combine costs more than it saves.
// A wave's share is fixed by the partition count alone, not by the context,
// so that its (m, l) values and its first kPrefetch accumulator rows go out
// together with the context length: the merge of a share of up to kPrefetch
// partitions waits on memory once.  Partitions past the context hold stale
// data; they get no weight and their rows are skipped, never multiplied.
template <int QT, int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_reduce_kernel(DecodeParams p) {
  constexpr int PER = (D + 63) / 64;
  constexpr int kPrefetch = 16;
  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_acc[NW][D];
  const int row = blockIdx.x;            // s * Hq + h
  const int s = row / p.Hq;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p0 = p.num_parts * w / NW, p1 = p.num_parts * (w + 1) / NW;   // this wave's share
  const float* m = p.ws_m + (int64_t)row * p.num_parts;
  const float* l = p.ws_l + (int64_t)row * p.num_parts;
  const float* a = p.ws_acc + (int64_t)row * p.num_parts * D;
  const int ctx = clamped_ctx(p, s);
  float x0[kPrefetch][PER];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      x0[u][k] = (p0 + u < p1 && d < D) ? a[(int64_t)(p0 + u) * D + d] : 0.f;
    }
  const int i0 = p0 + lane;
  const float m0 = i0 < p1 ? m[i0] : kNegInf, l0 = i0 < p1 ? l[i0] : 0.f;
  const int part_tokens = p.part_blocks * pkv::kBlockSize;
  int np = (ctx + part_tokens - 1) / part_tokens;
  np = np < 1 ? 1 : (np > p.num_parts ? p.num_parts : np);
  const int q1 = min(p1, np);            // this wave's partitions inside the context
  float M = (i0 < q1 && l0 > 0.f) ? m0 : kNegInf;
  for (int i = i0 + 64; i < q1; i += 64) M = fmaxf(M, l[i] > 0.f ? m[i] : kNegInf);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float L = 0.f;
  auto add_row = [&](float wgt, int j, const float* x) {   // lane j of wgt weighs row x
    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), j));
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = fmaf(wj, x[k], acc[k]);
  };
  if (M != kNegInf) {
    for (int base = p0; base < q1; base += 64) {
      const int i = base + lane;
      float wgt = 0.f;
      if (i < q1) {
        const float li = base == p0 ? l0 : l[i];
        const float mi = base == p0 ? m0 : m[i];
        wgt = li > 0.f ? __builtin_amdgcn_exp2f(mi - M) : 0.f;
        L += wgt * li;
      }
      const int cnt = min(64, q1 - base);
      int j0 = 0;
      if (base == p0) {
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u)
          if (u < cnt) add_row(wgt, u, x0[u]);
        j0 = kPrefetch;
      }
      // 8 rows per round, loads issued together
      const float* ab = a + (int64_t)base * D;
      for (; j0 < cnt; j0 += 8) {
        float x[8][PER];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int d = lane + 64 * k;
            x[u][k] = (j0 + u < cnt && d < D) ? ab[(int64_t)(j0 + u) * D + d] : 0.f;
          }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u < cnt) add_row(wgt, j0 + u, x[u]);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
  if constexpr (NW == 1) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      if (d < D) store_out<QT>(p.out, (int64_t)row * D + d, L > 0.f ? acc[k] / L : 0.f);
    }
    return;
  }
  // combine the waves' partial merges
  if (lane == 0) {
    sm_m[w] = M;
    sm_l[w] = L;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    if (d < D) sm_acc[w][d] = acc[k];
  }
  __syncthreads();
  float Mt = kNegInf;
#pragma unroll
  for (int v = 0; v < NW; ++v) Mt = fmaxf(Mt, sm_l[v] > 0.f ? sm_m[v] : kNegInf);
  float f[NW], Lt = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    f[v] = (Mt != kNegInf && sm_l[v] > 0.f) ? __builtin_amdgcn_exp2f(sm_m[v] - Mt) : 0.f;
    Lt += f[v] * sm_l[v];
  }
  for (int d = threadIdx.x; d < D; d += 64 * NW) {
    float o = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) o = fmaf(f[v], sm_acc[v][d], o);
    store_out<QT>(p.out, (int64_t)row * D + d, Lt > 0.f ? o / Lt : 0.f);
  }
}

template <int QT, int KVT, int D, int GMAX>
int launch_vec_t(const pkv::DecodeArgs& a) {
  const DecodeParams kp = make_params(a, GMAX);
  dim3 grid(kp.num_parts, a.num_kv_heads * kp.hchunks, a.num_seqs);
  return pkv::launch_kernel(decode_vec_kernel<QT, KVT, D, GMAX>, grid, dim3(64 * kVecWaves),
                            a.stream, kp, a.ev_start, a.ev_stop);
}

template <int QT, int KVT, int D>
int launch_vec_g(const pkv::DecodeArgs& a) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g <= 1) return launch_vec_t<QT, KVT, D, 1>(a);
  if (g <= 2) return launch_vec_t<QT, KVT, D, 2>(a);
  if (g <= 4) return launch_vec_t<QT, KVT, D, 4>(a);
  return launch_vec_t<QT, KVT, D, 8>(a);   // larger groups run in chunks of 8 heads
}

template <int QT, int D>
int launch_reduce_t(const pkv::DecodeArgs& a) {
  const DecodeParams kp = make_params(a, 16);
  // four waves per row only when rows can have many partitions
  const dim3 grid(a.num_seqs * a.num_q_heads);
  if (kp.num_parts > 16)
    return pkv::launch_kernel(decode_reduce_kernel<QT, D, 4>, grid, dim3(256), a.stream, kp,
                              a.ev_start, a.ev_stop);
  return pkv::launch_kernel(decode_reduce_kernel<QT, D, 1>, grid, dim3(64), a.stream, kp,
                            a.ev_start, a.ev_stop);
}

}  // namespace

namespace pkv {

int launch_decode_vector(const DecodeArgs& a) {
  const int q = a.q_dtype, kv = a.kv_dtype, D = a.head_dim;
#define PKV_VEC_CASE(QT, KVT, DD) \
  if (q == QT && kv == KVT && D == DD) return launch_vec_g<QT, KVT, DD>(a);
  PKV_VEC_CASE(PKV_F32, PKV_F32, 64)
  PKV_VEC_CASE(PKV_F32, PKV_F32, 128)
  PKV_VEC_CASE(PKV_BF16, PKV_BF16, 64)
  PKV_VEC_CASE(PKV_BF16, PKV_BF16, 128)
  PKV_VEC_CASE(PKV_F16, PKV_F16, 64)
  PKV_VEC_CASE(PKV_F16, PKV_F16, 128)
  PKV_VEC_CASE(PKV_BF16, PKV_FP8_E4M3, 64)
  PKV_VEC_CASE(PKV_BF16, PKV_FP8_E4M3, 128)
  PKV_VEC_CASE(PKV_F16, PKV_FP8_E4M3, 64)
  PKV_VEC_CASE(PKV_F16, PKV_FP8_E4M3, 128)
  PKV_VEC_CASE(PKV_BF16, PKV_INT8, 64)
  PKV_VEC_CASE(PKV_BF16, PKV_INT8, 128)
  PKV_VEC_CASE(PKV_F16, PKV_INT8, 64)
  PKV_VEC_CASE(PKV_F16, PKV_INT8, 128)
#undef PKV_VEC_CASE
  return (int)hipErrorInvalidValue;
}

int launch_decode_reduce(const DecodeArgs& a) {
  const int q = a.q_dtype, D = a.head_dim;
#define PKV_RED_CASE(QT, DD) \
  if (q == QT && D == DD) return launch_reduce_t<QT, DD>(a);
  PKV_RED_CASE(PKV_F32, 64)
  PKV_RED_CASE(PKV_F32, 128)
  PKV_RED_CASE(PKV_BF16, 64)
  PKV_RED_CASE(PKV_BF16, 128)
  PKV_RED_CASE(PKV_F16, 64)
  PKV_RED_CASE(PKV_F16, 128)
#undef PKV_RED_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace pkv
