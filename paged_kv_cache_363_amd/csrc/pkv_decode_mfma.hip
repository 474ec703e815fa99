// Paged decode attention on the CDNA4 matrix cores (MFMA).
//
// With grouped-query attention the g q-heads that share one kv-head all read
// the same 16-token K and V tiles, so per tile QK^T is a [16 tokens x d] by
// [d x g] product and PV a [g x 16] by [16 x d] product: dense contractions.
// The kernel pads the g heads to 16 MFMA columns (zero queries) and runs, per
// 16-token block:
//   S  [16 tok x 16 heads] = K_tile . Q^T     v_mfma_f32_16x16x32_{bf16,f16}
//   O^T[d x 16 heads]     += V_tile^T . P^T   v_mfma_f32_16x16x16_{bf16,f16}
// The accumulator layout of the first product (lane l holds rows 4(l/16)+i,
// column l%16) is exactly the B-operand layout the second product needs, so
// the softmax probabilities never leave their registers, and the output
// accumulator keeps one head per lane column, so the online-softmax rescale
// is a per-lane multiply.
//
// Math: softmax(q K^T * scale) V over the block-table-gathered context
// ("KV Cache 与 PageAttention深度实战", sections 1.2 and 3.2), evaluated with
// an online softmax in base 2.  E4M3 caches ("大语言模型推理引擎深度剖析",
// sections 4.2-4.3) are widened to the q type in registers (every E4M3 value
// is exact in bf16 and f16); k_scale is folded into the logit scale and
// v_scale into the final normalisation.
#include <hip/hip_runtime.h>

#include "pkv_decode_common.h"

namespace {

using namespace pkvd;

__device__ __forceinline__ float wave_max4(float x) {
  // max over the 4 lanes l, l^16, l^32, l^48 (same lane column)
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int QT>
struct Mfma;

template <>
struct Mfma<PKV_BF16> {
  using v8 = bf16x8;
  using v4 = i16x4;
  __device__ static f32x4 qk(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 pv(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // two E4M3 bytes (word `hi` of w) -> two bf16 in a 32-bit word
  __device__ static uint32_t fp8x2(uint32_t w, bool hi) {
    return __builtin_bit_cast(uint32_t,
                              hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
  __device__ static uint32_t pack2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
  }
  __device__ static float rounded(float a) { return (float)(__bf16)a; }
};

template <>
struct Mfma<PKV_F16> {
  using v8 = f16x8;
  using v4 = f16x4;
  __device__ static f32x4 qk(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 pv(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  __device__ static uint32_t fp8x2(uint32_t w, bool hi) {
    return __builtin_bit_cast(uint32_t,
                              hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
  __device__ static uint32_t pack2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
  }
  __device__ static float rounded(float a) { return (float)(_Float16)a; }
};

template <typename V>
__device__ __forceinline__ V as_v8(uint4 r) {
  return __builtin_bit_cast(V, r);
}
template <typename V>
__device__ __forceinline__ V as_v4(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(V, make_uint2(a, b));
}

// Row of V for one token as seen by one lane: DPL elements of the kv type.
template <int BYTES>
struct Row;
template <>
struct Row<4> {
  uint32_t w[1];
};
template <>
struct Row<8> {
  uint32_t w[2];
};
template <>
struct Row<16> {
  uint32_t w[4];
};

template <int BYTES>
__device__ __forceinline__ Row<BYTES> load_row(const uint8_t* ptr) {
  Row<BYTES> r;
  if constexpr (BYTES == 16) {
    uint4 v = *reinterpret_cast<const uint4*>(ptr);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (BYTES == 8) {
    uint2 v = *reinterpret_cast<const uint2*>(ptr);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    r.w[0] = *reinterpret_cast<const uint32_t*>(ptr);
  }
  return r;
}

template <int QT, int KVT, int D, int HS>
__global__ __launch_bounds__(64 * pkv::kWaves) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_mfma_kernel(DecodeParams p) {
  using M = Mfma<QT>;
  using V8 = typename M::v8;
  using V4 = typename M::v4;
  constexpr int LD = D + 4;
  constexpr int DPL = D / 16;        // dims per lane in a V row = PV m-tiles
  constexpr int KSTEPS = D / 32;     // QK k-steps of 32
  constexpr bool FP8 = (KVT == PKV_FP8_E4M3);
  constexpr int KVB = FP8 ? 1 : 2;
  constexpr int64_t TILE = 16 * D * KVB;   // bytes of one (block, kv-head) tile
  constexpr int ROWB = DPL * KVB;          // bytes of a lane's slice of one V row
  constexpr int KL = FP8 ? D / 64 : KSTEPS;  // 16-byte K loads per lane

  // raw bytes of one block as loaded by one lane
  struct Raw {
    uint4 k[KL];
    Row<ROWB> v[4];
  };

  __shared__ float sm_m[pkv::kWaves * HS];
  __shared__ float sm_l[pkv::kWaves * HS];
  __shared__ float sm_o[pkv::kWaves * HS * LD];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int part = blockIdx.x, s = blockIdx.z;
  const int hk = blockIdx.y / p.hchunks, hc = blockIdx.y % p.hchunks;
  const int h_first = hk * p.g + hc * p.chunk_heads;
  const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
  const int ctx = clamped_ctx(p, s);
  const int nblk = (ctx + 15) >> 4;
  const int b_begin = part * p.part_blocks;
  if (part > 0 && b_begin >= nblk) return;
  const int b_end = min(b_begin + p.part_blocks, nblk);

  // B operand of QK: lane (G, c) holds q-head c, the 8 dims of k-slot G.
  V8 qop[KSTEPS];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)s * p.Hq + h_first + c) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int dim0 = FP8 ? (64 * (kk / 2) + 16 * G + 8 * (kk % 2)) : (32 * kk + 8 * G);
      uint4 r = make_uint4(0, 0, 0, 0);
      if (c < nh) r = *reinterpret_cast<const uint4*>(qrow + dim0);
      qop[kk] = as_v8<V8>(r);
    }
  }

  f32x4 o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int64_t blk_stride = (int64_t)p.Hkv * TILE;
  const int64_t head_off = (int64_t)hk * TILE;
  const int32_t* btrow = p.bt + (int64_t)s * p.mb;

  auto issue = [&](Raw& r, int phys) {
    const uint8_t* kt = p.kc + phys * blk_stride + head_off;
    const uint8_t* vt = p.vc + phys * blk_stride + head_off;
    if constexpr (FP8) {
#pragma unroll
      for (int mm = 0; mm < KL; ++mm)
        r.k[mm] = *reinterpret_cast<const uint4*>(kt + c * D + 64 * mm + 16 * G);
    } else {
#pragma unroll
      for (int kk = 0; kk < KL; ++kk)
        r.k[kk] = *reinterpret_cast<const uint4*>(kt + (c * D + 32 * kk + 8 * G) * 2);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      r.v[rr] = load_row<ROWB>(vt + ((4 * G + rr) * D + DPL * c) * KVB);
  };

  auto consume = [&](Raw& r, int valid) {
    // A operand of QK: lane (G, c) holds token c, the dims of k-slot G.
    V8 kop[KSTEPS];
    if constexpr (FP8) {
#pragma unroll
      for (int mm = 0; mm < KL; ++mm) {
        const uint4 x = r.k[mm];
        kop[2 * mm] = as_v8<V8>(make_uint4(M::fp8x2(x.x, false), M::fp8x2(x.x, true),
                                           M::fp8x2(x.y, false), M::fp8x2(x.y, true)));
        kop[2 * mm + 1] = as_v8<V8>(make_uint4(M::fp8x2(x.z, false), M::fp8x2(x.z, true),
                                               M::fp8x2(x.w, false), M::fp8x2(x.w, true)));
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) kop[kk] = as_v8<V8>(r.k[kk]);
    }
    if (valid < 16) {
      // tokens past the context hold stale data (possibly NaN): zero their V
      // so that a zero weight cannot meet a NaN in the PV product
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (4 * G + rr >= valid)
#pragma unroll
          for (int i = 0; i < ROWB / 4; ++i) r.v[rr].w[i] = 0u;
    }

    // S = K Q^T: lane (G, c) gets tokens 4G+i, head c.
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) sacc = M::qk(kop[kk], qop[kk], sacc);

    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (4 * G + i < valid) ? sacc[i] * p.sl2 : kNegInf;
    float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    bm = wave_max4(bm);
    const float m_new = fmaxf(m_run, bm);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(z[i] - m_new);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] *= alpha;
    }
    // B operand of PV: k-slot (G, i) = token 4G+i, column c = head c.  The
    // weights go in as a 16-bit head plus a 16-bit remainder, so the product
    // keeps about 16 bits of each weight instead of 8 (bf16) or 11 (f16).
    const V4 pb = as_v4<V4>(M::pack2(pr[0], pr[1]), M::pack2(pr[2], pr[3]));
    float lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = pr[i] - M::rounded(pr[i]);
    const V4 pl = as_v4<V4>(M::pack2(lo[0], lo[1]), M::pack2(lo[2], lo[3]));

    // A operand of PV for m-tile e: dim DPL*c + e of tokens 4G..4G+3.
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const int wi = e / 4, k = e % 4;
        const uint32_t sel = (uint32_t)k | ((4u + k) << 8) | ((k + 1u) << 16) | ((5u + k) << 24);
        const uint32_t x01 = __builtin_amdgcn_perm(r.v[1].w[wi], r.v[0].w[wi], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(r.v[3].w[wi], r.v[2].w[wi], sel);
        const V4 a0 = as_v4<V4>(M::fp8x2(x01, false), M::fp8x2(x23, false));
        const V4 a1 = as_v4<V4>(M::fp8x2(x01, true), M::fp8x2(x23, true));
        o[e] = M::pv(a0, pl, M::pv(a0, pb, o[e]));
        o[e + 1] = M::pv(a1, pl, M::pv(a1, pb, o[e + 1]));
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int wi = e / 2;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t x01 = __builtin_amdgcn_perm(r.v[1].w[wi], r.v[0].w[wi], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(r.v[3].w[wi], r.v[2].w[wi], sel);
        const V4 a0 = as_v4<V4>(x01, x23);
        o[e] = M::pv(a0, pl, M::pv(a0, pb, o[e]));
      }
    }
  };

  // This wave's blocks are b_begin + w + 4*i, i < n_it.  Their physical ids
  // are fetched 64 at a time into one VGPR (lane i holds block i), then read
  // back with readlane; the K/V loads of block i+1 are issued before block i
  // is consumed so that every wave keeps a block in flight.
  const int n_it = b_end - b_begin - w > 0 ? (b_end - b_begin - w + pkv::kWaves - 1) / pkv::kWaves
                                           : 0;
  for (int base = 0; base < n_it; base += 64) {
    const int cnt = min(64, n_it - base);
    const int ids = lane < cnt ? btrow[b_begin + w + pkv::kWaves * (base + lane)] : -1;
    auto tokens = [&](int i) {
      return min(16, ctx - 16 * (b_begin + w + pkv::kWaves * (base + i)));
    };
    Raw ra, rb;
    int pa = __builtin_amdgcn_readlane(ids, 0);
    bool va = (unsigned)pa < (unsigned)p.nb;   // bad table entry: no weight
    if (va) issue(ra, pa);
    for (int i = 0; i < cnt; i += 2) {
      bool vb = false;
      if (i + 1 < cnt) {
        const int pb = __builtin_amdgcn_readlane(ids, i + 1);
        vb = (unsigned)pb < (unsigned)p.nb;
        if (vb) issue(rb, pb);
      }
      if (va) consume(ra, tokens(i));
      if (i + 1 >= cnt) break;
      va = false;
      if (i + 2 < cnt) {
        pa = __builtin_amdgcn_readlane(ids, i + 2);
        va = (unsigned)pa < (unsigned)p.nb;
        if (va) issue(ra, pa);
      }
      if (vb) consume(rb, tokens(i + 1));
    }
  }

  // lane (G, c) holds O[head c][dim DPL*(4G+i) + e]; l needs the 4 G lanes
  l_run = wave_sum4(l_run);
  if (c < nh) {
    if (G == 0) {
      sm_m[w * HS + c] = m_run;
      sm_l[w * HS + c] = l_run;
    }
    float* dst = sm_o + (w * HS + c) * LD + DPL * 4 * G;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[DPL * i + e] = o[e][i];
  }
  __syncthreads();
  merge_waves_and_store<QT, D, HS>(p, sm_m, sm_l, sm_o, nh, s, h_first, part);
}

template <int QT, int KVT, int D, int HS>
int launch_t(const pkv::DecodeArgs& a, const DecodeParams& kp) {
  dim3 grid(kp.num_parts, a.num_kv_heads * kp.hchunks, a.num_seqs);
  decode_mfma_kernel<QT, KVT, D, HS>
      <<<grid, dim3(64 * pkv::kWaves), 0, (hipStream_t)a.stream>>>(kp);
  return (int)hipGetLastError();
}

template <int QT, int KVT, int D>
int launch_hs(const pkv::DecodeArgs& a, const DecodeParams& kp) {
  if (kp.chunk_heads <= 4) return launch_t<QT, KVT, D, 4>(a, kp);
  if (kp.chunk_heads <= 8) return launch_t<QT, KVT, D, 8>(a, kp);
  return launch_t<QT, KVT, D, 16>(a, kp);
}

}  // namespace

namespace pkv {

int launch_decode_mfma(const DecodeArgs& a) {
  const pkvd::DecodeParams kp = pkvd::make_params(a, 16);
  const int q = a.q_dtype, kv = a.kv_dtype, D = a.head_dim;
#define PKV_MFMA_CASE(QT, KVT, DD) \
  if (q == QT && kv == KVT && D == DD) return launch_hs<QT, KVT, DD>(a, kp);
  PKV_MFMA_CASE(PKV_BF16, PKV_BF16, 128)
  PKV_MFMA_CASE(PKV_BF16, PKV_BF16, 64)
  PKV_MFMA_CASE(PKV_F16, PKV_F16, 128)
  PKV_MFMA_CASE(PKV_F16, PKV_F16, 64)
  PKV_MFMA_CASE(PKV_BF16, PKV_FP8_E4M3, 128)
  PKV_MFMA_CASE(PKV_BF16, PKV_FP8_E4M3, 64)
  PKV_MFMA_CASE(PKV_F16, PKV_FP8_E4M3, 128)
  PKV_MFMA_CASE(PKV_F16, PKV_FP8_E4M3, 64)
#undef PKV_MFMA_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace pkv
