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

template <int QT, int KVT, int D>
__global__ __launch_bounds__(64 * pkv::kWaves) void decode_mfma_kernel(DecodeParams p) {
  using M = Mfma<QT>;
  using V8 = typename M::v8;
  using V4 = typename M::v4;
  constexpr int HP = 16;             // MFMA columns = q-heads per workgroup
  constexpr int LD = D + 4;
  constexpr int DPL = D / 16;        // dims per lane in a V row = PV m-tiles
  constexpr int KSTEPS = D / 32;     // QK k-steps of 32
  constexpr bool FP8 = (KVT == PKV_FP8_E4M3);
  constexpr int KVB = FP8 ? 1 : 2;
  constexpr int64_t TILE = 16 * D * KVB;   // bytes of one (block, kv-head) tile
  constexpr int ROWB = DPL * KVB;          // bytes of a lane's slice of one V row

  __shared__ float sm_m[pkv::kWaves * HP];
  __shared__ float sm_l[pkv::kWaves * HP];
  __shared__ float sm_o[pkv::kWaves * HP * LD];

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

  for (int b = b_begin + w; b < b_end; b += pkv::kWaves) {
    const int phys = btrow[b];
    if ((unsigned)phys >= (unsigned)p.nb) continue;   // bad table entry: no weight
    const int valid = min(16, ctx - b * 16);
    const uint8_t* kt = p.kc + phys * blk_stride + head_off;
    const uint8_t* vt = p.vc + phys * blk_stride + head_off;

    // A operand of QK: lane (G, c) holds token c, the dims of k-slot G.
    V8 kop[KSTEPS];
    if constexpr (FP8) {
#pragma unroll
      for (int mm = 0; mm < D / 64; ++mm) {
        const uint4 r = *reinterpret_cast<const uint4*>(kt + c * D + 64 * mm + 16 * G);
        kop[2 * mm] = as_v8<V8>(make_uint4(M::fp8x2(r.x, false), M::fp8x2(r.x, true),
                                           M::fp8x2(r.y, false), M::fp8x2(r.y, true)));
        kop[2 * mm + 1] = as_v8<V8>(make_uint4(M::fp8x2(r.z, false), M::fp8x2(r.z, true),
                                               M::fp8x2(r.w, false), M::fp8x2(r.w, true)));
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        kop[kk] = as_v8<V8>(
            *reinterpret_cast<const uint4*>(kt + (c * D + 32 * kk + 8 * G) * 2));
    }

    // V rows: lane (G, c) reads tokens 4G..4G+3, dims DPL*c .. DPL*c+DPL-1.
    Row<ROWB> vr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vr[r] = load_row<ROWB>(vt + ((4 * G + r) * D + DPL * c) * KVB);
    if (valid < 16) {
      // tokens past the context hold stale data (possibly NaN): zero them so
      // that a zero weight cannot meet a NaN in the PV product
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * G + r >= valid)
#pragma unroll
          for (int i = 0; i < ROWB / 4; ++i) vr[r].w[i] = 0u;
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
    // B operand of PV: k-slot (G, i) = token 4G+i, column c = head c.
    const V4 pb = as_v4<V4>(M::pack2(pr[0], pr[1]), M::pack2(pr[2], pr[3]));

    // A operand of PV for m-tile e: dim DPL*c + e of tokens 4G..4G+3.
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const int wi = e / 4, k = e % 4;
        const uint32_t sel = (uint32_t)k | ((4u + k) << 8) | ((k + 1u) << 16) | ((5u + k) << 24);
        const uint32_t x01 = __builtin_amdgcn_perm(vr[1].w[wi], vr[0].w[wi], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(vr[3].w[wi], vr[2].w[wi], sel);
        o[e] = M::pv(as_v4<V4>(M::fp8x2(x01, false), M::fp8x2(x23, false)), pb, o[e]);
        o[e + 1] = M::pv(as_v4<V4>(M::fp8x2(x01, true), M::fp8x2(x23, true)), pb, o[e + 1]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int wi = e / 2;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t x01 = __builtin_amdgcn_perm(vr[1].w[wi], vr[0].w[wi], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(vr[3].w[wi], vr[2].w[wi], sel);
        o[e] = M::pv(as_v4<V4>(x01, x23), pb, o[e]);
      }
    }
  }

  // lane (G, c) holds O[head c][dim DPL*(4G+i) + e]; l needs the 4 G lanes
  l_run = wave_sum4(l_run);
  if (c < nh) {
    if (G == 0) {
      sm_m[w * HP + c] = m_run;
      sm_l[w * HP + c] = l_run;
    }
    float* dst = sm_o + (w * HP + c) * LD + DPL * 4 * G;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[DPL * i + e] = o[e][i];
  }
  __syncthreads();
  merge_waves_and_store<QT, D, HP>(p, sm_m, sm_l, sm_o, nh, s, h_first, part);
}

template <int QT, int KVT, int D>
int launch_t(const pkv::DecodeArgs& a, const DecodeParams& kp) {
  dim3 grid(kp.num_parts, a.num_kv_heads * kp.hchunks, a.num_seqs);
  decode_mfma_kernel<QT, KVT, D>
      <<<grid, dim3(64 * pkv::kWaves), 0, (hipStream_t)a.stream>>>(kp);
  return (int)hipGetLastError();
}

}  // namespace

namespace pkv {

int launch_decode_mfma(const DecodeArgs& a) {
  const pkvd::DecodeParams kp = pkvd::make_params(a, 16);
  const int q = a.q_dtype, kv = a.kv_dtype, D = a.head_dim;
#define PKV_MFMA_CASE(QT, KVT, DD) \
  if (q == QT && kv == KVT && D == DD) return launch_t<QT, KVT, DD>(a, kp);
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
