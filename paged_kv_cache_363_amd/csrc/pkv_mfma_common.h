// Matrix-core building blocks shared by the MFMA decode kernels: operand
// types, the per-lane loads of one 16-token K/V tile and the per-tile update
// (QK^T on v_mfma_f32_16x16x32, online softmax, PV on v_mfma_f32_16x16x16).
//
// With grouped-query attention the g q-heads sharing one kv-head read the
// same K and V tiles, so per tile QK^T is a [16 tokens x d] by [d x g]
// product and PV a [g x 16] by [16 x d] product.  The g heads are padded to
// the 16 MFMA columns with zero queries.  The accumulator layout of the first
// product (lane l holds rows 4(l/16)+i, column l%16) is the B-operand layout
// of the second one (PV computed as O^T = V^T P^T), so the softmax weights
// stay in registers, and O^T keeps one head per lane column, which makes the
// online-softmax rescale a per-lane multiply.
//
// Precision of the weights in PV: with an f16 cache, or a cache of one-byte
// codes (E4M3, INT8; f16 holds every such value exactly), PV runs in f16 and
// each weight is rounded once to f16 (11 significant bits, relative error at
// most 2^-11).  bf16 holds only 8 bits, so with a bf16 cache a weight enters
// PV as a bf16 head plus a bf16 remainder (two MFMAs, about 16 bits).
//
// One-byte K codes are widened to the q type in registers (every E4M3 value
// and every INT8 code is exact in bf16 and f16); k_scale is folded into the
// logit scale and v_scale into the final normalisation.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pkv_decode_common.h"

#ifndef PKV_LAZY_RESCALE
#define PKV_LAZY_RESCALE 8.0f   // see MfmaTile::consume
#endif
#ifndef PKV_ID_VGPRS
#define PKV_ID_VGPRS 2   // block-id windows of 64 * PKV_ID_VGPRS blocks
#endif

namespace pkvd {

__device__ __forceinline__ float wave_max4(float x) {
  // max over the 4 lanes l, l^16, l^32, l^48 (same lane column)
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) x = min(x, __shfl_xor(x, k));
  return x;
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
  // both halves rounded to nearest even in one v_cvt_pk_bf16_f32 (two
  // scalar conversions cost two of them plus a shift and an or)
  __device__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  }
  __device__ static uint32_t pack2_one(float a, float b) { return pack2(a, b); }
  // two INT8 codes (bytes 2*hi and 2*hi+1 of w) -> two bf16 (exact: |code| <= 127)
  __device__ static uint32_t i8x2(uint32_t w, bool hi) {
    const uint32_t h = hi ? w >> 16 : w;
    return pack2((float)(int32_t)(int8_t)h, (float)(int32_t)(int8_t)(h >> 8));
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
  // The same rounding (nearest, ties to even) in one v_cvt_pk_f16_f32: fewer
  // instructions for the multi-query kernels, which are bound by their
  // per-tile instructions; decode on the 70B-shaped E4M3 cache measured
  // 0.3 us slower with it, so decode keeps pack2.
  __device__ static uint32_t pack2_one(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
  __device__ static uint32_t i8x2(uint32_t w, bool hi) {
    const uint32_t h = hi ? w >> 16 : w;
    return pack2((float)(int32_t)(int8_t)h, (float)(int32_t)(int8_t)(h >> 8));
  }
  __device__ static float rounded(float a) { return (float)(_Float16)a; }
  // two INT8 codes (bytes 2*hi and 2*hi+1 of w) -> two f16, exact: the byte
  // c ^ 0x80 = c + 128 becomes the low mantissa bits of f16 1024 (0x6400),
  // and subtracting 1152 in f16 leaves c
  __device__ static uint32_t i8x2_magic(uint32_t w, bool hi) {
    const uint32_t x = w ^ 0x80808080u;
    const uint32_t m = __builtin_amdgcn_perm(0x64646464u, x, hi ? 0x04030402u : 0x04010400u);
    const f16x2 r = __builtin_bit_cast(f16x2, m) - f16x2{(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, r);
  }
};

template <typename V>
__device__ __forceinline__ V as_v8(uint4 r) {
  return __builtin_bit_cast(V, r);
}
template <typename V>
__device__ __forceinline__ V as_v8(u32x4 r) {
  return __builtin_bit_cast(V, r);
}
template <typename V>
__device__ __forceinline__ V as_v4(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(V, make_uint2(a, b));
}

// Row of V for one token as seen by one lane: DPL elements of the kv type,
// held in the loaded vector type (see ld_vec16).
template <int BYTES>
struct Row;
template <>
struct Row<4> {
  uint32_t w[1];
};
template <>
struct Row<8> {
  u32x2 w;
};
template <>
struct Row<16> {
  u32x4 w;
};

template <int BYTES, bool NT>
__device__ __forceinline__ Row<BYTES> load_row(const uint8_t* ptr) {
  Row<BYTES> r;
  if constexpr (BYTES == 16) {
    r.w = ld_vec16<NT>(ptr);
  } else if constexpr (BYTES == 8) {
    r.w = ld_vec8<NT>(ptr);
  } else {
    r.w[0] = ld_tile4<NT>(ptr);
  }
  return r;
}


// One 16-token tile of one kv-head, as seen by one lane of a wave.
//   K loads: lane (G = l/16, c = l%16) reads token c, the dims of k-slot G.
//   V loads: lane (G, c) reads tokens 4G..4G+3, dims DPL*c .. DPL*c+DPL-1.
template <int QT, int KVT, int D>
struct MfmaTile {
  using M = Mfma<QT>;
  using V8 = typename M::v8;
  using V4 = typename M::v4;
  static constexpr int DPL = D / 16;        // dims per lane in a V row = PV m-tiles
  static constexpr int KSTEPS = D / 32;     // QK k-steps of 32
  // one-byte codes (E4M3 or INT8) widened to the q dtype in registers
  static constexpr bool BYTE = (KVT == PKV_FP8_E4M3 || KVT == PKV_INT8);
  static constexpr int KVB = BYTE ? 1 : 2;
  static constexpr int64_t TILE = 16 * D * KVB;   // bytes of one (block, kv-head) tile
  static constexpr int ROWB = DPL * KVB;          // bytes of a lane's slice of one V row
  static constexpr int KL = BYTE ? D / 64 : KSTEPS;  // 16-byte K loads per lane
  // PV in f16 with one f16 weight (f16 and one-byte caches), else in the
  // q type with a head + remainder pair of weights
  static constexpr bool PVH = BYTE || KVT == PKV_F16;
  using PM = Mfma<PVH ? PKV_F16 : QT>;
  using P4 = typename PM::v4;

  // two one-byte codes (half-word `hi` of w) -> two q-dtype values, exact
  __device__ static uint32_t cvt2(uint32_t w, bool hi) {
    if constexpr (KVT == PKV_INT8) return M::i8x2(w, hi);
    else return M::fp8x2(w, hi);
  }
  // the same, to f16 (the PV operand)
  __device__ static uint32_t cvt2_f16(uint32_t w, bool hi) {
    if constexpr (KVT == PKV_INT8) return PM::i8x2_magic(w, hi);
    else return PM::fp8x2(w, hi);
  }

  using VRow = Row<ROWB>;
  struct Raw {
    u32x4 k[KL];
    VRow v[4];
  };

  // dim of element i of k-slot G in QK step kk (the same map for q and K)
  __device__ static int qk_dim0(int kk, int G) {
    return BYTE ? (64 * (kk / 2) + 16 * G + 8 * (kk % 2)) : (32 * kk + 8 * G);
  }

  // raw q row slice of q-head `row` (or zeros when !live) for every QK step
  __device__ static void load_q(uint4* qr, const void* q, int64_t row, bool live, int G) {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(q) + row * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qr[kk] = make_uint4(0, 0, 0, 0);
      if (live) qr[kk] = *reinterpret_cast<const uint4*>(qrow + qk_dim0(kk, G));
    }
  }

  // The same for a cache with per-channel K scales: q_i * ks_i in fp32, as a
  // q-dtype head (qhi) plus its remainder (qlo), so that two MFMAs keep about
  // 16 mantissa bits of each product.  ks: the kv-head's row of scales.
  __device__ static void load_q_scaled(uint4* qhi, uint4* qlo, const void* q, int64_t row,
                                       bool live, int G, const float* ks) {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(q) + row * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qhi[kk] = make_uint4(0, 0, 0, 0);
      qlo[kk] = make_uint4(0, 0, 0, 0);
      if (live) {
        const int d0 = qk_dim0(kk, G);
        const uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = (QT == PKV_F16 ? f16_lo(w[i]) : bf16_lo(w[i])) * ks[d0 + 2 * i];
          const float b = (QT == PKV_F16 ? f16_hi(w[i]) : bf16_hi(w[i])) * ks[d0 + 2 * i + 1];
          hi[i] = M::pack2(a, b);
          lo[i] = M::pack2(a - M::rounded(a), b - M::rounded(b));
        }
        qhi[kk] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        qlo[kk] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
    }
  }

  // Byte offsets of a lane's first K and V element inside a tile; the other
  // loads of the lane sit at fixed distances from them.  Unsigned 32-bit, so
  // that a load is a wave-uniform base plus one lane offset (the SGPR-base
  // form of global_load) with no per-lane 64-bit address arithmetic.
  __device__ static uint32_t k_lane_off(int c, int G) {
    return BYTE ? (uint32_t)(c * D + 16 * G) : (uint32_t)((c * D + 8 * G) * 2);
  }
  __device__ static uint32_t v_lane_off(int c, int G) {
    return (uint32_t)((4 * G * D + DPL * c) * KVB);
  }

  // NT: non-temporal (streaming) loads, see ld_tile16
  template <bool NT>
  __device__ static void issue(Raw& r, const uint8_t* kt, const uint8_t* vt, uint32_t koff,
                               uint32_t voff) {
    const uint8_t* kp = kt + koff;
    const uint8_t* vp = vt + voff;
#pragma unroll
    for (int kk = 0; kk < KL; ++kk) r.k[kk] = ld_vec16<NT>(kp + 64 * kk);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.v[rr] = load_row<ROWB, NT>(vp + rr * D * KVB);
  }

  // Online-softmax update of NTL column tiles with one K/V tile holding
  // `valid` live tokens (0 = none: the state does not change, and the tile's
  // registers are still read, so the caller need not branch around it).
  // Column tile j has its own q operand qr[j][KSTEPS] and state m_run[j],
  // l_run[j], o[j][DPL].  In the multi-query form (NTL > 1 or CAUSAL) l_run
  // holds one f32x4 per column tile (4 NTL floats, 16-byte aligned), which
  // accumulates on the matrix cores: every element is the column's whole
  // sum of weights.  Otherwise l_run[j] is this lane's share of it (tokens
  // 4G..4G+3), summed over the lanes of a column by the caller.  CAUSAL: the lane's column of tile j sits at
  // position pos[j] and attends to min(valid, pos[j] - tok0 + 1) tokens of
  // the tile, whose first token is at position tok0; otherwise to `valid`.
  // whole (wave-uniform): every column of the wave attends to all 16 tokens,
  // so the per-token limits need not be taken (the multi-query form).  K and
  // V are widened once and serve every column tile.  V rows past `valid` are
  // zeroed; rows below `valid` past a column's limit are finite and get
  // weight zero.
  // PC (one column tile only): qlo holds the remainder of per-channel-scaled
  // q (load_q_scaled), a second QK pass.
  template <int NTL = 1, bool PC = false, bool CAUSAL = false>
  __device__ static void consume(Raw& r, int valid, bool whole, const int* pos, int tok0,
                                 const uint4* qr, float sl2, float* m_run, float* l_run,
                                 f32x4* o, int c, int G, const uint4* qlo = nullptr) {
    static_assert(!PC || NTL == 1, "per-channel scales take one column tile");
    V8 kop[KSTEPS];
    if constexpr (BYTE) {
#pragma unroll
      for (int mm = 0; mm < KL; ++mm) {
        const u32x4 x = r.k[mm];
        kop[2 * mm] = as_v8<V8>(make_uint4(cvt2(x.x, false), cvt2(x.x, true),
                                           cvt2(x.y, false), cvt2(x.y, true)));
        kop[2 * mm + 1] = as_v8<V8>(make_uint4(cvt2(x.z, false), cvt2(x.z, true),
                                               cvt2(x.w, false), cvt2(x.w, true)));
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) kop[kk] = as_v8<V8>(r.k[kk]);
    }
    // Several column tiles or a causal limit: the multi-query kernels, whose
    // time goes to the per-tile update; one tile without it: decode, bound
    // by memory.  The two keep separate forms of the steps below, each the
    // faster one measured for its kernels.
    constexpr bool MQ = NTL > 1 || CAUSAL;
    // Tokens past the context hold stale data (possibly NaN): zero their V
    // so that a zero weight cannot meet a NaN in the PV product.  Only a
    // context's last block has fewer than 16 valid tokens: the multi-query
    // form skips the others with a branch (12 instructions per block saved;
    // with two blocks in flight its join adds no wait), decode selects on
    // every tile.
    if constexpr (MQ) {
      if (valid < 16) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (4 * G + rr >= valid)
#pragma unroll
            for (int i = 0; i < ROWB / 4; ++i) r.v[rr].w[i] = 0u;
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const bool live = 4 * G + rr < valid;
#pragma unroll
        for (int i = 0; i < ROWB / 4; ++i) r.v[rr].w[i] = live ? r.v[rr].w[i] : 0u;
      }
    }

    P4 pb[NTL];            // PV weights of each column tile
    [[maybe_unused]] V4 pl[NTL];   // their bf16 remainders (bf16 caches)
    // Multi-query form on bf16 caches: head and remainder side by side, the
    // B operand of one 16x16x32 MFMA (see the PV step below)
    constexpr bool PV32 = MQ && !PVH;
    [[maybe_unused]] uint4 phl[PV32 ? NTL : 1];
    // S = K Q^T of every column tile first (independent MFMA chains, one
    // basic block): lane (G, c) gets tokens 4G+i, column c.
    f32x4 sacc[NTL];
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
      sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        sacc[j] = M::qk(kop[kk], as_v8<V8>(qr[j * KSTEPS + kk]), sacc[j]);
      if constexpr (PC) {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) sacc[j] = M::qk(kop[kk], as_v8<V8>(qlo[kk]), sacc[j]);
      }
    }
    // the PV B operand of column tile j from its weights
    auto weights = [&](int j, const float* pr) {
      if constexpr (PV32) {
        // the heads' values read back from their packed bf16 words
        const uint32_t h01 = M::pack2(pr[0], pr[1]), h23 = M::pack2(pr[2], pr[3]);
        const float lo0 = pr[0] - __uint_as_float(h01 << 16);
        const float lo1 = pr[1] - __uint_as_float(h01 & 0xFFFF0000u);
        const float lo2 = pr[2] - __uint_as_float(h23 << 16);
        const float lo3 = pr[3] - __uint_as_float(h23 & 0xFFFF0000u);
        phl[j] = make_uint4(h01, h23, M::pack2(lo0, lo1), M::pack2(lo2, lo3));
        return;
      }
      // k-slot (G, i) = token 4G+i, column c
      if constexpr (MQ)
        pb[j] = as_v4<P4>(PM::pack2_one(pr[0], pr[1]), PM::pack2_one(pr[2], pr[3]));
      else
        pb[j] = as_v4<P4>(PM::pack2(pr[0], pr[1]), PM::pack2(pr[2], pr[3]));
      if constexpr (!PVH) {
        // bf16: the weight as a bf16 head plus its bf16 remainder
        float lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = pr[i] - M::rounded(pr[i]);
        pl[j] = as_v4<V4>(M::pack2(lo[0], lo[1]), M::pack2(lo[2], lo[3]));
      }
    };
    // The reference the weights are taken against moves only when the
    // tile's maximum exceeds it by more than PKV_LAZY_RESCALE (base-2 units):
    // weights up to 2^PKV_LAZY_RESCALE, no rescale of l and acc for small
    // rises.  l and acc keep one common reference, so the final acc / l (and
    // the log-sum-exp merges) are the same in real arithmetic.  A tile with
    // no valid token so far (m_keep still -inf) shifts by 0, so that it
    // leaves the state at zero instead of producing NaN.  acc is rescaled in
    // one branch for every column tile (a tile whose factor is 1 is
    // multiplied by 1, which changes nothing), so that the tiles' MFMA chains
    // above stay in one basic block.
    if constexpr (!MQ) {
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = (4 * G + i < valid) ? sacc[0][i] * sl2 : kNegInf;
      float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      bm = wave_max4(bm);
      const float m_new = fmaxf(m_run[0], bm);
      const float m_keep =
          (m_run[0] != kNegInf && m_new <= m_run[0] + PKV_LAZY_RESCALE) ? m_run[0] : m_new;
      const float m_ref = m_keep == kNegInf ? 0.f : m_keep;
      const float alpha = __builtin_amdgcn_exp2f(m_run[0] - m_ref);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(z[i] - m_ref);
      l_run[0] = l_run[0] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m_run[0] = m_keep;
      weights(0, pr);
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] *= alpha;
      }
    } else {
      // Most tiles are seen whole by every column: then the per-token test
      // of the causal limit is skipped (a wave-uniform branch with no load
      // inside).  Logits are taken against the running references first, one
      // fma each: while no logit of the wave exceeds its column's reference
      // by more than PKV_LAZY_RESCALE (the common case once a piece has
      // started), every reference stays, as the lazy rule above keeps it, and
      // the wave needs no maximum across lanes, no rescale and no test of an
      // empty state (a reference of -inf puts any live logit at +inf, and a
      // column with none live so far gets weights exp2(-inf) = 0).  Otherwise
      // the references are updated by the lazy rule, acc and l rescaled, and
      // the logits retaken.
      float t[NTL][4];
      auto lim = [&](int j) { return CAUSAL ? min(valid, pos[j] - tok0 + 1) : valid; };
      auto logits = [&](const float* mr) {
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) t[j][i] = __builtin_fmaf(sacc[j][i], sl2, -mr[j]);
        if (!whole) {
#pragma unroll
          for (int j = 0; j < NTL; ++j) {
            const int v = lim(j);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * G + i >= v) t[j][i] = kNegInf;
          }
        }
      };
      logits(m_run);
      float tmax = kNegInf;
#pragma unroll
      for (int j = 0; j < NTL; ++j)
        tmax = fmaxf(tmax, fmaxf(fmaxf(t[j][0], t[j][1]), fmaxf(t[j][2], t[j][3])));
      if (__any(tmax > PKV_LAZY_RESCALE)) {
        float m_rf[NTL];
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          float bm = kNegInf;
          const int v = whole ? 16 : lim(j);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * G + i < v) bm = fmaxf(bm, sacc[j][i] * sl2);
          bm = wave_max4(bm);
          const float m_new = fmaxf(m_run[j], bm);
          const bool keep = m_run[j] != kNegInf && m_new <= m_run[j] + PKV_LAZY_RESCALE;
          const float m_keep = keep ? m_run[j] : m_new;
          m_rf[j] = m_keep == kNegInf ? 0.f : m_keep;
          const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_rf[j]);
          reinterpret_cast<f32x4*>(l_run)[j] *= alpha;
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[j * DPL + e] *= alpha;
          m_run[j] = m_keep;
        }
        logits(m_rf);
      }
#pragma unroll
      for (int j = 0; j < NTL; ++j) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(t[j][i]);
        weights(j, pr);
      }
    }

    // A operand of PV for m-tile e: dim DPL*c + e of tokens 4G..4G+3, built
    // once for every column tile.
    if constexpr (BYTE) {
#pragma unroll
      for (int e = 0; e < DPL; e += 2) {
        const int wi = e / 4, k = e % 4;
        const uint32_t sel = (uint32_t)k | ((4u + k) << 8) | ((k + 1u) << 16) | ((5u + k) << 24);
        const uint32_t x01 = __builtin_amdgcn_perm(r.v[1].w[wi], r.v[0].w[wi], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(r.v[3].w[wi], r.v[2].w[wi], sel);
        const P4 a0 = as_v4<P4>(cvt2_f16(x01, false), cvt2_f16(x23, false));
        const P4 a1 = as_v4<P4>(cvt2_f16(x01, true), cvt2_f16(x23, true));
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          o[j * DPL + e] = PM::pv(a0, pb[j], o[j * DPL + e]);
          o[j * DPL + e + 1] = PM::pv(a1, pb[j], o[j * DPL + e + 1]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int wi = e / 2;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t x01 = __builtin_amdgcn_perm(r.v[1].w[wi], r.v[0].w[wi], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(r.v[3].w[wi], r.v[2].w[wi], sel);
        const P4 a0 = as_v4<P4>(x01, x23);
        if constexpr (PV32) {
          // o += V (w_hi + w_lo) as one MFMA with k = 32: k-slots 8G..8G+3
          // hold tokens 4G..4G+3 against the weights' heads, 8G+4..8G+7 the
          // same tokens against their remainders; the A operand carries the
          // V values twice.  One full-rate 16x16x32 instead of two half-rate
          // 16x16x16.
          const V8 a2 = as_v8<V8>(make_uint4(x01, x23, x01, x23));
#pragma unroll
          for (int j = 0; j < NTL; ++j) o[j * DPL + e] = M::qk(a2, as_v8<V8>(phl[j]), o[j * DPL + e]);
          continue;
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          if constexpr (PVH)
            o[j * DPL + e] = PM::pv(a0, pb[j], o[j * DPL + e]);
          else
            o[j * DPL + e] = M::pv(a0, pl[j], M::pv(a0, pb[j], o[j * DPL + e]));
        }
      }
    }
    // Multi-query form: l += the weights of the tile's 16 tokens, as one
    // MFMA against an all-ones A operand (the same weights as PV, so l and
    // acc sum identical terms; no VALU adds)
    if constexpr (MQ) {
      f32x4* la = reinterpret_cast<f32x4*>(l_run);
      if constexpr (PV32) {
        const V8 ones = as_v8<V8>(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
        for (int j = 0; j < NTL; ++j) la[j] = M::qk(ones, as_v8<V8>(phl[j]), la[j]);
      } else {
        static_assert(PVH, "the multi-query form takes f16 weights or bf16 head/remainder pairs");
        const P4 ones = as_v4<P4>(0x3C003C00u, 0x3C003C00u);   // f16 1.0
#pragma unroll
        for (int j = 0; j < NTL; ++j) la[j] = PM::pv(ones, pb[j], la[j]);
      }
    }
  }
};


// The step's new K/V row of one (sequence, kv-head), appended inside a decode
// kernel: the row goes to its slot and attention reads the context with it
// ("Transformer 推理优化", sections 2.2 and 3.3).  Lane l of a wave takes the
// row's elements EPL l .. EPL l + EPL - 1 (EPL = D / 64): it loads them raw
// (16-bit, the q dtype), encodes them to the cache's type with the bytes the
// cache append stores, and stages the encoded K row, then V row, in LDS
// (STAGE bytes).  sub() puts the staged row into a loaded tile of the slot's
// block, at the slot's position, in the tile's register layout: a wave that
// does so before consuming the tile sees the new row whether its loads ran
// before or after the row's store, so no read waits for the write.
template <int QT, int KVT, int D>
struct NewRow {
  using T = MfmaTile<QT, KVT, D>;
  static constexpr int EPL = D / 64;
  static constexpr int LB = EPL * T::KVB;   // encoded bytes per lane and row
  static constexpr int STAGE = 2 * D * T::KVB;

  // row: (sequence * num_kv_heads + kv-head)
  __device__ static void load(const uint8_t* kn, const uint8_t* vn, int64_t row, int lane,
                              uint32_t& kraw, uint32_t& vraw) {
    const int64_t e0 = row * D + EPL * lane;
    if constexpr (EPL == 2) {
      kraw = reinterpret_cast<const uint32_t*>(kn)[e0 / 2];
      vraw = reinterpret_cast<const uint32_t*>(vn)[e0 / 2];
    } else {
      kraw = reinterpret_cast<const uint16_t*>(kn)[e0];
      vraw = reinterpret_cast<const uint16_t*>(vn)[e0];
    }
  }
  __device__ static void put(uint8_t* dst, uint32_t x) {
    if constexpr (LB == 4) *reinterpret_cast<uint32_t*>(dst) = x;
    else if constexpr (LB == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)x;
    else *dst = (uint8_t)x;
  }
  __device__ static void encode(uint32_t kraw, uint32_t vraw, float k_inv, float v_inv,
                                uint32_t& ke, uint32_t& ve) {
    encode_new_chunk<QT, KVT, EPL>(make_uint4(kraw, 0u, 0u, 0u), k_inv, &ke);
    encode_new_chunk<QT, KVT, EPL>(make_uint4(vraw, 0u, 0u, 0u), v_inv, &ve);
  }
  // lds: STAGE bytes, 16-byte aligned
  __device__ static void stage(uint8_t* lds, int lane, uint32_t ke, uint32_t ve) {
    put(lds + LB * lane, ke);
    put(lds + D * T::KVB + LB * lane, ve);
  }
  // the row's store at `slot` (0 <= slot < num_blocks * 16)
  __device__ static void store(uint8_t* kc, uint8_t* vc, int64_t slot, int Hkv, int hk, int lane,
                               uint32_t ke, uint32_t ve) {
    const int64_t row0 = (((slot >> 4) * Hkv + hk) * pkv::kBlockSize + (slot & 15)) * D;
    put(kc + row0 * T::KVB + LB * lane, ke);
    put(vc + row0 * T::KVB + LB * lane, ve);
  }
  // r: a loaded tile of the slot's block; tn: the slot's position in it.
  // Every lane reads the staged row (the empty asm takes the values in all
  // lanes): otherwise the compiler turns the selects into exec-masked LDS
  // reads straight into the tile's registers, whose branches leave the load
  // counter's order unknown in the block loop, which then waits for every
  // load in flight.
  __device__ static void sub(typename T::Raw& r, const uint8_t* lds, int tn, int lane) {
    const int c = lane & 15, G = lane >> 4;
    const bool kl = c == tn, vl = G == (tn >> 2);
    u32x4 ek[T::KL];
#pragma unroll
    for (int kk = 0; kk < T::KL; ++kk) {
      const int d0 = T::BYTE ? 64 * kk + 16 * G : 32 * kk + 8 * G;   // as MfmaTile::issue
      ek[kk] = *reinterpret_cast<const u32x4*>(lds + d0 * T::KVB);
      asm volatile("" ::"v"(ek[kk]));
    }
#pragma unroll
    for (int kk = 0; kk < T::KL; ++kk) r.k[kk] = kl ? ek[kk] : r.k[kk];
    const typename T::VRow e =
        *reinterpret_cast<const typename T::VRow*>(lds + (D + T::DPL * c) * T::KVB);
    if constexpr (T::ROWB == 4)
      asm volatile("" ::"v"(e.w[0]));
    else
      asm volatile("" ::"v"(e.w));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const bool take = vl && rr == (tn & 3);
      if constexpr (T::ROWB == 4)
        r.v[rr].w[0] = take ? e.w[0] : r.v[rr].w[0];
      else
        r.v[rr].w = take ? e.w : r.v[rr].w;
    }
  }
};


// Online-softmax pass of one wave over the blocks [b0, b1) of one
// (sequence, kv-head) segment, continuing the running state of NTL column
// tiles (m_run[j], l_run[j], o[j][DPL], q operand qr[j][KSTEPS]).
//   kc, vc   : the caches, already offset to the segment's kv-head tile
//   row      : the sequence's block-table row
//   last     : index of the sequence's last block, tail its token count
// Block ids come 64 * PKV_ID_VGPRS at a time, one per lane of each of
// PKV_ID_VGPRS VGPRs, and are read back with readlane: a window boundary
// stalls the loads (the next window's ids must arrive first), so windows are
// wider than most pieces.  K/V loads run DEPTH blocks ahead of the block being
// consumed.
// Every load is issued unconditionally (ids past the chunk repeat its last
// block, invalid ids read block 0 and carry no weight), so the load counter
// can be waited on per block instead of drained.  nb must be > 0.
// stride: step i of the piece reads the block whose id is row[i * stride]
// (1: consecutive blocks; a wave taking every stride-th block of a run gets
// row offset to its first one).  Steps b0, b1, last and the hook's period
// count steps.  ids_first: the first window's ids, already loaded by the
// caller (lane l of ids_first[w] = row[(b0 + 64 w + l) * stride], any
// in-bounds id past the piece's end); nullptr: loaded here.
// CAUSAL: column tile j of the lane attends to positions <= pos[j] only
// (several queries of one sequence in one pass); otherwise pos is ignored.
// PC: per-channel K scales, qlo the remainder of the scaled q (load_q_scaled).
// Hook: with Hook::active, hook() runs after the last block of every run of
// hook.period blocks (runs aligned to multiples of the period) and after the
// piece's last block; it may read and reset the running state.  The loads of
// the next blocks stay in flight across it.  With Hook::subst,
// hook.prepare() runs once after the piece's first loads are issued, and
// hook.sub(tile, id) before each tile of block `id` is consumed (it may
// change the tile's registers).
struct NoHook {
  static constexpr bool active = false;
  static constexpr bool subst = false;
  int period = 0;
  __device__ void operator()() const {}
};

// A hook that calls f every `period` blocks.
template <typename F>
struct PeriodHook {
  static constexpr bool active = true;
  static constexpr bool subst = false;
  int period;
  F f;
  __device__ void operator()() const { f(); }
};

template <int QT, int KVT, int D, int DEPTH, bool NT, bool CAUSAL = false, bool PC = false,
          int NTL = 1, typename Hook = NoHook>
__device__ __forceinline__ void mfma_piece(const uint8_t* kc, const uint8_t* vc,
                                           int64_t blk_stride, const int32_t* row, int b0,
                                           int b1, int last, int tail, int nb, const uint4* qr,
                                           float sl2, float* m_run, float* l_run, f32x4* o,
                                           int lane, const int* pos = nullptr,
                                           const uint4* qlo = nullptr,
                                           const Hook& hook = Hook{}, int stride = 1,
                                           const int* ids_first = nullptr) {
  using T = MfmaTile<QT, KVT, D>;
  using Raw = typename T::Raw;
  const int c = lane & 15, G = lane >> 4;
  const uint32_t koff = T::k_lane_off(c, G), voff = T::v_lane_off(c, G);
  constexpr int NW = PKV_ID_VGPRS;
  [[maybe_unused]] int rem = Hook::active ? hook.period - b0 % hook.period : 0;
  // ids of the window of steps starting at c0 (in bounds: the step index is
  // clamped to the piece's last one)
  auto load_ids = [&](int* ids, int c0) {
    const int n = min(64 * NW, b1 - c0);
#pragma unroll
    for (int w = 0; w < NW; ++w) ids[w] = row[(int64_t)(c0 + min(64 * w + lane, n - 1)) * stride];
  };
  // CAUSAL: steps before whole_end are seen whole by every column (block b
  // is whole for a column at position q when 16 b + 15 <= q)
  int whole_end = 0;
  if constexpr (CAUSAL) {
    int pm = pos[0];
#pragma unroll
    for (int j = 1; j < NTL; ++j) pm = min(pm, pos[j]);
    whole_end = __builtin_amdgcn_readfirstlane((wave_min(pm) + 1) >> 4);
  }
  int ids[NW];
  if (ids_first) {
#pragma unroll
    for (int w = 0; w < NW; ++w) ids[w] = ids_first[w];
  } else {
    load_ids(ids, b0);
  }
  for (int c0 = b0; c0 < b1; c0 += 64 * NW) {
    const int n = min(64 * NW, b1 - c0);
    // The step index, the id and the tile's address are wave-uniform: kept
    // in scalar registers, the loads take the SGPR-base form and none of it
    // costs vector instructions.
    auto id_at = [&](int i) {
      const int k = __builtin_amdgcn_readfirstlane(i < n ? i : n - 1);
      int v = __builtin_amdgcn_readlane(ids[0], k & 63);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const int vw = __builtin_amdgcn_readlane(ids[w], k & 63);
        v = (k >> 6) == w ? vw : v;
      }
      return v;
    };
    auto addr = [&](int id) { return (int64_t)((unsigned)id < (unsigned)nb ? id : 0) * blk_stride; };
    Raw buf[DEPTH];
    int idc[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      idc[d] = id_at(d);
      const int64_t a = addr(idc[d]);
      T::template issue<NT>(buf[d], kc + a, vc + a, koff, voff);
      // Keep the blocks' loads in consumption order: the scheduler would
      // otherwise issue buf[0] last, and at the loop entry the load counter
      // would then be waited down to the newest block only.
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (Hook::subst) {
      if (c0 == b0) hook.prepare();
    }
    // Groups of DEPTH steps, each step issuing the step DEPTH ahead (past
    // the window's end: its last block again).
    if constexpr (NTL == 1) {
      // step ii from slot d: consume it, then (ISSUE) issue the loads of
      // step ii + DEPTH into the slot
      auto step = [&](int d, int ii, auto issue_c) {
        const int valid = (ii < n && (unsigned)idc[d] < (unsigned)nb)
                              ? (c0 + ii == last ? tail : 16) : 0;
        const bool whole = valid == 16 && (!CAUSAL || c0 + ii < whole_end);
        if constexpr (Hook::subst) hook.sub(buf[d], idc[d]);
        T::template consume<NTL, PC, CAUSAL>(buf[d], valid, whole, pos, 16 * (c0 + ii), qr, sl2,
                                             m_run, l_run, o, c, G, qlo);
        if constexpr (Hook::active) {
          if (ii < n && (--rem == 0 || c0 + ii == b1 - 1)) {
            hook();
            rem = hook.period;
          }
        }
        if constexpr (decltype(issue_c)::value) {
          const int idn = id_at(ii + DEPTH);
          const int64_t a = addr(idn);
          T::template issue<NT>(buf[d], kc + a, vc + a, koff, voff);
          idc[d] = idn;
        }
      };
      // In the piece's last window the final group issues nothing, so that
      // no unused load is left in flight when the piece ends (it would sit
      // ahead of the next loads in the load counter, and hold up the wave's
      // end).  The issuing and the final groups are separate code, so every
      // load counter wait stays exact.
      const bool last_win = c0 + 64 * NW >= b1;
      int i = 0;
      for (; last_win ? i + DEPTH < n : i < n; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) step(d, i + d, std::true_type{});
      }
      if (last_win) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) step(d, i + d, std::false_type{});
      }
    } else {
      // Several column tiles: every group issues (a second copy of the
      // group measured slower there: 64-row chunks 397 -> 418 us).
      for (int i = 0; i < n; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          const int ii = i + d;
          const int idn = id_at(ii + DEPTH);
          const int valid = (ii < n && (unsigned)idc[d] < (unsigned)nb)
                                ? (c0 + ii == last ? tail : 16) : 0;
          const bool whole = valid == 16 && (!CAUSAL || c0 + ii < whole_end);
          if constexpr (Hook::subst) hook.sub(buf[d], idc[d]);
          T::template consume<NTL, PC, CAUSAL>(buf[d], valid, whole, pos, 16 * (c0 + ii), qr,
                                               sl2, m_run, l_run, o, c, G, qlo);
          if constexpr (Hook::active) {
            if (ii < n && (--rem == 0 || c0 + ii == b1 - 1)) {
              hook();
              rem = hook.period;
            }
          }
          const int64_t a = addr(idn);
          T::template issue<NT>(buf[d], kc + a, vc + a, koff, voff);
          idc[d] = idn;
        }
      }
    }
    if (c0 + 64 * NW < b1) load_ids(ids, c0 + 64 * NW);
  }
}

}  // namespace pkvd
