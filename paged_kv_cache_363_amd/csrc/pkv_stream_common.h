// Pieces shared by the kernels of the work-balanced schedule (decode and
// multi-query): the share arithmetic and the log-sum-exp merge of a segment
// that several waves computed in pieces.
//
// A persistent grid of W waves splits U units into equal contiguous shares:
// wave k owns units [floor(U k / W), floor(U (k+1) / W)).  A segment cut by
// share boundaries leaves one (m, l, acc) piece per wave in the partial slots
// of the workspace (slot 2k: the wave's first piece, 2k+1: its last), and the
// merge kernel combines them:
//   M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k acc_k 2^(m_k - M) / L.
#pragma once
#include <hip/hip_runtime.h>

#include "pkv_mfma_common.h"

namespace pkvd {

// floor(n / c) for 0 <= n < 2^53 and c >= 1.  n and c are exact in double,
// and a correctly rounded quotient cannot reach an integer that the exact
// quotient lies below (that would take n >= 2^53), so truncation gives the
// floor.  Far cheaper on the GPU than 64-bit integer division, which expands
// into a long VALU sequence.  Every share boundary goes through here, in the
// decode and the merge kernels alike.
__device__ __forceinline__ int64_t floor_div53(int64_t n, int64_t c) {
  return (int64_t)((double)n / (double)c);
}

// Log-sum-exp merge of the pieces of one column (one q-head of one query row)
// of a segment whose units the workers wa..wb share (wa < wb), and the store
// of its normalised row.  The first worker's piece sits in slot sl0, worker
// wa + k's (k > 0) in slot 2 (wa + k), its first piece.
//   part : [2W][HS][D] accumulators,  ml : [2W][HS][2] (m, l)
//   col  : the column inside a slot (< HS)
//   out_off : element offset of the row in out
// One wave; lane j holds piece j's (m, l) and weight, and the accumulator rows
// of all pieces are read with independent loads, eight at a time.
template <int QT, int D>
__device__ __forceinline__ void merge_split_column(const float* part, const float* ml, int HS,
                                                   int col, int64_t wa, int64_t wb, int64_t sl0,
                                                   void* out, int64_t out_off) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = (D + 63) / 64;
  const int np = (int)(wb - wa + 1);
  auto slot_of = [&](int k) { return k == 0 ? sl0 : 2 * (wa + k); };
  auto ml_of = [&](int k) {
    return *reinterpret_cast<const float2*>(ml + (slot_of(k) * HS + col) * 2);
  };
  // Accumulator rows of pieces base+j0 .. base+j0+7 (the last valid piece
  // repeated past cnt; its weight is zero there).
  auto load_rows = [&](float (&x)[8][PER], int base, int j0, int cnt) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t sl = slot_of(base + min(j0 + u, cnt - 1));
#pragma unroll
      for (int k2 = 0; k2 < PER; ++k2) {
        const int d = lane + 64 * k2;
        x[u][k2] = d < D ? part[(sl * HS + col) * D + d] : 0.f;
      }
    }
  };
  float acc[PER];
#pragma unroll
  for (int k2 = 0; k2 < PER; ++k2) acc[k2] = 0.f;
  auto add_rows = [&](const float (&x)[8][PER], float wgt, int j0, int cnt) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wj =
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), min(j0 + u, 63)));
      const float wu = (j0 + u < cnt) ? wj : 0.f;
#pragma unroll
      for (int k2 = 0; k2 < PER; ++k2) acc[k2] = fmaf(wu, x[u][k2], acc[k2]);
    }
  };
  // Lane k holds piece k's (m, l).  Those and the first eight accumulator
  // rows go out together: none depends on another, so the merge of a
  // segment split over at most eight workers waits on memory once.
  const int cnt0 = min(64, np);
  float x0[8][PER];
  load_rows(x0, 0, 0, cnt0);
  float m0 = kNegInf, l0 = 0.f;
  if (lane < np) {
    const float2 v = ml_of(lane);
    m0 = v.x;
    l0 = v.y;
  }
  float M = l0 > 0.f ? m0 : kNegInf;
  for (int k = lane + 64; k < np; k += 64) {
    const float2 v = ml_of(k);
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
  if (M != kNegInf) {
    for (int base = 0; base < np; base += 64) {
      float wgt = 0.f;
      if (base + lane < np) {
        const float2 v = base == 0 ? make_float2(m0, l0) : ml_of(base + lane);
        wgt = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - M) : 0.f;
        L += wgt * v.y;
      }
      const int cnt = min(64, np - base);
      int j0 = 0;
      if (base == 0) {
        add_rows(x0, wgt, 0, cnt);
        j0 = 8;
      }
      for (; j0 < cnt; j0 += 8) {
        float x[8][PER];
        load_rows(x, base, j0, cnt);
        add_rows(x, wgt, j0, cnt);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
#pragma unroll
  for (int k2 = 0; k2 < PER; ++k2) {
    const int d = lane + 64 * k2;
    if (d < D) store_out<QT>(out, out_off + d, L > 0.f ? acc[k2] / L : 0.f);
  }
}

}  // namespace pkvd
