// Paged decode attention on the matrix cores with a work-balanced schedule.
//
// The contexts of a decode batch are ragged, so a grid of one workgroup per
// (sequence, kv-head, partition) leaves many workgroups empty or short and
// the last ones run on an almost idle GPU.  Here the step's work is
// flattened into units -- one 16-token block of one segment, a segment being
// the q-heads of one kv-head (at most 16 of them) of one sequence, segments
// in sequence order -- and a fixed grid of waves splits the units into equal
// contiguous shares.  Every wave streams its share with the per-tile update
// of MfmaTile, keeping the next block's loads (and, at a segment change, the
// next q rows) in flight while it works on the current block.
//
// A share covers the tail of one segment, whole segments and the head of
// another.  A whole segment is normalised and stored by its wave.  A piece of
// a segment is stored as (m, l, acc) in the wave's partial slot (its first
// piece in slot 0, its last in slot 1) and counted on the segment's arrival
// counter; the wave that completes the count merges the pieces with the
// log-sum-exp rule
//   M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k acc_k 2^(m_k - M) / L.
// Counters are tagged with a per-call epoch in their high 32 bits, so a
// counter left by an earlier call reads as zero and the workspace needs no
// clearing.
//
// Math: softmax(q K^T * scale) V over the block-table-gathered context
// ("KV Cache 与 PageAttention深度实战", sections 1.2 and 3.2).
#include <hip/hip_runtime.h>

#include "pkv_mfma_common.h"

namespace {

using namespace pkvd;

constexpr int kSkWaves = 4;   // waves per workgroup; each wave is its own worker

struct StreamParams {
  void* out;
  const void* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  const int32_t* cl;
  int S, Hq, Hkv, g, Y, hchunks, chunk_heads, nb, mb;
  float sl2, vsc;
  uint32_t epoch;
  float* part;                 // [2 W][chunk_heads][D]
  float* ml;                   // [2 W][chunk_heads][2]
  unsigned long long* cnt;     // [S][Y]
};

template <int QT, int KVT, int D>
__global__ __launch_bounds__(64 * kSkWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void decode_stream_kernel(StreamParams p) {
  using T = MfmaTile<QT, KVT, D>;
  using Raw = typename T::Raw;
  constexpr int DPL = T::DPL;
  constexpr int KS = T::KSTEPS;

  __shared__ int sm_pref[pkv::kMaxStreamSeqs + 1];   // blocks before sequence s
  __shared__ int sm_ctx[pkv::kMaxStreamSeqs];        // clamped context lengths

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int S = p.S;
  const int cap = p.mb * pkv::kBlockSize;
  for (int i = threadIdx.x; i < S; i += 64 * kSkWaves) {
    const int n = p.cl[i];
    sm_ctx[i] = n < 0 ? 0 : (n > cap ? cap : n);
  }
  __syncthreads();
  if (w == 0) {
    int carry = 0;
    for (int base = 0; base < S; base += 64) {
      const int i = base + lane;
      int x = i < S ? (sm_ctx[i] + 15) >> 4 : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      if (i < S) sm_pref[i + 1] = carry + x;
      carry += __shfl(x, 63);
    }
    if (lane == 0) sm_pref[0] = 0;
  }
  __syncthreads();

  const int64_t Y = p.Y;
  const int64_t U = Y * sm_pref[S];
  const int W = gridDim.x * kSkWaves;
  const int wk = blockIdx.x * kSkWaves + w;

  // sequences without context get zero rows
  for (int s = wk; s < S; s += W)
    if (sm_ctx[s] == 0)
      for (int i = lane; i < p.Hq * D; i += 64) store_out<QT>(p.out, (int64_t)s * p.Hq * D + i, 0.f);

  const int64_t We = U < W ? U : W;   // workers with a non-empty share
  if (wk >= We) return;
  auto share = [&](int64_t k) { return (U * k) / We; };
  auto worker_of = [&](int64_t u) { return ((u + 1) * We - 1) / U; };
  const int64_t u_lo = share(wk), u_hi = share(wk + 1);

  // unit u -> (sequence s, segment y, block b): s is the last sequence whose
  // first unit is <= u (sequences without blocks own no unit)
  auto locate = [&](int64_t u, int& s, int& y, int& b) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (Y * sm_pref[mid] <= u) lo = mid;
      else hi = mid - 1;
    }
    s = lo;
    const int nbk = sm_pref[s + 1] - sm_pref[s];
    const int64_t r = u - Y * sm_pref[s];
    y = (int)(r / nbk);
    b = (int)(r - (int64_t)y * nbk);
  };

  // per-lane descriptors of 64 consecutive units (lane i: unit base + i)
  struct Info {
    int s, y, b, phys, ntok;
  };
  auto fetch = [&](int64_t base, Info& f) {
    const int64_t u = base + lane;
    f.s = 0;
    f.y = 0;
    f.b = 0;
    f.phys = -1;
    f.ntok = 0;
    if (u < u_hi) {
      locate(u, f.s, f.y, f.b);
      f.phys = p.bt[(int64_t)f.s * p.mb + f.b];
      f.ntok = min(16, sm_ctx[f.s] - 16 * f.b);
    }
  };
  Info cur, nxt;
  int64_t cur_base = u_lo;
  fetch(u_lo, cur);
  fetch(u_lo + 64, nxt);
  auto info = [&](int64_t u, int& s, int& y, int& b, int& phys, int& ntok) {
    const int64_t d = u - cur_base;
    const Info& f = d < 64 ? cur : nxt;
    const int i = (int)(d < 64 ? d : d - 64);
    s = __builtin_amdgcn_readlane(f.s, i);
    y = __builtin_amdgcn_readlane(f.y, i);
    b = __builtin_amdgcn_readlane(f.b, i);
    phys = __builtin_amdgcn_readlane(f.phys, i);
    ntok = __builtin_amdgcn_readlane(f.ntok, i);
  };

  const int64_t blk_stride = (int64_t)p.Hkv * T::TILE;
  auto issue = [&](Raw& r, int phys, int y) {
    const int64_t off = phys * blk_stride + (int64_t)(y / p.hchunks) * T::TILE;
    T::issue(r, p.kc + off, p.vc + off, c, G);
  };
  auto q_rows = [&](uint4* qr, int s, int y) {
    const int hc = y % p.hchunks;
    const int h_first = (y / p.hchunks) * p.g + hc * p.chunk_heads;
    const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
    T::load_q(qr, p.q, (int64_t)s * p.Hq + h_first + c, c < nh, G);
  };

  uint4 qr[KS], qn[KS];
  f32x4 o[DPL];
  float m_run = kNegInf, l_run = 0.f;
  auto reset = [&]() {
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
  };
  reset();

  // Close the piece [b0, b_last] of segment (s, y): store or merge.
  auto finish = [&](int s, int y, int b0, int b_last, bool first_piece) {
    const int nbk = sm_pref[s + 1] - sm_pref[s];
    const int hc = y % p.hchunks;
    const int h_first = (y / p.hchunks) * p.g + hc * p.chunk_heads;
    const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
    const int HS = p.chunk_heads;
    const float l_tot = wave_sum4(l_run);
    if (b0 == 0 && b_last == nbk - 1) {
      if (c < nh) {
        const float inv = l_tot > 0.f ? p.vsc / l_tot : 0.f;
        const int64_t row = ((int64_t)s * p.Hq + h_first + c) * D + DPL * 4 * G;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < DPL; ++e) store_out<QT>(p.out, row + DPL * i + e, o[e][i] * inv);
      }
      return;
    }
    const int64_t slot = 2 * (int64_t)wk + (first_piece ? 0 : 1);
    if (c < nh) {
      float* dst = p.part + (slot * HS + c) * D + DPL * 4 * G;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DPL; ++e) dst[DPL * i + e] = o[e][i] * p.vsc;
      if (G == 0) {
        p.ml[(slot * HS + c) * 2] = m_run;
        p.ml[(slot * HS + c) * 2 + 1] = l_tot;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int64_t seg_start = Y * sm_pref[s] + (int64_t)y * nbk;
    const int64_t wa = worker_of(seg_start), wb = worker_of(seg_start + nbk - 1);
    unsigned mine = 0;
    if (lane == 0) {
      unsigned long long* ctr = p.cnt + (int64_t)s * p.Y + y;
      unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while (true) {
        const unsigned have = (unsigned)(old >> 32) == p.epoch ? (unsigned)old : 0u;
        const unsigned long long nw = ((unsigned long long)p.epoch << 32) | (have + 1u);
        if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_ACQ_REL, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
          mine = have + 1u;
          break;
        }
      }
    }
    mine = __shfl(mine, 0);
    if ((int64_t)mine != wb - wa + 1) return;
    // last piece in: merge every piece of the segment
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const bool wa_first = share(wa) == seg_start;
    for (int h = 0; h < nh; ++h) {
      float M = kNegInf;
      for (int64_t k = wa; k <= wb; ++k) {
        const int64_t sl = 2 * k + ((k == wa && !wa_first) ? 1 : 0);
        if (p.ml[(sl * HS + h) * 2 + 1] > 0.f) M = fmaxf(M, p.ml[(sl * HS + h) * 2]);
      }
      constexpr int PER = (D + 63) / 64;
      float acc[PER];
#pragma unroll
      for (int k2 = 0; k2 < PER; ++k2) acc[k2] = 0.f;
      float L = 0.f;
      if (M != kNegInf) {
        for (int64_t k = wa; k <= wb; ++k) {
          const int64_t sl = 2 * k + ((k == wa && !wa_first) ? 1 : 0);
          const float lk = p.ml[(sl * HS + h) * 2 + 1];
          if (!(lk > 0.f)) continue;
          const float f = __builtin_amdgcn_exp2f(p.ml[(sl * HS + h) * 2] - M);
          L += f * lk;
          const float* src = p.part + (sl * HS + h) * D;
#pragma unroll
          for (int k2 = 0; k2 < PER; ++k2) {
            const int d = lane + 64 * k2;
            if (d < D) acc[k2] = fmaf(f, src[d], acc[k2]);
          }
        }
      }
      const int64_t row = (int64_t)s * p.Hq + h_first + h;
#pragma unroll
      for (int k2 = 0; k2 < PER; ++k2) {
        const int d = lane + 64 * k2;
        if (d < D) store_out<QT>(p.out, row * D + d, L > 0.f ? acc[k2] / L : 0.f);
      }
    }
  };

  // current unit's descriptor; its loads and q rows are requested before the loop
  int s_, y_, b_, ph_, nt_;
  info(u_lo, s_, y_, b_, ph_, nt_);
  bool v_ = (unsigned)ph_ < (unsigned)p.nb;   // bad table entry: no weight
  int64_t piece_u0 = u_lo;
  int piece_b0 = b_;
  q_rows(qn, s_, y_);

  Raw ra, rb;
  if (v_) issue(ra, ph_, y_);

  // one unit: prefetch the next, consume the current, close the piece if the
  // next unit belongs to another segment
  auto step = [&](Raw& rc, Raw& rn, int64_t u) {
    if (u == piece_u0) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qr[kk] = qn[kk];
    }
    const bool has_next = u + 1 < u_hi;
    int ns = 0, ny = 0, nbb = 0, nph = -1, nnt = 0;
    if (has_next) info(u + 1, ns, ny, nbb, nph, nnt);
    const bool nv = has_next && (unsigned)nph < (unsigned)p.nb;
    const bool new_seg = has_next && (ns != s_ || ny != y_);
    if (nv) issue(rn, nph, ny);
    if (new_seg) q_rows(qn, ns, ny);
    if (v_) T::consume(rc, nt_, qr, p.sl2, m_run, l_run, o, c, G);
    if (!has_next || new_seg) {
      finish(s_, y_, piece_b0, b_, piece_u0 == u_lo);
      reset();
      piece_u0 = u + 1;
      piece_b0 = nbb;
    }
    s_ = ns;
    y_ = ny;
    b_ = nbb;
    ph_ = nph;
    nt_ = nnt;
    v_ = nv;
    if (u + 1 - cur_base == 64) {   // the next unit opens the next descriptor batch
      cur = nxt;
      cur_base += 64;
      fetch(cur_base + 64, nxt);
    }
  };

  for (int64_t u = u_lo; u < u_hi; u += 2) {
    step(ra, rb, u);
    if (u + 1 >= u_hi) break;
    step(rb, ra, u + 1);
  }
}

template <int QT, int KVT, int D>
int launch_t(const pkv::DecodeArgs& a, const StreamParams& sp, int grid) {
  decode_stream_kernel<QT, KVT, D>
      <<<dim3(grid), dim3(64 * kSkWaves), 0, (hipStream_t)a.stream>>>(sp);
  return (int)hipGetLastError();
}

}  // namespace

namespace pkv {

int launch_decode_stream(const DecodeArgs& a, int grid, uint32_t epoch, void* ws,
                         size_t off_ml, size_t off_part) {
  const pkvd::DecodeParams kp = pkvd::make_params(a, 16);
  StreamParams sp;
  sp.out = a.out;
  sp.q = a.q;
  sp.kc = kp.kc;
  sp.vc = kp.vc;
  sp.bt = a.block_tables;
  sp.cl = a.context_lens;
  sp.S = a.num_seqs;
  sp.Hq = a.num_q_heads;
  sp.Hkv = a.num_kv_heads;
  sp.g = kp.g;
  sp.hchunks = kp.hchunks;
  sp.chunk_heads = kp.chunk_heads;
  sp.Y = a.num_kv_heads * kp.hchunks;
  sp.nb = a.num_blocks;
  sp.mb = a.max_blocks_per_seq;
  sp.sl2 = kp.sl2;
  sp.vsc = kp.vsc;
  sp.epoch = epoch;
  char* w = static_cast<char*>(ws);
  sp.cnt = reinterpret_cast<unsigned long long*>(w);
  sp.ml = reinterpret_cast<float*>(w + off_ml);
  sp.part = reinterpret_cast<float*>(w + off_part);
  const int q = a.q_dtype, kv = a.kv_dtype, D = a.head_dim;
#define PKV_STREAM_CASE(QT, KVT, DD) \
  if (q == QT && kv == KVT && D == DD) return launch_t<QT, KVT, DD>(a, sp, grid);
  PKV_STREAM_CASE(PKV_BF16, PKV_BF16, 128)
  PKV_STREAM_CASE(PKV_BF16, PKV_BF16, 64)
  PKV_STREAM_CASE(PKV_F16, PKV_F16, 128)
  PKV_STREAM_CASE(PKV_F16, PKV_F16, 64)
  PKV_STREAM_CASE(PKV_BF16, PKV_FP8_E4M3, 128)
  PKV_STREAM_CASE(PKV_BF16, PKV_FP8_E4M3, 64)
  PKV_STREAM_CASE(PKV_F16, PKV_FP8_E4M3, 128)
  PKV_STREAM_CASE(PKV_F16, PKV_FP8_E4M3, 64)
#undef PKV_STREAM_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace pkv
