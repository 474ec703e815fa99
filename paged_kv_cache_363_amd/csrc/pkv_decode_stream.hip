// Paged decode attention on the matrix cores with a work-balanced schedule.
//
// The contexts of a decode batch are ragged, so a grid of one workgroup per
// (sequence, kv-head, partition) leaves many workgroups empty or short and
// the last ones run on an almost idle GPU.  Here the step's work is
// flattened into units -- one 16-token block of one segment, a segment being
// the q-heads of one kv-head (at most 16 of them) of one sequence, segments
// in sequence order -- and a fixed grid of waves splits the units into equal
// contiguous shares.  Every wave walks its share one piece (the part of one
// segment inside the share) at a time with mfma_piece, which keeps the K/V
// loads of the next blocks in flight while it works on the current one.
//
// A share covers the tail of one segment, whole segments and the head of
// another.  A whole segment is normalised and stored by its wave.  A piece of
// a segment is stored as (m, l, acc) in the wave's partial slot (its first
// piece in slot 0, its last in slot 1).  The waves never signal each other:
// across the XCDs of an MI355X that would need the L2 written back and
// invalidated at every signal.  Instead decode_split_merge_kernel runs next
// on the stream and merges the pieces of every split segment with the
// log-sum-exp rule
//   M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k acc_k 2^(m_k - M) / L.
// Both kernels derive the shares from the same prefix sums of the block
// counts, so the workspace carries nothing but the partial slots.
//
// Fixed partitions (partition mode): when the caller fixes the split-K
// partition size, the same persistent grid computes one (m, l, acc) per
// partition of P blocks into the fixed-partition workspace, and the
// split-K reduction kernel merges them.  The shares' boundaries are moved up
// to the next partition boundary, so every partition belongs to one wave,
// and a wave closes each of its partitions when it has consumed the
// partition's last block, with the loads of the next blocks in flight: the
// load pipeline runs through a wave's whole share instead of restarting for
// every partition, as one workgroup per partition would.  A closed partition
// goes to a stash in LDS, not to memory: a store issued between two loads in
// flight holds up the wait for the older load until the store is
// acknowledged (vector loads and stores share one counter on CDNA), so the
// stash is written out only when it is full and at the end of the piece.
//
// Math: softmax(q K^T * scale) V over the block-table-gathered context
// ("KV Cache 与 PageAttention深度实战", sections 1.2 and 3.2).
#include <hip/hip_runtime.h>

#include "pkv_stream_common.h"
#include "pkv_launch.h"

#ifndef PKV_PIPE_DEPTH
#define PKV_PIPE_DEPTH 2       // K/V blocks in flight per wave, 16-bit caches
#endif
#ifndef PKV_PIPE_DEPTH_FP8
#define PKV_PIPE_DEPTH_FP8 2   // same for E4M3 caches
#endif
#ifndef PKV_NT_FP8
#define PKV_NT_FP8 1           // non-temporal K/V loads for one-byte codes
#endif
#ifndef PKV_NT_16
#define PKV_NT_16 1            // non-temporal K/V loads for 16-bit caches
#endif

namespace {

using namespace pkvd;

constexpr int kSkWaves = 4;   // waves per workgroup; each wave is its own worker
// partition mode: LDS stash of closed partitions, per wave
constexpr int kStashFloats = 8192;   // accumulators (32 KiB)
constexpr int kStashSlots = 16;      // at most this many partitions

struct StreamParams {
  void* out;
  const void* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  const int32_t* cl;
  int S, Hq, Hkv, g, Y, hchunks, chunk_heads, nb, mb;
  float sl2, vsc;
  float* part;                 // [2 W][chunk_heads][D]
  float* ml;                   // [2 W][chunk_heads][2]
  int W;                       // waves of the decode grid
  int R;                       // restart units counted at the start of every segment
  const float* ks;             // per-channel K scales [Hkv][D] (nullptr: per tensor)
  const float* vs;             // per-channel V scales [Hkv][D]
  // partition mode: P blocks per partition, the reduction's workspace
  // (m, l: [S][Hq][num_parts], acc: [S][Hq][num_parts][D])
  int P, num_parts;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
};

// Unit prefix sums in LDS, computed by one workgroup of 4 waves.  A segment
// of a sequence with nbk blocks spans nbk + R units: R units that stand for
// the cost of starting a piece (the q rows and block ids must arrive before
// the first K/V loads can go out) followed by one unit per block.  Equal
// shares of units are then equal in time, not just in blocks.
// pref[s] = units of one segment of each sequence before s (0 for a
// sequence without context).
__device__ __forceinline__ void block_prefix(const StreamParams& p, int* sm_pref, int* sm_ctx) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
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
      const int nbk = i < S ? (sm_ctx[i] + 15) >> 4 : 0;
      int x = nbk > 0 ? nbk + p.R : 0;
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
}

// PC: a one-byte-code cache with per-channel scales (p.ks, p.vs).
// PM: partition mode (p.P blocks per partition).
template <int QT, int KVT, int D, bool PC, bool PM>
__global__ __launch_bounds__(64 * kSkWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void decode_stream_kernel(StreamParams p) {
  using T = MfmaTile<QT, KVT, D>;
  constexpr int DPL = T::DPL;
  constexpr int KS = T::KSTEPS;

  __shared__ int sm_pref[pkv::kMaxStreamSeqs + 1];   // segment units before sequence s
  __shared__ int sm_ctx[pkv::kMaxStreamSeqs];        // clamped context lengths
  // partition mode: closed partitions of each wave, [slot][head][D] and
  // [slot][head][2] (m, l)
  __shared__ float sm_stash[PM ? kSkWaves * kStashFloats : 1];
  __shared__ float sm_stml[PM ? kSkWaves * kStashSlots * 16 * 2 : 1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, G = lane >> 4;
  const int S = p.S;
  block_prefix(p, sm_pref, sm_ctx);

  const int64_t Y = p.Y;
  const int64_t U = Y * sm_pref[S];
  const int W = p.W;
  const int wk = blockIdx.x * kSkWaves + w;

  // sequences without context get zero rows (in partition mode: an empty
  // first partition, which the reduction turns into zeros)
  for (int s = wk; s < S; s += W) {
    if (sm_ctx[s] != 0) continue;
    if constexpr (PM) {
      for (int h = lane; h < p.Hq; h += 64) {
        const int64_t prow = ((int64_t)s * p.Hq + h) * p.num_parts;
        p.ws_m[prow] = kNegInf;
        p.ws_l[prow] = 0.f;
      }
    } else {
      for (int i = lane; i < p.Hq * D; i += 64) store_out<QT>(p.out, (int64_t)s * p.Hq * D + i, 0.f);
    }
  }

  const int64_t We = U < W ? U : W;   // workers with a non-empty share
  if (wk >= We) return;
  const int64_t u_lo = floor_div53(U * wk, We), u_hi = floor_div53(U * (wk + 1), We);

  // unit u -> (sequence s, segment y, position j in the segment's units): s
  // is the last sequence whose first unit is <= u (sequences without blocks
  // own no unit).  The prefix sums are non-decreasing, so the lanes that pass
  // the test form a prefix of the wave: a 64-way search, two rounds of LDS
  // reads for up to 4096 sequences.
  auto locate = [&](int64_t u, int& s, int& y, int& j) {
    int lo = 0, span = S;   // Y * pref[lo] <= u
    while (span > 1) {
      const int step = (span + 63) >> 6;
      const int i = lo + lane * step;
      const bool ok = lane * step < span && Y * sm_pref[i] <= u;
      const int cnt = __popcll(__ballot(ok));
      lo += (cnt - 1) * step;
      span = min(step, span - (cnt - 1) * step);
    }
    s = lo;
    // U < 2^31 (checked by the host), so 32-bit division suffices
    const uint32_t len = (uint32_t)(sm_pref[s + 1] - sm_pref[s]);
    const uint32_t r = (uint32_t)(u - Y * sm_pref[s]);
    y = (int)(r / len);
    j = (int)(r - (uint32_t)y * len);
  };

  const int64_t blk_stride = (int64_t)p.Hkv * T::TILE;
  uint4 qr[KS];
  uint4 qlo[PC ? KS : 1];
  f32x4 o[DPL];
  float m_run = kNegInf, l_run = 0.f;
  auto reset = [&]() {
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
  };

  // Close the piece [b0, b_last] of segment (s, y): store or merge.
  auto finish = [&](int s, int y, int b0, int b_last, bool first_piece) {
    const int nbk = sm_pref[s + 1] - sm_pref[s] - p.R;
    const int hc = y % p.hchunks;
    const int h_first = (y / p.hchunks) * p.g + hc * p.chunk_heads;
    const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
    const int HS = p.chunk_heads;
    const float l_tot = wave_sum4(l_run);
    if (b0 == 0 && b_last == nbk - 1) {
      if (c < nh) {
        const int64_t row = ((int64_t)s * p.Hq + h_first + c) * D + DPL * 4 * G;
        // lane (G, c) holds dims DPL*(4G+i) + e, e < DPL: DPL consecutive
        // outputs per i, written with one store each
        if constexpr (PC) {
          const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
          const float* vs = p.vs + (int64_t)(y / p.hchunks) * D + DPL * 4 * G;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) v[e] = o[e][i] * vs[DPL * i + e] * inv;
            store_out_n<QT, DPL>(p.out, row + DPL * i, v);
          }
        } else {
          const float inv = l_tot > 0.f ? p.vsc / l_tot : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) v[e] = o[e][i] * inv;
            store_out_n<QT, DPL>(p.out, row + DPL * i, v);
          }
        }
      }
      return;
    }
    const int64_t slot = 2 * (int64_t)wk + (first_piece ? 0 : 1);
    if (c < nh) {
      float* dst = p.part + (slot * HS + c) * D + DPL * 4 * G;
      const float* vs = PC ? p.vs + (int64_t)(y / p.hchunks) * D + DPL * 4 * G : nullptr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DPL; e += 4)
          *reinterpret_cast<float4*>(dst + DPL * i + e) =
              make_float4(o[e][i] * (PC ? vs[DPL * i + e] : p.vsc),
                          o[e + 1][i] * (PC ? vs[DPL * i + e + 1] : p.vsc),
                          o[e + 2][i] * (PC ? vs[DPL * i + e + 2] : p.vsc),
                          o[e + 3][i] * (PC ? vs[DPL * i + e + 3] : p.vsc));
      if (G == 0) {
        p.ml[(slot * HS + c) * 2] = m_run;
        p.ml[(slot * HS + c) * 2 + 1] = l_tot;
      }
    }
  };

  // Walk the share piece by piece: a piece is the part of one segment's
  // blocks that lies in [u_lo, u_hi).  Segments follow each other in
  // (sequence, y) order; sequences without blocks own no segment.  A piece
  // made of restart units only has no block and is skipped.
  int64_t u = u_lo;
  int s, y, j;
  locate(u, s, y, j);
  bool first_piece = true;
  while (true) {
    const int len = sm_pref[s + 1] - sm_pref[s];
    const int64_t seg_start = Y * sm_pref[s] + (int64_t)y * len;
    const int64_t pe = seg_start + len < u_hi ? seg_start + len : u_hi;
    int b = max(j - p.R, 0);
    int b1 = max((int)(pe - seg_start) - p.R, 0);
    if constexpr (PM) {
      // both ends up to the next partition boundary (or the segment's end);
      // the neighbouring share moves the same boundary the same way
      const int nbk = len - p.R;
      b = min((b + p.P - 1) / p.P * p.P, nbk);
      b1 = min((b1 + p.P - 1) / p.P * p.P, nbk);
    }
    if (b1 > b) {
      const int hc = y % p.hchunks;
      const int hk = y / p.hchunks;
      const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
      if constexpr (PC)
        T::load_q_scaled(qr, qlo, p.q, (int64_t)s * p.Hq + hk * p.g + hc * p.chunk_heads + c,
                         c < nh, G, p.ks + (int64_t)hk * D);
      else
        T::load_q(qr, p.q, (int64_t)s * p.Hq + hk * p.g + hc * p.chunk_heads + c, c < nh, G);
      reset();
      const int ctx = sm_ctx[s];
      const int last = ((ctx + 15) >> 4) - 1;
      constexpr int DEPTH = pkv::byte_codes(KVT) ? PKV_PIPE_DEPTH_FP8 : PKV_PIPE_DEPTH;
      constexpr bool NT = pkv::byte_codes(KVT) ? PKV_NT_FP8 : PKV_NT_16;
      const int64_t off = (int64_t)hk * T::TILE;
      if constexpr (PM) {
        // Close partition kp0 + n_st into stash slot n_st and start the next
        // partition; write the stash out when it is full and at the end.
        // Lane (G, c) stashes and later stores its own 4 * DPL accumulators,
        // so no other lane reads what it wrote.
        const int h_first = hk * p.g + hc * p.chunk_heads;
        const int HS = p.chunk_heads;
        const int slots = min(kStashSlots, kStashFloats / (HS * D));
        float* st = sm_stash + w * kStashFloats + c * D + DPL * 4 * G;
        float* stml = sm_stml + w * kStashSlots * 32 + 2 * c;
        int kp0 = b / p.P, n_st = 0;
        auto write_out = [&]() {
          if (c < nh) {
            const int64_t row = (int64_t)s * p.Hq + h_first + c;
            for (int k = 0; k < n_st; ++k) {
              const int64_t prow = row * p.num_parts + kp0 + k;
              const float* src = st + k * HS * D;
              float* dst = p.ws_acc + prow * D + DPL * 4 * G;
#pragma unroll
              for (int i = 0; i < 4 * DPL; ++i) dst[i] = src[i];
              if (G == 0) {
                p.ws_m[prow] = stml[k * 32];
                p.ws_l[prow] = stml[k * 32 + 1];
              }
            }
          }
          kp0 += n_st;
          n_st = 0;
        };
        auto close = [&]() {
          const float l_tot = wave_sum4(l_run);
          if (c < nh) {
            float* dst = st + n_st * HS * D;
            const float* vs = PC ? p.vs + (int64_t)hk * D + DPL * 4 * G : nullptr;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int e = 0; e < DPL; ++e)
                dst[DPL * i + e] = o[e][i] * (PC ? vs[DPL * i + e] : p.vsc);
            if (G == 0) {
              stml[n_st * 32] = m_run;
              stml[n_st * 32 + 1] = l_tot;
            }
          }
          if (++n_st == slots) write_out();
          reset();
        };
        const PeriodHook<decltype(close)> hook{p.P, close};
        if (p.nb > 0)
          mfma_piece<QT, KVT, D, DEPTH, NT, false, PC, 1, PeriodHook<decltype(close)>>(
              p.kc + off, p.vc + off, blk_stride, p.bt + (int64_t)s * p.mb, b, b1, last,
              ctx - 16 * last, p.nb, qr, p.sl2, &m_run, &l_run, o, lane, nullptr, qlo, hook);
        else   // no block can be valid: every partition is empty
          for (int k = b / p.P; k < (b1 + p.P - 1) / p.P; ++k) close();
        write_out();
      } else {
        if (p.nb > 0)
          mfma_piece<QT, KVT, D, DEPTH, NT, false, PC>(
              p.kc + off, p.vc + off, blk_stride, p.bt + (int64_t)s * p.mb, b, b1, last,
              ctx - 16 * last, p.nb, qr, p.sl2, &m_run, &l_run, o, lane, nullptr, qlo);
        finish(s, y, b, b1 - 1, first_piece);
      }
      first_piece = false;
    }
    u = pe;
    if (u >= u_hi) break;
    j = 0;
    if (++y == p.Y) {
      y = 0;
      do {
        ++s;
      } while (sm_pref[s + 1] == sm_pref[s]);
    }
  }
}

// Merge the pieces of every segment that the decode grid split between
// waves.  One wave per (segment, q-head of the segment); segments kept whole
// by one wave were already stored by it.  The shares are recomputed exactly
// as the decode kernel computed them: worker k owns units
// [U k / We, U (k+1) / We).
template <int QT, int D>
__global__ __launch_bounds__(64 * kSkWaves) void decode_split_merge_kernel(StreamParams p) {
  __shared__ int sm_pref[pkv::kMaxStreamSeqs + 1];
  __shared__ int sm_ctx[pkv::kMaxStreamSeqs];
  block_prefix(p, sm_pref, sm_ctx);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int64_t Y = p.Y;
  const int64_t U = Y * sm_pref[p.S];
  const int64_t We = U < p.W ? U : p.W;
  if (We == 0) return;
  const int HS = p.chunk_heads;
  const int64_t nitems = (int64_t)p.S * Y * HS;
  for (int64_t it = (int64_t)blockIdx.x * kSkWaves + w; it < nitems;
       it += (int64_t)gridDim.x * kSkWaves) {
    const int h = (int)(it % HS);
    const int64_t seg = it / HS;
    const int s = (int)(seg / Y), y = (int)(seg % Y);
    const int hc = y % p.hchunks;
    const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
    if (h >= nh) continue;
    const int len = sm_pref[s + 1] - sm_pref[s];
    if (len == 0) continue;
    // the segment's blocks are its units [seg_start + R, seg_start + len)
    const int64_t seg_start = Y * sm_pref[s] + (int64_t)y * len;
    const int64_t wa = floor_div53((seg_start + p.R + 1) * We - 1, U);
    const int64_t wb = floor_div53((seg_start + len) * We - 1, U);
    if (wa == wb) continue;
    // the first worker's piece is its first piece with blocks unless its
    // share holds blocks of the segment before (units below seg_start)
    const int64_t sl0 = 2 * wa + (floor_div53(U * wa, We) >= seg_start ? 0 : 1);
    const int h_first = (y / p.hchunks) * p.g + hc * p.chunk_heads;
    const int64_t row = (int64_t)s * p.Hq + h_first + h;
    merge_split_column<QT, D>(p.part, p.ml, HS, h, wa, wb, sl0, p.out, row * D);
  }
}

template <int QT, int KVT, int D, bool PM>
int launch_pm(const pkv::DecodeArgs& a, const StreamParams& sp, int grid) {
  const dim3 block(64 * kSkWaves);
  if constexpr (pkv::byte_codes(KVT)) {
    if (sp.ks)
      return pkv::launch_kernel(decode_stream_kernel<QT, KVT, D, true, PM>, dim3(grid), block,
                                a.stream, sp, a.ev_start, a.ev_stop);
  }
  return pkv::launch_kernel(decode_stream_kernel<QT, KVT, D, false, PM>, dim3(grid), block,
                            a.stream, sp, a.ev_start, a.ev_stop);
}

template <int QT, int KVT, int D>
int launch_t(const pkv::DecodeArgs& a, const StreamParams& sp, int grid) {
  if (sp.P > 0) return launch_pm<QT, KVT, D, true>(a, sp, grid);
  return launch_pm<QT, KVT, D, false>(a, sp, grid);
}

template <int QT, int D>
int launch_merge_t(const pkv::DecodeArgs& a, const StreamParams& sp) {
  const int64_t nitems = (int64_t)sp.S * sp.Y * sp.chunk_heads;
  int64_t grid = (nitems + kSkWaves - 1) / kSkWaves;
  if (grid > 4096) grid = 4096;
  return pkv::launch_kernel(decode_split_merge_kernel<QT, D>, dim3((unsigned)grid),
                            dim3(64 * kSkWaves), a.stream, sp, a.ev_start, a.ev_stop);
}

StreamParams make_stream_params(const pkv::DecodeArgs& a, int grid, void* ws, size_t off_ml,
                                size_t off_part) {
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
  char* w = static_cast<char*>(ws);
  sp.ml = reinterpret_cast<float*>(w + off_ml);
  sp.part = reinterpret_cast<float*>(w + off_part);
  sp.W = grid * kSkWaves;
  sp.R = pkv::kv_restart_units(a.kv_dtype);
  sp.ks = kp.ks;
  sp.vs = kp.vs;
  sp.P = 0;
  sp.num_parts = 0;
  sp.ws_m = sp.ws_l = sp.ws_acc = nullptr;
  return sp;
}

}  // namespace

namespace pkv {

int launch_decode_stream(const DecodeArgs& a, int grid, void* ws, size_t off_ml,
                         size_t off_part) {
  const StreamParams sp = make_stream_params(a, grid, ws, off_ml, off_part);
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
  PKV_STREAM_CASE(PKV_BF16, PKV_INT8, 128)
  PKV_STREAM_CASE(PKV_BF16, PKV_INT8, 64)
  PKV_STREAM_CASE(PKV_F16, PKV_INT8, 128)
  PKV_STREAM_CASE(PKV_F16, PKV_INT8, 64)
#undef PKV_STREAM_CASE
  return (int)hipErrorInvalidValue;
}

int launch_decode_stream_parts(const DecodeArgs& a, int grid) {
  StreamParams sp = make_stream_params(a, grid, nullptr, 0, 0);
  sp.ml = sp.part = nullptr;
  sp.P = a.partition / kBlockSize;
  sp.num_parts = a.num_parts;
  sp.ws_m = a.ws_m;
  sp.ws_l = a.ws_l;
  sp.ws_acc = a.ws_acc;
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
  PKV_STREAM_CASE(PKV_BF16, PKV_INT8, 128)
  PKV_STREAM_CASE(PKV_BF16, PKV_INT8, 64)
  PKV_STREAM_CASE(PKV_F16, PKV_INT8, 128)
  PKV_STREAM_CASE(PKV_F16, PKV_INT8, 64)
#undef PKV_STREAM_CASE
  return (int)hipErrorInvalidValue;
}

int launch_decode_split_merge(const DecodeArgs& a, int grid, void* ws, size_t off_ml,
                              size_t off_part) {
  const StreamParams sp = make_stream_params(a, grid, ws, off_ml, off_part);
  const int q = a.q_dtype, D = a.head_dim;
  if (q == PKV_BF16 && D == 128) return launch_merge_t<PKV_BF16, 128>(a, sp);
  if (q == PKV_BF16 && D == 64) return launch_merge_t<PKV_BF16, 64>(a, sp);
  if (q == PKV_F16 && D == 128) return launch_merge_t<PKV_F16, 128>(a, sp);
  if (q == PKV_F16 && D == 64) return launch_merge_t<PKV_F16, 64>(a, sp);
  return (int)hipErrorInvalidValue;
}

}  // namespace pkv
