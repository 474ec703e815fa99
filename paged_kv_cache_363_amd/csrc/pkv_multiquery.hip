// Paged multi-query attention on the CDNA4 matrix cores: several query rows
// per sequence in one pass, each attending causally through the block table.
// A sequence's rows are the last positions of its context (a chunk of a long
// prompt, "vLLM推理引擎深度解析" section 3.3 and "推理加速三板斧" section 4.5;
// or the draft tokens a target model verifies in one pass,
// "大语言模型推理引擎深度剖析" section 4.1).  Row i of a sequence with n rows
// and ctx tokens sits at position ctx - n + i and attends to positions
// 0 .. ctx - n + i; the chunk's own K/V are appended before the call.
//
// The MFMA tile of the decode kernels has 16 columns.  Here a column is a
// (query row, q-head) pair of one kv-head: chunk = min(g, 16) q-heads times
// qpt = 16 / chunk rows (4 rows x 4 heads at g = 4, 16 rows x 1 head for
// MHA).  A wave carries ntl <= 4 such column tiles (a row tile of ntl x qpt
// rows), so one K/V load, widened once, serves up to 64 (row, q-head)
// columns.  Each lane masks its column's logits at that row's position.
//
// One workgroup per (partition, sequence, kv-head, head chunk, row tile),
// ordered so that a group's row tiles share an XCD (see the kernel).  A workgroup
// walks the blocks its last row can see; its four waves take contiguous
// quarters of them and merge in LDS.  With several partitions each workgroup
// writes (m, l, acc) partials, an empty partition writing m = -inf, l = 0, and
// multiquery_reduce_kernel merges every row's partitions by log-sum-exp.
//
// With partition_size 0 the work-balanced schedule runs instead
// (multiquery_stream_kernel, then multiquery_split_merge_kernel): ragged
// contexts leave no CU idle at the end of the call.
#include <hip/hip_runtime.h>

#include "pkv_stream_common.h"
#include "pkv_launch.h"

#ifndef PKV_PIPE_DEPTH
#define PKV_PIPE_DEPTH 2       // K/V blocks in flight per wave, 16-bit caches
#endif
#ifndef PKV_PIPE_DEPTH_FP8
#define PKV_PIPE_DEPTH_FP8 2   // same for E4M3 caches
#endif

namespace {

using namespace pkvd;

constexpr int kCols = 16;   // MFMA tile columns
constexpr int kSeesAll = 1 << 30;   // causal position of a column that is not stored

struct MQParams {
  void* out;
  const void* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  const int32_t* cl;
  const int32_t* qs;
  int S, rows, max_q;
  int Hq, Hkv, g, nb, mb;
  int chunk;         // q-heads per column group
  int hchunks;       // column groups per kv-head
  int qpt;           // query rows per column tile (16 / chunk)
  int ntl;           // column tiles per wave (its template argument)
  int rpt;           // rows per row tile: qpt * ntl
  int qtiles;        // row tiles per (sequence, kv-head, head chunk) in the grid
  int part_blocks;   // 16-token blocks per partition
  int num_parts;     // partitions in the grid (1 = single pass)
  float sl2;         // scale * log2(e) * k_scale
  float vsc;         // v_scale (1 unless FP8)
  float* ws_m;       // [rows][Hq][P]
  float* ws_l;       // [rows][Hq][P]
  float* ws_acc;     // [rows][Hq][P][D]
  int nx;            // XCDs of the device (workgroup placement, see below)
  int64_t groups;    // (partition, sequence, kv-head, head chunk) groups
};

// Rows [r0, r0 + n) of sequence s, clamped so that every row index lies in
// [0, rows) and n <= max_q.
__device__ __forceinline__ void seq_rows(const MQParams& p, int s, int& r0, int& n) {
  int a = p.qs[s], b = p.qs[s + 1];
  a = a < 0 ? 0 : (a > p.rows ? p.rows : a);
  b = b < a ? a : (b > p.rows ? p.rows : b);
  r0 = a;
  n = min(b - a, p.max_q);
}

// NTL column tiles per wave: the rows of a row tile share every K/V load.
template <int QT, int KVT, int D, int NTL>
__global__ __launch_bounds__(64 * pkv::kWaves)
__attribute__((amdgpu_waves_per_eu(NTL > 1 ? 1 : 2, 8)))
void multiquery_mfma_kernel(MQParams p) {
  using T = MfmaTile<QT, KVT, D>;
  constexpr int LD = D + 4;
  constexpr int DPL = T::DPL;
  constexpr int KS = T::KSTEPS;

  __shared__ float sm_m[pkv::kWaves * kCols];
  __shared__ float sm_l[pkv::kWaves * kCols];
  __shared__ float sm_o[pkv::kWaves * kCols * LD];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, G = lane >> 4;
  // The row tiles of one (partition, sequence, kv-head, head chunk) group
  // read the same K/V.  Workgroups are dealt to the XCDs round robin by
  // index, each XCD with its own L2, so the grid is ordered to put all row
  // tiles of a group on one XCD: runs of nx * qtiles workgroups hold nx
  // groups, group x of a run taking the indices congruent to x mod nx.
  // (Any order computes the same result; this one lets one XCD's L2 serve
  // a group's repeated reads.)
  // (The integer divisions below expand to vector code; their uniform
  // results are moved to scalar registers, so that the block loop's
  // addresses are scalar arithmetic.)
  const int64_t run = (int64_t)p.nx * p.qtiles;
  const int64_t g0 = blockIdx.x / run;
  const int rr = (int)(blockIdx.x - g0 * run);
  const int qt = __builtin_amdgcn_readfirstlane(rr / p.nx);
  const int64_t grp = g0 * p.nx + rr % p.nx;
  if (grp >= p.groups) return;
  const int part = __builtin_amdgcn_readfirstlane((int)(grp % p.num_parts));
  int64_t yy64 = grp / p.num_parts;
  const int Yg = p.Hkv * p.hchunks;
  const int s = __builtin_amdgcn_readfirstlane((int)(yy64 / Yg));
  const int yy = (int)(yy64 % Yg);
  const int hc = __builtin_amdgcn_readfirstlane(yy % p.hchunks);
  const int hk = __builtin_amdgcn_readfirstlane(yy / p.hchunks);
  int r0, n;
  seq_rows(p, s, r0, n);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  n = __builtin_amdgcn_readfirstlane(n);
  const int i0 = qt * p.rpt;
  if (i0 >= n) return;   // no row of this sequence in the tile
  const int cap = p.mb * pkv::kBlockSize;
  const int ctx = __builtin_amdgcn_readfirstlane(min(max(p.cl[s], 0), cap));

  // this lane's column in column tile j: row i0 + j qpt + c / chunk, q-head
  // hk*g + hc*chunk + c % chunk
  const int h = hc * p.chunk + c % p.chunk;
  auto row_of = [&](int j) { return i0 + j * p.qpt + c / p.chunk; };
  auto live_of = [&](int j) { return c < p.qpt * p.chunk && row_of(j) < n && h < p.g; };
  int pos[NTL];
  uint4 qr[NTL * KS];
#pragma unroll
  for (int j = 0; j < NTL; ++j) {
    // < 0: the column attends to nothing.  A column that is not stored
    // (q zero) is taken to see every token, so that it never asks for the
    // per-token causal limits.
    pos[j] = live_of(j) ? ctx - n + row_of(j) : kSeesAll;
    T::load_q(qr + j * KS, p.q, (int64_t)(r0 + row_of(j)) * p.Hq + hk * p.g + h, live_of(j), G);
  }
  // blocks any row of the tile can see: up to its last row's position
  const int p_last = ctx - n + min(i0 + p.rpt, n) - 1;
  const int nblk = p_last >= 0 ? (p_last >> 4) + 1 : 0;
  const int b_begin = part * p.part_blocks;
  const int b_end = min(b_begin + p.part_blocks, nblk);
  const int nblk_p = max(b_end - b_begin, 0);

  f32x4 o[NTL * DPL];
#pragma unroll
  for (int e = 0; e < NTL * DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  // l of column tile j: every element of l_acc[j] holds the column's sum
  float m_run[NTL];
  f32x4 l_acc[NTL];
#pragma unroll
  for (int j = 0; j < NTL; ++j) {
    m_run[j] = kNegInf;
    l_acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int w0 = b_begin + (nblk_p * w) / pkv::kWaves;
  const int w1 = b_begin + (nblk_p * (w + 1)) / pkv::kWaves;
  if (p.nb > 0 && w1 > w0) {
    const int64_t blk_stride = (int64_t)p.Hkv * T::TILE;
    const int64_t head_off = (int64_t)hk * T::TILE;
    const int last = ((ctx + 15) >> 4) - 1;
    mfma_piece<QT, KVT, D, pkv::byte_codes(KVT) ? PKV_PIPE_DEPTH_FP8 : PKV_PIPE_DEPTH, false,
               true, false, NTL>(p.kc + head_off, p.vc + head_off, blk_stride,
                                 p.bt + (int64_t)s * p.mb, w0, w1, last, ctx - 16 * last, p.nb,
                                 qr, p.sl2, m_run, reinterpret_cast<float*>(l_acc), o, lane,
                                 pos);
  }

  // One column tile at a time through LDS: lane (G, c) holds O[column c][dim
  // DPL*(4G+i) + e]; l needs the 4 G lanes.  The merge gives each thread one
  // column and DPT consecutive dims: the column's factors and 1 / L are taken
  // once, and its outputs leave in one store.
  constexpr int DPT = D / 16;
  static_assert(kCols * 16 == 64 * pkv::kWaves, "one thread per (column, run of dims)");
  const int mc = threadIdx.x >> 4, md0 = (threadIdx.x & 15) * DPT;
#pragma unroll
  for (int j = 0; j < NTL; ++j) {
    const float lj = l_acc[j][0];
    if (j > 0) __syncthreads();   // the previous tile's reads are done
    if (G == 0) {
      sm_m[w * kCols + c] = m_run[j];
      sm_l[w * kCols + c] = lj;
    }
    {
      float* dst = sm_o + (w * kCols + c) * LD + DPL * 4 * G;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DPL; ++e) dst[DPL * i + e] = o[j * DPL + e][i];
    }
    __syncthreads();

    const int ic = i0 + j * p.qpt + mc / p.chunk, hh = hc * p.chunk + mc % p.chunk;
    if (mc < p.qpt * p.chunk && ic < n && hh < p.g) {
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < pkv::kWaves; ++v) M = fmaxf(M, sm_m[v * kCols + mc]);
      float L = 0.f, acc[DPT];
#pragma unroll
      for (int k = 0; k < DPT; ++k) acc[k] = 0.f;
#pragma unroll
      for (int v = 0; v < pkv::kWaves; ++v) {
        const float mv = sm_m[v * kCols + mc];
        const float f = (mv == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        L += f * sm_l[v * kCols + mc];
        const float4* src = reinterpret_cast<const float4*>(sm_o + (v * kCols + mc) * LD + md0);
#pragma unroll
        for (int k4 = 0; k4 < DPT / 4; ++k4) {
          const float4 x = src[k4];
          acc[4 * k4] += f * x.x;
          acc[4 * k4 + 1] += f * x.y;
          acc[4 * k4 + 2] += f * x.z;
          acc[4 * k4 + 3] += f * x.w;
        }
      }
      const int64_t row = (int64_t)(r0 + ic) * p.Hq + hk * p.g + hh;
      if (p.num_parts == 1) {
        const float inv = L > 0.f ? p.vsc / L : 0.f;
#pragma unroll
        for (int k = 0; k < DPT; ++k) acc[k] *= inv;
        store_out_n<QT, DPT>(p.out, row * D + md0, acc);
      } else {
        const int64_t pr = row * p.num_parts + part;
        float4* dst = reinterpret_cast<float4*>(p.ws_acc + pr * D + md0);
#pragma unroll
        for (int k4 = 0; k4 < DPT / 4; ++k4)
          dst[k4] = make_float4(acc[4 * k4] * p.vsc, acc[4 * k4 + 1] * p.vsc,
                                acc[4 * k4 + 2] * p.vsc, acc[4 * k4 + 3] * p.vsc);
        if (md0 == 0) {
          p.ws_m[pr] = M;
          p.ws_l[pr] = L;
        }
      }
    }
  }
}


template <int QT, int D>
__global__ __launch_bounds__(64) void multiquery_reduce_kernel(MQParams p) {
  const int64_t rh = blockIdx.x;   // row * Hq + head
  const int r = (int)(rh / p.Hq);
  int first = p.qs[0], end = p.qs[p.S];
  first = first < 0 ? 0 : (first > p.rows ? p.rows : first);
  end = end < first ? first : (end > p.rows ? p.rows : end);
  if (r < first || r >= end) return;
  const int np = p.num_parts;
  const float* m = p.ws_m + rh * np;
  const float* l = p.ws_l + rh * np;
  const float* a = p.ws_acc + rh * np * D;
  const int lane = threadIdx.x;
  float M = kNegInf;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, l[i] > 0.f ? m[i] : kNegInf);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  constexpr int PER = (D + 63) / 64;
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
    for (int base = 0; base < np; base += 64) {
      const int i = base + lane;
      float wgt = 0.f;
      if (i < np) {
        const float li = l[i];
        wgt = li > 0.f ? __builtin_amdgcn_exp2f(m[i] - M) : 0.f;
        L += wgt * li;
      }
      const int cnt = min(64, np - base);
      const float* ab = a + (int64_t)base * D;
      // 8 partitions per round, their loads issued together (rows past cnt
      // are not read and carry no weight)
      for (int j0 = 0; j0 < cnt; j0 += 8) {
        float x[8][PER];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int d = lane + 64 * k;
            x[u][k] = (j0 + u < cnt && d < D) ? ab[(int64_t)(j0 + u) * D + d] : 0.f;
          }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wj = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(wgt), min(j0 + u, 63)));
          const float wu = (j0 + u < cnt) ? wj : 0.f;
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[k] = fmaf(wu, x[u][k], acc[k]);
        }
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    if (d < D) store_out<QT>(p.out, rh * D + d, L > 0.f ? acc[k] / L : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Work-balanced schedule.  As in the balanced decode kernel, the call's work
// is flattened into units and a persistent grid of waves takes equal
// contiguous shares of them.  A tile is one row tile (rpt = ntl x qpt rows,
// ntl column tiles of 16 columns) of one sequence; it has Y = kv-heads x head
// chunks segments, each of nbk + R units: R restart units (the cost of
// starting a piece) and one unit per 16-token block its last row can see.  Tiles follow each other in
// (sequence, row tile) order; the prefix sums of their units sit in LDS, and
// both kernels derive every share from them.

struct MQStreamParams {
  MQParams b;
  int Y;         // segments per tile: kv-heads x head chunks
  int W;         // waves of the grid
  int R;         // restart units at the start of every segment
  float* ml;     // [2 W][16 ntl][2]
  float* part;   // [2 W][16 ntl][D]
};

struct MQStreamSmem {
  int pref[pkv::kMaxStreamTiles + 1];      // units of one segment of each tile before tile t
  int tb[pkv::kMaxStreamSeqs + 1];         // first tile of sequence s
  int ctx[pkv::kMaxStreamSeqs];            // clamped context lengths
  int r0[pkv::kMaxStreamSeqs];             // first row of sequence s
  int n[pkv::kMaxStreamSeqs];              // rows of sequence s (clamped, <= max_q)
  uint16_t tseq[pkv::kMaxStreamTiles];     // sequence of tile t
};

// 16-token blocks the last row of row tile qt of a sequence (ctx tokens, n
// rows) can see; 0 when every row of the tile sits before position 0.
__device__ __forceinline__ int mq_tile_blocks(const MQParams& p, int ctx, int n, int qt) {
  const int p_last = ctx - n + min(qt * p.rpt + p.rpt, n) - 1;
  return p_last >= 0 ? (p_last >> 4) + 1 : 0;
}

// Inclusive scan of x over the lanes of one wave.
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Sequence data, tile bases and the unit prefix sums in LDS, computed by the
// whole workgroup.  The host bounds the sequences by kMaxStreamSeqs and the
// tiles (sequences x row tiles of max_query_len rows) by kMaxStreamTiles.
__device__ void mq_tile_prefix(const MQStreamParams& sp, MQStreamSmem& sm) {
  const MQParams& p = sp.b;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.S;
  const int cap = p.mb * pkv::kBlockSize;
  for (int i = threadIdx.x; i < S; i += 64 * pkv::kWaves) {
    const int c = p.cl[i];
    sm.ctx[i] = c < 0 ? 0 : (c > cap ? cap : c);
    int r0, n;
    seq_rows(p, i, r0, n);
    sm.r0[i] = r0;
    sm.n[i] = n;
  }
  __syncthreads();
  if (w == 0) {
    int carry = 0;
    for (int base = 0; base < S; base += 64) {
      const int i = base + lane;
      const int x = wave_scan(i < S ? (sm.n[i] + p.rpt - 1) / p.rpt : 0, lane);
      if (i < S) sm.tb[i + 1] = carry + x;
      carry += __shfl(x, 63);
    }
    if (lane == 0) sm.tb[0] = 0;
  }
  __syncthreads();
  // each tile's units, stored one place up for the in-place scan below
  if (p.qtiles > 16) {
    // long prompt chunks: a wave per sequence, its lanes over the row tiles
    for (int i = w; i < S; i += pkv::kWaves) {
      const int t0 = sm.tb[i], nt = sm.tb[i + 1] - t0;
      for (int qt = lane; qt < nt; qt += 64) {
        const int nbk = mq_tile_blocks(p, sm.ctx[i], sm.n[i], qt);
        sm.tseq[t0 + qt] = (uint16_t)i;
        sm.pref[t0 + qt + 1] = nbk > 0 ? nbk + sp.R : 0;
      }
    }
  } else {
    for (int i = threadIdx.x; i < S; i += 64 * pkv::kWaves) {
      const int t0 = sm.tb[i], nt = sm.tb[i + 1] - t0;
      for (int qt = 0; qt < nt; ++qt) {
        const int nbk = mq_tile_blocks(p, sm.ctx[i], sm.n[i], qt);
        sm.tseq[t0 + qt] = (uint16_t)i;
        sm.pref[t0 + qt + 1] = nbk > 0 ? nbk + sp.R : 0;
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    const int T = sm.tb[S];
    int carry = 0;
    for (int base = 0; base < T; base += 64) {
      const int t = base + lane;
      const int x = wave_scan(t < T ? sm.pref[t + 1] : 0, lane);
      if (t < T) sm.pref[t + 1] = carry + x;
      carry += __shfl(x, 63);
    }
    if (lane == 0) sm.pref[0] = 0;
  }
  __syncthreads();
}

// One wave per worker.  A share covers the tail of one segment, whole
// segments and the head of another; a whole segment is normalised and stored
// by its wave, a piece of a split segment goes to the wave's partial slot
// (its first piece in slot 2 wk, its last in slot 2 wk + 1).  NTL column
// tiles per wave, as in the fixed kernel.
template <int QT, int KVT, int D, int NTL>
__global__ __launch_bounds__(64 * pkv::kWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void multiquery_stream_kernel(MQStreamParams sp) {
  using T = MfmaTile<QT, KVT, D>;
  constexpr int DPL = T::DPL;
  constexpr int KS = T::KSTEPS;
  constexpr int NC = kCols * NTL;   // columns of a row tile
  __shared__ MQStreamSmem sm;
  const MQParams& p = sp.b;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, G = lane >> 4;
  mq_tile_prefix(sp, sm);
  const int Tn = sm.tb[p.S];
  const int64_t Y = sp.Y;
  const int64_t U = Y * sm.pref[Tn];
  const int W = sp.W;
  const int wk = blockIdx.x * pkv::kWaves + w;

  // the rows of a tile that sees no block attend to nothing: zeros
  for (int t = wk; t < Tn; t += W) {
    if (sm.pref[t + 1] != sm.pref[t]) continue;
    const int s = sm.tseq[t];
    const int i0 = (t - sm.tb[s]) * p.rpt, i1 = min(i0 + p.rpt, sm.n[s]);
    const int64_t base = (int64_t)(sm.r0[s] + i0) * p.Hq * D;
    const int64_t cnt = (int64_t)(i1 - i0) * p.Hq * D;
    for (int64_t i = lane; i < cnt; i += 64) store_out<QT>(p.out, base + i, 0.f);
  }

  const int64_t We = U < W ? U : W;   // workers with a non-empty share
  if (wk >= We) return;
  const int64_t u_lo = floor_div53(U * wk, We), u_hi = floor_div53(U * (wk + 1), We);

  // unit u -> (tile t, segment y, position j in the segment's units): t is
  // the last tile whose first unit is <= u (tiles without blocks own no
  // unit); a 64-way search over the non-decreasing prefix sums.
  auto locate = [&](int64_t u, int& t, int& y, int& j) {
    int lo = 0, span = Tn;   // Y * pref[lo] <= u
    while (span > 1) {
      const int step = (span + 63) >> 6;
      const int i = lo + lane * step;
      const bool ok = lane * step < span && Y * sm.pref[i] <= u;
      const int cnt = __popcll(__ballot(ok));
      lo += (cnt - 1) * step;
      span = min(step, span - (cnt - 1) * step);
    }
    t = lo;
    // U < 2^31 (checked by the host), so 32-bit division suffices
    const uint32_t len = (uint32_t)(sm.pref[t + 1] - sm.pref[t]);
    const uint32_t r = (uint32_t)(u - Y * sm.pref[t]);
    y = (int)(r / len);
    j = (int)(r - (uint32_t)y * len);
  };

  const int64_t blk_stride = (int64_t)p.Hkv * T::TILE;
  uint4 qr[NTL * KS];
  f32x4 o[NTL * DPL];
  float m_run[NTL];
  f32x4 l_acc[NTL];   // every element: the column's sum of weights
  int pos[NTL];

  // The piece after the one ending at unit u0 in segment (t0, y0): the next
  // segment of the share that holds blocks (a segment's first R units are
  // restart units).  False if the share has none.
  auto next_piece = [&](int t0, int y0, int64_t u0, int& t1, int& y1, int& b1n) -> bool {
    int tt = t0, yy = y0;
    int64_t uu = u0;
    while (uu < u_hi) {
      if (++yy == Y) {
        yy = 0;
        do {
          ++tt;
        } while (sm.pref[tt + 1] == sm.pref[tt]);
      }
      const int ln = sm.pref[tt + 1] - sm.pref[tt];
      const int64_t st = Y * sm.pref[tt] + (int64_t)yy * ln;
      const int64_t en = st + ln < u_hi ? st + ln : u_hi;
      const int bb1 = max((int)(en - st) - sp.R, 0);
      if (bb1 > 0) {
        t1 = tt;
        y1 = yy;
        b1n = bb1;
        return true;
      }
      uu = en;
    }
    return false;
  };
  // q rows of the piece's column tiles, and the first window of its block
  // ids (steps b0.., as mfma_piece reads them), for segment (tt, yy)
  constexpr int NW = PKV_ID_VGPRS;
  auto piece_loads = [&](int tt, int yy, int b0, int b1p, uint4* qd, int* idd) {
    const int ss = sm.tseq[tt];
    const int hc = yy % p.hchunks, hk = yy / p.hchunks;
    const int n = sm.n[ss], r0 = sm.r0[ss];
    const int h = hc * p.chunk + c % p.chunk;
    const int i0 = (tt - sm.tb[ss]) * p.rpt + c / p.chunk;
#pragma unroll
    for (int k = 0; k < NTL; ++k) {
      const int iqk = i0 + k * p.qpt;
      const bool lv = c < p.qpt * p.chunk && iqk < n && h < p.g;
      T::load_q(qd + k * KS, p.q, (int64_t)(r0 + iqk) * p.Hq + hk * p.g + h, lv, G);
    }
    const int32_t* row = p.bt + (int64_t)ss * p.mb;
    const int nn = min(64 * NW, b1p - b0);
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) idd[w2] = row[b0 + min(64 * w2 + lane, nn - 1)];
  };
  uint4 qn[NTL * KS];   // the next piece's, loaded while this one streams
  int idc0[NW], idn[NW];
  bool have_next = false;

  int64_t u = u_lo;
  int t, y, j;
  locate(u, t, y, j);
  int s = sm.tseq[t];
  bool first_piece = true;
  while (true) {
    const int len = sm.pref[t + 1] - sm.pref[t];
    const int64_t seg_start = Y * sm.pref[t] + (int64_t)y * len;
    const int64_t pe = seg_start + len < u_hi ? seg_start + len : u_hi;
    const int b = max(j - sp.R, 0);
    const int b1 = max((int)(pe - seg_start) - sp.R, 0);
    if (b1 > b) {
      const int hc = y % p.hchunks, hk = y / p.hchunks;
      const int n = sm.n[s], ctx = sm.ctx[s], r0 = sm.r0[s];
      // this lane's column in column tile k: row iq(k) of the sequence,
      // q-head h of the kv-head
      const int h = hc * p.chunk + c % p.chunk;
      const int i0 = (t - sm.tb[s]) * p.rpt + c / p.chunk;
      auto iq = [&](int k) { return i0 + k * p.qpt; };
      auto live = [&](int k) { return c < p.qpt * p.chunk && iq(k) < n && h < p.g; };
      // this piece's q and first ids: loaded ahead by the previous piece
      // (which started at step 0 of this segment), else now
      if (have_next) {
#pragma unroll
        for (int k = 0; k < NTL * KS; ++k) qr[k] = qn[k];
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) idc0[w2] = idn[w2];
      } else {
        piece_loads(t, y, b, b1, qr, idc0);
      }
      // the next piece's loads go out before this piece's blocks
      int tn = t, yn = y, b1n = 0;
      have_next = p.nb > 0 && next_piece(t, y, pe, tn, yn, b1n);
      if (have_next) piece_loads(tn, yn, 0, b1n, qn, idn);
#pragma unroll
      for (int k = 0; k < NTL; ++k) {
        // < 0: the column attends to nothing; one not stored sees every token
        pos[k] = live(k) ? ctx - n + iq(k) : kSeesAll;
        m_run[k] = kNegInf;
        l_acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int e = 0; e < NTL * DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int last = ((ctx + 15) >> 4) - 1;
      if (p.nb > 0) {
        const int64_t off = (int64_t)hk * T::TILE;
        mfma_piece<QT, KVT, D, pkv::byte_codes(KVT) ? PKV_PIPE_DEPTH_FP8 : PKV_PIPE_DEPTH,
                   !pkv::byte_codes(KVT), true, false, NTL>(
            p.kc + off, p.vc + off, blk_stride, p.bt + (int64_t)s * p.mb, b, b1, last,
            ctx - 16 * last, p.nb, qr, p.sl2, m_run, reinterpret_cast<float*>(l_acc), o, lane,
            pos, nullptr, NoHook{}, 1, idc0);
      }
      // close the piece: store the rows, or leave (m, l, acc) for the merge
      const bool whole = b == 0 && b1 == len - sp.R;
      const int64_t slot = 2 * (int64_t)wk + (first_piece ? 0 : 1);
#pragma unroll
      for (int k = 0; k < NTL; ++k) {
        const float l_tot = l_acc[k][0];
        if (!live(k)) continue;
        // each lane's DPL consecutive dims of a row leave in one store
        if (whole) {
          const int64_t row = ((int64_t)(r0 + iq(k)) * p.Hq + hk * p.g + h) * D + DPL * 4 * G;
          const float inv = l_tot > 0.f ? p.vsc / l_tot : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float vals[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) vals[e] = o[k * DPL + e][i] * inv;
            store_out_n<QT, DPL>(p.out, row + DPL * i, vals);
          }
        } else {
          const int64_t col = slot * NC + k * kCols + c;
          float4* dst = reinterpret_cast<float4*>(sp.part + col * D + DPL * 4 * G);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < DPL; e += 4)
              dst[(DPL * i + e) / 4] =
                  make_float4(o[k * DPL + e][i] * p.vsc, o[k * DPL + e + 1][i] * p.vsc,
                              o[k * DPL + e + 2][i] * p.vsc, o[k * DPL + e + 3][i] * p.vsc);
          if (G == 0) {
            sp.ml[col * 2] = m_run[k];
            sp.ml[col * 2 + 1] = l_tot;
          }
        }
      }
      first_piece = false;
    }
    u = pe;
    if (u >= u_hi) break;
    j = 0;
    if (++y == Y) {
      y = 0;
      do {
        ++t;
      } while (sm.pref[t + 1] == sm.pref[t]);
      s = sm.tseq[t];
    }
  }
}

// Merge the pieces of every segment the grid above split between waves, the
// shares recomputed exactly as there.  One wave per (split segment, column
// tile, quarter of the head dim): lane l takes column l / 4 of the column
// tile and a sixteenth of its dims, and folds the pieces in order with the
// running log-sum-exp rescale, the loads of four pieces at a time in flight
// together.  (The partials of 16 columns make this merge four times the
// decode merge's traffic per segment; the split gives it enough waves to
// keep that many loads in flight.)
template <int QT, int D>
__global__ __launch_bounds__(64 * pkv::kWaves) void multiquery_split_merge_kernel(
    MQStreamParams sp) {
  constexpr int kDimSplit = 4;          // waves per (segment, column tile)
  constexpr int DQ = D / (4 * kDimSplit);   // dims per lane
  constexpr int NV = DQ / 4;            // float4 loads per lane and piece
  __shared__ MQStreamSmem sm;
  mq_tile_prefix(sp, sm);
  const MQParams& p = sp.b;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int cc = lane >> 2;
  const int Tn = sm.tb[p.S];
  const int64_t Y = sp.Y;
  const int64_t U = Y * sm.pref[Tn];
  const int64_t We = U < sp.W ? U : sp.W;
  if (We == 0) return;
  const int64_t nitems = (int64_t)Tn * Y * p.ntl * kDimSplit;
  for (int64_t it = (int64_t)blockIdx.x * pkv::kWaves + w; it < nitems;
       it += (int64_t)gridDim.x * pkv::kWaves) {
    const int dq = (int)(it % kDimSplit);
    const int d0 = dq * (D / kDimSplit) + (lane & 3) * DQ;
    const int ct = (int)(it / kDimSplit % p.ntl);
    const int64_t seg = it / kDimSplit / p.ntl;
    const int t = (int)(seg / Y), y = (int)(seg % Y);
    const int len = sm.pref[t + 1] - sm.pref[t];
    if (len == 0) continue;
    // the segment's blocks are its units [seg_start + R, seg_start + len)
    const int64_t seg_start = Y * sm.pref[t] + (int64_t)y * len;
    const int64_t wa = floor_div53((seg_start + sp.R + 1) * We - 1, U);
    const int64_t wb = floor_div53((seg_start + len) * We - 1, U);
    if (wa == wb) continue;
    // the first worker's piece is its first piece with blocks unless its
    // share holds blocks of the segment before (units below seg_start)
    const int64_t sl0 = 2 * wa + (floor_div53(U * wa, We) >= seg_start ? 0 : 1);
    const int np = (int)(wb - wa + 1);
    const int s = sm.tseq[t];
    const int hc = y % p.hchunks, hk = y / p.hchunks;
    const int h = hc * p.chunk + cc % p.chunk;
    const int nc = kCols * p.ntl;   // columns of a slot
    {
      const int iq = (t - sm.tb[s]) * p.rpt + ct * p.qpt + cc / p.chunk;
      const bool live = cc < p.qpt * p.chunk && iq < sm.n[s] && h < p.g;
      auto slot_of = [&](int k) { return k == 0 ? sl0 : 2 * (wa + k); };
      // (m, l) and this lane's accumulator dims of piece k (zeros for a dead
      // column, which never reads)
      auto load_piece = [&](int k, float2& v, float4 (&x)[NV]) {
        const int64_t sl = slot_of(k) * nc + ct * kCols + cc;
        v = make_float2(kNegInf, 0.f);
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) {
          v = *reinterpret_cast<const float2*>(sp.ml + sl * 2);
          const float4* src = reinterpret_cast<const float4*>(sp.part + sl * D + d0);
#pragma unroll
          for (int i = 0; i < NV; ++i) x[i] = src[i];
        }
      };
      float M = kNegInf, L = 0.f;
      float4 acc[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      // kBatch pieces' loads go out together, then fold in order (pieces
      // past np repeat the last one and are not folded)
      constexpr int kBatch = 4;
      for (int base = 0; base < np; base += kBatch) {
        float2 v[kBatch];
        float4 x[kBatch][NV];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) load_piece(min(base + u, np - 1), v[u], x[u]);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (base + u < np && v[u].y > 0.f) {
            const float Mn = fmaxf(M, v[u].x);
            const float a = __builtin_amdgcn_exp2f(M - Mn);   // 0 while M = -inf
            const float b = __builtin_amdgcn_exp2f(v[u].x - Mn);
            L = L * a + v[u].y * b;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
              acc[i].x = acc[i].x * a + x[u][i].x * b;
              acc[i].y = acc[i].y * a + x[u][i].y * b;
              acc[i].z = acc[i].z * a + x[u][i].z * b;
              acc[i].w = acc[i].w * a + x[u][i].w * b;
            }
            M = Mn;
          }
        }
      }
      if (live) {
        const int64_t row = ((int64_t)(sm.r0[s] + iq) * p.Hq + hk * p.g + h) * D + d0;
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
          store_out4<QT>(p.out, row + 4 * i, acc[i].x * inv, acc[i].y * inv, acc[i].z * inv,
                         acc[i].w * inv);
      }
    }
  }
}

MQParams make_mq_params(const pkv::MQArgs& a) {
  MQParams p;
  p.out = a.out;
  p.q = a.q;
  p.kc = static_cast<const uint8_t*>(a.k_cache);
  p.vc = static_cast<const uint8_t*>(a.v_cache);
  p.bt = a.block_tables;
  p.cl = a.context_lens;
  p.qs = a.query_start;
  p.S = a.num_seqs;
  p.rows = a.num_rows;
  p.max_q = a.max_query_len;
  p.Hq = a.num_q_heads;
  p.Hkv = a.num_kv_heads;
  p.g = a.num_q_heads / a.num_kv_heads;
  p.nb = a.num_blocks;
  p.mb = a.max_blocks_per_seq;
  const pkv::MQTiles t = pkv::mq_tiles(p.g, a.max_query_len, a.max_ntl);
  p.chunk = t.chunk;
  p.hchunks = t.hchunks;
  p.qpt = t.qpt;
  p.ntl = t.ntl;
  p.rpt = t.qpt * t.ntl;
  p.qtiles = t.qtiles;
  p.part_blocks = a.partition / pkv::kBlockSize;
  p.num_parts = a.num_parts;
  const bool fp8 = pkv::byte_codes(a.kv_dtype);   // scaled one-byte codes
  p.sl2 = a.scale * kLog2e * (fp8 ? a.k_scale : 1.0f);
  p.vsc = fp8 ? a.v_scale : 1.0f;
  p.ws_m = a.ws_m;
  p.ws_l = a.ws_l;
  p.ws_acc = a.ws_acc;
  p.nx = pkv::device_xccs();
  p.groups = (int64_t)p.num_parts * p.S * p.Hkv * p.hchunks;
  return p;
}

template <int QT, int KVT, int D>
int launch_mq_t(const pkv::MQArgs& a) {
  const MQParams p = make_mq_params(a);
  const int64_t runs = (p.groups + p.nx - 1) / p.nx;
  const int64_t nwg = runs * p.nx * p.qtiles;
  if (nwg > INT32_MAX) return (int)hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nwg);
  const dim3 block(64 * pkv::kWaves);
  auto k = p.ntl == 4   ? multiquery_mfma_kernel<QT, KVT, D, 4>
           : p.ntl == 2 ? multiquery_mfma_kernel<QT, KVT, D, 2>
                        : multiquery_mfma_kernel<QT, KVT, D, 1>;
  return pkv::launch_kernel(k, grid, block, a.stream, p, a.ev_start, a.ev_stop);
}

template <int QT, int D>
int launch_mq_reduce_t(const pkv::MQArgs& a) {
  const MQParams p = make_mq_params(a);
  return pkv::launch_kernel(multiquery_reduce_kernel<QT, D>,
                            dim3((unsigned)((int64_t)p.rows * p.Hq)), dim3(64), a.stream, p,
                            a.ev_start, a.ev_stop);
}

MQStreamParams make_mq_stream_params(const pkv::MQArgs& a) {
  MQStreamParams sp;
  sp.b = make_mq_params(a);
  sp.Y = sp.b.Hkv * sp.b.hchunks;
  sp.W = a.stream_grid * pkv::kWaves;
  sp.R = pkv::kv_restart_units(a.kv_dtype);
  sp.ml = a.st_ml;
  sp.part = a.st_part;
  return sp;
}

template <int QT, int KVT, int D>
int launch_mq_stream_t(const pkv::MQArgs& a) {
  const MQStreamParams sp = make_mq_stream_params(a);
  const dim3 grid(a.stream_grid), block(64 * pkv::kWaves);
  auto k = sp.b.ntl == 4   ? multiquery_stream_kernel<QT, KVT, D, 4>
           : sp.b.ntl == 2 ? multiquery_stream_kernel<QT, KVT, D, 2>
                           : multiquery_stream_kernel<QT, KVT, D, 1>;
  return pkv::launch_kernel(k, grid, block, a.stream, sp, a.ev_start, a.ev_stop);
}

template <int QT, int D>
int launch_mq_split_merge_t(const pkv::MQArgs& a) {
  const MQStreamParams sp = make_mq_stream_params(a);
  // one wave per (segment, column tile, quarter of the head dim), bounded
  // by sequences x row tiles.  At most two workgroups per CU: each one
  // rebuilds the tile prefix sums in LDS first (57 KB, so two fit on a CU),
  // and one round of that is cheaper than several, the waves looping over
  // the items instead.
  const int64_t nitems = (int64_t)sp.b.S * sp.b.qtiles * sp.Y * sp.b.ntl * 4;
  int64_t grid = (nitems + pkv::kWaves - 1) / pkv::kWaves;
  const int64_t cap = 2 * (int64_t)pkv::device_cus();
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  return pkv::launch_kernel(multiquery_split_merge_kernel<QT, D>, dim3((unsigned)grid),
                            dim3(64 * pkv::kWaves), a.stream, sp, a.ev_start, a.ev_stop);
}

}  // namespace

namespace pkv {

int launch_multiquery_stream(const MQArgs& a) {
  const int q = a.q_dtype, kv = a.kv_dtype, D = a.head_dim;
#define PKV_MQ_CASE(QT, KVT, DD) \
  if (q == QT && kv == KVT && D == DD) return launch_mq_stream_t<QT, KVT, DD>(a);
  PKV_MQ_CASE(PKV_BF16, PKV_BF16, 64)
  PKV_MQ_CASE(PKV_BF16, PKV_BF16, 128)
  PKV_MQ_CASE(PKV_F16, PKV_F16, 64)
  PKV_MQ_CASE(PKV_F16, PKV_F16, 128)
  PKV_MQ_CASE(PKV_BF16, PKV_FP8_E4M3, 64)
  PKV_MQ_CASE(PKV_BF16, PKV_FP8_E4M3, 128)
  PKV_MQ_CASE(PKV_F16, PKV_FP8_E4M3, 64)
  PKV_MQ_CASE(PKV_F16, PKV_FP8_E4M3, 128)
  PKV_MQ_CASE(PKV_BF16, PKV_INT8, 64)
  PKV_MQ_CASE(PKV_BF16, PKV_INT8, 128)
  PKV_MQ_CASE(PKV_F16, PKV_INT8, 64)
  PKV_MQ_CASE(PKV_F16, PKV_INT8, 128)
#undef PKV_MQ_CASE
  return (int)hipErrorInvalidValue;
}

int launch_multiquery_split_merge(const MQArgs& a) {
  const int q = a.q_dtype, D = a.head_dim;
  if (q == PKV_BF16 && D == 128) return launch_mq_split_merge_t<PKV_BF16, 128>(a);
  if (q == PKV_BF16 && D == 64) return launch_mq_split_merge_t<PKV_BF16, 64>(a);
  if (q == PKV_F16 && D == 128) return launch_mq_split_merge_t<PKV_F16, 128>(a);
  if (q == PKV_F16 && D == 64) return launch_mq_split_merge_t<PKV_F16, 64>(a);
  return (int)hipErrorInvalidValue;
}

int launch_multiquery(const MQArgs& a) {
  const int q = a.q_dtype, kv = a.kv_dtype, D = a.head_dim;
#define PKV_MQ_CASE(QT, KVT, DD) \
  if (q == QT && kv == KVT && D == DD) return launch_mq_t<QT, KVT, DD>(a);
  PKV_MQ_CASE(PKV_BF16, PKV_BF16, 64)
  PKV_MQ_CASE(PKV_BF16, PKV_BF16, 128)
  PKV_MQ_CASE(PKV_F16, PKV_F16, 64)
  PKV_MQ_CASE(PKV_F16, PKV_F16, 128)
  PKV_MQ_CASE(PKV_BF16, PKV_FP8_E4M3, 64)
  PKV_MQ_CASE(PKV_BF16, PKV_FP8_E4M3, 128)
  PKV_MQ_CASE(PKV_F16, PKV_FP8_E4M3, 64)
  PKV_MQ_CASE(PKV_F16, PKV_FP8_E4M3, 128)
  PKV_MQ_CASE(PKV_BF16, PKV_INT8, 64)
  PKV_MQ_CASE(PKV_BF16, PKV_INT8, 128)
  PKV_MQ_CASE(PKV_F16, PKV_INT8, 64)
  PKV_MQ_CASE(PKV_F16, PKV_INT8, 128)
#undef PKV_MQ_CASE
  return (int)hipErrorInvalidValue;
}

int launch_multiquery_reduce(const MQArgs& a) {
  const int q = a.q_dtype, D = a.head_dim;
  if (q == PKV_BF16 && D == 128) return launch_mq_reduce_t<PKV_BF16, 128>(a);
  if (q == PKV_BF16 && D == 64) return launch_mq_reduce_t<PKV_BF16, 64>(a);
  if (q == PKV_F16 && D == 128) return launch_mq_reduce_t<PKV_F16, 128>(a);
  if (q == PKV_F16 && D == 64) return launch_mq_reduce_t<PKV_F16, 64>(a);
  return (int)hipErrorInvalidValue;
}

}  // namespace pkv
