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
// 16 / chunk rows (4 rows x 4 heads at g = 4, 16 rows x 1 head for MHA), so
// one K/V tile load serves every row of the tile.  Each lane masks its
// column's logits at that row's position.
//
// Grid (partition, kv-head x head chunk x row tile, sequence).  A workgroup
// walks the blocks its last row can see; its four waves take contiguous
// quarters of them and merge in LDS.  With several partitions each workgroup
// writes (m, l, acc) partials, an empty partition writing m = -inf, l = 0, and
// multiquery_reduce_kernel merges every row's partitions by log-sum-exp.
#include <hip/hip_runtime.h>

#include "pkv_mfma_common.h"

#ifndef PKV_PIPE_DEPTH
#define PKV_PIPE_DEPTH 2       // K/V blocks in flight per wave, 16-bit caches
#endif
#ifndef PKV_PIPE_DEPTH_FP8
#define PKV_PIPE_DEPTH_FP8 2   // same for E4M3 caches
#endif

namespace {

using namespace pkvd;

constexpr int kCols = 16;   // MFMA tile columns

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
  int qpt;           // query rows per tile (16 / chunk)
  int qtiles;        // row tiles per (sequence, kv-head, head chunk) in the grid
  int part_blocks;   // 16-token blocks per partition
  int num_parts;     // partitions in the grid (1 = single pass)
  float sl2;         // scale * log2(e) * k_scale
  float vsc;         // v_scale (1 unless FP8)
  float* ws_m;       // [rows][Hq][P]
  float* ws_l;       // [rows][Hq][P]
  float* ws_acc;     // [rows][Hq][P][D]
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

template <int QT, int KVT, int D>
__global__ __launch_bounds__(64 * pkv::kWaves) __attribute__((amdgpu_waves_per_eu(2, 8)))
void multiquery_mfma_kernel(MQParams p) {
  using T = MfmaTile<QT, KVT, D>;
  constexpr int LD = D + 4;
  constexpr int DPL = T::DPL;

  __shared__ float sm_m[pkv::kWaves * kCols];
  __shared__ float sm_l[pkv::kWaves * kCols];
  __shared__ float sm_o[pkv::kWaves * kCols * LD];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, G = lane >> 4;
  const int part = blockIdx.x, s = blockIdx.z;
  int yy = blockIdx.y;
  const int qt = yy % p.qtiles;
  yy /= p.qtiles;
  const int hc = yy % p.hchunks, hk = yy / p.hchunks;
  int r0, n;
  seq_rows(p, s, r0, n);
  const int i0 = qt * p.qpt;
  if (i0 >= n) return;   // no row of this sequence in the tile
  const int cap = p.mb * pkv::kBlockSize;
  const int ctx = min(max(p.cl[s], 0), cap);

  // this lane's column: row i0 + c / chunk, q-head hk*g + hc*chunk + c % chunk
  const int iq = i0 + c / p.chunk;
  const int h = hc * p.chunk + c % p.chunk;
  const bool live = c < p.qpt * p.chunk && iq < n && h < p.g;
  const int pos = live ? ctx - n + iq : -1;   // < 0: the row attends to nothing
  // blocks any row of the tile can see: up to its last row's position
  const int p_last = ctx - n + min(i0 + p.qpt, n) - 1;
  const int nblk = p_last >= 0 ? (p_last >> 4) + 1 : 0;
  const int b_begin = part * p.part_blocks;
  const int b_end = min(b_begin + p.part_blocks, nblk);
  const int nblk_p = max(b_end - b_begin, 0);

  uint4 qr[T::KSTEPS];
  T::load_q(qr, p.q, (int64_t)(r0 + iq) * p.Hq + hk * p.g + h, live, G);
  f32x4 o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int w0 = b_begin + (nblk_p * w) / pkv::kWaves;
  const int w1 = b_begin + (nblk_p * (w + 1)) / pkv::kWaves;
  if (p.nb > 0 && w1 > w0) {
    const int64_t blk_stride = (int64_t)p.Hkv * T::TILE;
    const int64_t head_off = (int64_t)hk * T::TILE;
    const int last = ((ctx + 15) >> 4) - 1;
    mfma_piece<QT, KVT, D, pkv::byte_codes(KVT) ? PKV_PIPE_DEPTH_FP8 : PKV_PIPE_DEPTH, false,
               true>(p.kc + head_off, p.vc + head_off, blk_stride, p.bt + (int64_t)s * p.mb,
                     w0, w1, last, ctx - 16 * last, p.nb, qr, p.sl2, m_run, l_run, o, lane,
                     pos);
  }

  // lane (G, c) holds O[column c][dim DPL*(4G+i) + e]; l needs the 4 G lanes
  l_run = wave_sum4(l_run);
  if (G == 0) {
    sm_m[w * kCols + c] = m_run;
    sm_l[w * kCols + c] = l_run;
  }
  {
    float* dst = sm_o + (w * kCols + c) * LD + DPL * 4 * G;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[DPL * i + e] = o[e][i];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < kCols * D; idx += 64 * pkv::kWaves) {
    const int cc = idx / D, d = idx % D;
    const int ic = i0 + cc / p.chunk, hh = hc * p.chunk + cc % p.chunk;
    if (cc >= p.qpt * p.chunk || ic >= n || hh >= p.g) continue;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < pkv::kWaves; ++v) M = fmaxf(M, sm_m[v * kCols + cc]);
    float L = 0.f, acc = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int v = 0; v < pkv::kWaves; ++v) {
        const float mv = sm_m[v * kCols + cc];
        const float f = (mv == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        L += f * sm_l[v * kCols + cc];
        acc += f * sm_o[(v * kCols + cc) * LD + d];
      }
    }
    const int64_t row = (int64_t)(r0 + ic) * p.Hq + hk * p.g + hh;
    if (p.num_parts == 1) {
      store_out<QT>(p.out, row * D + d, L > 0.f ? acc * p.vsc / L : 0.f);
    } else {
      const int64_t pr = row * p.num_parts + part;
      p.ws_acc[pr * D + d] = acc * p.vsc;
      if (d == 0) {
        p.ws_m[pr] = M;
        p.ws_l[pr] = L;
      }
    }
  }
}

// One wave per (row, q-head) of the rows some sequence owns: the log-sum-exp
// merge of the row's partitions, every one of which the kernel above wrote.
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
  const pkv::MQTiles t = pkv::mq_tiles(p.g, a.max_query_len);
  p.chunk = t.chunk;
  p.hchunks = t.hchunks;
  p.qpt = t.qpt;
  p.qtiles = t.qtiles;
  p.part_blocks = a.partition / pkv::kBlockSize;
  p.num_parts = a.num_parts;
  const bool fp8 = pkv::byte_codes(a.kv_dtype);   // scaled one-byte codes
  p.sl2 = a.scale * kLog2e * (fp8 ? a.k_scale : 1.0f);
  p.vsc = fp8 ? a.v_scale : 1.0f;
  p.ws_m = a.ws_m;
  p.ws_l = a.ws_l;
  p.ws_acc = a.ws_acc;
  return p;
}

template <int QT, int KVT, int D>
int launch_mq_t(const pkv::MQArgs& a) {
  const MQParams p = make_mq_params(a);
  dim3 grid(p.num_parts, p.Hkv * p.hchunks * p.qtiles, p.S);
  multiquery_mfma_kernel<QT, KVT, D>
      <<<grid, dim3(64 * pkv::kWaves), 0, (hipStream_t)a.stream>>>(p);
  return (int)hipGetLastError();
}

template <int QT, int D>
int launch_mq_reduce_t(const pkv::MQArgs& a) {
  const MQParams p = make_mq_params(a);
  multiquery_reduce_kernel<QT, D>
      <<<dim3((unsigned)((int64_t)p.rows * p.Hq)), dim3(64), 0, (hipStream_t)a.stream>>>(p);
  return (int)hipGetLastError();
}

}  // namespace

namespace pkv {

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
