// Paged decode attention on the CDNA4 matrix cores, fixed partitions.
//
// Each workgroup owns one (partition, kv-head, head chunk, sequence); its
// waves take the partition's 16-token blocks in turn (wave w every NWG-th
// block from the w-th), each with an online softmax (mfma_piece,
// pkv_mfma_common.h), and merge through LDS at the end (see
// pkv_decode_common.h).
//
// Math: softmax(q K^T * scale) V over the block-table-gathered context
// ("KV Cache 与 PageAttention深度实战", sections 1.2 and 3.2).
#include <hip/hip_runtime.h>

#include "pkv_mfma_common.h"
#include "pkv_launch.h"

#ifndef PKV_PIPE_DEPTH
#define PKV_PIPE_DEPTH 2       // K/V blocks in flight per wave, 16-bit caches
#endif
#ifndef PKV_PIPE_DEPTH_FP8
#define PKV_PIPE_DEPTH_FP8 2   // same for E4M3 caches
#endif
#ifndef PKV_MFMA_NT16
#define PKV_MFMA_NT16 false    // non-temporal K/V loads, 16-bit caches
#endif
#ifndef PKV_MFMA_NT8
#define PKV_MFMA_NT8 true      // non-temporal K/V loads, one-byte codes
#endif
#ifndef PKV_MFMA_WPE
#define PKV_MFMA_WPE 2     // minimum waves per SIMD the register budget must allow
#endif
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4   // waves per workgroup (they split the partition's blocks)
#endif

namespace {

using namespace pkvd;

constexpr int NWG = PKV_MFMA_WAVES;

// The step's new K/V row of one (sequence, kv-head) (NewRow), appended by
// the decode kernel itself.  prepare() encodes the lane's raw elements and
// stages the encoded rows in the wave's own part of the LDS merge area (not
// used until the wave's blocks are done); the writer wave also stores them
// to the slot.  sub() runs before each loaded tile is consumed and puts the
// row into the tile when its block holds the slot.
template <int QT, int KVT, int D>
struct AppendRow {
  using N = NewRow<QT, KVT, D>;
  static constexpr bool active = false;
  static constexpr bool subst = true;
  uint32_t kraw, vraw;
  float k_inv, v_inv;
  int64_t slot;    // the row's slot (negative: no row)
  bool writer;
  uint8_t* lds;    // N::STAGE bytes of the wave's LDS, 16-byte aligned
  uint8_t* kc;
  uint8_t* vc;
  int nb, Hkv, hk, lane;
  int period = 0;
  __device__ void operator()() const {}

  __device__ void prepare() const {
    uint32_t ke, ve;
    N::encode(kraw, vraw, k_inv, v_inv, ke, ve);
    N::stage(lds, lane, ke, ve);
    if (writer && slot >= 0 && slot < (int64_t)nb * pkv::kBlockSize)
      N::store(kc, vc, slot, Hkv, hk, lane, ke, ve);
  }

  // r: the tile of block `id` (wave-uniform)
  __device__ void sub(typename N::T::Raw& r, int id) const {
    if (slot < 0 || (int64_t)id != slot >> 4) return;
    N::sub(r, lds, (int)(slot & 15), lane);
  }
};

// PC: a one-byte-code cache with per-channel scales (p.ks, p.vs).
// APP: the kernel appends the step's new K/V rows itself (p.kn, p.vn,
// p.slots; AppendRow).
template <int QT, int KVT, int D, int HS, bool PC, bool APP = false>
__global__ __launch_bounds__(64 * NWG) __attribute__((amdgpu_waves_per_eu(PKV_MFMA_WPE, 8)))
void decode_mfma_kernel(DecodeParams p) {
  using T = MfmaTile<QT, KVT, D>;
  constexpr int LD = D + 4;
  constexpr int DPL = T::DPL;

  __shared__ float sm_m[NWG * HS];
  __shared__ float sm_l[NWG * HS];
  __shared__ __align__(16) float sm_o[NWG * HS * LD];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, G = lane >> 4;
  const int part = blockIdx.x, s = blockIdx.z;
  const int hk = blockIdx.y / p.hchunks, hc = blockIdx.y % p.hchunks;
  const int h_first = hk * p.g + hc * p.chunk_heads;
  const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
  const int b_begin = part * p.part_blocks;
  const int32_t* row = p.bt + (int64_t)s * p.mb;

  // Wave w takes blocks b_begin + w, b_begin + w + NWG, ... of the partition.
  // Which ids those are does not depend on the context length, so the first
  // window of them (and q) is requested before the length arrives: the
  // first K/V loads wait for one round trip less.  Indices past the table
  // row are clamped to its last entry (never used: the piece stops at the
  // context).
  // APP: the new row's slot (AppendRow), read first: before any store of
  // the kernel, so that it stays a scalar load
  [[maybe_unused]] int64_t slot = -1;
  if constexpr (APP) slot = p.slots[s];
  int ids0[PKV_ID_VGPRS];
  if (p.mb > 0) {
#pragma unroll
    for (int k = 0; k < PKV_ID_VGPRS; ++k)
      ids0[k] = row[min(b_begin + w + NWG * (64 * k + lane), p.mb - 1)];
  }
  uint4 qr[T::KSTEPS];
  uint4 qlo[PC ? T::KSTEPS : 1];
  if constexpr (PC)
    T::load_q_scaled(qr, qlo, p.q, (int64_t)s * p.Hq + h_first + c, c < nh, G,
                     p.ks + (int64_t)hk * D);
  else
    T::load_q(qr, p.q, (int64_t)s * p.Hq + h_first + c, c < nh, G);

  // APP: the raw new row of this (sequence, kv-head), lane l's elements
  // (AppendRow), requested with q, before the context length, which it does
  // not depend on.
  [[maybe_unused]] uint32_t kraw = 0u, vraw = 0u;
  if constexpr (APP)
    NewRow<QT, KVT, D>::load(p.kn, p.vn, (int64_t)s * p.Hkv + hk, lane, kraw, vraw);
  const int ctx = clamped_ctx(p, s);
  const int nblk = (ctx + 15) >> 4;
  if (part > 0 && b_begin >= nblk) {
    // the new row is used on this path too, so the compiler keeps its loads
    // above the branch (sunk below it, they would be issued after the
    // length's round trip, and the first K/V loads would wait for them)
    if constexpr (APP) asm volatile("" ::"v"(kraw), "v"(vraw), "s"(slot));
    return;
  }
  const int b_end = min(b_begin + p.part_blocks, nblk);

  f32x4 o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // this wave's steps, and the step holding the context's last block (if any)
  const int nblk_p = b_end - b_begin;
  const int steps = nblk_p > w ? (nblk_p - w + NWG - 1) / NWG : 0;
  const int lb = nblk - 1 - b_begin - w;
  const int last_step = (b_end == nblk && lb >= 0 && lb % NWG == 0) ? lb / NWG : -1;
  [[maybe_unused]] const AppendRow<QT, KVT, D> app{
      kraw, vraw, p.k_inv, p.v_inv, slot, part == 0 && hc == 0 && w == 0,
      reinterpret_cast<uint8_t*>(sm_o + w * HS * LD), const_cast<uint8_t*>(p.kc),
      const_cast<uint8_t*>(p.vc), p.nb, p.Hkv, hk, lane};
  if (p.nb > 0 && steps > 0) {
    const int64_t blk_stride = (int64_t)p.Hkv * T::TILE;
    const int64_t head_off = (int64_t)hk * T::TILE;
    constexpr int DEPTH = pkv::byte_codes(KVT) ? PKV_PIPE_DEPTH_FP8 : PKV_PIPE_DEPTH;
    constexpr bool NT = pkv::byte_codes(KVT) ? PKV_MFMA_NT8 : PKV_MFMA_NT16;
    if constexpr (APP) {
      mfma_piece<QT, KVT, D, DEPTH, NT, false, PC>(
          p.kc + head_off, p.vc + head_off, blk_stride, row + b_begin + w, 0, steps, last_step,
          ctx - 16 * (nblk - 1), p.nb, qr, p.sl2, &m_run, &l_run, o, lane, nullptr, qlo, app,
          NWG, ids0);
    } else {
      mfma_piece<QT, KVT, D, DEPTH, NT, false, PC>(
          p.kc + head_off, p.vc + head_off, blk_stride, row + b_begin + w, 0, steps, last_step,
          ctx - 16 * (nblk - 1), p.nb, qr, p.sl2, &m_run, &l_run, o, lane, nullptr, qlo,
          NoHook{}, NWG, ids0);
    }
  } else if constexpr (APP) {
    if (app.writer) app.prepare();   // no blocks here: only the store remains
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
  merge_waves_and_store<QT, D, HS, NWG>(p, sm_m, sm_l, sm_o, nh, s, h_first, part);
}

template <int QT, int KVT, int D, int HS>
int launch_t(const pkv::DecodeArgs& a, const DecodeParams& kp) {
  dim3 grid(kp.num_parts, a.num_kv_heads * kp.hchunks, a.num_seqs);
  const dim3 block(64 * NWG);
  if constexpr (pkv::byte_codes(KVT)) {
    if (kp.ks)
      return pkv::launch_kernel(decode_mfma_kernel<QT, KVT, D, HS, true>, grid, block, a.stream,
                                kp, a.ev_start, a.ev_stop);
  }
  if (kp.kn)
    return pkv::launch_kernel(decode_mfma_kernel<QT, KVT, D, HS, false, true>, grid, block,
                              a.stream, kp, a.ev_start, a.ev_stop);
  return pkv::launch_kernel(decode_mfma_kernel<QT, KVT, D, HS, false>, grid, block, a.stream, kp,
                            a.ev_start, a.ev_stop);
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
  PKV_MFMA_CASE(PKV_BF16, PKV_INT8, 128)
  PKV_MFMA_CASE(PKV_BF16, PKV_INT8, 64)
  PKV_MFMA_CASE(PKV_F16, PKV_INT8, 128)
  PKV_MFMA_CASE(PKV_F16, PKV_INT8, 64)
#undef PKV_MFMA_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace pkv
