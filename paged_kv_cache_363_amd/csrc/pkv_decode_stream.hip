// Paged decode attention on the matrix cores with a work-balanced schedule.
//
// The contexts of a decode batch are ragged, so a grid of one workgroup per
// (sequence, kv-head, partition) leaves many workgroups empty or short and
// the last ones run on an almost idle GPU.  Here the step's work is
// flattened into units -- one 16-token block of one segment, a segment being
// the q-heads of one kv-head (at most 16 of them) of one sequence, segments
// in sequence order -- and a fixed grid of waves splits the units into equal
// contiguous shares.  A share covers the tail of one segment, whole segments
// and the head of another: a wave's pieces (the part of one segment inside
// the share).
//
// One load pipeline runs through a wave's whole share.  Before the first
// block the wave turns its steps (blocks, in share order) into cache tile
// indices in LDS (block id * kv-heads + kv-head, so one index addresses a
// block of any segment) and stages the q rows of its first pieces in LDS.
// Every step then consumes one block and issues the loads of the block
// DEPTH steps ahead, whichever piece it belongs to; a new piece only closes
// the running softmax state and takes its q rows from LDS, with the next
// blocks' loads in flight.  (A pipeline per piece paid about one loaded
// round trip at every piece.)
//
// A closed piece goes to an LDS stash, not to memory: a store issued between
// loads in flight holds up the wait for the next block until the store is
// acknowledged (vector loads and stores share one counter on CDNA).  The
// stash is written out when full and after the share's last block.  A whole
// segment is normalised and stored; a piece of a split segment is stored as
// (m, l, acc) in the wave's partial slot (its first piece in slot 0, its last
// in slot 1).  The waves never signal each other: across the XCDs of an
// MI355X that would need the L2 written back and invalidated at every
// signal.  Instead decode_split_merge_kernel runs next on the stream and
// merges the pieces of every split segment with the log-sum-exp rule
//   M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k acc_k 2^(m_k - M) / L.
// Both kernels derive the shares from the same prefix sums of the block
// counts, so the workspace carries nothing but the partial slots.
//
// Fixed partitions (partition mode): when the caller fixes the split-K
// partition size, the same persistent grid computes one (m, l, acc) per
// partition of P blocks into the fixed-partition workspace, and the
// split-K reduction kernel merges them.  There the units are whole
// partitions, so every partition belongs to one wave, and a wave closes each
// of its partitions into the stash when it has consumed the partition's last
// block.
//
// Math: softmax(q K^T * scale) V over the block-table-gathered context
// ("KV Cache 与 PageAttention深度实战", sections 1.2 and 3.2).
#include <hip/hip_runtime.h>

#include <type_traits>

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
// per wave in LDS: the stash of closed pieces (partitions), the tile list of
// the share's next steps, the q rows of the share's first pieces
constexpr int kStashFloats = 4096;   // accumulators (16 KiB)
constexpr int kStashSlots = 16;      // at most this many closed pieces
constexpr int kTileCap = 512;        // steps (2 KiB)
constexpr int kQStage = 768;         // uint4 (12 KiB): 3 pieces at D = 128
// s_waitcnt vmcnt(0) (lgkmcnt and expcnt left at their maxima)
constexpr int kVmcnt0 = 0x0F70;

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
  // the step's new K/V rows ([S][Hkv][D] in the q dtype) and their slots,
  // appended by the decode kernel itself (nullptr: none)
  const uint8_t* kn;
  const uint8_t* vn;
  const int64_t* slots;
  float k_inv, v_inv;
};

// Unit prefix sums in LDS, computed by one workgroup of 4 waves.  A segment
// of a sequence with nbk blocks spans nbk + R units: R units that stand for
// the cost of starting a piece (closing the previous one and taking the new
// q rows) followed by one unit per block.  Equal shares of units are then
// equal in time, not just in blocks.  In partition mode a unit is a whole
// partition of the segment instead, so that no partition is split between
// waves and no share needs rounding.
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
      // partition mode: one unit per partition of the segment
      int x = nbk > 0 ? (p.P > 0 ? (nbk + p.P - 1) / p.P : nbk + p.R) : 0;
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
// APP: the kernel appends the step's new K/V rows itself (p.kn, p.vn,
// p.slots; NewRow): a piece stages the new row of its (sequence, kv-head)
// in LDS, puts it into the tile of the slot's block before consuming it,
// and the piece holding the last block of its sequence's kv-head (head
// chunk 0) stores it to the slot.
template <int QT, int KVT, int D, bool PC, bool PM, bool APP = false>
__global__ __launch_bounds__(64 * kSkWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void decode_stream_kernel(StreamParams p) {
  using T = MfmaTile<QT, KVT, D>;
  using Raw = typename T::Raw;
  constexpr int DPL = T::DPL;
  constexpr int KS = T::KSTEPS;
  constexpr int NW = PKV_ID_VGPRS;
  constexpr int WIN = 64 * NW;                 // steps per register window of tiles
  constexpr int QU4 = KS * 64 * (PC ? 2 : 1);  // uint4 of one piece's staged q
  constexpr int NQ = kQStage / QU4 < 4 ? kQStage / QU4 : 4;
  static_assert(NQ >= 1, "q stage holds at least one piece");
  static_assert(kTileCap % WIN == 0, "tile list holds whole windows");
  constexpr int DEPTH = pkv::byte_codes(KVT) ? PKV_PIPE_DEPTH_FP8 : PKV_PIPE_DEPTH;
  constexpr bool NT = pkv::byte_codes(KVT) ? PKV_NT_FP8 : PKV_NT_16;

  __shared__ int sm_pref[pkv::kMaxStreamSeqs + 1];   // segment units before sequence s
  __shared__ int sm_ctx[pkv::kMaxStreamSeqs];        // clamped context lengths
  // per wave: closed pieces or partitions ([slot][head][D] accumulators,
  // [slot][head][2] (m, l), [slot] destination), the tile list of the
  // share's next steps, and the q rows of its first pieces
  __shared__ float sm_stash[kSkWaves * kStashFloats];
  __shared__ float sm_stml[kSkWaves * kStashSlots * 16 * 2];
  __shared__ int4 sm_meta[kSkWaves * kStashSlots];
  __shared__ int sm_tiles[kSkWaves * kTileCap];
  __shared__ uint4 sm_q[kSkWaves * kQStage];
  // APP: the new rows and slots of the pieces being staged (piece k in
  // place k % NQ)
  using NR = NewRow<QT, KVT, D>;
  __shared__ __align__(16) uint8_t sm_new[APP ? kSkWaves * NQ * NR::STAGE : 16];
  __shared__ int64_t sm_nslot[APP ? kSkWaves * NQ : 1];

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
    if constexpr (APP) {   // no piece reads the row, only the store remains
      const int64_t sl = p.slots[s];
      if (sl >= 0 && sl < (int64_t)p.nb * pkv::kBlockSize) {
        for (int hk = 0; hk < p.Hkv; ++hk) {
          uint32_t kr, vr, ke, ve;
          NR::load(p.kn, p.vn, (int64_t)s * p.Hkv + hk, lane, kr, vr);
          NR::encode(kr, vr, p.k_inv, p.v_inv, ke, ve);
          NR::store(const_cast<uint8_t*>(p.kc), const_cast<uint8_t*>(p.vc), sl, p.Hkv, hk, lane,
                    ke, ve);
        }
      }
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

  // The share piece by piece: a piece is the part of one segment's blocks
  // that lies in [u_lo, u_hi).  Segments follow each other in (sequence, y)
  // order; sequences without blocks own no segment.  A piece made of restart
  // units only has no block and is skipped.  Three walkers go over the same
  // pieces: one counts them, one feeds the tile list, one follows the
  // consumed blocks.
  struct Walk {
    int64_t u;
    int s, y, j;
    bool more;
  };
  struct Piece {
    int s, y, b, b1;
  };
  Walk w0;
  w0.u = u_lo;
  w0.more = true;
  locate(u_lo, w0.s, w0.y, w0.j);
  auto walk_next = [&](Walk& wv, Piece& pc) -> bool {
    while (wv.more) {
      const int p0 = __builtin_amdgcn_readfirstlane(sm_pref[wv.s]);
      const int len = __builtin_amdgcn_readfirstlane(sm_pref[wv.s + 1]) - p0;
      const int64_t seg_start = Y * p0 + (int64_t)wv.y * len;
      const int64_t pe = seg_start + len < u_hi ? seg_start + len : u_hi;
      int b, b1;
      if constexpr (PM) {
        // units are whole partitions: the piece is partitions [j, pe)
        const int nbk = (sm_ctx[wv.s] + 15) >> 4;
        b = wv.j * p.P;
        b1 = min((int)(pe - seg_start) * p.P, nbk);
      } else {
        b = max(wv.j - p.R, 0);
        b1 = max((int)(pe - seg_start) - p.R, 0);
      }
      const Piece found{wv.s, wv.y, b, b1};
      wv.u = pe;
      if (wv.u >= u_hi) {
        wv.more = false;
      } else {
        wv.j = 0;
        if (++wv.y == p.Y) {
          wv.y = 0;
          do {
            ++wv.s;
          } while (sm_pref[wv.s + 1] == sm_pref[wv.s]);
        }
      }
      if (b1 > b) {
        pc = found;
        return true;
      }
    }
    return false;
  };

  // ---- stash of closed pieces (partitions), written out at the end ----
  // A closed piece goes to LDS, not to memory, and the stash is written out
  // after the share's last block (or when full).  Writes mixed into the read
  // stream cost far more than their bytes: flushing every partition as it
  // closes made the 32K partitioned step 11% slower, and a fifth wave per
  // workgroup that wrote the stash out while the other four streamed made
  // it 12% slower, although no streaming wave then waited on a store.
  // Lane (G, c) stashes its own 4 * DPL accumulators (row c of the slot).
  const int HS = p.chunk_heads;
  const int slots = min(kStashSlots, kStashFloats / (HS * D));
  float* st = sm_stash + w * kStashFloats + c * D + DPL * 4 * G;
  float* stml = sm_stml + w * kStashSlots * 32 + 2 * c;
  int4* meta = sm_meta + w * kStashSlots;
  int n_st = 0;
  enum { kOut = 0, kPart = 1, kWsPart = 2 };
  // Written out row by row: a slot is HS rows of D floats in LDS, and every
  // lane takes 4 consecutive floats of it, so each store instruction writes
  // whole rows (the lanes' own 4 * DPL accumulators are scattered over 16
  // rows and would leave most lanes idle and most lines partly written).
  const float* stw = sm_stash + w * kStashFloats;
  const float* stmw = sm_stml + w * kStashSlots * 32;
  auto flush = [&]() {
    for (int k = 0; k < n_st; ++k) {
      const int4 mt = meta[k];
      const int kind = __builtin_amdgcn_readfirstlane(mt.x);
      const int s = __builtin_amdgcn_readfirstlane(mt.y);
      const int y = __builtin_amdgcn_readfirstlane(mt.z);
      const int idx = __builtin_amdgcn_readfirstlane(mt.w);
      const int hc = y % p.hchunks, hk = y / p.hchunks;
      const int nh = min(p.chunk_heads, p.g - hc * p.chunk_heads);
      const int64_t row0 = (int64_t)s * p.Hq + hk * p.g + hc * p.chunk_heads;   // first q-head
      for (int e = 4 * lane; e < nh * D; e += 256) {
        const int h = e / D, dim = e % D;
        const float4 a = *reinterpret_cast<const float4*>(stw + k * HS * D + e);
        const float m = stmw[k * 32 + 2 * h], l = stmw[k * 32 + 2 * h + 1];
        float4 sc;
        if constexpr (PC) {   // the caller's scale rows need only 4-byte alignment
          const float* vr = p.vs + (int64_t)hk * D + dim;
          sc = make_float4(vr[0], vr[1], vr[2], vr[3]);
        } else {
          sc = make_float4(p.vsc, p.vsc, p.vsc, p.vsc);
        }
        if (!PM && kind == kOut) {
          const float inv = l > 0.f ? (PC ? 1.f / l : p.vsc / l) : 0.f;
          if constexpr (PC)
            store_out4<QT>(p.out, (row0 + h) * D + dim, a.x * sc.x * inv, a.y * sc.y * inv,
                           a.z * sc.z * inv, a.w * sc.w * inv);
          else
            store_out4<QT>(p.out, (row0 + h) * D + dim, a.x * inv, a.y * inv, a.z * inv,
                           a.w * inv);
        } else if (PM) {
          const int64_t prow = (row0 + h) * p.num_parts + idx;
          *reinterpret_cast<float4*>(p.ws_acc + prow * D + dim) =
              make_float4(a.x * sc.x, a.y * sc.y, a.z * sc.z, a.w * sc.w);
          if (dim == 0) {
            p.ws_m[prow] = m;
            p.ws_l[prow] = l;
          }
        } else {
          const int64_t prow = (int64_t)idx * HS + h;
          *reinterpret_cast<float4*>(p.part + prow * D + dim) =
              make_float4(a.x * sc.x, a.y * sc.y, a.z * sc.z, a.w * sc.w);
          if (dim == 0) *reinterpret_cast<float2*>(p.ml + prow * 2) = make_float2(m, l);
        }
      }
    }
    n_st = 0;
  };

  f32x4 o[DPL];
  float m_run = kNegInf, l_run = 0.f;
  auto reset = [&]() {
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
  };
  // close the running state into the stash with its destination
  auto close = [&](int kind, int s, int y, int idx) {
    const float l_tot = wave_sum4(l_run);
    if (c < HS) {   // rows past the chunk would run into the next slot
      float* dst = st + n_st * HS * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DPL; ++e) dst[DPL * i + e] = o[e][i];
    }
    if (G == 0) {
      stml[n_st * 32] = m_run;
      stml[n_st * 32 + 1] = l_tot;
    }
    if (lane == 0) meta[n_st] = make_int4(kind, s, y, idx);
    if (++n_st == slots) flush();
    reset();
  };

  // ---- setup ----
  // The first K/V loads wait on the shares, the first piece and its block
  // ids; everything else (counting the share's pieces and blocks, the q rows
  // of later pieces) is done while those loads are in flight.
  Piece first;
  {
    Walk tw = w0;
    if (!walk_next(tw, first)) return;   // a share of restart units only
  }
  reset();

  if (p.nb == 0) {
    // no block id can be valid: every piece (partition) closes empty
    Walk tw = w0;
    Piece pc;
    int pi = 0;
    while (walk_next(tw, pc)) {
      if constexpr (PM) {
        for (int k = pc.b / p.P; k < (pc.b1 + p.P - 1) / p.P; ++k) close(kWsPart, pc.s, pc.y, k);
      } else {
        const int nbk = (sm_ctx[pc.s] + 15) >> 4;
        if (pc.b == 0 && pc.b1 == nbk) close(kOut, pc.s, pc.y, 0);
        else close(kPart, pc.s, pc.y, 2 * wk + (pi == 0 ? 0 : 1));
      }
      ++pi;
    }
    flush();
    return;
  }

  auto q_row = [&](const Piece& pc) {
    const int hc = pc.y % p.hchunks, hk = pc.y / p.hchunks;
    return (int64_t)pc.s * p.Hq + hk * p.g + hc * p.chunk_heads + c;
  };
  auto q_live = [&](const Piece& pc) {
    const int hc = pc.y % p.hchunks;
    return c < min(p.chunk_heads, p.g - hc * p.chunk_heads);
  };
  auto load_q_of = [&](const Piece& pc, uint4* qh, uint4* ql) {
    if constexpr (PC)
      T::load_q_scaled(qh, ql, p.q, q_row(pc), q_live(pc), G,
                       p.ks + (int64_t)(pc.y / p.hchunks) * D);
    else
      T::load_q(qh, p.q, q_row(pc), q_live(pc), G);
  };
  // the first piece's q rows go out with its block ids (the scaled form for
  // per-channel caches computes on them, so it waits until the first K/V
  // loads are out)
  uint4 qr[KS];
  uint4 qlo[PC ? KS : 1];
  if constexpr (!PC) load_q_of(first, qr, qlo);

  // ---- tile list: the share's steps as cache tile indices ----
  // tile = id * Hkv + hk for a valid block id, -1 for an invalid one (its
  // loads read tile 0 and it carries no weight).  Filled kTileCap steps at a
  // time by all lanes (lane t of window v: step 64 v + t), steps past the
  // share's end repeating its last one; read back a window of WIN steps at
  // a time into registers.
  int* tiles = sm_tiles + w * kTileCap;
  Walk lw = w0;
  Piece lp;
  bool lp_ok = walk_next(lw, lp);
  int lo_off = 0;
  uint32_t last_roff = 0;
  int last_hk = 0;
  // fills CAP steps (the first fill one window, so that the first loads go
  // out sooner; later ones the whole list); returns how many of the share's
  // steps it found
  auto fill = [&](auto cap) -> int {
    constexpr int CAP = decltype(cap)::value;
    constexpr int NV = CAP / 64;
    uint32_t roff[NV];
    int hkv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      roff[v] = 0;
      hkv[v] = 0;
    }
    int acc = 0;
    while (lp_ok && acc < CAP) {
      const int L = lp.b1 - lp.b - lo_off;
      const int take = min(L, CAP - acc);
      // step t of this fill (acc <= t < acc + take) is block lp.b + lo_off + t - acc
      const uint32_t base = (uint32_t)lp.s * (uint32_t)p.mb + (uint32_t)(lp.b + lo_off) - (uint32_t)acc;
      const int hkp = lp.y / p.hchunks;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int t = 64 * v + lane;
        if (t >= acc && t < acc + take) {
          roff[v] = base + (uint32_t)t;
          hkv[v] = hkp;
        }
      }
      last_roff = base + (uint32_t)(acc + take - 1);
      last_hk = hkp;
      acc += take;
      lo_off += take;
      if (lo_off == lp.b1 - lp.b) {
        lo_off = 0;
        lp_ok = walk_next(lw, lp);
      }
    }
    int id[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int t = 64 * v + lane;
      if (t >= acc) {
        roff[v] = last_roff;
        hkv[v] = last_hk;
      }
      id[v] = p.bt[roff[v]];
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
      tiles[64 * v + lane] = (unsigned)id[v] < (unsigned)p.nb ? id[v] * p.Hkv + hkv[v] : -1;
    return acc;
  };
  int idw[NW];
  int wk0 = 0, fill_base = 0;
  auto read_window = [&]() {
#pragma unroll
    for (int v = 0; v < NW; ++v) idw[v] = tiles[wk0 - fill_base + 64 * v + lane];
  };
  const int filled = fill(std::integral_constant<int, WIN>{});
  int fe = WIN;
  read_window();
  // The share's step count: known now when the first fill took all of it,
  // else at least WIN (> DEPTH) and counted below.
  int total = lp_ok ? INT32_MAX : filled;

  // tile of the next step to issue (steps past the end repeat the last)
  int kiss = 0;
  auto next_tile = [&]() -> int {
    const int k = min(kiss, total - 1);
    ++kiss;
    if (k >= wk0 + WIN) {
      wk0 += WIN;
      if (wk0 == fe) {
        fill_base = fe;
        fill(std::integral_constant<int, kTileCap>{});
        fe += kTileCap;
      }
      read_window();
    }
    const int i = k - wk0;
    int v = __builtin_amdgcn_readlane(idw[0], i & 63);
#pragma unroll
    for (int vv = 1; vv < NW; ++vv) {
      const int x = __builtin_amdgcn_readlane(idw[vv], i & 63);
      v = (i >> 6) == vv ? x : v;
    }
    return v;
  };

  const uint32_t koff = T::k_lane_off(c, G), voff = T::v_lane_off(c, G);
  auto issue = [&](Raw& r, int tile) {
    const int64_t a = (int64_t)(tile < 0 ? 0 : tile) * T::TILE;
    T::template issue<NT>(r, p.kc + a, p.vc + a, koff, voff);
  };

  Raw buf[DEPTH];
  int idc[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    idc[d] = next_tile();
    issue(buf[d], idc[d]);
    // keep the blocks' loads in consumption order
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- with the first loads in flight ----
  if constexpr (PC) load_q_of(first, qr, qlo);
  // the share's pieces and steps, and the q rows of its first pieces after
  // the first, staged in LDS
  int npieces = 0;
  Piece pq[NQ];
  {
    Walk tw = w0;
    Piece pc;
    int t = 0;
    while (walk_next(tw, pc)) {
#pragma unroll
      for (int i = 0; i < NQ; ++i)
        if (npieces == i) pq[i] = pc;
      ++npieces;
      t += pc.b1 - pc.b;
    }
    total = t;
  }
  const int nq = min(npieces, NQ);
  // APP: the new rows of the first pieces: loaded here, ahead of the q rows
  // of the staging below, unconditionally (places past the share's pieces
  // repeat the first), so that no branch leaves the load counter's order
  // unknown; encoded and staged in LDS after the q rows
  // (the places live in LDS, addressed from the wave index, so that the
  // block loop carries no more than one scalar for them: the slot's tile)
  [[maybe_unused]] auto place_row = [&](int k) { return sm_new + (w * NQ + k) * NR::STAGE; };
  [[maybe_unused]] auto place_slot = [&](int k) {
    const int64_t v = sm_nslot[w * NQ + k];
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
  };
  [[maybe_unused]] uint32_t nkr[APP ? NQ : 1], nvr[APP ? NQ : 1];
  [[maybe_unused]] int64_t nsl_r[APP ? NQ : 1];
  [[maybe_unused]] Piece pcs[APP ? NQ : 1];
  if constexpr (APP) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i < nq) pcs[i] = pq[i];
      else pcs[i] = pq[0];
      nsl_r[i] = p.slots[pcs[i].s];
      NR::load(p.kn, p.vn, (int64_t)pcs[i].s * p.Hkv + pcs[i].y / p.hchunks, lane, nkr[i],
               nvr[i]);
    }
  }
  // piece pc's new row (raw elements kr, vr; slot sl) into place k; the
  // piece holding the last block of its sequence's kv-head (head chunk 0)
  // also stores it to the slot
  // (real = false: only the row is staged, into a place no piece reads)
  [[maybe_unused]] auto stage_piece = [&](const Piece& pc, int k, uint32_t kr, uint32_t vr,
                                          int64_t sl, bool real = true) {
    uint32_t ke, ve;
    NR::encode(kr, vr, p.k_inv, p.v_inv, ke, ve);
    NR::stage(place_row(k), lane, ke, ve);
    if (!real) return;
    if (lane == 0) sm_nslot[w * NQ + k] = sl;
    if (pc.y % p.hchunks == 0 && pc.b1 == (sm_ctx[pc.s] + 15) >> 4 && sl >= 0 &&
        sl < (int64_t)p.nb * pkv::kBlockSize)
      NR::store(const_cast<uint8_t*>(p.kc), const_cast<uint8_t*>(p.vc), sl, p.Hkv,
                pc.y / p.hchunks, lane, ke, ve);
  };
  uint4* qs = sm_q + w * kQStage;
#pragma unroll
  for (int i = 1; i < NQ; ++i)
    if (i < nq) {
      uint4 qt[KS];
      uint4 qtl[PC ? KS : 1];
      load_q_of(pq[i], qt, qtl);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        qs[(i * KS + k) * 64 + lane] = qt[k];
        if constexpr (PC) qs[((NQ + i) * KS + k) * 64 + lane] = qtl[k];
      }
    }

  // APP: the new rows of the first pieces, staged in LDS (their loads went
  // out before the q rows above).  Every place is written, so that every
  // load is consumed here: a load left unconsumed on some paths would still
  // count as in flight in the block loop, which would then wait for it.
  if constexpr (APP) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) stage_piece(pcs[i], i, nkr[i], nvr[i], nsl_r[i], i < nq);
  }

  // ---- the consumed piece ----
  Walk cw = w0;
  Piece cur;
  walk_next(cw, cur);
  int pi = 0;          // index of the current piece
  int cb = cur.b;      // block of the segment consumed next
  int c_last = ((sm_ctx[cur.s] + 15) >> 4) - 1;
  int c_tail = sm_ctx[cur.s] - 16 * c_last;
  int rem = PM ? p.P : 0;   // blocks left in the current partition
  // APP: the tile index of the current piece's slot block (-2, which no
  // tile has, when there is no row); its row and slot sit in place pi % NQ
  [[maybe_unused]] int cur_tile = -2;
  [[maybe_unused]] auto take_row = [&](int k) {
    const int64_t sl = place_slot(k);
    const bool ok = sl >= 0 && sl < (int64_t)p.nb * pkv::kBlockSize;
    cur_tile = ok ? (int)(sl >> 4) * p.Hkv + cur.y / p.hchunks : -2;
  };
  if constexpr (APP) take_row(0);

  // step kc from slot d: consume, then close / switch pieces as due
  int kc = 0;
  auto consume_step = [&](int d) {
    const bool live = kc < total;
    const int valid = live && idc[d] >= 0 ? (cb == c_last ? c_tail : 16) : 0;
    if constexpr (APP) {
      if (idc[d] == cur_tile) {
        const int k = pi % NQ;
        NR::sub(buf[d], place_row(k), (int)(place_slot(k) & 15), lane);
      }
    }
    T::template consume<1, PC, false>(buf[d], valid, valid == 16, nullptr, 0, qr, p.sl2, &m_run,
                                      &l_run, o, c, G, qlo);
    if (live) {
      ++cb;
      if constexpr (PM) {
        if (--rem == 0 || cb == cur.b1) {
          close(kWsPart, cur.s, cur.y, (cb - 1) / p.P);
          rem = p.P;
        }
      }
      if (cb == cur.b1) {
        if constexpr (!PM) {
          if (cur.b == 0 && cur.b1 == c_last + 1) close(kOut, cur.s, cur.y, 0);
          else close(kPart, cur.s, cur.y, 2 * wk + (pi == 0 ? 0 : 1));
        }
        if (++pi < npieces) {
          walk_next(cw, cur);
          cb = cur.b;
          c_last = ((sm_ctx[cur.s] + 15) >> 4) - 1;
          c_tail = sm_ctx[cur.s] - 16 * c_last;
          if (pi < NQ) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
              qr[k] = qs[(pi * KS + k) * 64 + lane];
              if constexpr (PC) qlo[k] = qs[((NQ + pi) * KS + k) * 64 + lane];
            }
          } else {
            load_q_of(cur, qr, qlo);
            [[maybe_unused]] uint32_t kr = 0u, vr = 0u;
            [[maybe_unused]] int64_t sl = -1;
            if constexpr (APP) {
              sl = p.slots[cur.s];
              NR::load(p.kn, p.vn, (int64_t)cur.s * p.Hkv + cur.y / p.hchunks, lane, kr,
                       vr);
            }

            // wait here: q registers left in flight on this rare path would
            // make every later block wait for the newest loads
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
            if constexpr (APP) stage_piece(cur, pi % NQ, kr, vr, sl);
          }
          if constexpr (APP) take_row(pi % NQ);
        }
      }
    }
    ++kc;
  };

  // Groups of DEPTH steps.  While the share has steps beyond the group's
  // loads, every step issues the loads of the step DEPTH ahead (past the
  // share's end they repeat its last tile), and a group runs to its end
  // (a step past the end consumes nothing): a branch that skipped an issue
  // would join the loop again and make the compiler wait for the newest
  // loads at every block.  The last group issues nothing, so that nothing
  // is left in flight when the stash is written out.
  while (kc + DEPTH < total) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      consume_step(d);
      const int tn = next_tile();
      issue(buf[d], tn);
      idc[d] = tn;
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) consume_step(d);
  flush();
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
  if (sp.kn)
    return pkv::launch_kernel(decode_stream_kernel<QT, KVT, D, false, PM, true>, dim3(grid), block,
                              a.stream, sp, a.ev_start, a.ev_stop);
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
  sp.R = pkv::stream_restart_units(a.kv_dtype);
  sp.ks = kp.ks;
  sp.vs = kp.vs;
  sp.P = 0;
  sp.num_parts = 0;
  sp.ws_m = sp.ws_l = sp.ws_acc = nullptr;
  sp.kn = kp.kn;
  sp.vn = kp.vn;
  sp.slots = kp.slots;
  sp.k_inv = kp.k_inv;
  sp.v_inv = kp.v_inv;
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
