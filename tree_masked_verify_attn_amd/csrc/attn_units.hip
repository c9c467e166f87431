// bf16 tree-masked verify/expand attention over balanced units of work
// (gfx950), for batches whose sequences differ in length.
//
// Same mathematics and MFMA formulation as attn_stream.hip (SwiftSpec summary,
// Section 3.1.3 Figure 3 and Section 3.2; split heads combined as in
// Section 3.3), but the work is cut differently:
//  * The tiles (32 KV positions) of every job (sequence, row tile, KV head)
//    are laid end to end in one stream: sequences outermost, then KV heads,
//    then row tiles.  Neighbouring ranges then read the same sequence's
//    blocks, whose rows interleave the KV heads (measured 2 us faster on the
//    paged alternating batches than KV heads outermost, 126.0 against 128.0
//    and 128.5 us).  Each job also counts kJobCost tiles that are never loaded:
//    what a job costs beyond its tiles (its mask set-up, the change of job,
//    a partly filled last tile), so that a range of many short jobs holds
//    fewer tiles.  With N such units and G work groups, group g takes the
//    contiguous range [g*U, (g+1)*U), U = ceil(N / G): every group gets the
//    same amount of work whatever the length mix, and all G groups are
//    resident at once (two per compute unit).
//  * A range holds pieces of one or more jobs ("segments").  The LDS-DMA ring
//    runs across segment boundaries: the loads of the next segment's first
//    stages are in flight while the current one finishes, so a group pays
//    the ring's start-up latency once, not once per piece.  At a boundary only
//    the compute side changes job (results out, state reset, next queries in).
//  * A segment that covers a whole job writes the final rows.  A job cut by a
//    range boundary leaves one partial (max, sum, output) state per group it
//    touches, in slot 2g (the piece that starts the group's range) or 2g + 1
//    (the piece that ends it), in half precision (partial_f16.h); the combine
//    launch (merge_units_kernel) adds them up.
//  * Segments are set up in batches (at most kMaxSeg segments, a few of them
//    reaching a tree cache, kUnitBlocks paged block ids); a group whose
//    range needs more drains the ring and sets up the next batch, carrying
//    the running state of a job cut by the batch boundary.
#include "stream_common.h"

namespace ta {
namespace {

constexpr int kMaxSeg = 16;
constexpr int kJobCost = kUnitJobCost;
constexpr int kUnitBlocks = 512;
// Row masks of the segments that reach a tree cache: as many as fit in 12 KiB.
template <int RPT>
constexpr int max_tree_seg() {
  return 12288 / (RPT * 32) < 8 ? 12288 / (RPT * 32) : 8;
}
constexpr int kS = 4;  // ring stages

// Segment flags.
constexpr int kContPrev = 1;       // continues the previous batch's last segment
constexpr int kContNext = 2;       // continues into the next batch
constexpr int kFromJobStart = 4;   // the job's first tile is in this (logical) segment
constexpr int kToJobEnd = 8;       // the job's last tile is in this segment
constexpr int kFromRangeStart = 16;  // the segment starts at the group's first tile

struct USeg {
  int b, rtile, hkv;
  int j0, j1;           // batch-local tiles [j0, j1)
  int t_begin, t_end;   // KV positions of sequence b covered by [j0, j1)
  int P, n;
  int blk0, blk_off;    // paged: t_begin / block_size and where its ids start in sBlk
  int tree;             // row-mask table index, or -1
  int flags;
};

// Stream geometry of sequence b (shared with the combine launch).
struct SeqJobs {
  int P, n, T;
  int tiles;   // ceil(T / 32), 0 for a sequence with nothing to do
  int rt_lo;   // first row tile with a valid row
  int rts;     // row tiles with valid rows (jobs per KV head)
};
// (from the raw prefix_len[b] and n_nodes[b])
__device__ __forceinline__ SeqJobs seq_jobs_of(const AttnParams& p, int P_raw, int n_raw, int RPT) {
  SeqJobs s{0, 0, 0, 0, 0, 0};
  SeqBounds sb;
  if (!seq_bounds_of(P_raw, n_raw, p.n_max, p.T_cap, sb)) return s;
  const int R = p.n_q * p.G;
  int r_lo = 0, r_hi = R;
  if (p.expand) {
    const int fs = p.n_q - sb.n;  // first query slot holding an existing node
    r_lo = fs > 0 ? fs * p.G : 0;
  } else {
    r_hi = min(sb.n, p.n_q) * p.G;
  }
  if (r_lo >= r_hi) return s;
  s.P = sb.P;
  s.n = sb.n;
  s.T = sb.T;
  s.tiles = (sb.T + kTile - 1) / kTile;
  s.rt_lo = r_lo / RPT;
  s.rts = (r_hi + RPT - 1) / RPT - s.rt_lo;
  return s;
}
__device__ __forceinline__ SeqJobs seq_jobs(const AttnParams& p, int b, int RPT) {
  return seq_jobs_of(p, p.prefix_len[b], p.n_nodes[b], RPT);
}

template <int D, int NRG>
__global__ __launch_bounds__(kThreads, 2) void attn_units_kernel(AttnParams p) {
  using C = SCfg<D, NRG, kS>;
  constexpr int RPT = C::RPT;
  constexpr int kMaxTreeSeg = max_tree_seg<RPT>();
  // With at most two row groups the two other waves issue every ring load, so
  // the computing waves' own load counter sees only their query loads: the
  // next job's queries can be fetched while the current job's last tile is
  // consumed and waited for without draining the ring.
  constexpr int kDmaWaves = NRG <= 2 ? 2 : 4;
  constexpr int kInst = C::HALF / 1024 / kDmaWaves;  // 1 KiB loads per loading wave, K or V
  constexpr int kNL = 2 * kInst;                    // loads per loading wave per stage
  static_assert(C::HALF % (1024 * kDmaWaves) == 0, "stage split over the loading waves");
  // Between batches the ring's LDS holds the set-up tables: per sequence its
  // stream start and geometry; later the tree segments' parents and one
  // ancestor table.
  static_assert(6 * (kUnitMaxSeqs + 1) * 4 <= C::RING, "sequence tables must fit in the ring");
  static_assert(kMaxTreeSeg * kMaxNodes * 4 + kMaxNodes * (kMaskWords * 8 + 4) <= C::RING,
                "tree set-up tables must fit in the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t sRing[C::RING];
  __shared__ int sBlk[kUnitBlocks];
  __shared__ USeg sSeg[kMaxSeg];
  __shared__ uint64_t sRowMask[kMaxTreeSeg][RPT][kMaskWords];
  __shared__ int sScan[kThreads / 64];
  __shared__ int sNumSeg, sBatchTiles, sNext;

  const int g = blockIdx.x;
  const int G = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lhi = lane >> 5;
  const int l32 = lane & 31;
  const int rg = wave < NRG ? wave : -1;           // computing waves own a 32-row group
  const bool loader = wave >= 4 - kDmaWaves;        // waves that issue ring loads
  const int dma_rank = wave - (4 - kDmaWaves);      // index among the loading waves
  const int row_in_tile = (rg < 0 ? 0 : rg) * 32 + l32;
  const int B = p.B;
  const int bs = p.block_size;
  // block sizes that are powers of two (16 in the usual serving layouts) split
  // a position into (block, row) with a shift and a mask
  const int bs_shift = (bs & (bs - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(bs)) : -1;
  const bool paged = p.block_table != nullptr;

  // per sequence: start of its tiles (all KV heads) in the stream
  int* sS = reinterpret_cast<int*>(sRing);  // [B + 1]
  int* sTiles = sS + (kUnitMaxSeqs + 1);
  int* sRtlo = sTiles + (kUnitMaxSeqs + 1);
  int* sP = sRtlo + (kUnitMaxSeqs + 1);
  int* sN = sP + (kUnitMaxSeqs + 1);
  int* sRts = sN + (kUnitMaxSeqs + 1);

  // ---- the stream: per-sequence tiles and starts (four sequences per thread) ----
  auto load_stream = [&]() -> int {
    int cnt[4];
    int tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = 4 * tid + k;
      cnt[k] = 0;
      if (b < B) {
        const SeqJobs s = seq_jobs(p, b, RPT);
        cnt[k] = s.tiles > 0 ? p.Hkv * s.rts * (s.tiles + kJobCost) : 0;
        sTiles[b] = s.tiles;
        sRts[b] = s.rts;
        sRtlo[b] = s.rt_lo;
        sP[b] = s.P;
        sN[b] = s.n;
      }
      tot += cnt[k];
    }
    // exclusive scan of the threads' totals
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) sScan[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += sScan[w];
    int run = before + incl - tot;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = 4 * tid + k;
      if (b < B) sS[b] = run;
      run += cnt[k];
    }
    int total = 0;
    for (int w = 0; w < kThreads / 64; ++w) total += sScan[w];
    if (tid == 0) sS[B] = total;
    __syncthreads();
    return total;
  };

  int Sh = load_stream();  // stream units (all KV heads)
  if (g == 0) {  // the combine launch reads, per sequence, one 16-byte record
    for (int b = tid; b < B; b += kThreads)
      reinterpret_cast<int4*>(p.ws_seq)[b] = int4{sS[b], sS[B], sP[b], sN[b]};
  }
  const int N = Sh;
  const int U = (N + G - 1) / G;
  const int x0 = g * U;
  const int x1 = min(N, x0 + U);
  if (x0 >= x1) return;  // uniform

  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const uint8_t* Kg = static_cast<const uint8_t*>(p.k);
  const uint8_t* Vg = static_cast<const uint8_t*>(p.v);
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_u8*)sRing));
  const float cs = p.scale_log2;

  // running state of the current job piece (computing waves)
  f32x16 acc[C::MB];
  float m_ref = -INFINITY, l_sum = 0.f;
  bf16x8 qreg[C::KS];
  int slot = 0, gq = 0, node = -1;
  int from_job_start = 0, from_range_start = 0;  // of the current logical segment

  int x = x0;  // next stream tile to set up
  bool first_batch = true;
  while (x < x1) {
    if (!first_batch) load_stream();  // the ring overwrote the tables
    first_batch = false;

    // ---- batch set-up: segments (one thread), block ids, row masks ----
    if (tid == 0) {
      // sequence holding tile x: the last b with sS[b] <= x
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sS[mid] <= x) lo = mid; else hi = mid - 1;
      }
      int b = lo;
      int k = 0, jl = 0, nblk = 0, ntree = 0;
      int xs = x;
      while (xs < x1 && k < kMaxSeg) {
        while (b < B && sS[b + 1] <= xs) ++b;  // skip sequences with no tiles
        const int tiles = sTiles[b];
        const int stride = tiles + kJobCost;  // a job's units in the stream
        const int per_head = sRts[b] * stride;
        const int off0 = xs - sS[b];
        const int hkv = off0 / per_head;
        const int off = off0 - hkv * per_head;
        const int job = off / stride;  // row tile within the sequence
        const int jt = off - job * stride;
        if (jt >= tiles) {  // the job's cost units: nothing to load
          xs = min(x1, xs + stride - jt);
          continue;
        }
        int take = min(tiles - jt, x1 - xs);
        const int P = sP[b], n = sN[b], T = P + n;
        const int tb = jt * kTile;
        int te = min(T, (jt + take) * kTile);
        if (paged) {
          const int blk0 = tb / bs;
          int need = (te - 1) / bs - blk0 + 1;
          if (nblk + need > kUnitBlocks) {  // keep the whole tiles whose blocks fit
            const int fit = ((blk0 + kUnitBlocks - nblk) * bs - tb) / kTile;
            if (fit <= 0) break;
            take = min(take, fit);
            te = min(T, (jt + take) * kTile);
          }
        }
        const bool tree = te > P;
        if (tree && ntree == kMaxTreeSeg) break;
        USeg s;
        s.b = b;
        s.rtile = sRtlo[b] + job;
        s.hkv = hkv;
        s.j0 = jl;
        s.j1 = jl + take;
        s.t_begin = tb;
        s.t_end = te;
        s.P = P;
        s.n = n;
        s.blk0 = paged ? tb / bs : 0;
        s.blk_off = nblk;
        s.tree = tree ? ntree++ : -1;
        int f = 0;
        if (k == 0 && xs > x0 && jt > 0) f |= kContPrev;
        if (jt == 0) f |= kFromJobStart;
        if (jt + take == tiles) f |= kToJobEnd;
        if (xs == x0) f |= kFromRangeStart;
        if (jt + take < tiles && xs + take < x1) f |= kContNext;
        s.flags = f;
        sSeg[k] = s;
        if (paged) nblk += (te - 1) / bs - tb / bs + 1;
        jl += take;
        xs += take;
        if (jt + take == tiles) xs = min(x1, xs + kJobCost);  // past the job's cost units
        ++k;
      }
      sNumSeg = k;
      sBatchTiles = jl;
      sNext = xs;
    }
    __syncthreads();
    const int nseg = sNumSeg;
    const int L = sBatchTiles;
    x = sNext;
    if (nseg == 0) continue;  // uniform: the rest of the range held cost units only
    // Block ids (paged) and the parents of the segments that reach a tree
    // cache, in one round of loads (the sequence tables are done with).
    int* sPar = reinterpret_cast<int*>(sRing);  // [kMaxTreeSeg][kMaxNodes]
    auto sAnc = reinterpret_cast<uint64_t(*)[kMaskWords]>(sRing + kMaxTreeSeg * kMaxNodes * 4);
    int* sJump = reinterpret_cast<int*>(sRing + kMaxTreeSeg * kMaxNodes * 4 + kMaxNodes * kMaskWords * 8);
    {
      static_assert(kUnitBlocks <= 2 * kThreads, "two block ids per thread");
      int nb = 0;
      if (paged)
        for (int k = 0; k < nseg; ++k) nb += (sSeg[k].t_end - 1) / bs - sSeg[k].blk0 + 1;
      int bv[2] = {0, 0};
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = tid + r * kThreads;
        if (i < nb) {
          int k = 0;
          while (k + 1 < nseg && sSeg[k + 1].blk_off <= i) ++k;
          bv[r] = p.block_table[static_cast<size_t>(sSeg[k].b) * p.max_blocks + sSeg[k].blk0 +
                                (i - sSeg[k].blk_off)];
        }
      }
      int pv[kMaxTreeSeg];
#pragma unroll
      for (int t = 0; t < kMaxTreeSeg; ++t) pv[t] = -1;
      for (int k = 0; k < nseg; ++k) {
        const int tr = sSeg[k].tree;
#pragma unroll
        for (int t = 0; t < kMaxTreeSeg; ++t)
          if (tr == t && tid < sSeg[k].n)
            pv[t] = p.parent[static_cast<size_t>(sSeg[k].b) * p.n_max + tid];
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = tid + r * kThreads;
        if (i < nb) sBlk[i] = bv[r] < 0 ? 0 : (bv[r] >= p.num_blocks ? p.num_blocks - 1 : bv[r]);
      }
#pragma unroll
      for (int t = 0; t < kMaxTreeSeg; ++t) sPar[t * kMaxNodes + tid] = pv[t];
    }
    __syncthreads();
    for (int k = 0; k < nseg; ++k) {
      const int tr = sSeg[k].tree;  // uniform
      if (tr < 0) continue;
      const int n = sSeg[k].n, rtile = sSeg[k].rtile;
      build_ancestor_masks(sPar + tr * kMaxNodes, n, sAnc, sJump);
      for (int r = tid; r < RPT; r += kThreads) {
        const int grow = rtile * RPT + r;
        int nd = -1;
        if (grow < p.n_q * p.G) {
          const int sl = grow / p.G;
          nd = p.expand ? n - p.n_q + sl : sl;
          if (nd < 0 || nd >= n) nd = -1;
        }
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) sRowMask[tr][r][w] = nd >= 0 ? sAnc[nd][w] : 0ull;
      }
      __syncthreads();
    }
    __syncthreads();  // the ring may now overwrite the tables

    // ---- segment state ----
    // compute side: the segment of the tile being consumed
    int kc = 0;
    int c_j1, c_tb0, c_te, c_P, c_tree, c_flags, c_b, c_hkv;
    auto load_c = [&](int k) {
      c_j1 = __builtin_amdgcn_readfirstlane(sSeg[k].j1);
      c_tb0 = __builtin_amdgcn_readfirstlane(sSeg[k].t_begin - sSeg[k].j0 * kTile);
      c_te = __builtin_amdgcn_readfirstlane(sSeg[k].t_end);
      c_P = __builtin_amdgcn_readfirstlane(sSeg[k].P);
      c_tree = __builtin_amdgcn_readfirstlane(sSeg[k].tree);
      c_flags = __builtin_amdgcn_readfirstlane(sSeg[k].flags);
      c_b = __builtin_amdgcn_readfirstlane(sSeg[k].b);
      c_hkv = __builtin_amdgcn_readfirstlane(sSeg[k].hkv);
    };
    // issue side: the segment of the next stage to load
    int ki = 0;
    int i_j1, i_tb0, i_te, i_b, i_hkv, i_blk0, i_blkoff;
    auto load_i = [&](int k) {
      i_j1 = __builtin_amdgcn_readfirstlane(sSeg[k].j1);
      i_tb0 = __builtin_amdgcn_readfirstlane(sSeg[k].t_begin - sSeg[k].j0 * kTile);
      i_te = __builtin_amdgcn_readfirstlane(sSeg[k].t_end);
      i_b = __builtin_amdgcn_readfirstlane(sSeg[k].b);
      i_hkv = __builtin_amdgcn_readfirstlane(sSeg[k].hkv);
      i_blk0 = __builtin_amdgcn_readfirstlane(sSeg[k].blk0);
      i_blkoff = __builtin_amdgcn_readfirstlane(sSeg[k].blk_off);
    };
    load_c(0);
    load_i(0);

    // Issues stage j (the stages are issued in order) into ring slot `sl`.
    // Every address of the stage first (a paged stage reads its block ids
    // from LDS in one round), then the loads: the DMA's memory clobber would
    // otherwise hold each block-id read behind the previous row's loads.
    auto issue_stage = [&](int j, int sl) {
      if (!loader) return;  // wave-uniform
      while (j >= i_j1) load_i(++ki);  // uniform; ki < nseg since j < L
      const uint32_t sbase = ring_base + sl * C::STAGE;
      const int tb = i_tb0 + j * kTile;
      size_t off[kInst];
      auto addresses = [&](auto pow2_tag) {
#pragma unroll
        for (int q = 0; q < kInst; ++q) {
          const int r = (dma_rank * kInst + q) * C::ROWS_PER_INST + lane / C::CH;
          const int c = (lane % C::CH) ^ swz<D>(r);
          int tok = tb + r;
          tok = tok < i_te ? tok : i_te - 1;
          size_t row;
          if (paged) {
            int bi, in;
            if constexpr (decltype(pow2_tag)::value) {
              bi = tok >> bs_shift;
              in = tok & (bs - 1);
            } else {
              bi = tok / bs;
              in = tok - bi * bs;
            }
            const int blk = sBlk[i_blkoff + bi - i_blk0];
            row = (static_cast<size_t>(blk) * bs + in) * p.Hkv + i_hkv;
          } else {
            row = (static_cast<size_t>(i_b) * p.T_cap + tok) * p.Hkv + i_hkv;
          }
          off[q] = row * C::ROW + c * 16;
        }
      };
      if (bs_shift >= 0) addresses(std::true_type{});
      else addresses(std::false_type{});
#pragma unroll
      for (int q = 0; q < kInst; ++q) {
        const int r0 = (dma_rank * kInst + q) * C::ROWS_PER_INST;
        const uint32_t lk = __builtin_amdgcn_readfirstlane(sbase + r0 * C::ROW);
        dma16(Kg + off[q], lk);
        dma16(Vg + off[q], lk + C::HALF);
      }
    };

    // Rows of segment k's job: row -> (query slot, head), node (-1: none).
    auto rows_of = [&](int k, int& sl_, int& g_, int& nd_) {
      const int grow = __builtin_amdgcn_readfirstlane(sSeg[k].rtile) * RPT + row_in_tile;
      const int n = __builtin_amdgcn_readfirstlane(sSeg[k].n);
      nd_ = -1;
      sl_ = 0;
      g_ = 0;
      if (rg >= 0 && grow < p.n_q * p.G) {
        sl_ = grow / p.G;
        g_ = grow % p.G;
        nd_ = p.expand ? n - p.n_q + sl_ : sl_;
        if (nd_ < 0 || nd_ >= n) nd_ = -1;
      }
    };
    auto set_rows = [&]() { rows_of(kc, slot, gq, node); };
    // Queries of the rows (sl_, g_, nd_) of job (b_, h_) into qreg.
    auto issue_q = [&](int b_, int h_, int sl_, int g_, int nd_) {
      const size_t qrow = ((static_cast<size_t>(b_) * p.n_q + sl_) * p.Hq + h_ * p.G + g_) * D;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (nd_ >= 0) v = *reinterpret_cast<const u32x4*>(Q + qrow + (2 * ks + lhi) * 8);
        qreg[ks] = __builtin_bit_cast(bf16x8, v);
      }
    };
    auto load_q = [&]() {
      issue_q(c_b, c_hkv, slot, gq, node);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every load of this wave done
    };
    auto reset_state = [&]() {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
      m_ref = -INFINITY;
      l_sum = 0.f;
    };
    // A new logical segment starts (not the continuation of the previous batch's).
    auto begin_segment = [&]() {
      from_job_start = (c_flags & kFromJobStart) != 0;
      from_range_start = (c_flags & kFromRangeStart) != 0;
      if (rg >= 0) {
        set_rows();
        reset_state();
        load_q();
      }
    };
    // Results of the compute-side segment, which ends here.
    auto end_segment = [&]() {
      if (rg < 0) return;  // wave-uniform
      if (from_job_start && (c_flags & kToJobEnd)) {  // the whole job: final rows
        if (node < 0) return;
        uint16_t* Out = static_cast<uint16_t*>(p.out);
        const size_t orow = ((static_cast<size_t>(c_b) * p.n_q + slot) * p.Hq + c_hkv * p.G + gq) * D;
        const float inv = 1.f / l_sum;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * mb + 8 * q4 + 4 * lhi;
            const uint32_t lo = f32_to_bf16_bits(acc[mb][4 * q4 + 0] * inv) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(acc[mb][4 * q4 + 1] * inv)) << 16);
            const uint32_t hi = f32_to_bf16_bits(acc[mb][4 * q4 + 2] * inv) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(acc[mb][4 * q4 + 3] * inv)) << 16);
            *reinterpret_cast<u32x2*>(Out + orow + d) = u32x2{lo, hi};
          }
        if (p.lse != nullptr && lhi == 0) {
          const size_t lrow = (static_cast<size_t>(c_b) * p.Hq + c_hkv * p.G + gq) * p.n_q + slot;
          p.lse[lrow] = (m_ref + log2f(l_sum)) * kLn2;
        }
        return;
      }
      // a piece of a cut job: its partial state in slot 2g or 2g + 1
      const int e = partial_exp(acc);  // every lane of the wave
      if (node < 0) return;
      const size_t pr = (2 * static_cast<size_t>(g) + (from_range_start ? 0 : 1)) * RPT + row_in_tile;
      store_partial_f16(acc, m_ref, l_sum, e, lhi, reinterpret_cast<uint16_t*>(p.ws_o) + pr * D,
                        reinterpret_cast<PartialRec*>(p.ws_ml) + pr);
    };

    // S^T = K . Q^T for the tile in ring slot `sl`.
    auto qk = [&](int sl) -> f32x16 {
      const uint8_t* sK = sRing + sl * C::STAGE;
      f32x16 Sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) Sc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sK + lds_off<D>(l32, 2 * ks + lhi));
        Sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qreg[ks], Sc,
                                                     0, 0, 0);
      }
      return Sc;
    };
    int v_base_p, v_base_m;
    {
      const int gi = lane >> 4, jl = lane & 15;
      const int xx = (jl >> 3) & 1;
      const int s_lo = (((jl >> 2) & 1) << 1) | ((gi >> 1) & 1);
      const int y = (2 * (gi & 1) + ((jl & 3) >> 1)) ^ s_lo;
      const int Lb = (4 * (gi >> 1) + (jl >> 2)) * C::ROW + 16 * y + 8 * (jl & 1);
      v_base_p = Lb + 64 * xx;
      v_base_m = Lb - 64 * xx;
    }
    // Mask (tiles that reach the tree cache or the segment's end), online
    // softmax and O^T += V^T . P^T for the tile at positions tb.. in slot sl.
    auto softmax_pv = [&](f32x16 Sc, int tb, int sl, auto masked_tag) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      const uint8_t* sV = sRing + sl * C::STAGE + C::HALF;
      if constexpr (kMasked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = tb + 8 * (r >> 2) + 4 * lhi + (r & 3);
          const int jj = t - c_P;
          const bool tree_col = jj >= 0 && t < c_te && c_tree >= 0;
          const uint64_t word = tree_col ? sRowMask[c_tree < 0 ? 0 : c_tree][row_in_tile][jj >> 6] : 0ull;
          const bool in_tree = ((word >> (jj & 63)) & 1ull) != 0ull;
          const bool vis = t < c_te && (jj < 0 || in_tree);
          if (!vis) Sc[r] = -INFINITY;
        }
      }
      float mx = Sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, Sc[r]);
      mx = halves_max(mx) * cs;
      const bool bump = mx > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(bump) != 0ull) {
        const float m_new = bump ? mx : m_ref;
        const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
        l_sum *= alpha;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
        m_ref = m_new;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      float rs = 0.f;
      bf16x8 pk[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(Sc[r], cs, -m_use));
        rs += pr;
        pk[r >> 3][r & 7] = static_cast<__bf16>(pr);
      }
      l_sum += halves_sum(rs);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const int m1 = mb, m2 = mb ^ (D == 128 ? 2 : 0);
          const int o1 = ((m1 & 1) ? v_base_m : v_base_p) + (16 * kk) * C::ROW + 64 * m1;
          const int o2 = ((m2 & 1) ? v_base_m : v_base_p) + (16 * kk + 8) * C::ROW + 64 * m2;
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + o1));
          const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + o2));
          const u32x2 w1 = __builtin_bit_cast(u32x2, v1), w2 = __builtin_bit_cast(u32x2, v2);
          const u32x4 w = {w1[0], w1[1], w2[0], w2[1]};
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pk[kk],
                                                            acc[mb], 0, 0, 0);
        }
      }
    };
    // Tile j visible to every wave (stage j landed, barrier); then stage j+2
    // goes into the slot of tile j-2, which no wave reads any more.
    auto arrive = [&](int j, int sl) {
      const int issued_last = min(j == 0 ? kS - 2 : j + kS - 3, L - 1);
      if (loader) wait_stage<kS - 2, kNL>(issued_last - j);
      raw_barrier();
      if (j >= 1 && j + kS - 2 < L) issue_stage(j + kS - 2, (sl + kS - 2) % kS);
    };

    // ---- the ring over the batch's L tiles, one compute segment at a time ----
    // Tile jj sits in ring slot jj % 4.  Iteration jj makes tile jj + 1
    // visible (issuing stage jj + 3), starts its scores on the matrix cores
    // when it belongs to the same segment, then runs tile jj's softmax and
    // P.V; between segments the results go out and the next job's queries
    // come in while the ring keeps loading.
    for (int j = 0; j < kS - 1 && j < L; ++j) issue_stage(j, j);
    arrive(0, 0);
    bool prepared = false;  // the next segment's state is already set up
    for (int k = 0; k < nseg; ++k) {
      if (!prepared) {
        if (k > 0) load_c(k);
        kc = k;
        if (!(c_flags & kContPrev)) begin_segment();
      }
      prepared = false;
      const int j0 = k == 0 ? 0 : __builtin_amdgcn_readfirstlane(sSeg[k].j0);
      const int j1 = c_j1;
      const bool next = k + 1 < nseg;  // another segment of this batch follows
      // tiles before jc need no mask: they end at or before min(P, t_end)
      const int lim = min(c_P, c_te);
      const int jc = j0 + max(0, min(j1 - j0, (lim - (c_tb0 + j0 * kTile)) / kTile));
      const int jend = next ? j1 - 1 : j1;  // with a next segment its last tile is peeled
      f32x16 s_cur = rg >= 0 ? qk(j0 & (kS - 1)) : f32x16{};
      int jj = j0;
      for (; jj < min(jc, jend); ++jj) {
        if (jj + 1 < L) arrive(jj + 1, (jj + 1) & (kS - 1));
        if (rg >= 0) {
          f32x16 s_next = {};
          if (jj + 1 < j1) s_next = qk((jj + 1) & (kS - 1));
          softmax_pv(s_cur, c_tb0 + jj * kTile, jj & (kS - 1), std::false_type{});
          s_cur = s_next;
        }
      }
      for (; jj < jend; ++jj) {
        if (jj + 1 < L) arrive(jj + 1, (jj + 1) & (kS - 1));
        if (rg >= 0) {
          f32x16 s_next = {};
          if (jj + 1 < j1) s_next = qk((jj + 1) & (kS - 1));
          softmax_pv(s_cur, c_tb0 + jj * kTile, jj & (kS - 1), std::true_type{});
          s_cur = s_next;
        }
      }
      if (next) {
        // tile j1 - 1: the next job's queries load while it is consumed
        arrive(j1, j1 & (kS - 1));
        int n_slot, n_gq, n_node;
        rows_of(k + 1, n_slot, n_gq, n_node);
        if (rg >= 0) {
          issue_q(__builtin_amdgcn_readfirstlane(sSeg[k + 1].b),
                  __builtin_amdgcn_readfirstlane(sSeg[k + 1].hkv), n_slot, n_gq, n_node);
          if constexpr (kDmaWaves == 4) __builtin_amdgcn_s_waitcnt(0x0F70);  // ring loads too
          // (the masked form is exact for any tile; this one ends a job, so
          // it holds tree positions anyway)
          softmax_pv(s_cur, c_tb0 + (j1 - 1) * kTile, (j1 - 1) & (kS - 1), std::true_type{});
        }
        if (!(c_flags & kContNext)) end_segment();
        load_c(k + 1);
        kc = k + 1;
        slot = n_slot;
        gq = n_gq;
        node = n_node;
        from_job_start = (c_flags & kFromJobStart) != 0;
        from_range_start = (c_flags & kFromRangeStart) != 0;
        if (rg >= 0) reset_state();
        prepared = true;
      } else if (!(c_flags & kContNext)) {
        end_segment();
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // the ring is idle: the next batch may use its LDS
  }
}

// Combine launch of a units call: for every job cut by a range boundary, the
// log-sum-exp combination of its pieces (slots 2g / 2g + 1 of the groups its
// tiles fall in).  One thread per (row, 4 channels) of a job.
template <int RPT>
__global__ __launch_bounds__(kThreads) void merge_units_kernel(AttnParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv;
  const int hkv = bh % p.Hkv;
  // One load brings the sequence's stream start, the stream's length and the
  // bounds the attention launch took (P, n; 0, 0 for a sequence with nothing
  // to do), instead of dependent rounds of loads.
  const int4 rec = reinterpret_cast<const int4*>(p.ws_seq)[b];
  const int seq0 = rec.x;
  const int Sh = rec.y;  // stream units (all KV heads)
  const SeqJobs s = seq_jobs_of(p, rec.z, rec.w, RPT);
  if (s.rts == 0) return;
  const int groups = p.d / 4;
  const int per_tile = RPT * groups;
  const int e = blockIdx.y * kThreads + threadIdx.x;
  const int rtile = e / per_tile;
  if (rtile < s.rt_lo || rtile >= s.rt_lo + s.rts) return;
  const int r = (e % per_tile) / groups;
  const int dg = e % groups;
  const int gr = rtile * RPT + r;
  if (gr >= p.n_q * p.G) return;
  const int slot = gr / p.G, gq = gr % p.G;
  const int node = p.expand ? s.n - p.n_q + slot : slot;
  if (node < 0 || node >= s.n) return;

  const int N = Sh;
  const int G = p.n_split;  // work groups of the attention launch
  const int U = (N + G - 1) / G;
  const int J0 = seq0 + hkv * s.rts * (s.tiles + kJobCost) + (rtile - s.rt_lo) * (s.tiles + kJobCost);
  const int J1 = J0 + s.tiles;  // the job's tiles (its cost units follow)
  const int g0 = J0 / U, g1 = (J1 - 1) / U;
  if (g0 == g1) return;  // one group held the whole job and wrote its rows

  float M = -INFINITY, Lsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  constexpr int kBatch = 4;
  for (int q0 = g0; q0 <= g1; q0 += kBatch) {
    float ms[kBatch], ls[kBatch];
    PartialF16 hs[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {  // the whole batch's loads first
      const int gg = q0 + k <= g1 ? q0 + k : g1;
      const size_t ps = 2 * static_cast<size_t>(gg) + ((gg == g0 && J0 != g0 * U) ? 1 : 0);
      const size_t pr = ps * RPT + r;
      hs[k] = load_partial_f16(reinterpret_cast<const uint16_t*>(p.ws_o) + pr * p.d + 4 * dg,
                               reinterpret_cast<const PartialRec*>(p.ws_ml) + pr);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      ms[k] = hs[k].rec[0];
      ls[k] = hs[k].rec[1];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (q0 + k > g1) ms[k] = -INFINITY;
    // (no early continue when every state is empty: all weights are then
    // zero and the loads of the outputs stay ahead of the row records' use)
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) Mb = fmaxf(Mb, ms[k]);
    const float a = (M == -INFINITY) ? 0.f : exp2f(M - Mb);
    Lsum *= a;
    o *= a;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wgt = (ms[k] == -INFINITY) ? 0.f : exp2f(ms[k] - Mb);
      Lsum = fmaf(ls[k], wgt, Lsum);
      add_partial_f16(o, hs[k], wgt);
    }
    M = Mb;
  }
  const float inv = 1.f / Lsum;
  uint16_t* out = static_cast<uint16_t*>(p.out) +
                  ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + gq) * p.d + 4 * dg;
  const f32x4 v = o * inv;
  const uint32_t lo = f32_to_bf16_bits(v[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  const uint32_t hi = f32_to_bf16_bits(v[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  *reinterpret_cast<u32x2*>(out) = u32x2{lo, hi};
  if (p.lse != nullptr && dg == 0)
    p.lse[(static_cast<size_t>(b) * p.Hq + hkv * p.G + gq) * p.n_q + slot] = (M + log2f(Lsum)) * kLn2;
}

template <int D>
hipError_t launch_du(const AttnParams& p, hipStream_t s) {
  const dim3 grid(p.n_split);
  const dim3 block(kThreads);
  switch (p.rows_per_tile / 32) {
    case 1: return launch(attn_units_kernel<D, 1>, grid, block, s, p);
    case 2: return launch(attn_units_kernel<D, 2>, grid, block, s, p);
    case 3: return launch(attn_units_kernel<D, 3>, grid, block, s, p);
    case 4: return launch(attn_units_kernel<D, 4>, grid, block, s, p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_units(const AttnParams& p, hipStream_t s) {
  if (p.d == 128) return launch_du<128>(p, s);
  if (p.d == 64) return launch_du<64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge_units(const AttnParams& p, hipStream_t s) {
  const long long items = static_cast<long long>(p.n_row_tiles) * p.rows_per_tile * (p.d / 4);
  const dim3 grid(p.B * p.Hkv, static_cast<unsigned>((items + kThreads - 1) / kThreads));
  switch (p.rows_per_tile / 32) {
    case 1: return launch(merge_units_kernel<32>, grid, dim3(kThreads), s, p);
    case 2: return launch(merge_units_kernel<64>, grid, dim3(kThreads), s, p);
    case 3: return launch(merge_units_kernel<96>, grid, dim3(kThreads), s, p);
    case 4: return launch(merge_units_kernel<128>, grid, dim3(kThreads), s, p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ta
