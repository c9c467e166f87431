// bf16 tree-masked verify/expand attention, streaming variant for gfx950.
//
// Same mathematics and the same MFMA formulation as attn_mfma.hip (S^T = K .
// Q^T and O^T = V^T . P^T on v_mfma_f32_32x32x16_bf16, one query row per lane
// pair, lazy rescale, ancestor bitmask only on the tile that reaches the tree
// cache; SwiftSpec summary, Section 3.1.3 Figure 3 and Section 3.2), but built
// to keep many KV bytes in flight per compute unit:
//  * K/V move from HBM straight into a ring of S LDS stages of 32 positions
//    with global_load_lds_dwordx4 (no staging registers).  Lane i of a load
//    fetches the global 16-byte chunk that belongs at LDS position
//    base + 16 * i of the XOR-swizzled layout.
//  * The loads are issued from inline assembly and waited for with explicit
//    s_waitcnt vmcnt(N) + s_barrier, so the compiler cannot add a blanket
//    vmcnt(0) in front of every LDS read: S-2 stages stay in flight while two
//    are read (a tile's P.V and the next tile's scores run in the same
//    step).
//  * Each computing wave owns one 32-row group of the tile's rows and
//    consumes every stage; waves beyond the row groups only issue loads.
//  * Paged caches: the split's block ids are copied to LDS first, so the
//    ring loop issues no other vector-memory loads.
//  * A split sequence leaves partial (max, sum, output) states in the
//    workspace; the combine launch (attn_merge.hip) finishes it.
//  * RoPE variant (kRope; SwiftSpec summary, Section 3.3: the masked
//    attention takes the position embedding): the queries are rotated as
//    they are loaded, to the positions P - 1 + depth of their nodes.  The ring
//    then streams the prefix only; after it, the split's tree positions are
//    staged in the ring's LDS, 32 at a time, the new nodes' keys rotated from
//    k_new and their values from v_new (older nodes, when expanding, read
//    from the cache), and attended as one more masked tile.  The work group
//    of row tile 0 also writes the new nodes' rows to the cache (one writer
//    per row); the others never read those rows from the cache.  At set-up
//    only the first two stages are in flight: the other two slots hold the
//    ancestor masks and the cos/sin table of the tile's query slots.
#include "rope_common.h"
#include "stream_common.h"

namespace ta {
namespace {

// S = 4: a 64 KiB ring, two work groups per compute unit.  (A three-stage
// ring for three groups per CU does not fit: 128 query rows need the
// registers of two.)
template <int D, int NRG, int S, bool kRope>
__global__ __launch_bounds__(kThreads, 2) void attn_stream_kernel(AttnParams p) {
  using C = SCfg<D, NRG, S>;
  static_assert(S >= 2 && S <= 4, "ring depth");
  static_assert(!kRope || S == 4, "the RoPE set-up uses two of four ring slots");
  __shared__ __attribute__((aligned(1024))) uint8_t sRing[C::LDS];
  __shared__ int sBlk[kRope ? 1 : kMaxSplitBlocks];   // paged block ids (not with RoPE)
  __shared__ uint64_t sRowMask[C::RPT][kMaskWords];  // ancestor mask of each row's node
  __shared__ int sDepth[kRope ? kMaxNodes : 1];      // RoPE: depth of every node
  __shared__ double sInv[kRope ? D / 2 : 1];         // RoPE: base^(-2j/d)

  // grid = (sequence x KV head, split, row tile): consecutive work groups are
  // different (sequence, KV head) pairs, which the dispatcher deals round
  // robin to the eight XCDs, so every XCD gets an even share of every split
  // (with the split fastest, split s of all sequences would land on one XCD).
  const int bh = blockIdx.x;
  const int split = blockIdx.y;
  const int rtile = blockIdx.z;
  const int b = bh / p.Hkv;
  const int hkv = bh % p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: load bases in SGPRs
  const int lhi = lane >> 5;
  const int l32 = lane & 31;
  const int t_begin = split * p.chunk;
  const uint8_t* Kg = static_cast<const uint8_t*>(p.k);
  const uint8_t* Vg = static_cast<const uint8_t*>(p.v);
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_u8*)sRing));
  const size_t pos_stride = static_cast<size_t>(p.Hkv) * C::ROW;  // contiguous: bytes per position

  // computing waves own one 32-row group each (with NRG = 4, every wave)
  constexpr bool kAllCompute = NRG == kThreads / 64;
  const int rg = (kAllCompute || wave < NRG) ? wave : -1;
  const int R = p.n_q * p.G;
  const int row_in_tile = (rg < 0 ? 0 : rg) * 32 + l32;
  const int grow = rtile * C::RPT + row_in_tile;
  const bool row_exists = rg >= 0 && grow < R;  // a query slot of q (its node may not exist)
  const int slot = row_exists ? grow / p.G : 0;
  const int g = row_exists ? grow % p.G : 0;

  // Q^T operand (B side of S^T = K . Q^T): lane holds row l32, chunk 2*ks + lhi.
  bf16x8 qreg[C::KS];
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const size_t qrow = ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * D;

  // A split of a contiguous cache starts at t_begin whatever the sequence's
  // length, and its first two tiles lie inside the allocation when
  // t_begin + 64 <= T_cap: their K/V and the tile's query rows are loaded
  // before the lengths are known, so that the ring's first memory latency
  // overlaps the lengths' load and the mask set-up.  (Every return below
  // waits for these loads first: the LDS they land in must not be handed to
  // another work group while they are in flight.)
  const bool spec = !kRope && p.block_table == nullptr && t_begin + 2 * kTile <= p.T_cap;
  if (spec) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < C::INST_PER_WAVE; ++q) {
        const int r0 = (wave * C::INST_PER_WAVE + q) * C::ROWS_PER_INST;
        const int r = r0 + lane / C::CH;
        const int c = (lane % C::CH) ^ swz<D>(r);
        const size_t off = (static_cast<size_t>(b) * p.T_cap + t_begin + j * kTile + r) * pos_stride +
                           static_cast<size_t>(hkv) * C::ROW + c * 16;
        const uint32_t lk = __builtin_amdgcn_readfirstlane(ring_base + j * C::STAGE + r0 * C::ROW);
        dma16(Kg + off, lk);
        dma16(Vg + off, lk + C::HALF);
      }
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_exists) v = *reinterpret_cast<const u32x4*>(Q + qrow + (2 * ks + lhi) * 8);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  SeqBounds sb;
  if (!seq_bounds(p.prefix_len, p.n_nodes, b, p.n_max, p.T_cap, sb)) {
    if (spec) wait_vmcnt<0>();
    return;
  }
  const int nsplit = (sb.T + p.chunk - 1) / p.chunk;
  if (split >= nsplit) {
    if (spec) wait_vmcnt<0>();
    return;
  }
  const int t_end = min(sb.T, t_begin + p.chunk);

  int node = -1;
  if (row_exists) {
    node = p.expand ? sb.n - p.n_q + slot : slot;
    if (node < 0 || node >= sb.n) node = -1;
  }
  if (!__syncthreads_or(node >= 0)) {
    if (spec) wait_vmcnt<0>();
    return;
  }

  // With RoPE the ring streams the prefix part of the split; the tree part
  // follows it (staged, not streamed).
  const int t_ring_end = kRope ? min(t_end, sb.P) : t_end;
  int vis_end = t_ring_end;  // the masked path's end of visible positions
  const bool has_tree = t_end > sb.P;

  // ---- setup: ancestor masks (in ring slots 2-3, which no load has
  // reached yet), paged block ids ------------
  static_assert(C::SETUP <= 2 * C::STAGE, "the set-up tables fit in ring slots 2 and 3");
  if constexpr (!kRope) {
    auto sAnc = reinterpret_cast<uint64_t(*)[kMaskWords]>(sRing + 2 * C::STAGE);
    int* sJump = reinterpret_cast<int*>(sRing + 2 * C::STAGE + kMaxNodes * kMaskWords * 8);
    if (has_tree) build_ancestor_masks(p.parent + static_cast<size_t>(b) * p.n_max, sb.n, sAnc, sJump);
    if (p.block_table != nullptr) {
      const int blk0 = t_begin / p.block_size;
      const int nblk = (t_end - 1) / p.block_size - blk0 + 1;  // <= kMaxSplitBlocks (planner)
      for (int i = tid; i < nblk && i < kMaxSplitBlocks; i += kThreads) {
        int v = p.block_table[static_cast<size_t>(b) * p.max_blocks + blk0 + i];
        sBlk[i] = v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
      }
    }
    __syncthreads();
    // keep each row's mask (only the tail tile reads it) outside the ring
    if (has_tree && rg >= 0 && lhi == 0) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) sRowMask[row_in_tile][w] = node >= 0 ? sAnc[node][w] : 0ull;
    }
    __syncthreads();  // the ring may now overwrite the ancestor table
  }

  // The queries, loaded once the first ring stages are in flight (below), so
  // that both latencies overlap.
  auto load_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (node >= 0) v = *reinterpret_cast<const u32x4*>(Q + qrow + (2 * ks + lhi) * 8);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
    // Complete every load with a wait the compiler can see (vmcnt(0), other
    // counters untouched); otherwise it would re-wait for the Q loads inside
    // the ring loop, where the outstanding loads are the ring's.
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  // ---- ring of stages ----------------------------------------------------
  const int ntiles = max(0, (t_ring_end - t_begin + kTile - 1) / kTile);
  const int blk0 = (!kRope && p.block_table != nullptr) ? t_begin / p.block_size : 0;

  // Byte offset of row `tok` (clamped into the split) of the K or V cache.
  auto row_bytes_off = [&](int tok) -> size_t {
    tok = tok < t_ring_end ? tok : t_ring_end - 1;
    size_t row;
    if (!kRope && p.block_table != nullptr) {
      const int blk = sBlk[tok / p.block_size - blk0];
      row = (static_cast<size_t>(blk) * p.block_size + tok % p.block_size) * p.Hkv + hkv;
    } else {
      row = (static_cast<size_t>(b) * p.T_cap + tok) * p.Hkv + hkv;
    }
    return row * C::ROW;
  };
  // Per-lane DMA sources: lane (row r, physical chunk pc) of load q fetches
  // logical chunk pc ^ swz(r).  In the contiguous layout the byte offset of the
  // next stage to issue just advances by one tile of positions per stage.
  const bool contiguous = kRope || p.block_table == nullptr;
  size_t dma_off[C::INST_PER_WAVE];
#pragma unroll
  for (int q = 0; q < C::INST_PER_WAVE; ++q) {
    const int r = (wave * C::INST_PER_WAVE + q) * C::ROWS_PER_INST + lane / C::CH;
    const int c = (lane % C::CH) ^ swz<D>(r);
    dma_off[q] = (static_cast<size_t>(b) * p.T_cap + t_begin + r) * pos_stride +
                 static_cast<size_t>(hkv) * C::ROW + c * 16;
  }
  // Issues stage j (the stages are issued in order) into ring slot `slot`;
  // whole_tag true: the stage is known to be a whole tile inside the split.
  auto issue_stage = [&](int j, int slot, auto whole_tag) {
    const int tb = t_begin + j * kTile;
    const uint32_t sbase = ring_base + slot * C::STAGE;
    const bool fast = contiguous && (decltype(whole_tag)::value || tb + kTile <= t_ring_end);
    if (fast) {
#pragma unroll
      for (int q = 0; q < C::INST_PER_WAVE; ++q) {
        const uint32_t lk = sbase + (wave * C::INST_PER_WAVE + q) * C::ROWS_PER_INST * C::ROW;
        dma16(Kg + dma_off[q], lk);
        dma16(Vg + dma_off[q], lk + C::HALF);
        dma_off[q] += kTile * pos_stride;
      }
    } else {
#pragma unroll
      for (int q = 0; q < C::INST_PER_WAVE; ++q) {
        const int r0 = (wave * C::INST_PER_WAVE + q) * C::ROWS_PER_INST;
        const int r = r0 + lane / C::CH;
        const int c = (lane % C::CH) ^ swz<D>(r);
        const size_t off = row_bytes_off(tb + r) + c * 16;
        const uint32_t lk = sbase + r0 * C::ROW;
        dma16(Kg + off, lk);
        dma16(Vg + off, lk + C::HALF);
        dma_off[q] += kTile * pos_stride;
      }
    }
  };

  f32x16 acc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  float m_ref = -INFINITY;
  float m_hi = -INFINITY;  // the largest tile maximum seen (log2 units)
  float l_sum = 0.f;
  const float cs = p.scale_log2;
  const int lim = min(sb.P, t_ring_end);

  // S^T = K . Q^T for the tile in ring `slot` (M = 32 positions, N = 32 rows,
  // K = d).  The MFMAs run while the previous tile's softmax uses the VALU.
  auto qk = [&](int slot) -> f32x16 {
    const uint8_t* sK = sRing + slot * C::STAGE;
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
  // Per-lane bases of the transposed V reads: lane (group gi, index jl) reads
  // positions 16kk + 8h + 4(gi/2) + jl/4 at channels 32mb + 16(gi%2) + 4(jl%4);
  // under the swizzle that is base +- 64 x + (16kk + 8h) ROW + 64 (mb ^ 2h).
  int v_base_p, v_base_m;
  {
    const int gi = lane >> 4, jl = lane & 15;
    const int x = (jl >> 3) & 1;
    const int s_lo = (((jl >> 2) & 1) << 1) | ((gi >> 1) & 1);
    const int y = (2 * (gi & 1) + ((jl & 3) >> 1)) ^ s_lo;
    const int L = (4 * (gi >> 1) + (jl >> 2)) * C::ROW + 16 * y + 8 * (jl & 1);
    v_base_p = L + 64 * x;
    v_base_m = L - 64 * x;
  }
  // Mask (tiles that reach the tree cache or the split's end), online
  // softmax and O^T += V^T . P^T for the tile of positions tb.. held in ring
  // `slot`.  Lane l holds positions tb + 8*(r/4) + 4*lhi + r%4 of row l32.
  // No branch: the exponentials take as reference m_use = max(m_ref, tile
  // maximum - kRescaleMax) (the tile's own maximum while the row has seen
  // nothing), so every p stays below 2^kRescaleMax, and the mask, the
  // maximum, the exponentials and P.V form one block with the next tile's
  // QK^T MFMAs, which the compiler interleaves.  The running maximum of the
  // tiles' maxima (m_hi) is folded into the state by settle(), called after
  // every tile: a maximum more than kRescaleSlack above m_ref rescales the
  // state to it, so that at every tile's start the state's p are at most
  // 2^kRescaleSlack.  When m_use passes m_ref (a jump of more than
  // kRescaleMax), the state is left as it is: next to this tile's largest p
  // (2^kRescaleMax) it weighs below 2^-(kRescaleMax - kRescaleSlack - 20) for
  // up to 2^20 positions, far below fp32 resolution, scaled down or not.
  auto softmax_pv = [&](f32x16 Sc, int tb, int slot, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const uint8_t* sV = sRing + slot * C::STAGE + C::HALF;
    if constexpr (kMasked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tb + 8 * (r >> 2) + 4 * lhi + (r & 3);
        const int jj = t - sb.P;  // tree column (negative: prefix)
        const bool tree_col = jj >= 0 && t < vis_end;  // then jj < n <= 256
        const uint64_t word = tree_col ? sRowMask[row_in_tile][jj >> 6] : 0ull;
        const bool in_tree = ((word >> (jj & 63)) & 1ull) != 0ull;
        const bool vis = t < vis_end && (jj < 0 || in_tree);
        if (!vis) Sc[r] = -INFINITY;
      }
    }
    float mx = Sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, Sc[r]);
    mx = halves_max(mx) * cs;  // the tile's row maximum (log2 units)
    float m_use = m_ref == -INFINITY ? mx : fmaxf(m_ref, mx - kRescaleMax);
    m_use = m_use == -INFINITY ? 0.f : m_use;  // nothing visible yet: every p is 0
    float rs = 0.f;
    bf16x8 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(Sc[r], cs, -m_use));  // v_exp_f32; args <= 64
      rs += pr;
      pk[r >> 3][r & 7] = static_cast<__bf16>(pr);
    }
    l_sum += halves_sum(rs);
    m_ref = m_ref == -INFINITY ? mx : m_use;  // the state's reference from here on
    m_hi = fmaxf(m_hi, mx);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        // 16-lane group: 4 positions x 16 channels, transposed on read.  With
        // the swizzle, every address is one of two per-lane bases (by parity of
        // the swizzled channel block) plus a constant.
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
  // After each tile (a rarely taken, wave-uniform branch, which measured
  // cheapest there): fold m_hi into the state.  m_ref is finite whenever
  // m_hi passes it.
  auto settle = [&]() {
    const bool bump = m_hi > m_ref + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(bump) != 0ull) {
      const float alpha = bump ? exp2f(m_ref - m_hi) : 1.f;
      l_sum *= alpha;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
      m_ref = bump ? m_hi : m_ref;
    }
  };
  // Makes tile j visible to every wave: wait until stage j has landed (at most
  // (stages issued after it) x NL loads of this wave pending), then barrier.
  // After the barrier no wave still reads the slot of tile j-2, which then
  // receives stage j+S-2.
  auto arrive = [&](int j, int slot) {
    // stages issued so far: 0 .. S-2 by the prologue, then t+S-2 by arrive(t), t = 1 .. j-1
    const int issued_last = min(j == 0 ? S - 2 : j + S - 3, ntiles - 1);
    wait_stage<S - 2, C::NL>(issued_last - j);
    raw_barrier();
    if (j >= 1 && j + S - 2 < ntiles) issue_stage(j + S - 2, (slot + S - 2) % S, std::false_type{});
  };
  // arrive() inside the dense loop (1 <= j, j + 3 < ntiles): exactly S - 3
  // stages after j are in flight and stage j + S - 2 exists, so the wait and
  // the issue need no run-time cases.
  auto arrive_dense = [&](int j, int slot) {
    wait_vmcnt<(S - 3) * C::NL>();
    raw_barrier();
    issue_stage(j + S - 2, (slot + S - 2) % S, std::true_type{});
  };

  // Prologue: stages 0 .. S-2 and the queries in flight, tile 0's scores started.
  if constexpr (!kRope) {
    static_assert(S == 4, "the early start covers stages 0 and 1 of four");
    if (spec) {
      if (t_begin + 2 * kTile > t_ring_end) {
        // the early tiles ran past the split's end (rows there may hold
        // anything): load them again, clamped to the split
        wait_vmcnt<0>();
        for (int j = 0; j < 2 && j < ntiles; ++j) issue_stage(j, j, std::false_type{});
      } else {
#pragma unroll
        for (int q = 0; q < C::INST_PER_WAVE; ++q) dma_off[q] += 2 * kTile * pos_stride;
      }
      // the early query loads have landed; rows without a node take zeros
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      if (node < 0) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
      if (2 < ntiles) issue_stage(2, 2, std::false_type{});
    } else {
      for (int j = 0; j < S - 1 && j < ntiles; ++j) issue_stage(j, j, std::false_type{});
      load_q();
    }
  } else {
    // Stages 0 .. S-3 go out first; ring slots S-2 and S-1 hold the set-up.
    for (int j = 0; j < S - 2 && j < ntiles; ++j) issue_stage(j, j, std::false_type{});
    uint8_t* setup = sRing + (S - 2) * C::STAGE;
    auto sAnc = reinterpret_cast<uint64_t(*)[kMaskWords]>(setup);
    int* sJump = reinterpret_cast<int*>(setup + kMaxNodes * kMaskWords * 8);
    if (tid < D / 2) sInv[tid] = rope_inv_freq(p.rope_base, tid, D);
    build_ancestor_masks(p.parent + static_cast<size_t>(b) * p.n_max, sb.n, sAnc, sJump);
    if (has_tree && rg >= 0 && lhi == 0) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) sRowMask[row_in_tile][w] = node >= 0 ? sAnc[node][w] : 0ull;
    }
    for (int i = tid; i < sb.n; i += kThreads) {
      int dep = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) dep += __popcll(sAnc[i][w]);
      sDepth[i] = dep;  // the node and its ancestors: its depth below the root
    }
    __syncthreads();
    // cos/sin of the tile's query slots (they overwrite the masks)
    const int slot_lo = rtile * C::RPT / p.G;
    const int slot_hi = min(p.n_q, ((rtile + 1) * C::RPT - 1) / p.G + 1);
    float2* sTab = reinterpret_cast<float2*>(setup);
    for (int e = tid; e < (slot_hi - slot_lo) * (D / 2); e += kThreads) {
      const int sl = slot_lo + e / (D / 2), j = e % (D / 2);
      const int nd = p.expand ? sb.n - p.n_q + sl : sl;
      float c = 1.f, sn = 0.f;
      if (nd >= 0 && nd < sb.n) rope_cos_sin(sb.P - 1 + sDepth[nd], sInv[j], c, sn);
      sTab[e] = float2{c, sn};
    }
    __syncthreads();
    // queries: each lane holds chunks 2ks + lhi; chunk c pairs with c + D/16
    // (channels j and j + d/2), which is qreg[ks + KS/2] of the same lane
    {
      u32x4 raw[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        raw[ks] = u32x4{0u, 0u, 0u, 0u};
        if (node >= 0) raw[ks] = *reinterpret_cast<const u32x4*>(Q + qrow + (2 * ks + lhi) * 8);
      }
      const float2* tab = sTab + (slot - slot_lo) * (D / 2);
#pragma unroll
      for (int ks = 0; ks < C::KS / 2; ++ks) {
        const uint32_t w0[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
        const uint32_t w1[4] = {raw[ks + C::KS / 2].x, raw[ks + C::KS / 2].y,
                                raw[ks + C::KS / 2].z, raw[ks + C::KS / 2].w};
        uint32_t o0[4], o1[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          float y[2][2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = (2 * ks + lhi) * 8 + 2 * h + e;
            const float x0 = __uint_as_float(e ? (w0[h] & 0xffff0000u) : (w0[h] << 16));
            const float x1 = __uint_as_float(e ? (w1[h] & 0xffff0000u) : (w1[h] << 16));
            const float2 cs2 = node >= 0 ? tab[j] : float2{1.f, 0.f};
            rope_rotate(x0, x1, cs2.x, cs2.y, y[0][e], y[1][e]);
          }
          o0[h] = f32_to_bf16_bits(y[0][0]) | (static_cast<uint32_t>(f32_to_bf16_bits(y[0][1])) << 16);
          o1[h] = f32_to_bf16_bits(y[1][0]) | (static_cast<uint32_t>(f32_to_bf16_bits(y[1][1])) << 16);
        }
        qreg[ks] = __builtin_bit_cast(bf16x8, u32x4{o0[0], o0[1], o0[2], o0[3]});
        qreg[ks + C::KS / 2] = __builtin_bit_cast(bf16x8, u32x4{o1[0], o1[1], o1[2], o1[3]});
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query loads (and the first stages)
    }
    __syncthreads();  // the table is done with: slot S-2 takes its stage
    if (S - 2 < ntiles) issue_stage(S - 2, S - 2, std::false_type{});
  }
  if (ntiles > 0) arrive(0, 0);
  f32x16 s_cur = (rg >= 0 && ntiles > 0) ? qk(0) : f32x16{};
  // Iteration j: tile j+1 arrives and its scores start on the matrix cores,
  // then tile j's softmax and P.V run.  Tiles below lim = min(P, t_end) need no
  // mask; the dense part is unrolled by the ring depth so that every slot
  // offset is a constant.  Its tiles go in pairs whose scores live in two
  // alternating registers (s_cur, s_odd): with one "next scores" value copied
  // into s_cur every tile, the compiler emitted eight 64-bit moves per tile.
  static_assert(S % 2 == 0, "the dense loop takes tiles in pairs");
  const int n_clean = max(0, min(ntiles, (lim - t_begin) / kTile));
  int j = 0;
  for (; j + S <= n_clean && j + S + 3 < ntiles; j += S) {  // arrive_dense's range
#pragma unroll
    for (int u = 0; u < S; u += 2) {
      f32x16 s_odd;
      arrive_dense(j + u + 1, (u + 1) % S);
      if (kAllCompute || rg >= 0) {
        s_odd = qk((u + 1) % S);
        softmax_pv(s_cur, t_begin + (j + u) * kTile, u, std::false_type{});
        settle();
      }
      arrive_dense(j + u + 2, (u + 2) % S);
      if (kAllCompute || rg >= 0) {
        s_cur = qk((u + 2) % S);
        softmax_pv(s_odd, t_begin + (j + u + 1) * kTile, u + 1, std::false_type{});
        settle();
      }
    }
  }
  // The rest (the masked tail, the last tiles), unrolled the same way: j is a
  // multiple of S here, so tile j + u sits in slot u.
  for (; j < ntiles; j += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int jj = j + u;
      if (jj < ntiles) {
        const bool more = jj + 1 < ntiles;
        if (more) arrive(jj + 1, (u + 1) % S);
        if (kAllCompute || rg >= 0) {
          f32x16 s_next = {};
          if (more) s_next = qk((u + 1) % S);
          if (jj < n_clean)
            softmax_pv(s_cur, t_begin + jj * kTile, u, std::false_type{});
          else
            softmax_pv(s_cur, t_begin + jj * kTile, u, std::true_type{});
          settle();
          s_cur = s_next;
        }
      }
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // ---- RoPE: the split's tree positions, 32 at a time, staged in slot 0 ----
  if constexpr (kRope) {
    const int first_new = p.expand ? sb.n - p.n_q : 0;  // new nodes: [first_new, n)
    const uint16_t* Kn = static_cast<const uint16_t*>(p.k_new);
    const uint16_t* Vn = static_cast<const uint16_t*>(p.v_new);
    uint16_t* Kc = static_cast<uint16_t*>(const_cast<void*>(p.k));
    uint16_t* Vc = static_cast<uint16_t*>(const_cast<void*>(p.v));
    const bool writer = rtile == 0;
    float2* sTab = reinterpret_cast<float2*>(sRing + 2 * C::STAGE);  // [32][D/2]
    uint8_t* sK = sRing;
    uint8_t* sV = sRing + C::HALF;
    vis_end = t_end;
    for (int c0 = max(sb.P, t_begin); c0 < t_end; c0 += kTile) {
      for (int e = tid; e < kTile * (D / 2); e += kThreads) {
        const int r = e / (D / 2), j = e % (D / 2);
        const int nd = c0 + r - sb.P;
        float c = 1.f, sn = 0.f;
        if (c0 + r < t_end && nd >= first_new) rope_cos_sin(sb.P - 1 + sDepth[nd], sInv[j], c, sn);
        sTab[e] = float2{c, sn};
      }
      __syncthreads();
      // keys: (row, chunk pair) items; values: (row, chunk) items
      for (int e = tid; e < kTile * (C::CH / 2); e += kThreads) {
        const int r = e / (C::CH / 2), cp = e % (C::CH / 2);
        const int t = c0 + r, nd = t - sb.P;
        u32x4 a = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
        if (t < t_end) {
          const size_t crow = ((static_cast<size_t>(b) * p.T_cap + t) * p.Hkv + hkv) * D;
          if (nd >= first_new) {
            const size_t nrow =
                ((static_cast<size_t>(b) * p.n_q + (nd - first_new)) * p.Hkv + hkv) * D;
            const u32x4 x = *reinterpret_cast<const u32x4*>(Kn + nrow + cp * 8);
            const u32x4 y = *reinterpret_cast<const u32x4*>(Kn + nrow + (cp + C::CH / 2) * 8);
            const uint32_t wx[4] = {x.x, x.y, x.z, x.w}, wy[4] = {y.x, y.y, y.z, y.w};
            uint32_t ox[4], oy[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              float r0[2], r1[2];
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                const float x0 = __uint_as_float(q ? (wx[h] & 0xffff0000u) : (wx[h] << 16));
                const float x1 = __uint_as_float(q ? (wy[h] & 0xffff0000u) : (wy[h] << 16));
                const float2 cs2 = sTab[r * (D / 2) + cp * 8 + 2 * h + q];
                rope_rotate(x0, x1, cs2.x, cs2.y, r0[q], r1[q]);
              }
              ox[h] = f32_to_bf16_bits(r0[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(r0[1])) << 16);
              oy[h] = f32_to_bf16_bits(r1[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(r1[1])) << 16);
            }
            a = u32x4{ox[0], ox[1], ox[2], ox[3]};
            z = u32x4{oy[0], oy[1], oy[2], oy[3]};
            if (writer) {
              *reinterpret_cast<u32x4*>(Kc + crow + cp * 8) = a;
              *reinterpret_cast<u32x4*>(Kc + crow + (cp + C::CH / 2) * 8) = z;
            }
          } else {  // an older node (expanding): already rotated in the cache
            a = *reinterpret_cast<const u32x4*>(Kc + crow + cp * 8);
            z = *reinterpret_cast<const u32x4*>(Kc + crow + (cp + C::CH / 2) * 8);
          }
        }
        *reinterpret_cast<u32x4*>(sK + lds_off<D>(r, cp)) = a;
        *reinterpret_cast<u32x4*>(sK + lds_off<D>(r, cp + C::CH / 2)) = z;
      }
      for (int e = tid; e < kTile * C::CH; e += kThreads) {
        const int r = e / C::CH, c = e % C::CH;
        const int t = c0 + r, nd = t - sb.P;
        u32x4 a = {0u, 0u, 0u, 0u};
        if (t < t_end) {
          const size_t crow = ((static_cast<size_t>(b) * p.T_cap + t) * p.Hkv + hkv) * D;
          if (nd >= first_new) {
            const size_t nrow =
                ((static_cast<size_t>(b) * p.n_q + (nd - first_new)) * p.Hkv + hkv) * D;
            a = *reinterpret_cast<const u32x4*>(Vn + nrow + c * 8);
            if (writer) *reinterpret_cast<u32x4*>(Vc + crow + c * 8) = a;
          } else {
            a = *reinterpret_cast<const u32x4*>(Vc + crow + c * 8);
          }
        }
        *reinterpret_cast<u32x4*>(sV + lds_off<D>(r, c)) = a;
      }
      __syncthreads();
      if (rg >= 0) {
        softmax_pv(qk(0), c0, 0, std::true_type{});
        settle();
      }
      __syncthreads();  // before the next group of positions overwrites slot 0
    }
  }

  uint16_t* Out = static_cast<uint16_t*>(p.out);
  const size_t orow = ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * D;
  const size_t lrow = (static_cast<size_t>(b) * p.Hq + hkv * p.G + g) * p.n_q + slot;

  if (nsplit == 1) {
    if (rg >= 0 && node >= 0) {
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
      if (p.lse != nullptr && lhi == 0) p.lse[lrow] = (m_ref + log2f(l_sum)) * kLn2;
    }
    return;
  }

  const int tile_id = bh * p.n_row_tiles + rtile;
  const size_t part = static_cast<size_t>(tile_id) * p.n_split;
  if (rg >= 0) {  // wave-uniform: every lane takes part in the row maximum
    const size_t pr = (part + split) * C::RPT + row_in_tile;
    const int e = partial_exp(acc);
    store_partial_f16(acc, m_ref, l_sum, e, lhi, reinterpret_cast<uint16_t*>(p.ws_o) + pr * D,
                      reinterpret_cast<PartialRec*>(p.ws_ml) + pr);
  }
  // the combine launch (attn_merge.hip) finishes split sequences
}

template <int D, int S, bool R>
hipError_t launch_ds(const AttnParams& p, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv, p.n_split, p.n_row_tiles);
  const dim3 block(kThreads);
  switch (p.rows_per_tile / 32) {
    case 1: return launch(attn_stream_kernel<D, 1, S, R>, grid, block, s, p);
    case 2: return launch(attn_stream_kernel<D, 2, S, R>, grid, block, s, p);
    case 3: return launch(attn_stream_kernel<D, 3, S, R>, grid, block, s, p);
    case 4: return launch(attn_stream_kernel<D, 4, S, R>, grid, block, s, p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool stream_rope_fits(int d, int rows_per_tile, int G) {
  // cos/sin (8 bytes) of d/2 pairs for every query slot a row tile touches,
  // in two 32-position ring stages of d-wide bf16 K and V rows (256 d bytes);
  // the tree phase's table of 32 positions needs 128 d bytes of the same
  const long long slots = rows_per_tile / G + 1;
  return slots * (d / 2) * 8 <= 2LL * 4 * 32 * d && (d == 64 || d == 128);
}

hipError_t launch_attn_stream(const AttnParams& p, hipStream_t s) {
  if (p.rope) {
    if (p.block_table != nullptr || !stream_rope_fits(p.d, p.rows_per_tile, p.G))
      return hipErrorInvalidValue;
    if (p.d == 128) return launch_ds<128, 4, true>(p, s);
    if (p.d == 64) return launch_ds<64, 4, true>(p, s);
    return hipErrorInvalidValue;
  }
  if (p.d == 128) return launch_ds<128, 4, false>(p, s);
  if (p.d == 64) return launch_ds<64, 4, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ta
