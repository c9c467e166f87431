// Evolving-tree-cache re-root with in-place KV compaction (SwiftSpec summary,
// Section 3.2 and Figure 4: verified nodes join the prefix cache, the subtree
// under the last verified node is pulled forward to follow it, the rest is
// dropped; KV is moved, never recomputed).
//
// Launch 1 (move): one work group per (KV head x 64-byte column slice, K|V,
// sequence x layer).  The group rebuilds the move list itself from
// parent/path/keep (ancestor masks by pointer doubling, kept-node ranks by
// popcount); if no row changes place (a chain, or a path that is already in
// order) it stops there.  Otherwise it copies its own 64-byte slice of every
// moved row: all loads go to registers (at most 4 x 16 bytes per thread), the
// group synchronises, then all stores run.  Because a group owns its slice
// exclusively, a destination that is another move's source is never
// overwritten before it has been read.
// Launch 2 (metadata): one work group per sequence rewrites parent, n_nodes
// and prefix_len after every layer has been moved (stream order), and moves
// the draft's per-node tokens and weights when it is given them.
//
// Fused with the greedy acceptance (accept_reroot_kernel): the same move
// groups first take the accepted path themselves (tree_walk.h) from the
// target's argmax per node, so no launch has to hand the path over; and they
// read the tree from a copy the argmax launch took, so one of them can
// rewrite the live metadata at once instead of a separate launch after the
// moves.
#include "ta_device.h"
#include "tree_walk.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kSliceChunks = 4;  // 16-byte chunks per column slice (64 bytes)
constexpr int kMaxChunksPerThread = kMaxNodes * kSliceChunks / kThreads;

struct Plan {
  int P, n, k, keep, v_last, n_kept, valid;
};

// The kept set: descendants of the path's last node when the subtree is
// kept (a 256-bit mask in sKept), and its size.  Synchronises.
__device__ __forceinline__ void plan_kept(Plan& pl, const uint64_t (*sAnc)[kMaskWords],
                                          uint64_t* sKept) {
  const int tid = threadIdx.x;
  bool kept = false;
  if (pl.keep && pl.k > 0 && tid < pl.n && tid != pl.v_last) kept = mask_bit(sAnc[tid], pl.v_last);
  const unsigned long long bal = __ballot(kept);
  if ((tid & 63) == 0) sKept[tid >> 6] = bal;
  __syncthreads();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) nk += __popcll(sKept[w]);
  pl.n_kept = nk;
}

// Shared by both launches: sequence bounds, path, kept set (as a 256-bit mask
// in sKept) and each kept node's rank (popcount of kept bits below it).
__device__ __forceinline__ Plan make_plan(const int32_t* prefix_len, const int32_t* parent,
                                          const int32_t* n_nodes, const int32_t* path,
                                          const int32_t* path_len, const uint8_t* keep, int b,
                                          int n_max, uint64_t (*sAnc)[kMaskWords], int* sJump,
                                          uint64_t* sKept, int* sPath) {
  Plan pl;
  const int tid = threadIdx.x;
  // every global load first (slot index clamped), so the plan pays one
  // memory latency: the sequence's sizes and flag, this slot's path entry
  // and parent
  const int ic = tid < n_max ? tid : n_max - 1;
  int n = n_nodes[b];
  int k = path_len[b];
  const int P = prefix_len[b];
  const int kp = keep[b];
  const int v_i = path[static_cast<size_t>(b) * n_max + ic];
  const int par_i = parent[static_cast<size_t>(b) * n_max + ic];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  k = k < 0 ? 0 : (k > n ? n : k);
  pl.P = P;
  pl.n = n;
  pl.k = k;
  pl.keep = kp != 0;
  pl.valid = pl.P >= 0;
  if (tid < k) sPath[tid] = v_i < 0 ? 0 : (v_i >= n ? n - 1 : v_i);
  if (tid < kMaskWords) sKept[tid] = 0;
  build_ancestor_masks_of(par_i, n, sAnc, sJump);
  pl.v_last = k > 0 ? sPath[k - 1] : -1;
  plan_kept(pl, sAnc, sKept);
  return pl;
}

__device__ __forceinline__ int kept_rank(const uint64_t* sKept, int i) {
  int r = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) {
    if (w < (i >> 6))
      r += __popcll(sKept[w]);
    else if (w == (i >> 6))
      r += __popcll(sKept[w] & ((1ull << (i & 63)) - 1ull));
  }
  return r;
}

// Copies this work group's 64-byte column slice (K or V of one KV head of one
// layer of sequence b) of every row that changes place.  All threads call it
// (it synchronises); it stops early when no row moves.
__device__ __forceinline__ void move_slice(const RerootLayer& L, int b, int hkv, int which,
                                           int slice, int Hkv, int row_bytes, const Plan& pl,
                                           const int* sPath, const uint64_t* sKept, int* sSrc,
                                           int* sDst) {
  const int tid = threadIdx.x;
  // Move list: slot j < k promotes path node j; slot k + r takes kept node of rank r.
  const int n_moves = min(pl.k + pl.n_kept, kMaxNodes);
  if (tid < pl.k) {
    sDst[tid] = pl.P + tid;
    sSrc[tid] = pl.P + sPath[tid];
  }
  if (tid < pl.n && mask_bit(sKept, tid)) {
    const int r = pl.k + kept_rank(sKept, tid);
    if (r < kMaxNodes) {
      sDst[r] = pl.P + r;
      sSrc[r] = pl.P + tid;
    }
  }
  __syncthreads();
  if (!__syncthreads_or(tid < n_moves && sSrc[tid] != sDst[tid])) return;

  const int total = n_moves * kSliceChunks;
  uint8_t* base = static_cast<uint8_t*>(which == 0 ? L.k : L.v) + slice * (16 * kSliceChunks);
  const bool paged = L.block_table != nullptr;
  const int cap = paged ? L.max_blocks * L.block_size : L.T_cap;
  auto row_ptr = [&](int pos) -> uint8_t* {
    size_t row;
    if (paged) {
      int blk = L.block_table[static_cast<size_t>(b) * L.max_blocks + pos / L.block_size];
      blk = blk < 0 ? 0 : (blk >= L.num_blocks ? L.num_blocks - 1 : blk);
      row = (static_cast<size_t>(blk) * L.block_size + pos % L.block_size) * Hkv + hkv;
    } else {
      row = (static_cast<size_t>(b) * L.T_cap + pos) * Hkv + hkv;
    }
    return base + row * static_cast<size_t>(row_bytes);
  };

  // Element e = tid + c * kThreads of the move list: row e / kSliceChunks,
  // chunk e % kSliceChunks of the slice.  Four named registers (not an array,
  // which the compiler places in scratch memory).
  static_assert(kMaxChunksPerThread == 4, "one register per chunk below");
  auto src_of = [&](int c, int& m, int& ch) {
    const int e = tid + c * kThreads;
    m = e / kSliceChunks;
    ch = e % kSliceChunks;
    return e < total && sSrc[m] != sDst[m] && sSrc[m] < cap && sDst[m] < cap;
  };
  auto load = [&](int c, uint4& r) {
    int m, ch;
    if (src_of(c, m, ch)) r = *reinterpret_cast<const uint4*>(row_ptr(sSrc[m]) + ch * 16);
  };
  auto store = [&](int c, const uint4& r) {
    int m, ch;
    if (src_of(c, m, ch)) *reinterpret_cast<uint4*>(row_ptr(sDst[m]) + ch * 16) = r;
  };
  uint4 r0 = {}, r1 = {}, r2 = {}, r3 = {};
  load(0, r0);
  load(1, r1);
  load(2, r2);
  load(3, r3);
  __syncthreads();
  store(0, r0);
  store(1, r1);
  store(2, r2);
  store(3, r3);
}

// The metadata of sequence b after the move: kept node of rank r takes slot
// r, with its parent renumbered (-1 under the new root); the path's nodes
// join the prefix.  par_tid: the old parent entry of node tid (tid < n).
// tok_b / cum_b (either may be null): per-node arrays the draft keeps beside
// its tree.  They move with their nodes; cum is re-based to the new root (the
// last verified node), whose own weight is subtracted.  Entries at or past
// the new node count read -1 / -inf.  All threads call it (it synchronises):
// every old value is read before the first write.
__device__ __forceinline__ void rewrite_meta(const Plan& pl, int par_tid, int b, int n_max,
                                             int32_t* prefix_len, int32_t* par_b,
                                             int32_t* n_nodes, int32_t* tok_b, float* cum_b,
                                             const uint64_t* sKept) {
  const int tid = threadIdx.x;
  int newpar = -1, slot = -1, tk = -1;
  float w = 0.f;
  const float base = (cum_b != nullptr && pl.v_last >= 0) ? cum_b[pl.v_last] : 0.f;
  if (tid < pl.n && mask_bit(sKept, tid)) {
    const int pp = clamp_parent(par_tid, tid);
    slot = kept_rank(sKept, tid);
    newpar = (pp == pl.v_last || pp < 0) ? -1 : kept_rank(sKept, pp);
    if (tok_b != nullptr) tk = tok_b[tid];
    if (cum_b != nullptr) w = cum_b[tid];
  }
  __syncthreads();
  if (tid < n_max && tid >= pl.n_kept) {
    par_b[tid] = -1;
    if (tok_b != nullptr) tok_b[tid] = -1;
    if (cum_b != nullptr) cum_b[tid] = -INFINITY;
  }
  if (slot >= 0) {
    par_b[slot] = newpar;
    if (tok_b != nullptr) tok_b[slot] = tk;
    if (cum_b != nullptr) cum_b[slot] = w - base;
  }
  if (tid == 0) {
    prefix_len[b] = pl.P + pl.k;
    n_nodes[b] = pl.n_kept;
  }
}

__global__ __launch_bounds__(kThreads) void reroot_move_kernel(
    RerootLayers layers, int n_layers, const int32_t* prefix_len, const int32_t* parent,
    const int32_t* n_nodes, const int32_t* path, const int32_t* path_len, const uint8_t* keep,
    int n_max, int Hkv, int row_bytes) {
  __shared__ uint64_t sAnc[kMaxNodes][kMaskWords];
  __shared__ int sJump[kMaxNodes];
  __shared__ uint64_t sKept[kMaskWords];
  __shared__ int sPath[kMaxNodes];
  __shared__ int sSrc[kMaxNodes];
  __shared__ int sDst[kMaxNodes];

  const int n_slices = row_bytes / (16 * kSliceChunks);
  const int hkv = blockIdx.x / n_slices;
  const int slice = blockIdx.x % n_slices;
  const int which = blockIdx.y;  // 0: K, 1: V
  const int b = blockIdx.z / n_layers;
  const int layer = blockIdx.z % n_layers;

  const Plan pl = make_plan(prefix_len, parent, n_nodes, path, path_len, keep, b, n_max, sAnc,
                            sJump, sKept, sPath);
  if (!pl.valid || pl.k == 0) return;  // nothing moves (keep: no-op; drop: metadata only)
  move_slice(layers.l[layer], b, hkv, which, slice, Hkv, row_bytes, pl, sPath, sKept, sSrc, sDst);
}

__global__ __launch_bounds__(kThreads) void reroot_meta_kernel(int32_t* prefix_len,
                                                               int32_t* parent, int32_t* n_nodes,
                                                               const int32_t* path,
                                                               const int32_t* path_len,
                                                               const uint8_t* keep, int n_max,
                                                               int32_t* tok, float* cum) {
  __shared__ uint64_t sAnc[kMaxNodes][kMaskWords];
  __shared__ int sJump[kMaxNodes];
  __shared__ uint64_t sKept[kMaskWords];
  __shared__ int sPath[kMaxNodes];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* par_b = parent + static_cast<size_t>(b) * n_max;
  const Plan pl = make_plan(prefix_len, parent, n_nodes, path, path_len, keep, b, n_max, sAnc,
                            sJump, sKept, sPath);
  if (!pl.valid || (pl.k == 0 && pl.keep)) return;
  const int par_tid = tid < pl.n ? par_b[tid] : -1;
  rewrite_meta(pl, par_tid, b, n_max, prefix_len, par_b, n_nodes,
               tok != nullptr ? tok + static_cast<size_t>(b) * n_max : nullptr,
               cum != nullptr ? cum + static_cast<size_t>(b) * n_max : nullptr, sKept);
}

// Greedy acceptance, re-root move and metadata in one launch (grid as the
// move launch; with no layers, one group per sequence).  Every group reads the
// tree from the snapshot the argmax launch took (snap: prefix_len, parent,
// n_nodes before this call) and amax [B][n_max], the target's argmax per
// node.  first: this is the call's first launch; its (slice 0, K, layer 0)
// groups write path / path_len / bonus and the new metadata into the live
// arrays, which no group of any launch of the call reads.
__global__ __launch_bounds__(kThreads) void accept_reroot_kernel(
    RerootLayers layers, int n_layers, int32_t* prefix_len, int32_t* parent, int32_t* n_nodes,
    MetaSnapshot snap, const int32_t* tok, const int32_t* root_tok, const int32_t* amax,
    const uint8_t* keep, int n_max, int Hkv, int row_bytes, int32_t* path, int32_t* path_len,
    int32_t* bonus, int first) {
  __shared__ uint64_t sAnc[kMaxNodes][kMaskWords];
  __shared__ int sJump[kMaxNodes];
  __shared__ uint64_t sKept[kMaskWords];
  __shared__ int sPath[kMaxNodes];
  __shared__ int sSrc[kMaxNodes];
  __shared__ int sDst[kMaxNodes];
  __shared__ int sA[kMaxNodes];
  __shared__ uint64_t sAcc[kMaskWords];
  __shared__ unsigned long long sKey[kThreads / 64];
  static_assert(kThreads == kWalkThreads, "one thread per node slot");

  const bool moves = n_layers > 0;
  const int nl = moves ? n_layers : 1;
  const int n_slices = row_bytes / (16 * kSliceChunks);
  const int hkv = moves ? blockIdx.x / n_slices : 0;
  const int slice = moves ? blockIdx.x % n_slices : 0;
  const int which = blockIdx.y;  // 0: K, 1: V
  const int b = blockIdx.z / nl;
  const int layer = blockIdx.z % nl;
  const int tid = threadIdx.x;
  const bool writer = first && blockIdx.x == 0 && blockIdx.y == 0 && layer == 0;

  // every global load first (slot index clamped)
  const int ic = tid < n_max ? tid : n_max - 1;
  const size_t row = static_cast<size_t>(b) * n_max;
  int n = snap.n_nodes_out[b];
  const int P = snap.prefix_len_out[b];
  const int kp = keep[b];
  const int rt = root_tok[b];
  const int a_i = amax[row + ic];
  const int par_i = snap.parent_out[row + ic];
  const int tok_i = tok[row + ic];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);

  const Accepted r = greedy_accept(n, rt, a_i, par_i, tok_i, sAnc, sJump, sA, sAcc, sKey);
  const int pslot = path_slot(sAnc, r.best, tid, n);
  if (pslot >= 0) sPath[pslot] = tid;
  if (writer) {
    int32_t* path_b = path + row;
    if (tid < n_max) {
      if (pslot >= 0) path_b[pslot] = tid;
      if (tid >= r.len) path_b[tid] = -1;
    }
    if (tid == 0) {
      path_len[b] = r.len;
      bonus[b] = r.best >= 0 ? sA[r.best] : rt;
    }
  }
  Plan pl;
  pl.P = P;
  pl.n = n;
  pl.k = r.len;
  pl.keep = kp != 0;
  pl.valid = P >= 0;
  pl.v_last = r.len > 0 ? r.best : -1;
  plan_kept(pl, sAnc, sKept);  // synchronises (sPath complete)
  if (writer && pl.valid && !(pl.k == 0 && pl.keep))
    rewrite_meta(pl, par_i, b, n_max, prefix_len, parent + row, n_nodes, nullptr, nullptr, sKept);
  if (!moves || !pl.valid || pl.k == 0) return;
  move_slice(layers.l[layer], b, hkv, which, slice, Hkv, row_bytes, pl, sPath, sKept, sSrc, sDst);
}

}  // namespace

hipError_t launch_reroot_move(const RerootLayers& layers, int n_layers, const int32_t* prefix_len,
                              const int32_t* parent, const int32_t* n_nodes, const int32_t* path,
                              const int32_t* path_len, const uint8_t* keep, int B, int n_max,
                              int Hkv, int row_bytes, hipStream_t s) {
  // row_bytes is 128, 256 or 512 (d = 64 or 128, bf16 or fp32): whole slices.
  dim3 grid(Hkv * (row_bytes / (16 * kSliceChunks)), 2, B * n_layers);
  return launch(reroot_move_kernel, grid, dim3(kThreads), s, layers, n_layers, prefix_len, parent,
                n_nodes, path, path_len, keep, n_max, Hkv, row_bytes);
}

hipError_t launch_reroot_meta(int32_t* prefix_len, int32_t* parent, int32_t* n_nodes,
                              const int32_t* path, const int32_t* path_len, const uint8_t* keep,
                              int B, int n_max, int32_t* tok, float* cum, hipStream_t s) {
  return launch(reroot_meta_kernel, dim3(B), dim3(kThreads), s, prefix_len, parent, n_nodes, path,
                path_len, keep, n_max, tok, cum);
}

hipError_t launch_accept_reroot(const RerootLayers& layers, int n_layers, int32_t* prefix_len,
                                int32_t* parent, int32_t* n_nodes, const MetaSnapshot& snap,
                                const int32_t* tok, const int32_t* root_tok, const int32_t* amax,
                                const uint8_t* keep, int B, int n_max, int Hkv, int row_bytes,
                                int32_t* path, int32_t* path_len, int32_t* bonus, int first,
                                hipStream_t s) {
  // with no layers, one group per sequence; else the move launch's grid
  const dim3 grid = n_layers > 0 ? dim3(Hkv * (row_bytes / (16 * kSliceChunks)), 2, B * n_layers)
                                 : dim3(1, 1, B);
  return launch(accept_reroot_kernel, grid, dim3(kThreads), s, layers, n_layers, prefix_len,
                parent, n_nodes, snap, tok, root_tok, amax, keep, n_max, Hkv, row_bytes, path,
                path_len, bonus, first);
}

}  // namespace ta
