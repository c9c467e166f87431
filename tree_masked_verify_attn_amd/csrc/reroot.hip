// Evolving-tree-cache re-root with in-place KV compaction (SwiftSpec summary,
// Section 3.2 and Figure 4: verified nodes join the prefix cache, the subtree
// under the last verified node is pulled forward to follow it, the rest is
// dropped; KV is moved, never recomputed).
//
// Launch 1 (move): one work group per (KV head, K|V, sequence x layer).  The
// group rebuilds the move list itself from parent/path/keep (ancestor masks by
// pointer doubling, kept-node ranks by popcount), then copies every moved row
// of its own (layer, K|V, head) column slice: all rows are loaded into
// registers, the group synchronises, then all rows are stored.  Because a
// group owns its slice exclusively, a destination row that is another move's
// source is never overwritten before it has been read.
// Launch 2 (metadata): one work group per sequence rewrites parent, n_nodes
// and prefix_len after every layer has been moved (stream order).
#include "ta_device.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunksPerThread = 32;  // 256 rows x 512 B / (256 threads x 16 B)

struct Plan {
  int P, n, k, keep, v_last, n_kept, valid;
};

// Shared by both launches: sequence bounds, path, kept set (as a 256-bit mask
// in sKept) and each kept node's rank (popcount of kept bits below it).
__device__ __forceinline__ Plan make_plan(const int32_t* prefix_len, const int32_t* parent,
                                          const int32_t* n_nodes, const int32_t* path,
                                          const int32_t* path_len, const uint8_t* keep, int b,
                                          int n_max, uint64_t (*sAnc)[kMaskWords], int* sJump,
                                          uint64_t* sKept, int* sPath) {
  Plan pl;
  const int tid = threadIdx.x;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  int k = path_len[b];
  k = k < 0 ? 0 : (k > n ? n : k);
  pl.P = prefix_len[b];
  pl.n = n;
  pl.k = k;
  pl.keep = keep[b] != 0;
  pl.valid = pl.P >= 0;
  if (tid < k) {
    int v = path[static_cast<size_t>(b) * n_max + tid];
    sPath[tid] = v < 0 ? 0 : (v >= n ? n - 1 : v);
  }
  if (tid < kMaskWords) sKept[tid] = 0;
  build_ancestor_masks(parent + static_cast<size_t>(b) * n_max, n, sAnc, sJump);
  pl.v_last = k > 0 ? sPath[k - 1] : -1;
  bool kept = false;
  if (pl.keep && k > 0 && tid < n && tid != pl.v_last) kept = mask_bit(sAnc[tid], pl.v_last);
  const unsigned long long bal = __ballot(kept);
  if ((tid & 63) == 0) sKept[tid >> 6] = bal;
  __syncthreads();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) nk += __popcll(sKept[w]);
  pl.n_kept = nk;
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

  const int hkv = blockIdx.x;
  const int which = blockIdx.y;  // 0: K, 1: V
  const int b = blockIdx.z / n_layers;
  const int layer = blockIdx.z % n_layers;
  const int tid = threadIdx.x;
  const RerootLayer& L = layers.l[layer];

  const Plan pl = make_plan(prefix_len, parent, n_nodes, path, path_len, keep, b, n_max, sAnc,
                            sJump, sKept, sPath);
  if (!pl.valid || pl.k == 0) return;  // nothing moves (keep: no-op; drop: metadata only)

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

  const int cpr = row_bytes / 16;  // 16-byte chunks per row
  const int total = n_moves * cpr;
  uint8_t* base = static_cast<uint8_t*>(which == 0 ? L.k : L.v);
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

  uint4 buf[kMaxChunksPerThread];
#pragma unroll
  for (int c = 0; c < kMaxChunksPerThread; ++c) {
    const int e = tid + c * kThreads;
    if (e < total) {
      const int m = e / cpr, ch = e % cpr;
      const int src = sSrc[m], dst = sDst[m];
      if (src != dst && src < cap && dst < cap)
        buf[c] = *reinterpret_cast<const uint4*>(row_ptr(src) + ch * 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kMaxChunksPerThread; ++c) {
    const int e = tid + c * kThreads;
    if (e < total) {
      const int m = e / cpr, ch = e % cpr;
      const int src = sSrc[m], dst = sDst[m];
      if (src != dst && src < cap && dst < cap)
        *reinterpret_cast<uint4*>(row_ptr(dst) + ch * 16) = buf[c];
    }
  }
}

__global__ __launch_bounds__(kThreads) void reroot_meta_kernel(int32_t* prefix_len,
                                                               int32_t* parent, int32_t* n_nodes,
                                                               const int32_t* path,
                                                               const int32_t* path_len,
                                                               const uint8_t* keep, int n_max) {
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
  // Read every old parent before any write.
  int newpar = -1, slot = -1;
  if (tid < pl.n && mask_bit(sKept, tid)) {
    const int pp = clamp_parent(par_b[tid], tid);
    slot = kept_rank(sKept, tid);
    newpar = (pp == pl.v_last || pp < 0) ? -1 : kept_rank(sKept, pp);
  }
  __syncthreads();
  if (tid < n_max && tid >= pl.n_kept) par_b[tid] = -1;
  if (slot >= 0) par_b[slot] = newpar;
  if (tid == 0) {
    prefix_len[b] = pl.P + pl.k;
    n_nodes[b] = pl.n_kept;
  }
}

}  // namespace

hipError_t launch_reroot_move(const RerootLayers& layers, int n_layers, const int32_t* prefix_len,
                              const int32_t* parent, const int32_t* n_nodes, const int32_t* path,
                              const int32_t* path_len, const uint8_t* keep, int B, int n_max,
                              int Hkv, int row_bytes, hipStream_t s) {
  dim3 grid(Hkv, 2, B * n_layers);
  return launch(reroot_move_kernel, grid, dim3(kThreads), s, layers, n_layers, prefix_len, parent,
                n_nodes, path, path_len, keep, n_max, Hkv, row_bytes);
}

hipError_t launch_reroot_meta(int32_t* prefix_len, int32_t* parent, int32_t* n_nodes,
                              const int32_t* path, const int32_t* path_len, const uint8_t* keep,
                              int B, int n_max, hipStream_t s) {
  return launch(reroot_meta_kernel, dim3(B), dim3(kThreads), s, prefix_len, parent, n_nodes, path,
                path_len, keep, n_max);
}

}  // namespace ta
