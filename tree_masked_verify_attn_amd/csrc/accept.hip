// Greedy longest accepted path (draft-length co-design article: accept draft
// tokens up to the first mismatch with the target's greedy choice, then the
// target's own token; SwiftSpec summary, Section 3.1.2 Figure 2: the target
// returns the root, the accepted nodes and one new token).
//
// Two launches:
//   1. argmax: one 1024-thread work group per (node, sequence) scans the
//      node's logits row with batches of 16-byte loads issued back to back
//      and a wave64 (value, index) max-reduction; ties go to the lowest index.  The result a[i] is parked in path[b][i].
//   2. path: one work group per sequence, one thread per node.  Ancestor
//      bitmasks come from pointer doubling; "token matches the target's
//      choice after the parent" is a wave ballot into a 256-bit mask; a node
//      is accepted when its ancestor mask has no bit outside that mask; the
//      deepest accepted node (popcount of its mask, lowest index on ties)
//      wins and its mask, read in index order, is the path.
#include "ta_device.h"
#include "tree_walk.h"

namespace ta {
namespace {

constexpr int kThreads = 256;

struct ArgMax {
  float v;
  int i;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ __forceinline__ void consider(ArgMax& best, float v, int i) {
  if (v > best.v) {  // indices grow within a thread: strict '>' keeps the first
    best.v = v;
    best.i = i;
  }
}

// Loads per thread issued back to back before any of them is consumed: a row
// of 32000 fp32 logits is 8000 16-byte vectors, under 8 per thread of a
// 1024-thread group, so one batch of loads covers the row.
constexpr int kArgThreads = 1024;
constexpr int kArgUnroll = 8;

template <bool kBf16>
__global__ __launch_bounds__(kArgThreads) void argmax_kernel(const void* logits,
                                                             const int32_t* n_nodes, int n_max,
                                                             int V, int32_t* path,
                                                             MetaSnapshot snap) {
  const int i = blockIdx.x;
  const int b = blockIdx.y;
  if (snap.parent != nullptr && i == 0) {  // the sequence's metadata as it is now
    const size_t row = static_cast<size_t>(b) * n_max;
    for (int t = threadIdx.x; t < n_max; t += kArgThreads) snap.parent_out[row + t] = snap.parent[row + t];
    if (threadIdx.x == 0) {
      snap.prefix_len_out[b] = snap.prefix_len[b];
      snap.n_nodes_out[b] = n_nodes[b];
    }
  }
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  if (i >= n) return;
  const int tid = threadIdx.x;
  ArgMax best{-INFINITY, 0x7fffffff};
  const size_t row = (static_cast<size_t>(b) * n_max + i) * static_cast<size_t>(V);
  constexpr int kPer = kBf16 ? 8 : 4;  // logits per 16-byte vector
  const void* xrow = kBf16 ? static_cast<const void*>(static_cast<const uint16_t*>(logits) + row)
                           : static_cast<const void*>(static_cast<const float*>(logits) + row);
  const bool vec = (V % kPer == 0) && ((reinterpret_cast<uintptr_t>(xrow) & 15) == 0);
  int start = 0;
  if (vec) {
    const u32x4* x4 = static_cast<const u32x4*>(xrow);
    const int nv = V / kPer;
    for (int base = 0; base < nv; base += kArgThreads * kArgUnroll) {
      u32x4 w[kArgUnroll];
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int j = base + u * kArgThreads + tid;
        // -inf never replaces the running best (strict '>'), so padding is inert.
        constexpr uint32_t kNegInf = kBf16 ? 0xff80ff80u : 0xff800000u;
        w[u] = j < nv ? __builtin_nontemporal_load(x4 + j)
                      : u32x4{kNegInf, kNegInf, kNegInf, kNegInf};
      }
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int j0 = (base + u * kArgThreads + tid) * kPer;
        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (kBf16) {
            consider(best, __uint_as_float(ws[e] << 16), j0 + 2 * e);
            consider(best, __uint_as_float(ws[e] & 0xffff0000u), j0 + 2 * e + 1);
          } else {
            consider(best, __uint_as_float(ws[e]), j0 + e);
          }
        }
      }
    }
    start = V;
  }
  for (int j = start + tid; j < V; j += kArgThreads) {
    const float x = kBf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(xrow)[j])
                          : static_cast<const float*>(xrow)[j];
    consider(best, x, j);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ArgMax other{__shfl_xor(best.v, o, 64), __shfl_xor(best.i, o, 64)};
    best = better(best, other);
  }
  __shared__ ArgMax sBest[kArgThreads / 64];
  if ((tid & 63) == 0) sBest[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    ArgMax r = sBest[0];
    for (int w = 1; w < kArgThreads / 64; ++w) r = better(r, sBest[w]);
    // Every row has at least one element; an all-NaN row reports index 0.
    path[static_cast<size_t>(b) * n_max + i] = (r.i == 0x7fffffff) ? 0 : r.i;
  }
}

__global__ __launch_bounds__(kThreads) void accept_path_kernel(const int32_t* parent,
                                                               const int32_t* tok,
                                                               const int32_t* n_nodes,
                                                               const int32_t* root_tok, int n_max,
                                                               int32_t* path, int32_t* path_len,
                                                               int32_t* bonus) {
  __shared__ uint64_t sAnc[kMaxNodes][kMaskWords];
  __shared__ int sJump[kMaxNodes];
  __shared__ int sA[kMaxNodes];
  __shared__ uint64_t sAcc[kMaskWords];
  __shared__ unsigned long long sKey[kThreads / 64];
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int32_t* par_b = parent + static_cast<size_t>(b) * n_max;
  int32_t* path_b = path + static_cast<size_t>(b) * n_max;
  // every global load first (slot index clamped), so the launch pays one
  // memory latency: the node count, root token, and this slot's argmax
  // (parked by the first launch), parent and token
  const int ic = i < n_max ? i : n_max - 1;
  int n = n_nodes[b];
  const int rt = root_tok[b];
  const int a_i = path_b[ic];
  const int par_i = par_b[ic];
  const int tok_i = tok[static_cast<size_t>(b) * n_max + ic];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);

  const Accepted r = greedy_accept(n, rt, a_i, par_i, tok_i, sAnc, sJump, sA, sAcc, sKey);
  // Write the path: node j of best's mask goes to slot popcount(mask below j).
  if (i < n_max) {
    const int slot = path_slot(sAnc, r.best, i, n);
    if (slot >= 0) path_b[slot] = i;
    if (i >= r.len) path_b[i] = -1;
  }
  if (i == 0) {
    path_len[b] = r.len;
    bonus[b] = r.best >= 0 ? sA[r.best] : rt;
  }
}

}  // namespace

hipError_t launch_argmax(const void* logits, int logit_dtype, const int32_t* n_nodes, int B,
                         int n_max, int V, int32_t* out, const MetaSnapshot& snap, hipStream_t s) {
  dim3 g1(n_max, B);
  return logit_dtype == TA_BF16
             ? launch(argmax_kernel<true>, g1, dim3(kArgThreads), s, logits, n_nodes, n_max, V, out,
                      snap)
             : launch(argmax_kernel<false>, g1, dim3(kArgThreads), s, logits, n_nodes, n_max, V, out,
                      snap);
}

hipError_t launch_accept(const void* logits, int logit_dtype, const int32_t* parent,
                         const int32_t* tok, const int32_t* n_nodes, const int32_t* root_tok,
                         int B, int n_max, int V, int32_t* path, int32_t* path_len,
                         int32_t* bonus, hipStream_t s) {
  hipError_t e = launch_argmax(logits, logit_dtype, n_nodes, B, n_max, V, path, MetaSnapshot{}, s);
  if (e != hipSuccess) return e;
  return launch(accept_path_kernel, dim3(B), dim3(kThreads), s, parent, tok, n_nodes, root_tok,
                n_max, path, path_len, bonus);
}

}  // namespace ta
