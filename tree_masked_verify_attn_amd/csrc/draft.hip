// Draft side of one draft-worker iteration (SwiftSpec summary, Section 3.1.1
// Algorithm 1, steps Synchronize, Re-root and Select; Section 3.1.2
// Figure 2; Section 3.2, the update procedure).
//
//   token walk: the target's verified tokens are followed down the draft tree
//     from the root; each one found among the current node's children moves
//     the walk to that child (the lowest index among equal sibling tokens).
//     The matched nodes are the re-root path; keep = every token matched (the
//     last one is the new root and its subtree stays), otherwise the walk
//     stopped at a token that is not in the tree and a new tree starts.  The
//     outputs feed tree_cache_reroot unchanged.
//   select: the bs nodes of largest cumulative score (ties: lower index) are
//     the subtree to send: with scores that do not increase from a parent to
//     its child they are closed under ancestors and maximise the expected
//     accepted tokens (the sum of exp(cum)).  They are written in node order
//     with parents renumbered inside the selection.
//
// One work group per sequence, one thread per node (n_max <= 256).
#include <limits.h>

#include "ta_device.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void token_walk_kernel(
    const int32_t* parent, const int32_t* tok, const int32_t* n_nodes, const int32_t* verified,
    const int32_t* verified_len, int n_max, int m_max, int32_t* path, int32_t* path_len,
    uint8_t* keep) {
  __shared__ int sVer[kWalkMaxTokens];
  __shared__ int sMin[kWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  int len = verified_len[b];
  len = len < 0 ? 0 : (len > m_max ? m_max : len);
  for (int k = tid; k < len; k += kThreads) sVer[k] = verified[static_cast<size_t>(b) * m_max + k];
  const int my_par = tid < n ? clamp_parent(parent[static_cast<size_t>(b) * n_max + tid], tid) : -2;
  const int my_tok = tid < n ? tok[static_cast<size_t>(b) * n_max + tid] : 0;
  __syncthreads();

  int cur = -1;  // the root
  int k = 0;
  for (; k < len; ++k) {
    const bool match = tid < n && my_par == cur && my_tok == sVer[k];
    const uint64_t m = __ballot(match);
    if (lane == 0) sMin[wave] = m != 0 ? wave * 64 + __ffsll(static_cast<long long>(m)) - 1 : INT_MAX;
    __syncthreads();
    int nxt = sMin[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) nxt = min(nxt, sMin[w]);
    __syncthreads();  // sMin is rewritten by the next step
    if (nxt == INT_MAX) break;  // uniform: the token is not in the tree
    if (tid == 0) path[static_cast<size_t>(b) * n_max + k] = nxt;
    cur = nxt;
  }
  if (tid == 0) {
    path_len[b] = k;
    keep[b] = k == len ? 1 : 0;
  }
}

__global__ __launch_bounds__(kThreads) void select_subtree_kernel(
    const float* cum, const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
    int n_max, int bs, int32_t* sel_node, int32_t* sel_parent, int32_t* sel_tok,
    int32_t* sel_n) {
  __shared__ float sCum[kThreads];
  __shared__ int sPos[kThreads];
  __shared__ int sScan[kWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const int take = bs < n ? bs : n;
  float c = -INFINITY;
  int p = -1, t = 0;
  if (tid < n) {
    c = cum[static_cast<size_t>(b) * n_max + tid];
    c = c != c ? -INFINITY : c;  // NaN ranks last
    p = clamp_parent(parent[static_cast<size_t>(b) * n_max + tid], tid);
    t = tok[static_cast<size_t>(b) * n_max + tid];
  }
  sCum[tid] = c;
  __syncthreads();
  // rank under (score desc, index asc): a permutation of 0 .. n-1
  int rank = 0;
  if (tid < n) {
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float cj = sCum[j];
      rank += (cj > c || (cj == c && j < tid)) ? 1 : 0;
    }
  }
  const bool chosen = tid < n && rank < take;
  // position among the chosen nodes, in node order
  const uint64_t m = __ballot(chosen);
  if (lane == 0) sScan[wave] = __popcll(m);
  __syncthreads();
  int pos = __popcll(m & ((1ull << lane) - 1ull));
  for (int w = 0; w < wave; ++w) pos += sScan[w];
  sPos[tid] = chosen ? pos : -1;
  __syncthreads();
  const size_t o = static_cast<size_t>(b) * bs;
  if (chosen) {
    sel_node[o + pos] = tid;
    sel_parent[o + pos] = p >= 0 ? sPos[p] : -1;  // -1 also for a parent left out (rising scores)
    sel_tok[o + pos] = t;
  }
  for (int k = take + tid; k < bs; k += kThreads) {
    sel_node[o + k] = -1;
    sel_parent[o + k] = -1;
    sel_tok[o + k] = 0;
  }
  if (tid == 0) sel_n[b] = take;
}

}  // namespace

hipError_t launch_token_walk(const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
                             const int32_t* verified, const int32_t* verified_len, int B,
                             int n_max, int m_max, int32_t* path, int32_t* path_len,
                             uint8_t* keep, hipStream_t s) {
  return launch(token_walk_kernel, dim3(B), dim3(kThreads), s, parent, tok, n_nodes, verified,
                verified_len, n_max, m_max, path, path_len, keep);
}

hipError_t launch_select_subtree(const float* cum, const int32_t* parent, const int32_t* tok,
                                 const int32_t* n_nodes, int B, int n_max, int bs,
                                 int32_t* sel_node, int32_t* sel_parent, int32_t* sel_tok,
                                 int32_t* sel_n, hipStream_t s) {
  return launch(select_subtree_kernel, dim3(B), dim3(kThreads), s, cum, parent, tok, n_nodes, n_max,
                bs, sel_node, sel_parent, sel_tok, sel_n);
}

}  // namespace ta
