// Greedy acceptance of one sequence's draft tree by one 256-thread work group
// (draft-length co-design article: accept draft tokens up to the first
// mismatch with the target's greedy choice, then the target's own token;
// SwiftSpec summary, Section 3.1.2 Figure 2: the target returns the root, the
// accepted nodes and one new token).  Shared by the acceptance launch and the
// fused acceptance + re-root launch, so that both take the same path.
#pragma once
#include "ta_device.h"

namespace ta {

constexpr int kWalkThreads = kMaxNodes;  // one thread per node slot
static_assert(kWalkThreads / 64 == kMaskWords, "one ballot word per wave");

struct Accepted {
  int best;  // deepest accepted node (lowest index on ties), -1 when none
  int len;   // its depth (nodes on its root path), 0 when none
};

// Thread i of a kWalkThreads-thread group owns node i.  a_i: the target's
// argmax after node i; par_i, tok_i: node i's parent and draft token; rt: the
// target's token after the prefix.
// Builds the ancestor masks in sAnc (bit j of sAnc[i]: j is i or an ancestor
// of i) and leaves each node's argmax in sA.  Node i is accepted when every
// node u on its root path has tok[u] == (parent[u] < 0 ? rt : a[parent[u]]):
// "token matches the target's choice after the parent" is a wave ballot into
// a 256-bit mask, and a node is accepted when its ancestor mask has no bit
// outside it.  Synchronises; the result is the same in every thread.
__device__ __forceinline__ Accepted greedy_accept(int n, int rt, int a_i, int par_i, int tok_i,
                                                  uint64_t (*sAnc)[kMaskWords], int* sJump,
                                                  int* sA, uint64_t* sAcc,
                                                  unsigned long long* sKey) {
  const int i = threadIdx.x;
  if (i < n) sA[i] = a_i;
  if (i < kMaskWords) sAcc[i] = 0;
  build_ancestor_masks_of(par_i, n, sAnc, sJump);  // synchronises (also after the writes above)

  bool acc = false;
  if (i < n) {
    const int p = clamp_parent(par_i, i);
    acc = tok_i == (p < 0 ? rt : sA[p]);
  }
  const unsigned long long bal = __ballot(acc);  // 64 nodes per wave -> mask word (i >> 6)
  if ((i & 63) == 0) sAcc[i >> 6] = bal;
  __syncthreads();

  unsigned long long key = 0;  // (depth << 16) | (0xffff - node); 0 = not accepted
  if (i < n) {
    bool ok = true;
    int depth = 0;
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) {
      ok = ok && ((sAnc[i][w] & ~sAcc[w]) == 0);
      depth += __popcll(sAnc[i][w]);
    }
    if (ok) key = (static_cast<unsigned long long>(depth) << 16) | (0xffffu - i);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(key, o, 64);
    key = other > key ? other : key;
  }
  if ((i & 63) == 0) sKey[i >> 6] = key;
  __syncthreads();
  unsigned long long best_key = sKey[0];
#pragma unroll
  for (int w = 1; w < kWalkThreads / 64; ++w) best_key = sKey[w] > best_key ? sKey[w] : best_key;
  Accepted r;
  r.best = best_key ? static_cast<int>(0xffffu - (best_key & 0xffffu)) : -1;
  r.len = best_key ? static_cast<int>(best_key >> 16) : 0;
  return r;
}

// Position of node i on the accepted path (its ancestors come first, as a
// parent's index is below its child's): the number of path nodes below i, or
// -1 when i is not on the path.
__device__ __forceinline__ int path_slot(const uint64_t (*sAnc)[kMaskWords], int best, int i,
                                         int n) {
  if (best < 0 || i >= n || !mask_bit(sAnc[best], i)) return -1;
  int slot = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) {
    const uint64_t m = sAnc[best][w];
    if (w < (i >> 6))
      slot += __popcll(m);
    else if (w == (i >> 6))
      slot += __popcll(m & ((1ull << (i & 63)) - 1ull));
  }
  return slot;
}

}  // namespace ta
