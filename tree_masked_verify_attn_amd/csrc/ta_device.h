// Device helpers shared by the kernels of libtreeattn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ta_internal.h"

namespace ta {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxNodes = TA_MAX_NODES;        // 256
constexpr int kMaskWords = kMaxNodes / 64;     // 4 x 64-bit words per ancestor mask

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// wave64 reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---------------------------------------------------------------------------
// Sequence bounds, clamped so that no access leaves the documented buffers.
// Returns false when the sequence has nothing to do or its sizes are invalid.
// ---------------------------------------------------------------------------
struct SeqBounds {
  int P;  // prefix length
  int n;  // tree nodes
  int T;  // P + n, <= T_cap
};

// The same from the raw prefix_len[b] and n_nodes[b].
__device__ __forceinline__ bool seq_bounds_of(int P, int n, int n_max, int T_cap, SeqBounds& sb) {
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  if (P < 0 || n == 0) return false;
  if (static_cast<long long>(P) + n > T_cap) return false;
  sb.P = P;
  sb.n = n;
  sb.T = P + n;
  return true;
}
__device__ __forceinline__ bool seq_bounds(const int32_t* prefix_len, const int32_t* n_nodes,
                                           int b, int n_max, int T_cap, SeqBounds& sb) {
  return seq_bounds_of(prefix_len[b], n_nodes[b], n_max, T_cap, sb);
}

// Parent of node i with invalid entries read as -1 (child of the root).
__device__ __forceinline__ int clamp_parent(int p, int i) { return (p >= -1 && p < i) ? p : -1; }

// ---------------------------------------------------------------------------
// Ancestor bitmasks by pointer doubling, one node per thread (blockDim = 256).
// anc[i] gets bit j set iff j == i or j is an ancestor of i.  After round k
// each mask covers ancestors up to distance 2^k - 1, so 8 rounds reach any
// depth below 256; the loop stops once every jump pointer has left the tree.
// All threads of the block must call this (it synchronises).  par_i is this
// thread's parent entry (read only when threadIdx.x < n), so that callers can
// load it together with their other inputs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void build_ancestor_masks_of(int par_i, int n,
                                                        uint64_t (*anc)[kMaskWords], int* jump) {
  const int i = threadIdx.x;
  uint64_t a[kMaskWords] = {0, 0, 0, 0};
  int j = -1;
  if (i < n) {
    a[i >> 6] = 1ull << (i & 63);
    j = clamp_parent(par_i, i);
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) anc[i][w] = a[w];
    jump[i] = j;
  }
  int live = __syncthreads_or(j >= 0);
  while (live) {
    int jn = -1;
    if (i < n && j >= 0) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) a[w] |= anc[j][w];
      jn = jump[j];
    }
    __syncthreads();
    if (i < n) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) anc[i][w] = a[w];
      jump[i] = jn;
    }
    j = jn;
    live = __syncthreads_or(j >= 0);
  }
}
__device__ __forceinline__ void build_ancestor_masks(const int32_t* parent_b, int n,
                                                     uint64_t (*anc)[kMaskWords], int* jump) {
  build_ancestor_masks_of(threadIdx.x < n ? parent_b[threadIdx.x] : -1, n, anc, jump);
}

__device__ __forceinline__ bool mask_bit(const uint64_t* m, int j) {
  return (m[j >> 6] >> (j & 63)) & 1ull;
}

// Element offset of (sequence b, position t, kv head hkv, channel 0).
__device__ __forceinline__ size_t kv_offset(const int32_t* block_table, int block_size,
                                            int max_blocks, int num_blocks, int T_cap, int Hkv,
                                            int d, int b, int t, int hkv) {
  if (block_table != nullptr) {
    int blk = block_table[static_cast<size_t>(b) * max_blocks + t / block_size];
    blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    return ((static_cast<size_t>(blk) * block_size + (t % block_size)) * Hkv + hkv) *
           static_cast<size_t>(d);
  }
  return ((static_cast<size_t>(b) * T_cap + t) * Hkv + hkv) * static_cast<size_t>(d);
}

}  // namespace ta
