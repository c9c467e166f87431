// Generic tree-masked attention kernel: fp32 arithmetic on the vector ALUs,
// fp32 or bf16 storage, d in {64, 128}.  It serves the fp32 workloads and any
// shape the MFMA kernel does not take.
//
// What it computes (SwiftSpec summary, Section 3.1.3 Figure 3 and Section 3.2;
// draft-length co-design article, key mechanism): for each query row (tree
// node i, query head h) softmax attention over the P prefix positions and the
// tree positions of i's ancestors and i itself, with KV head h / G.
//
// Work decomposition: one work group per (sequence x KV head, split, row tile).
// A row tile is 32 query rows (node-major, the G heads of a node adjacent);
// a split is `chunk` consecutive KV positions.  Each of the 4 waves owns 8
// rows; a 64-position K/V tile is staged in LDS as fp32, lane j scores
// position j, and each lane accumulates 2 (d=128) or 1 (d=64) output
// channels.  A split sequence leaves partial (max, sum, output) triples in the
// workspace for the combine launch (attn_merge.hip).
#include "ta_device.h"

namespace ta {
namespace {

constexpr int kRows = 32;       // query rows per work group
constexpr int kTile = 64;       // KV positions per LDS tile
constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(AttnParams p) {
  constexpr int C = D / 64;  // output channels per lane
  __shared__ float sK[kTile][D + 1];
  __shared__ float sV[kTile][D];
  __shared__ float sQ[kRows][D];
  __shared__ float sP[kRows][kTile];
  __shared__ uint64_t sAnc[kMaxNodes][kMaskWords];
  __shared__ int sJump[kMaxNodes];
  __shared__ int sNode[kRows];

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
  const int wave = tid >> 6;

  SeqBounds sb;
  if (!seq_bounds(p.prefix_len, p.n_nodes, b, p.n_max, p.T_cap, sb)) return;
  const int nsplit = (sb.T + p.chunk - 1) / p.chunk;
  if (split >= nsplit) return;
  const int t_begin = split * p.chunk;
  const int t_end = min(sb.T, t_begin + p.chunk);

  // Query rows of this tile: row r -> (node slot r / G, head hkv*G + r % G).
  const int R = p.n_q * p.G;
  const int row0 = rtile * kRows;
  if (tid < kRows) {
    const int r = row0 + tid;
    int node = -1;
    if (r < R) {
      const int slot = r / p.G;
      node = p.expand ? sb.n - p.n_q + slot : slot;
      if (node < 0 || node >= sb.n) node = -1;
    }
    sNode[tid] = node;
  }
  __syncthreads();
  {
    bool any = false;
    for (int r = 0; r < kRows; ++r) any |= sNode[r] >= 0;
    if (!any) return;  // uniform across the block
  }

  const T* __restrict__ Q = static_cast<const T*>(p.q);
  const T* __restrict__ Kp = static_cast<const T*>(p.k);
  const T* __restrict__ Vp = static_cast<const T*>(p.v);

  // Stage the tile's queries, pre-multiplied by scale*log2(e).
  for (int e = tid; e < kRows * D; e += kThreads) {
    const int r = e / D, c = e % D;
    float val = 0.f;
    if (sNode[r] >= 0) {
      const int gr = row0 + r;
      const int slot = gr / p.G, g = gr % p.G;
      const size_t qo = ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * D + c;
      val = load_elem<T>(Q, qo) * p.scale_log2;
    }
    sQ[r][c] = val;
  }
  // Ancestor masks are only needed when this split reaches the tree cache.
  const bool has_tree = t_end > sb.P;
  if (has_tree) build_ancestor_masks(p.parent + static_cast<size_t>(b) * p.n_max, sb.n, sAnc, sJump);
  __syncthreads();

  float m[8], l[8], o[8][C];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    m[rr] = -INFINITY;
    l[rr] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) o[rr][c] = 0.f;
  }

  for (int tb = t_begin; tb < t_end; tb += kTile) {
    const int nt = min(kTile, t_end - tb);
    // K/V tile -> LDS (fp32); rows past the end are zero so that 0 * V stays 0.
    for (int e = tid; e < kTile * D; e += kThreads) {
      const int j = e / D, c = e % D;
      float kv = 0.f, vv = 0.f;
      if (j < nt) {
        const size_t off = kv_offset(p.block_table, p.block_size, p.max_blocks, p.num_blocks,
                                     p.T_cap, p.Hkv, D, b, tb + j, hkv);
        kv = load_elem<T>(Kp, off + c);
        vv = load_elem<T>(Vp, off + c);
      }
      sK[j][c] = kv;
      sV[j][c] = vv;
    }
    __syncthreads();

    const int t = tb + lane;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = wave * 8 + rr;
      const int node = sNode[r];
      float pj = 0.f;
      if (node >= 0) {  // wave-uniform
        float s = 0.f;
#pragma unroll 8
        for (int c = 0; c < D; ++c) s = fmaf(sQ[r][c], sK[lane][c], s);
        bool vis = lane < nt;
        if (vis && t >= sb.P) vis = mask_bit(sAnc[node], t - sb.P);
        s = vis ? s : -INFINITY;
        const float mx = wave_max(s);
        const float m_new = fmaxf(m[rr], mx);
        pj = vis ? exp2f(s - m_new) : 0.f;
        const float alpha = (m[rr] == -INFINITY) ? 0.f : exp2f(m[rr] - m_new);
        l[rr] = l[rr] * alpha + wave_sum(pj);
        m[rr] = m_new;
#pragma unroll
        for (int c = 0; c < C; ++c) o[rr][c] *= alpha;
      }
      sP[r][lane] = pj;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = wave * 8 + rr;
      if (sNode[r] < 0) continue;
      for (int j = 0; j < nt; ++j) {
        const float pj = sP[r][j];
#pragma unroll
        for (int c = 0; c < C; ++c) o[rr][c] = fmaf(pj, sV[j][lane + 64 * c], o[rr][c]);
      }
    }
    __syncthreads();
  }

  T* __restrict__ Out = static_cast<T*>(p.out);
  auto out_index = [&](int r, int c) -> size_t {
    const int gr = row0 + r;
    const int slot = gr / p.G, g = gr % p.G;
    return ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * D + c;
  };
  auto lse_index = [&](int r) -> size_t {
    const int gr = row0 + r;
    const int slot = gr / p.G, g = gr % p.G;
    return (static_cast<size_t>(b) * p.Hq + hkv * p.G + g) * p.n_q + slot;
  };
  constexpr float kLn2 = 0.69314718055994530942f;

  if (nsplit == 1) {
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = wave * 8 + rr;
      if (sNode[r] < 0) continue;
      const float inv = 1.f / l[rr];
#pragma unroll
      for (int c = 0; c < C; ++c) store_elem<T>(Out, out_index(r, lane + 64 * c), o[rr][c] * inv);
      if (p.lse != nullptr && lane == 0) p.lse[lse_index(r)] = (m[rr] + log2f(l[rr])) * kLn2;
    }
    return;
  }

  // Publish this split's partial result for the combine launch.
  const int tile_id = bh * p.n_row_tiles + rtile;
  const size_t part = static_cast<size_t>(tile_id) * p.n_split;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int r = wave * 8 + rr;
    float* po = p.ws_o + ((part + split) * kRows + r) * D;
#pragma unroll
    for (int c = 0; c < C; ++c) po[lane + 64 * c] = o[rr][c];
    if (lane == 0) {
      p.ws_ml[((part + split) * kRows + r) * 2 + 0] = m[rr];
      p.ws_ml[((part + split) * kRows + r) * 2 + 1] = l[rr];
    }
  }
  // the combine launch (attn_merge.hip) finishes split sequences
}

}  // namespace

hipError_t launch_attn_generic(const AttnParams& p, int dtype, hipStream_t s) {
  dim3 grid(p.B * p.Hkv, p.n_split, p.n_row_tiles);
  dim3 block(kThreads);
  if (dtype == TA_F32)
    return p.d == 64 ? launch(attn_generic_kernel<float, 64>, grid, block, s, p)
                     : launch(attn_generic_kernel<float, 128>, grid, block, s, p);
  return p.d == 64 ? launch(attn_generic_kernel<uint16_t, 64>, grid, block, s, p)
                   : launch(attn_generic_kernel<uint16_t, 128>, grid, block, s, p);
}

size_t attn_ws_bytes(int tiles, int n_split, int rows_per_tile, int d) {
  if (n_split <= 1) return 0;
  const size_t parts = static_cast<size_t>(tiles) * n_split * rows_per_tile;
  size_t bytes = parts * d * sizeof(float);        // ws_o
  bytes += parts * 2 * sizeof(float);              // ws_ml
  return bytes;
}

}  // namespace ta
