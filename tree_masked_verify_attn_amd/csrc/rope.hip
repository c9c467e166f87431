// Rotary position embedding at tree positions and the KV append of the new
// nodes (SwiftSpec summary, Section 3.3: the masked attention takes the
// position embedding, RoPE; Section 3.2: a node's KV stays where it was
// computed, so its position is that of its token in the sequence it
// continues).
//
// Node i of a sequence with prefix length P sits at position P - 1 + depth(i)
// (the root, the last prefix token, at P - 1).  Each channel pair (j, j + d/2)
// of a query row and of the node's key turns by position * base^(-2j/d); the
// rotated key and the value go to cache row P + i.  This runs as its own
// small launch before the attention call: the rows it touches are the new
// nodes' (a few hundred KiB at most), and the attention kernels keep their
// registers for the KV stream.
//
// One work group per (query slot, sequence): the node's depth from a walk up
// the parent links in LDS, the angles reduced modulo 2 pi in double precision
// (positions reach tens of thousands, where a float product would be off by
// ~1e-3 rad), cos/sin tabulated in LDS, then every query head, key head and
// value head of the slot.
#include "ta_device.h"

namespace ta {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_append_kernel(RopeParams p) {
  __shared__ int sPar[kMaxNodes];
  __shared__ float sCos[64], sSin[64];
  __shared__ int sDepth;
  const int s = blockIdx.x;  // query slot
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  SeqBounds sb;
  if (!seq_bounds(p.prefix_len, p.n_nodes, b, p.n_max, p.T_cap, sb)) return;
  const int node = p.expand ? sb.n - p.n_q + s : s;
  if (node < 0 || node >= sb.n) return;  // uniform: no node in this slot
  for (int i = tid; i < sb.n; i += kThreads)
    sPar[i] = clamp_parent(p.parent[static_cast<size_t>(b) * p.n_max + i], i);
  __syncthreads();
  if (tid == 0) {
    int dep = 0;
    for (int v = node; v >= 0; v = sPar[v]) ++dep;  // parents precede children: ends
    sDepth = dep;
  }
  __syncthreads();
  const int pos = sb.P - 1 + sDepth;
  const int half = p.d / 2;
  if (tid < half) {
    const double inv = pow(static_cast<double>(p.base), -2.0 * tid / p.d);
    const double two_pi = 6.283185307179586476925286766559;
    double a = fmod(static_cast<double>(pos) * inv, two_pi);
    sCos[tid] = static_cast<float>(cos(a));
    sSin[tid] = static_cast<float>(sin(a));
  }
  __syncthreads();

  const T* q = static_cast<const T*>(p.q_in);
  T* qo = static_cast<T*>(p.q_out);
  const size_t qrow = (static_cast<size_t>(b) * p.n_q + s) * p.Hq * p.d;
  // queries: Hq x half pairs
  for (int e = tid; e < p.Hq * half; e += kThreads) {
    const int h = e / half, j = e % half;
    const size_t o = qrow + static_cast<size_t>(h) * p.d + j;
    const float x0 = ld<T>(q, o), x1 = ld<T>(q, o + half);
    st<T>(qo, o, x0 * sCos[j] - x1 * sSin[j]);
    st<T>(qo, o + half, x1 * sCos[j] + x0 * sSin[j]);
  }
  // keys (rotated) and values (copied) into cache row P + node
  const T* kn = static_cast<const T*>(p.k_new);
  const T* vn = static_cast<const T*>(p.v_new);
  T* K = static_cast<T*>(p.k);
  T* Vc = static_cast<T*>(p.v);
  const size_t krow = (static_cast<size_t>(b) * p.n_q + s) * p.Hkv * p.d;
  for (int e = tid; e < p.Hkv * half; e += kThreads) {
    const int h = e / half, j = e % half;
    const size_t i = krow + static_cast<size_t>(h) * p.d + j;
    const size_t c = kv_offset(p.block_table, p.block_size, p.max_blocks, p.num_blocks, p.T_cap,
                               p.Hkv, p.d, b, sb.P + node, h) + j;
    const float x0 = ld<T>(kn, i), x1 = ld<T>(kn, i + half);
    st<T>(K, c, x0 * sCos[j] - x1 * sSin[j]);
    st<T>(K, c + half, x1 * sCos[j] + x0 * sSin[j]);
    Vc[c] = vn[i];
    Vc[c + half] = vn[i + half];
  }
}

}  // namespace

hipError_t launch_rope_append(const RopeParams& p, int dtype, hipStream_t s) {
  const dim3 grid(p.n_q, p.B);
  if (dtype == TA_F32) return launch(rope_append_kernel<float>, grid, dim3(kThreads), s, p);
  return launch(rope_append_kernel<uint16_t>, grid, dim3(kThreads), s, p);
}

}  // namespace ta
