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
// ~1e-3 rad; rope_common.h), cos/sin tabulated in LDS, then every query head, key head and
// value head of the slot.  With 16-byte aligned rows a thread moves whole
// 16-byte vectors (a vector of channels j.. and its partner j + d/2 ..), and
// its first four items are loaded before the depth walk and the angles, so
// that those latencies overlap.
#include "rope_common.h"
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
  if (tid < half) rope_cos_sin(pos, rope_inv_freq(p.base, tid, p.d), sCos[tid], sSin[tid]);
  __syncthreads();

  const T* q = static_cast<const T*>(p.q_in);
  T* qo = static_cast<T*>(p.q_out);
  const size_t qrow = (static_cast<size_t>(b) * p.n_q + s) * p.Hq * p.d;
  // queries: Hq x half pairs
  for (int e = tid; e < p.Hq * half; e += kThreads) {
    const int h = e / half, j = e % half;
    const size_t o = qrow + static_cast<size_t>(h) * p.d + j;
    const float x0 = ld<T>(q, o), x1 = ld<T>(q, o + half);
    float y0, y1;
    rope_rotate(x0, x1, sCos[j], sSin[j], y0, y1);
    st<T>(qo, o, y0);
    st<T>(qo, o + half, y1);
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
    float y0, y1;
    rope_rotate(x0, x1, sCos[j], sSin[j], y0, y1);
    st<T>(K, c, y0);
    st<T>(K, c + half, y1);
    Vc[c] = vn[i];
    Vc[c + half] = vn[i + half];
  }
}

// 16-byte vectors as floats (8 bf16 or 4 fp32 values) and back.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(u32x4 w, float (&f)[4]) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[4]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(u32x4 w, float (&f)[8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(ws[i] << 16);
      f[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
    uint32_t ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ws[i] = f32_to_bf16_bits(f[2 * i]) | (static_cast<uint32_t>(f32_to_bf16_bits(f[2 * i + 1])) << 16);
    return u32x4{ws[0], ws[1], ws[2], ws[3]};
  }
};

constexpr int kEarly = 4;  // items per thread whose loads go out before the angles

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_append_vec_kernel(RopeParams p) {
  using VT = Vec16<T>;
  constexpr int kV = VT::N;
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
  const int half = p.d / 2;
  const int hv = half / kV;  // vectors per half row
  // items: query pairs (head, vector), key pairs, value vectors
  const int nQ = p.Hq * hv, nK = p.Hkv * hv, nV = p.Hkv * 2 * hv;
  const int total = nQ + nK + nV;
  const size_t qrow = (static_cast<size_t>(b) * p.n_q + s) * p.Hq * p.d;
  const size_t krow = (static_cast<size_t>(b) * p.n_q + s) * p.Hkv * p.d;
  const T* qi = static_cast<const T*>(p.q_in);
  const T* kn = static_cast<const T*>(p.k_new);
  const T* vn = static_cast<const T*>(p.v_new);
  // source offset of item it: its first vector, and the partner half d/2 on
  auto src = [&](int it, const T*& base, size_t& off) {
    if (it < nQ) {
      base = qi;
      off = qrow + static_cast<size_t>(it / hv) * p.d + (it % hv) * kV;
    } else if (it < nQ + nK) {
      const int k = it - nQ;
      base = kn;
      off = krow + static_cast<size_t>(k / hv) * p.d + (k % hv) * kV;
    } else {
      const int k = it - nQ - nK;  // value vector k of 2 * hv per head
      base = vn;
      off = krow + static_cast<size_t>(k / (2 * hv)) * p.d + (k % (2 * hv)) * kV;
    }
  };
  auto ld = [&](const T* base, size_t off) {
    return *reinterpret_cast<const u32x4*>(base + off);
  };
  // rotate (queries, keys) or copy (values) item it and store it
  auto finish = [&](int it, u32x4 w0, u32x4 w1) {
    if (it >= nQ + nK) {  // value: copy into the cache
      const int k = it - nQ - nK;
      const int h = k / (2 * hv), e = (k % (2 * hv)) * kV;
      const size_t c = kv_offset(p.block_table, p.block_size, p.max_blocks, p.num_blocks, p.T_cap,
                                 p.Hkv, p.d, b, sb.P + node, h) + e;
      *reinterpret_cast<u32x4*>(static_cast<T*>(p.v) + c) = w0;
      return;
    }
    float x0[kV], x1[kV], y0[kV], y1[kV];
    VT::unpack(w0, x0);
    VT::unpack(w1, x1);
    const int j0 = (it < nQ ? it : it - nQ) % hv * kV;
#pragma unroll
    for (int e = 0; e < kV; ++e) rope_rotate(x0[e], x1[e], sCos[j0 + e], sSin[j0 + e], y0[e], y1[e]);
    T* dst;
    size_t o;
    if (it < nQ) {
      dst = static_cast<T*>(p.q_out);
      o = qrow + static_cast<size_t>(it / hv) * p.d + j0;
    } else {
      const int h = (it - nQ) / hv;
      dst = static_cast<T*>(p.k);
      o = kv_offset(p.block_table, p.block_size, p.max_blocks, p.num_blocks, p.T_cap, p.Hkv, p.d,
                    b, sb.P + node, h) + j0;
    }
    *reinterpret_cast<u32x4*>(dst + o) = VT::pack(y0);
    *reinterpret_cast<u32x4*>(dst + o + half) = VT::pack(y1);
  };

  // the first items' loads, then the parents
  u32x4 w0[kEarly], w1[kEarly];
#pragma unroll
  for (int i = 0; i < kEarly; ++i) {
    const int it = tid + i * kThreads;
    w0[i] = u32x4{0u, 0u, 0u, 0u};
    w1[i] = w0[i];
    if (it < total) {
      const T* base;
      size_t off;
      src(it, base, off);
      w0[i] = ld(base, off);
      if (it < nQ + nK) w1[i] = ld(base, off + half);
    }
  }
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
  if (tid < half) rope_cos_sin(pos, rope_inv_freq(p.base, tid, p.d), sCos[tid], sSin[tid]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kEarly; ++i) {
    const int it = tid + i * kThreads;
    if (it < total) finish(it, w0[i], w1[i]);
  }
  for (int it = tid + kEarly * kThreads; it < total; it += kThreads) {
    const T* base;
    size_t off;
    src(it, base, off);
    const u32x4 a = ld(base, off);
    const u32x4 c = it < nQ + nK ? ld(base, off + half) : a;
    finish(it, a, c);
  }
}

}  // namespace

hipError_t launch_rope_append(const RopeParams& p, int dtype, hipStream_t s) {
  const dim3 grid(p.n_q, p.B);
  // whole 16-byte vectors need 16-byte aligned rows and half rows
  auto al = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  const int eb = dtype == TA_F32 ? 4 : 2;
  const bool vec = al(p.q_in) && al(p.q_out) && al(p.k_new) && al(p.v_new) && al(p.k) &&
                   al(p.v) && (p.d / 2 * eb) % 16 == 0;
  if (dtype == TA_F32)
    return vec ? launch(rope_append_vec_kernel<float>, grid, dim3(kThreads), s, p)
               : launch(rope_append_kernel<float>, grid, dim3(kThreads), s, p);
  return vec ? launch(rope_append_vec_kernel<uint16_t>, grid, dim3(kThreads), s, p)
             : launch(rope_append_kernel<uint16_t>, grid, dim3(kThreads), s, p);
}

}  // namespace ta
