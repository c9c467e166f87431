// Split-KV combine (the second launch of a split attention call).
//
// Each split s of a (sequence, KV head, row tile) left, per query row, the
// running maximum m_s (log2 units of the scaled scores), the sum l_s of
// 2^(score - m_s) and the unnormalised output O_s.  The rows' results are the
// log-sum-exp combination (SwiftSpec summary, Section 3.3: one head split
// over several thread blocks, partial results combined):
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,
//   O = sum_s 2^(m_s - M) O_s / L,  LSE = (M + log2 L) * ln 2.
// The combine runs as its own launch: on gfx950 the kernel boundary makes the
// partial results visible to every compute unit once, whereas a device-scope
// release/acquire in each splitting work group writes back and invalidates
// the whole L2 of its XCD every time.  The bf16 MFMA kernels leave their
// partial outputs in half precision (partial_f16.h), the generic kernel in
// fp32.
#include "partial_f16.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;  // partial states in flight per thread
constexpr float kLn2 = 0.69314718055994530942f;

template <typename T>
__device__ __forceinline__ void store4(T* out, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* out, f32x4 v) {
  *reinterpret_cast<f32x4*>(out) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* out, f32x4 v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const uint32_t lo = f32_to_bf16_bits(v[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  const uint32_t hi = f32_to_bf16_bits(v[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  *reinterpret_cast<u32x2*>(out) = u32x2{lo, hi};
}

// grid = (sequence x KV head, row-tile x channel-group blocks); one thread
// per (row, 4 channels) of a tile.
template <typename T, bool F16>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv;
  const int hkv = bh % p.Hkv;
  const int groups = p.d / 4;
  const int per_tile = p.rows_per_tile * groups;
  const int e = blockIdx.y * kThreads + threadIdx.x;
  const int rtile = e / per_tile;
  if (rtile >= p.n_row_tiles) return;
  const int r = (e % per_tile) / groups;
  const int dg = e % groups;
  const size_t part = static_cast<size_t>(bh * p.n_row_tiles + rtile) * p.n_split;
  // Partial states are read kBatch at a time with unconditional loads (splits
  // past the last repeat one and get weight zero), so that a batch's loads are
  // all in flight before the first is used; batches combine online.  The
  // first batch does not wait for the sequence's length: its slots exist for
  // every plan (clamped to the allocated splits), and the slots past the
  // sequence's last split are discarded below.
  float ms[kBatch], ls[kBatch];
  f32x4 os[kBatch];
  PartialF16 hs[kBatch];  // half-precision states as loaded
  auto load_batch = [&](int s0, int last) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sp = s0 + k < last ? s0 + k : last;
      const size_t pr = (part + sp) * p.rows_per_tile + r;
      if constexpr (F16) {
        hs[k] = load_partial_f16(reinterpret_cast<const uint16_t*>(p.ws_o) + pr * p.d + 4 * dg,
                                 reinterpret_cast<const PartialRec*>(p.ws_ml) + pr);
      } else {
        const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + pr * 2);
        ms[k] = ml.x;
        ls[k] = ml.y;
        os[k] = *reinterpret_cast<const f32x4*>(p.ws_o + pr * p.d + 4 * dg);
      }
    }
  };
  load_batch(0, p.n_split - 1);
  // The exits below use the first batch, so that its loads stay ahead of the
  // sequence's bounds: the compiler would otherwise sink them past the exits,
  // and the two memory latencies would add up.
  static_assert(kBatch == 4, "keep_first_batch names four partial states");
  auto keep_first_batch = [&]() {
    if constexpr (F16) {
      asm volatile("" ::"v"(hs[0].rec), "v"(hs[1].rec), "v"(hs[2].rec), "v"(hs[3].rec));
      asm volatile("" ::"v"(hs[0].h), "v"(hs[1].h), "v"(hs[2].h), "v"(hs[3].h));
    } else {
      asm volatile("" ::"v"(ms[0]), "v"(ms[1]), "v"(ms[2]), "v"(ms[3]), "v"(ls[0]), "v"(ls[1]),
                   "v"(ls[2]), "v"(ls[3]));
      asm volatile("" ::"v"(os[0]), "v"(os[1]), "v"(os[2]), "v"(os[3]));
    }
  };
  SeqBounds sb;
  if (!seq_bounds(p.prefix_len, p.n_nodes, b, p.n_max, p.T_cap, sb)) return keep_first_batch();
  const int nsplit = (sb.T + p.chunk - 1) / p.chunk;
  if (nsplit <= 1) return keep_first_batch();  // the attention kernel wrote this sequence's results
  const int gr = rtile * p.rows_per_tile + r;
  const int R = p.n_q * p.G;
  if (gr >= R) return keep_first_batch();
  const int slot = gr / p.G, g = gr % p.G;
  const int node = p.expand ? sb.n - p.n_q + slot : slot;
  if (node < 0 || node >= sb.n) return keep_first_batch();

  float M = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    if (s0 > 0) load_batch(s0, nsplit - 1);
    if constexpr (F16) {
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        ms[k] = hs[k].rec[0];
        ls[k] = hs[k].rec[1];
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (s0 + k >= nsplit) {  // not a split of this sequence (may hold stale bytes)
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        os[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        hs[k].h = f16x4{0, 0, 0, 0};
      }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) Mb = fmaxf(Mb, ms[k]);
    if (Mb == -INFINITY) continue;  // no visible position so far
    const float a = (M == -INFINITY) ? 0.f : exp2f(M - Mb);
    L *= a;
    o *= a;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wgt = (ms[k] == -INFINITY) ? 0.f : exp2f(ms[k] - Mb);
      L = fmaf(ls[k], wgt, L);
      if constexpr (F16) add_partial_f16(o, hs[k], wgt);
      else o += os[k] * wgt;
    }
    M = Mb;
  }
  const float inv = 1.f / L;
  T* out = static_cast<T*>(p.out) +
           ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * p.d + 4 * dg;
  store4<T>(out, o * inv);
  if (p.lse != nullptr && dg == 0)
    p.lse[(static_cast<size_t>(b) * p.Hq + hkv * p.G + g) * p.n_q + slot] = (M + log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_attn_merge(const AttnParams& p, int dtype, hipStream_t s) {
  const long long items = static_cast<long long>(p.n_row_tiles) * p.rows_per_tile * (p.d / 4);
  const dim3 grid(p.B * p.Hkv, static_cast<unsigned>((items + kThreads - 1) / kThreads));
  if (dtype == TA_F32) return launch(merge_kernel<float, false>, grid, dim3(kThreads), s, p);
  if (p.ws_f16) return launch(merge_kernel<uint16_t, true>, grid, dim3(kThreads), s, p);
  return launch(merge_kernel<uint16_t, false>, grid, dim3(kThreads), s, p);
}

}  // namespace ta
