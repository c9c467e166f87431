// Tree verification by speculative sampling at temperature T > 0 (MineDraft
// notes, the PEARL walkthrough: a rejected draft token is replaced by a draw
// from norm(max(0, p - q)); the same notes sample at temperature 1.0;
// SwiftSpec summary, Section 3.1: the draft tree).
//
// At an accepted node v, with p = softmax(target[v] / T) and q =
// softmax(draft[v] / T), the children are tried in index order against a
// running distribution r (first p): child c with token x is accepted when
// u[c] * q(x) < r(x); a rejection replaces r by norm(max(0, r - q)).  When no
// child is accepted, the bonus token is drawn from r by the inverse CDF.
//
// Two launches:
//   1. stats: one 1024-thread work group per (node, sequence) reads the
//      node's target and draft rows with 16-byte loads issued back to back
//      and stores (max, 1/sum) of 2^(x c - max), c = log2(e) / T, for each:
//      this is the HBM-bound part, every row once.
//   2. walk: one 1024-thread work group per sequence.  Each node's own test
//      values p_parent(tok), q_parent(tok) come from one round of gathers, so
//      the walk is LDS work until a rejection: r is never stored; after k
//      rejections at v, r(x) is rebuilt element by element from p(x), q(x)
//      and the k normalisers, so a rejection with more siblings to try costs
//      one pass over v's rows (k steps per element).  The bonus costs one
//      more: every wave sums r over its own segment of the vocabulary, and
//      the wave whose segment holds the target walks it 64 tokens at a time
//      with wave prefix sums.  A rejection of the last sibling needs no pass
//      of its own: the bonus draws from the unnormalised residual
//      max(0, r - q) directly (or from r if that is all zero), whose sum the
//      same pass forms.
//   Probabilities use the hardware 2^x (v_exp_f32): a walk is one work group
//   per sequence, so its passes are bound by that CU's ALU, not by HBM.
#include <limits.h>

#include "ta_device.h"

namespace ta {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

template <bool kBf16>
__device__ __forceinline__ float logit_at(const void* base, size_t i) {
  if (kBf16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  return static_cast<const float*>(base)[i];
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) pairs of max and sum of 2^(z - m); -inf maxima carry no mass.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.f : s * exp2_hw(m - mm);
  const float c = m2 == -INFINITY ? 0.f : s2 * exp2_hw(m2 - mm);
  m = mm;
  s = a + c;
}

__device__ __forceinline__ void wave_lse(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
}

// Block-wide merge of two (m, s) pairs; every thread gets the result.
__device__ __forceinline__ void block_lse2(float& m0, float& s0, float& m1, float& s1,
                                           float4* sRed) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_lse(m0, s0);
  wave_lse(m1, s1);
  if (lane == 0) sRed[wave] = make_float4(m0, s0, m1, s1);
  __syncthreads();
  float4 a = sRed[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    const float4 c = sRed[w];
    lse_merge(a.x, a.y, c.x, c.y);
    lse_merge(a.z, a.w, c.z, c.w);
  }
  m0 = a.x;
  s0 = a.y;
  m1 = a.z;
  s1 = a.w;
  __syncthreads();  // sRed is reused
}

__device__ __forceinline__ float block_sum(float x, float* sRed) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  if (lane == 0) sRed[wave] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += sRed[w];
  __syncthreads();
  return t;
}

// One row: per-thread (max, sum) over 16-byte vectors (or scalars when the
// row is not a whole number of aligned vectors).
template <bool kBf16>
__device__ __forceinline__ void row_lse(const void* row, int V, float c2, float& m, float& s) {
  constexpr int kPer = kBf16 ? 8 : 4;
  const int tid = threadIdx.x;
  m = -INFINITY;
  s = 0.f;
  const bool vec = (V % kPer == 0) && ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (vec) {
    const u32x4* x4 = static_cast<const u32x4*>(row);
    const int nv = V / kPer;
    for (int base = 0; base < nv; base += kThreads * kUnroll) {
      u32x4 w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = base + u * kThreads + tid;
        w[u] = __builtin_nontemporal_load(x4 + (j < nv ? j : nv - 1));  // read once: streaming policy
      }
      float z[kUnroll * kPer];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const bool ok = base + u * kThreads + tid < nv;
        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          float x;
          if (kBf16)
            x = __uint_as_float((e & 1) ? (ws[e >> 1] & 0xffff0000u) : (ws[e >> 1] << 16));
          else
            x = __uint_as_float(ws[e]);
          z[u * kPer + e] = ok ? x * c2 : -INFINITY;
        }
      }
      float bm = -INFINITY;
#pragma unroll
      for (int e = 0; e < kUnroll * kPer; ++e) bm = fmaxf(bm, z[e]);
      float bs = 0.f;
      if (bm != -INFINITY) {
#pragma unroll
        for (int e = 0; e < kUnroll * kPer; ++e) bs += exp2_hw(z[e] - bm);
      }
      lse_merge(m, s, bm, bs);
    }
  } else {
    for (int x = tid; x < V; x += kThreads) {
      const float z = logit_at<kBf16>(row, x) * c2;
      lse_merge(m, s, z, 1.f);
    }
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void samp_stats_kernel(const void* tgt, const void* dft,
                                                               const int32_t* n_nodes, int n_max,
                                                               int V, float c2,
                                                               float4* stats) {
  __shared__ float4 sRed[kWaves];
  const int i = blockIdx.x, b = blockIdx.y;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  if (i >= n) return;  // uniform
  const size_t off = (static_cast<size_t>(b) * n_max + i) * static_cast<size_t>(V);
  constexpr size_t eb = kBf16 ? 2 : 4;
  float mp, sp, mq, sq;
  row_lse<kBf16>(static_cast<const char*>(tgt) + off * eb, V, c2, mp, sp);
  row_lse<kBf16>(static_cast<const char*>(dft) + off * eb, V, c2, mq, sq);
  block_lse2(mp, sp, mq, sq, sRed);
  if (threadIdx.x == 0)
    stats[static_cast<size_t>(b) * n_max + i] = make_float4(mp, 1.f / sp, mq, 1.f / sq);
}

// Probability of a logit under (max, 1/sum) with c = log2(e) / T.
__device__ __forceinline__ float prob(float x, float c, float m, float inv_s) {
  return exp2_hw(fmaf(x, c, -m)) * inv_s;
}

// r after k rejections at a node, from p(x), q(x) and the reciprocal
// normalisers (0: the excess summed to 0 and r stayed as it was).
__device__ __forceinline__ float running_r(float p, float q, const float* sZi, int k) {
  float r = p;
  for (int j = 0; j < k; ++j) {
    const float zi = sZi[j];
    r = zi > 0.f ? fmaxf(r - q, 0.f) * zi : r;
  }
  return r;
}

// Elements a thread loads before using any of them in the walk's passes.
constexpr int kG = 16;

// r(x) and q(x) for x = x0 + g * stride, g < kG (0 for x >= lim): all loads
// are issued first.
template <bool kBf16>
__device__ __forceinline__ void load_rq(const void* tgt, const void* dft, size_t row, int x0,
                                        int stride, int lim, int V, float c2, float4 st,
                                        const float* sZi, int k, float (&r)[kG], float (&q)[kG]) {
  float tl[kG], dl[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int x = min(x0 + g * stride, V - 1);
    tl[g] = logit_at<kBf16>(tgt, row + x);
    dl[g] = logit_at<kBf16>(dft, row + x);
  }
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const bool ok = x0 + g * stride < lim;
    const float px = prob(tl[g], c2, st.x, st.y);
    const float qx = prob(dl[g], c2, st.z, st.w);
    r[g] = ok ? running_r(px, qx, sZi, k) : 0.f;
    q[g] = ok ? qx : 0.f;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void samp_walk_kernel(
    const void* tgt, const void* dft, const int32_t* parent, const int32_t* tok,
    const int32_t* n_nodes, const int32_t* root_tok, const float* u_accept, const float* u_bonus,
    int n_max, int V, float c2, const float4* stats, int32_t* path, int32_t* path_len,
    int32_t* bonus) {
  __shared__ float4 sStat[kMaxNodes];
  __shared__ float sPv[kMaxNodes], sQv[kMaxNodes], sU[kMaxNodes], sZi[kMaxNodes];
  __shared__ int sFirst[kMaxNodes], sNext[kMaxNodes], sPar[kMaxNodes], sPath[kMaxNodes];
  __shared__ float sRed[kWaves], sRed2[kWaves];
  __shared__ int sLast[kWaves], sLast2[kWaves];
  __shared__ int sTop, sBonus;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const int rt = root_tok[b];
  const size_t rows = static_cast<size_t>(b) * n_max;

  // node i: parent, the parent's statistics, and its own test values
  int par = -1, x = 0;
  bool x_ok = false;
  if (tid < n) {
    par = clamp_parent(parent[rows + tid], tid);
    x = tok[rows + tid];
    x_ok = x >= 0 && x < V;
    sPar[tid] = par;
    sStat[tid] = stats[rows + tid];
    sU[tid] = u_accept[rows + tid];
  }
  if (tid == 0) {
    sTop = INT_MAX;
    sBonus = -1;
  }
  float tp = 0.f, dq = 0.f;
  if (tid < n && par >= 0 && x_ok) {
    const size_t e = (rows + par) * static_cast<size_t>(V) + x;
    tp = logit_at<kBf16>(tgt, e);
    dq = logit_at<kBf16>(dft, e);
  }
  __syncthreads();
  if (tid < n) {
    if (par >= 0) {
      const float4 st = sStat[par];
      sPv[tid] = x_ok ? prob(tp, c2, st.x, st.y) : 0.f;
      sQv[tid] = x_ok ? prob(dq, c2, st.z, st.w) : 0.f;
    } else if (x == rt) {
      atomicMin(&sTop, tid);
    }
    // next sibling (the next node with the same parent) and first child
    int nx = -1, fc = -1;
    for (int j = tid + 1; j < n; ++j) {
      const int pj = sPar[j];
      if (nx < 0 && pj == par) nx = j;
      if (fc < 0 && pj == tid) fc = j;
    }
    sNext[tid] = nx;
    sFirst[tid] = fc;
  }
  __syncthreads();

  const int top = sTop;
  if (top == INT_MAX) {  // uniform: nothing under the root carries root_tok
    for (int i = tid; i < n_max; i += kThreads) path[rows + i] = -1;
    if (tid == 0) {
      path_len[b] = 0;
      bonus[b] = rt;
    }
    return;
  }
  int v = top, len = 1;
  if (tid == 0) sPath[0] = top;
  int result = 0;
  for (;;) {
    const float4 st = sStat[v];
    const size_t rowv = (rows + v) * static_cast<size_t>(V);
    int k = 0;             // rejections at v folded into r
    bool excess = false;   // the last sibling was rejected: draw from max(0, r - q)
    int c = sFirst[v];
    while (c >= 0) {
      const float r = running_r(sPv[c], sQv[c], sZi, k);
      if (sU[c] * sQv[c] < r) break;  // uniform: every thread computes the same
      if (sNext[c] < 0) {  // no sibling left to test: the bonus pass takes the excess
        excess = true;
        c = -1;
        break;
      }
      // rejected: Z = sum over x of max(0, r(x) - q(x))
      float part = 0.f;
      for (int base = 0; base < V; base += kThreads * kG) {
        float rr[kG], q[kG];
        load_rq<kBf16>(tgt, dft, rowv, base + tid, kThreads, V, V, c2, st, sZi, k, rr, q);
#pragma unroll
        for (int g = 0; g < kG; ++g) part += fmaxf(rr[g] - q[g], 0.f);
      }
      const float z = block_sum(part, sRed);
      if (tid == 0) sZi[k] = z > 0.f ? 1.f / z : 0.f;
      __syncthreads();
      ++k;
      c = sNext[c];
    }
    if (c >= 0) {  // accepted: move down
      v = c;
      if (tid == 0) sPath[len] = c;
      ++len;
      continue;
    }
    // bonus: inverse CDF of w = r, or of max(0, r - q) after a last-sibling
    // rejection when that is not all zero.  Wave w owns tokens [w * seg,
    // (w + 1) * seg); lane l reads tokens w * seg + 64 j + l (coalesced).
    const int seg = ((V + kWaves - 1) / kWaves + 63) & ~63;
    const int s0 = wave * seg, s1 = min(V, s0 + seg);
    float Sr = 0.f, Se = 0.f;
    int lr = -1, le = -1;  // the segment's last token with r > 0 / excess > 0
    for (int js = s0; js < s1; js += 64 * kG) {
      float r[kG], q[kG];
      load_rq<kBf16>(tgt, dft, rowv, js + lane, 64, s1, V, c2, st, sZi, k, r, q);
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const float e = fmaxf(r[g] - q[g], 0.f);
        Sr += r[g];
        Se += e;
        lr = r[g] > 0.f ? js + g * 64 + lane : lr;
        le = e > 0.f ? js + g * 64 + lane : le;
      }
    }
    Sr = wave_sum(Sr);
    Se = wave_sum(Se);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lr = max(lr, __shfl_xor(lr, o, 64));
      le = max(le, __shfl_xor(le, o, 64));
    }
    if (lane == 0) {
      sRed[wave] = Sr;
      sRed2[wave] = Se;
      sLast[wave] = lr;
      sLast2[wave] = le;
    }
    __syncthreads();
    float tot_e = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot_e += sRed2[w];
    const bool use_e = excess && tot_e > 0.f;  // uniform
    const float* sumw = use_e ? sRed2 : sRed;
    const int* lastw = use_e ? sLast2 : sLast;
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += sumw[w];
    const float target = u_bonus[b] * total;
    // the first segment whose running total passes the target
    int ow = -1, glast = -1;
    float before = 0.f, ow_before = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float t = sumw[w];
      if (ow < 0 && t > 0.f && target < before + t) {
        ow = w;
        ow_before = before;
      }
      before += t;
      glast = max(glast, lastw[w]);
    }
    if (ow < 0) {  // uniform: rounding left the target at or past the total
      if (tid == 0) sBonus = glast;
    } else if (wave == ow) {
      // walk the segment 64 tokens at a time: a wave prefix sum per step
      const float local = target - ow_before;
      float acc = 0.f;
      int pick = -1;
      for (int js = s0; js < s1 && pick < 0; js += 64 * kG) {
        float r[kG], q[kG];
        load_rq<kBf16>(tgt, dft, rowv, js + lane, 64, s1, V, c2, st, sZi, k, r, q);
#pragma unroll
        for (int g = 0; g < kG; ++g) {
          float inc = use_e ? fmaxf(r[g] - q[g], 0.f) : r[g];
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
          }
          const uint64_t cross = __ballot(pick < 0 && acc + inc > local);
          if (cross != 0 && pick < 0) pick = js + g * 64 + __ffsll(static_cast<long long>(cross)) - 1;
          acc += __shfl(inc, 63, 64);
        }
      }
      if (lane == 0) sBonus = pick >= 0 ? pick : lastw[ow];
    }
    __syncthreads();
    result = sBonus;
    if (result < 0) result = V - 1;
    break;
  }
  __syncthreads();
  for (int i = tid; i < n_max; i += kThreads) path[rows + i] = i < len ? sPath[i] : -1;
  if (tid == 0) {
    path_len[b] = len;
    bonus[b] = result;
  }
}

}  // namespace

size_t samp_ws_bytes(int B, int n_max) {
  return static_cast<size_t>(B) * static_cast<size_t>(n_max) * sizeof(float4);
}

hipError_t launch_accept_sampling(const void* tgt, const void* dft, int logit_dtype,
                                  const int32_t* parent, const int32_t* tok,
                                  const int32_t* n_nodes, const int32_t* root_tok,
                                  const float* u_accept, const float* u_bonus, float c2, int B,
                                  int n_max, int V, int32_t* path, int32_t* path_len,
                                  int32_t* bonus, void* ws, hipStream_t s) {
  float4* stats = static_cast<float4*>(ws);
  const bool bf = logit_dtype == TA_BF16;
  hipError_t e = bf ? launch(samp_stats_kernel<true>, dim3(n_max, B), dim3(kThreads), s, tgt, dft,
                             n_nodes, n_max, V, c2, stats)
                    : launch(samp_stats_kernel<false>, dim3(n_max, B), dim3(kThreads), s, tgt,
                             dft, n_nodes, n_max, V, c2, stats);
  if (e != hipSuccess) return e;
  const float4* cs = stats;
  return bf ? launch(samp_walk_kernel<true>, dim3(B), dim3(kThreads), s, tgt, dft, parent, tok,
                     n_nodes, root_tok, u_accept, u_bonus, n_max, V, c2, cs, path, path_len,
                     bonus)
            : launch(samp_walk_kernel<false>, dim3(B), dim3(kThreads), s, tgt, dft, parent, tok,
                     n_nodes, root_tok, u_accept, u_bonus, n_max, V, c2, cs, path, path_len,
                     bonus);
}

}  // namespace ta
