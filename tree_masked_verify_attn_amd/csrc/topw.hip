// Maximum-likelihood draft-tree expansion on the device (SwiftSpec summary,
// Section 3.1.3: a node's value is the log-softmax probability of its token
// under its parent's distribution, its weight the sum of the values from the
// root down to it; an expansion step takes the w best new leaves).
//
// Candidate (p, t), p in {-1 (root), 0 .. n-1}, t a token that is not yet the
// token of a child of p, scores cum[p] + x_p[t] - lse_p with x_p the logits
// row of p and lse_p = log sum_v exp(x_p[v]) (cum[-1] = 0).  Within one row
// the order by score is the order by logit, so:
//
//   1. rows: one work group per (row, sequence) reads the row once and keeps,
//      at the same time, the online (max, sum of exp) and each thread's w
//      largest logits among the allowed tokens (a row's children are marked
//      in an LDS bitmap); the group then merges its threads' lists into the
//      row's w best candidates, scored, in the workspace;
//   2. select: one work group per sequence takes the w best of the rows'
//      candidates (higher score first; ties: lower parent, then the row's
//      order: higher logit, then lower token) and appends them as new nodes:
//      parent, token, cumulative score, and the new node count.
//
// Scores are fp32: lse_p in fp32 (max-shifted sum of exp), score = cum[p] +
// (x - lse_p).
#include "ta_device.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                   // 16-byte loads per thread in flight
constexpr int kBitmapWords = kTopwMaxVocab / 32;

struct Cand {
  float v;  // logit (rows pass) or score (select pass)
  int t;    // token (rows pass) or candidate index (select pass)
};

// a before b: higher value, then lower index
__device__ __forceinline__ bool before(float av, int at, float bv, int bt) {
  return av > bv || (av == bv && at < bt);
}

// Keeps list[0..W) sorted best first; inserts (v, t) if it belongs.
template <int W>
__device__ __forceinline__ void insert(Cand (&list)[W], float v, int t) {
  if (!before(v, t, list[W - 1].v, list[W - 1].t)) return;
  Cand c{v, t};
#pragma unroll
  for (int k = 0; k < W; ++k) {
    if (before(c.v, c.t, list[k].v, list[k].t)) {
      const Cand tmp = list[k];
      list[k] = c;
      c = tmp;
    }
  }
}

// Work-group arg-best of one candidate per thread (all threads call).
__device__ __forceinline__ Cand block_best(Cand c, Cand* scratch) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(c.v, o, 64);
    const int ot = __shfl_xor(c.t, o, 64);
    if (before(ov, ot, c.v, c.t)) c = Cand{ov, ot};
  }
  __syncthreads();  // scratch may still be read by the previous round
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = c;
  __syncthreads();
  Cand b = scratch[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w)
    if (before(scratch[w].v, scratch[w].t, b.v, b.t)) b = scratch[w];
  return b;
}

template <int W, bool kBf16>
__global__ __launch_bounds__(kThreads) void topw_rows_kernel(const void* logits,
                                                             const int32_t* parent,
                                                             const int32_t* tok,
                                                             const float* cum,
                                                             const int32_t* n_nodes, int n_max,
                                                             int V, int w, float* ws_score,
                                                             int32_t* ws_tok) {
  __shared__ uint32_t sTaken[kBitmapWords];
  __shared__ Cand sBest[kThreads / 64];
  __shared__ float sM[kThreads / 64], sS[kThreads / 64];
  const int r = blockIdx.x;  // row: 0 = root, 1 + i = node i
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  if (r > n) return;
  const int p = r - 1;
  const size_t cbase = (static_cast<size_t>(b) * (n_max + 1) + r) * w;

  // tokens already taken by children of p
  const int words = (V + 31) / 32;
  for (int i = tid; i < words; i += kThreads) sTaken[i] = 0u;
  __syncthreads();
  for (int c = tid; c < n; c += kThreads) {
    if (clamp_parent(parent[static_cast<size_t>(b) * n_max + c], c) == p) {
      const int t = tok[static_cast<size_t>(b) * n_max + c];
      if (t >= 0 && t < V) atomicOr(&sTaken[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();

  Cand list[W];
#pragma unroll
  for (int k = 0; k < W; ++k) list[k] = Cand{-INFINITY, 0x7fffffff};
  float m = -INFINITY, s = 0.f;  // online max and sum of exp(x - m)
  auto consider = [&](float x, int t) {
    if (x > m) {
      s = s * __expf(m - x) + 1.f;
      m = x;
    } else {
      s += __expf(x - m);
    }
    if (before(x, t, list[W - 1].v, list[W - 1].t) && !((sTaken[t >> 5] >> (t & 31)) & 1u))
      insert(list, x, t);
  };

  const size_t row = (static_cast<size_t>(b) * (n_max + 1) + r) * static_cast<size_t>(V);
  constexpr int kPer = kBf16 ? 8 : 4;  // logits per 16-byte vector
  const void* xrow = kBf16 ? static_cast<const void*>(static_cast<const uint16_t*>(logits) + row)
                           : static_cast<const void*>(static_cast<const float*>(logits) + row);
  const bool vec = (V % kPer == 0) && ((reinterpret_cast<uintptr_t>(xrow) & 15) == 0);
  int start = 0;
  if (vec) {
    const u32x4* x4 = static_cast<const u32x4*>(xrow);
    const int nv = V / kPer;
    for (int base = 0; base < nv; base += kThreads * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = base + u * kThreads + tid;
        v[u] = __builtin_nontemporal_load(x4 + (j < nv ? j : nv - 1));
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = base + u * kThreads + tid;
        if (j < nv) {
          const uint32_t ws[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (kBf16) {
              consider(__uint_as_float(ws[e] << 16), j * kPer + 2 * e);
              consider(__uint_as_float(ws[e] & 0xffff0000u), j * kPer + 2 * e + 1);
            } else {
              consider(__uint_as_float(ws[e]), j * kPer + e);
            }
          }
        }
      }
    }
    start = V;
  }
  for (int t = start + tid; t < V; t += kThreads) {
    const float x = kBf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(xrow)[t])
                          : static_cast<const float*>(xrow)[t];
    consider(x, t);
  }

  // log-sum-exp of the row
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64), os = __shfl_xor(s, o, 64);
    const float mm = fmaxf(m, om);
    s = (m == -INFINITY ? 0.f : s * __expf(m - mm)) + (om == -INFINITY ? 0.f : os * __expf(om - mm));
    m = mm;
  }
  if ((tid & 63) == 0) {
    sM[tid >> 6] = m;
    sS[tid >> 6] = s;
  }
  __syncthreads();
  float M = sM[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) M = fmaxf(M, sM[i]);
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) S += sM[i] == -INFINITY ? 0.f : sS[i] * __expf(sM[i] - M);
  const float lse = M + __logf(S);
  const float base = p < 0 ? 0.f : cum[static_cast<size_t>(b) * n_max + p];

  // the row's w best: w rounds of a work-group arg-best over the threads' heads
  for (int k = 0; k < w; ++k) {
    const Cand best = block_best(list[0], sBest);
    if (list[0].t == best.t && list[0].v == best.v && best.t != 0x7fffffff) {
      // this thread owned the winner (tokens are unique across threads)
#pragma unroll
      for (int i = 0; i + 1 < W; ++i) list[i] = list[i + 1];
      list[W - 1] = Cand{-INFINITY, 0x7fffffff};
    }
    if (tid == 0) {
      const bool ok = best.t != 0x7fffffff;
      ws_score[cbase + k] = ok ? base + (best.v - lse) : -INFINITY;
      ws_tok[cbase + k] = ok ? best.t : -1;
    }
  }
}

__global__ __launch_bounds__(kThreads) void topw_select_kernel(int32_t* parent, int32_t* tok,
                                                               float* cum, int32_t* n_nodes,
                                                               int n_max, int w,
                                                               const float* ws_score,
                                                               const int32_t* ws_tok) {
  __shared__ Cand sBest[kThreads / 64];
  __shared__ uint8_t sUsed[(kMaxNodes + 1) * kTopwMaxW];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const int room = n_max - n;
  const int take = w < room ? w : room;
  const int total = (n + 1) * w;  // candidates: row r, rank k -> index r * w + k
  const size_t cbase = static_cast<size_t>(b) * (n_max + 1) * w;
  for (int i = tid; i < total; i += kThreads) sUsed[i] = 0;
  __syncthreads();
  int appended = 0;
  for (int k = 0; k < take; ++k) {
    // Candidate i = row * w + rank.  Order: higher score, then lower index,
    // i.e. lower parent (row = parent + 1), then the rows pass's rank (higher
    // logit, then lower token).
    Cand mine{-INFINITY, 0x7fffffff};
    for (int i = tid; i < total; i += kThreads) {
      if (sUsed[i] || ws_tok[cbase + i] < 0) continue;
      const float v = ws_score[cbase + i];
      if (before(v, i, mine.v, mine.t)) mine = Cand{v, i};
    }
    const Cand best = block_best(mine, sBest);
    if (best.t == 0x7fffffff) break;  // uniform: fewer candidates than w
    if (tid == 0) {
      const int row = best.t / w;
      const int slot = n + appended;
      parent[static_cast<size_t>(b) * n_max + slot] = row - 1;
      tok[static_cast<size_t>(b) * n_max + slot] = ws_tok[cbase + best.t];
      cum[static_cast<size_t>(b) * n_max + slot] = best.v;
      sUsed[best.t] = 1;
    }
    ++appended;
    __syncthreads();  // sUsed visible before the next round
  }
  if (tid == 0) n_nodes[b] = n + appended;
}

}  // namespace

size_t topw_ws_bytes(int B, int n_max, int w) {
  return static_cast<size_t>(B) * (n_max + 1) * w * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_topw(const void* logits, int logit_dtype, int32_t* parent, int32_t* tok,
                       float* cum, int32_t* n_nodes, int B, int n_max, int V, int w, void* ws,
                       hipStream_t s) {
  float* ws_score = static_cast<float*>(ws);
  int32_t* ws_tok = reinterpret_cast<int32_t*>(ws_score + static_cast<size_t>(B) * (n_max + 1) * w);
  const dim3 g1(n_max + 1, B);
  hipError_t e;
  const bool bf = logit_dtype == TA_BF16;
  if (w <= 8)
    e = bf ? launch(topw_rows_kernel<8, true>, g1, dim3(kThreads), s, logits, parent, tok, cum,
                    n_nodes, n_max, V, w, ws_score, ws_tok)
           : launch(topw_rows_kernel<8, false>, g1, dim3(kThreads), s, logits, parent, tok, cum,
                    n_nodes, n_max, V, w, ws_score, ws_tok);
  else
    e = bf ? launch(topw_rows_kernel<kTopwMaxW, true>, g1, dim3(kThreads), s, logits, parent, tok,
                    cum, n_nodes, n_max, V, w, ws_score, ws_tok)
           : launch(topw_rows_kernel<kTopwMaxW, false>, g1, dim3(kThreads), s, logits, parent, tok,
                    cum, n_nodes, n_max, V, w, ws_score, ws_tok);
  if (e != hipSuccess) return e;
  return launch(topw_select_kernel, dim3(B), dim3(kThreads), s, parent, tok, cum, n_nodes, n_max,
                w, ws_score, ws_tok);
}

}  // namespace ta
