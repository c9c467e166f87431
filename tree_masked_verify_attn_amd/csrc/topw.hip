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
//   1. rows: one 1024-thread work group per (row, sequence) reads the row
//      once; each thread takes its maximum, then one sum of exponentials
//      against it, and its best allowed logit: the first occurrence of its
//      maximum unless a child of the row's node holds that token (then a full
//      scan; the children are marked in an LDS bitmap).  (Rows longer than
//      one load batch keep an online maximum and sum instead.)  The w-th best of the threads' best logits is a threshold no
//      worse than the row's w-th best allowed logit, and only the (at most w)
//      threads whose best reaches it can hold logits that reach it; those
//      threads put such logits in LDS, where each is ranked by counting the
//      ones before it, and ranks below w are the row's w best candidates,
//      scored, in the workspace;
//   2. select: one work group per sequence takes the w best of the rows'
//      candidates (higher score first; ties: lower parent, then the row's
//      order: higher logit, then lower token) the same way, with the rows'
//      first candidates setting the threshold (a row's candidates are in
//      that order already), and appends them as new nodes: parent, token,
//      cumulative score, and the new node count.
//
// Scores are fp32: lse_p in fp32 (max-shifted sum of exp), score = cum[p] +
// (x - lse_p).  Both kernels issue all their global loads before the first
// is used, so each pays one memory latency.
#include "ta_device.h"

#include <utility>

namespace ta {
namespace {

constexpr int kThreads = 1024;  // one load batch covers a 32000-way fp32 row
constexpr int kWaves = kThreads / 64;
static_assert(kTopwMaxW <= kWaves, "the threshold bound needs a wave maximum per selected key");
constexpr int kUnroll = 8;      // 16-byte loads per thread in flight
constexpr int kBitmapWords = kTopwMaxVocab / 32;
// Candidates past the threshold: at most w threads, each holding at most
// ceil(V / kThreads) logits of the row.
constexpr int kMaxCand = kTopwMaxW * (kTopwMaxVocab / kThreads);
constexpr int kNone = 0x7fffffff;  // "no token"
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;

// Candidates are ordered by a 64-bit key: the value (higher first) in the
// high word, mapped so that unsigned order is float order (-0 taken as +0),
// and the complement of the index (lower first) in the low word.  Every
// non-NaN value maps above 0, so key 0 means "no candidate".
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u ^= (u >> 31) ? 0xffffffffu : 0x80000000u;
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~idx);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  uint32_t u = static_cast<uint32_t>(k >> 32);
  u ^= (u >> 31) ? 0x80000000u : 0xffffffffu;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~static_cast<uint32_t>(k); }

// Cross-lane steps on the vector ALUs (no LDS): DPP within rows of 16
// lanes, the gfx950 32-lane swap, and one permute for lanes 16 apart.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t swap32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 63) < 32 ? r[1] : r[0];
}
// Step k of a wave all-reduce: the value of this lane's partner.  After
// steps 0..k every lane holds the combination of its group of 4, 4, 8, 16,
// 32 (lanes of rows r and r ^ 2) and finally all 64 lanes.
template <int kStep>
__device__ __forceinline__ uint32_t xchg(uint32_t x) {
  if constexpr (kStep == 0) return dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (kStep == 1) return dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (kStep == 2) return dpp<0x141>(x);  // row_half_mirror: the other quad of 8
  if constexpr (kStep == 3) return dpp<0x140>(x);  // row_mirror: the other half of 16
  if constexpr (kStep == 4) return swap32(x);      // lane ^ 32
  return static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), 16, 64));
}
template <int kStep = 0>
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, xchg<kStep>(x));
  if constexpr (kStep < 5) return wave_umax<kStep + 1>(x);
  return x;
}
// log2-domain (max, sum of 2^(x - max)) over the wave, in every lane
template <int kStep = 0>
__device__ __forceinline__ void wave_lse(float& m, float& s) {
  const float om = __uint_as_float(xchg<kStep>(__float_as_uint(m)));
  const float os = __uint_as_float(xchg<kStep>(__float_as_uint(s)));
  const float mm = fmaxf(m, om);
  const float msub = mm == -INFINITY ? 0.f : mm;
  s = s * __builtin_amdgcn_exp2f(m - msub) + os * __builtin_amdgcn_exp2f(om - msub);
  m = mm;
  if constexpr (kStep < 5) wave_lse<kStep + 1>(m, s);
}
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  const uint32_t hi = static_cast<uint32_t>(k >> 32), lo = static_cast<uint32_t>(k);
  const uint32_t mh = wave_umax(hi);
  const uint32_t ml = wave_umax(hi == mh ? lo : 0u);
  return (static_cast<uint64_t>(mh) << 32) | ml;
}
// row_ror:n of a 64-bit value (lane i of a row of 16 gets lane (i + n) % 16)
template <int N>
__device__ __forceinline__ uint64_t ror_key(uint32_t hi, uint32_t lo) {
  return (static_cast<uint64_t>(dpp<0x120 + N>(hi)) << 32) | dpp<0x120 + N>(lo);
}
template <int... N>
__device__ __forceinline__ int count_above_in_row(uint64_t e, std::integer_sequence<int, N...>) {
  const uint32_t hi = static_cast<uint32_t>(e >> 32), lo = static_cast<uint32_t>(e);
  return ((ror_key<N + 1>(hi, lo) > e ? 1 : 0) + ...);
}

// The w-th largest of the work group's keys (one per thread, 0 = none), or 0
// when fewer than w keys exist; the same for every thread (all threads call,
// 1 <= w <= kWaves).  The w-th largest wave maximum is a bound no larger than
// the answer (w keys reach it), so only the keys that reach the bound are
// ranked exactly: four threads per key, each counting a quarter of them.
// Keys must be unique apart from 0.  sSurv holds kThreads keys, sWmax
// kWaves + 1.
__device__ __forceinline__ uint64_t block_threshold(uint64_t key, int w, uint64_t* sSurv,
                                                    uint64_t* sWmax, uint64_t* sTau,
                                                    int* sCount) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const uint64_t wmax = wave_max_key(key);
  if (lane == 0) sWmax[wave] = wmax;
  if (tid == 0) {
    sWmax[kWaves] = 0;
    *sCount = 0;
    *sTau = 0;
  }
  __syncthreads();
  if (wave == 0) {  // the bound: each wave maximum ranked among the 16 (one row of lanes)
    const uint64_t e = sWmax[lane & 15];
    const int above = count_above_in_row(e, std::make_integer_sequence<int, 15>{});
    if (lane < kWaves && e != 0 && above == w - 1) sWmax[kWaves] = e;
  }
  __syncthreads();
  const uint64_t bound = sWmax[kWaves];
  const bool surv = key != 0 && key >= bound;
  const uint64_t mask = __ballot(surv);
  int base = 0;
  if (lane == 0 && mask != 0) base = atomicAdd(sCount, __popcll(mask));
  base = __builtin_amdgcn_readfirstlane(base);
  if (surv) sSurv[base + __popcll(mask & ((1ull << lane) - 1ull))] = key;
  __syncthreads();
  const int K = *sCount;  // <= kThreads
  for (int i = tid >> 2; i < K; i += kThreads / 4) {  // a quad shares i
    const uint64_t e = sSurv[i];
    const int q = tid & 3;
    const int f1 = (q + 1) * K / 4;
    int above = 0;
    for (int f = q * K / 4; f < f1; ++f) above += sSurv[f] > e ? 1 : 0;
    above += static_cast<int>(dpp<0xB1>(static_cast<uint32_t>(above)));
    above += static_cast<int>(dpp<0x4E>(static_cast<uint32_t>(above)));
    if (q == 0 && above == w - 1) *sTau = e;
  }
  __syncthreads();
  return *sTau;
}

// Number of keys in sKeys[0, C) above k.
__device__ __forceinline__ int keys_above(const uint64_t* sKeys, int C, uint64_t k) {
  int above = 0;
#pragma unroll 8
  for (int j = 0; j < C; ++j) above += sKeys[j] > k ? 1 : 0;
  return above;
}

// kVec: the rows are read as 16-byte vectors of kPer logits (V a multiple
// of kPer, the logits 16-byte aligned), else one logit per load.
template <bool kBf16, bool kVec>
__global__ __launch_bounds__(kThreads) void topw_rows_kernel(const void* logits,
                                                             const int32_t* parent,
                                                             const int32_t* tok,
                                                             const float* cum,
                                                             const int32_t* n_nodes, int n_max,
                                                             int V, int w, float* ws_score,
                                                             int32_t* ws_tok) {
  __shared__ uint32_t sTaken[kBitmapWords];
  __shared__ uint64_t sCand[kMaxCand];
  __shared__ uint64_t sSurv[kThreads];
  __shared__ uint64_t sWmax[kWaves + 1];
  __shared__ float sM[kWaves], sS[kWaves];
  __shared__ uint64_t sTau;
  __shared__ int sCount, sSurvCount;
  const int r = blockIdx.x;  // row: 0 = root, 1 + i = node i
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int p = r - 1;
  const size_t cbase = (static_cast<size_t>(b) * (n_max + 1) + r) * w;

  // Unit j of the row: a 16-byte vector of kPer logits (tokens j * kPer + e)
  // or, without kVec, the single logit j.
  constexpr int kPer = kVec ? (kBf16 ? 8 : 4) : 1;
  const size_t row = (static_cast<size_t>(b) * (n_max + 1) + r) * static_cast<size_t>(V);
  const int nunits = V / kPer;
  const int step = kThreads * kUnroll;
  u32x4 v[kUnroll];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int j = base + u * kThreads + tid;
      j = j < nunits ? j : nunits - 1;
      if (kVec) {
        const u32x4* x4 = kBf16 ? reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(logits) + row)
                                : reinterpret_cast<const u32x4*>(static_cast<const float*>(logits) + row);
        v[u] = __builtin_nontemporal_load(x4 + j);
      } else if (kBf16) {
        v[u] = u32x4{static_cast<uint32_t>((static_cast<const uint16_t*>(logits) + row)[j]), 0u, 0u, 0u};
      } else {
        v[u] = u32x4{(static_cast<const uint32_t*>(logits) + row)[j], 0u, 0u, 0u};
      }
    }
  };
  auto value = [&](const u32x4& x, int e) -> float {
    const uint32_t word = x[kBf16 ? (e >> 1) : e];
    if (!kBf16) return __uint_as_float(word);
    return __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
  };

  // --- every global load first: the row, the child slots, cum[p], n ---
  load_batch(0);
  const int cslot = tid < n_max ? tid : n_max - 1;
  const int c_par = parent[static_cast<size_t>(b) * n_max + cslot];
  const int c_tok = tok[static_cast<size_t>(b) * n_max + cslot];
  const float base_cum = cum[static_cast<size_t>(b) * n_max + (p < 0 ? 0 : p)];
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  if (r > n) return;  // uniform: the row of a node that does not exist

  // tokens already taken by children of p
  const int words = (V + 31) / 32;
  for (int i = tid; i < words; i += kThreads) sTaken[i] = 0u;
  if (tid == 0) sCount = 0;
  __syncthreads();
  if (tid < n && clamp_parent(c_par, tid) == p && c_tok >= 0 && c_tok < V)
    atomicOr(&sTaken[c_tok >> 5], 1u << (c_tok & 31));
  __syncthreads();
  // taken bits of unit j's kPer tokens (they share one bitmap word)
  auto taken_bits = [&](int j) -> uint32_t {
    const int t0 = j * kPer;
    return (sTaken[t0 >> 5] >> (t0 & 31)) & ((1u << kPer) - 1u);
  };

  // --- pass 1: online (max, sum) in log2 units, and the thread's best
  // allowed logit (its tokens rise, so a tie keeps the earlier one) ---
  float m = -INFINITY, s = 0.f;
  float kv = -INFINITY;
  int kt = kNone;
  float umax[kUnroll];  // each unit's largest logit (the last batch's)
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) umax[u] = -INFINITY;
  auto unit_max = [&](const u32x4& x) -> float {
    float vmax = value(x, 0);
#pragma unroll
    for (int e = 1; e < kPer; ++e) vmax = fmaxf(vmax, value(x, e));
    return vmax;
  };
  // The thread's best allowed logit over its units: ties keep the earlier
  // token (a thread's tokens rise with u and e).
  auto best_allowed = [&](int base) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = base + u * kThreads + tid;
      if (j >= nunits) break;
      const uint32_t tk = taken_bits(j);
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const float x = value(v[u], e);
        // bitwise, not short-circuit: no branch per logit
        const bool better = (((tk >> e) & 1u) == 0u) & ((x > kv) | ((x == kv) & (kt == kNone)));
        kv = better ? x : kv;
        kt = better ? j * kPer + e : kt;
      }
    }
  };
  if (nunits <= step) {
    // One batch holds the thread's whole share of the row: its maximum
    // first, then one sum of exponentials against it, and the best allowed
    // logit is the first occurrence of that maximum unless a child of p
    // took it (then the full scan).
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u * kThreads + tid >= nunits) break;
      umax[u] = unit_max(v[u]);
      tmax = fmaxf(tmax, umax[u]);
    }
    m = tmax * kLog2e;
    const float msub = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u * kThreads + tid >= nunits) break;
#pragma unroll
      for (int e = 0; e < kPer; ++e) s += __builtin_amdgcn_exp2f(value(v[u], e) * kLog2e - msub);
    }
    int first = kNone;  // the first token holding tmax
#pragma unroll
    for (int u = kUnroll - 1; u >= 0; --u) {
      if (u * kThreads + tid < nunits && umax[u] == tmax) {
#pragma unroll
        for (int e = kPer - 1; e >= 0; --e)
          first = value(v[u], e) == tmax ? (u * kThreads + tid) * kPer + e : first;
      }
    }
    if (first != kNone && ((taken_bits(first / kPer) >> (first % kPer)) & 1u) == 0u) {
      kv = tmax;
      kt = first;
    } else {
      best_allowed(0);
    }
  } else {
    for (int base = 0; base < nunits; base += step) {
      if (base > 0) load_batch(base);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = base + u * kThreads + tid;
        if (j >= nunits) break;
        const float vmax = unit_max(v[u]);
        umax[u] = vmax;
        const float mn = fmaxf(m, vmax * kLog2e);
        const float msub = mn == -INFINITY ? 0.f : mn;
        float add = 0.f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) add += __builtin_amdgcn_exp2f(value(v[u], e) * kLog2e - msub);
        s = s * __builtin_amdgcn_exp2f(m - msub) + add;
        m = mn;
      }
      best_allowed(base);
    }
  }

  // log-sum-exp of the row (log2 units until the end)
  wave_lse(m, s);
  if ((tid & 63) == 0) {
    sM[tid >> 6] = m;
    sS[tid >> 6] = s;
  }

  // --- threshold: the w-th best thread key (synchronises) ---
  const uint64_t key = kt == kNone ? 0ull : make_key(kv, static_cast<uint32_t>(kt));
  const uint64_t tau = block_threshold(key, w, sSurv, sWmax, &sTau, &sSurvCount);

  // --- pass 2: threads whose key reaches the threshold list their allowed
  // logits that reach it (the batch in registers is the row's only one,
  // else the row is read again) ---
  if (key != 0 && key >= tau) {
    const bool all = tau == 0;
    const float tv = key_value(tau);
    const int tt = static_cast<int>(key_index(tau));
    for (int base = 0; base < nunits; base += step) {
      if (nunits > step) {
        load_batch(base);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) umax[u] = unit_max(v[u]);
      }
      // units whose largest logit reaches the threshold's value
      uint32_t units = 0u;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        units |= (base + u * kThreads + tid < nunits && (all | (umax[u] >= tv))) ? (1u << u) : 0u;
      while (units != 0u) {
        const int u = __ffs(units) - 1;
        units &= units - 1u;
        u32x4 x = v[0];
#pragma unroll
        for (int k = 1; k < kUnroll; ++k) x = u == k ? v[k] : x;
        const int j = base + u * kThreads + tid;
        const uint32_t tk = taken_bits(j);
        uint32_t hit = 0u;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const float xv = value(x, e);
          const bool reach = all | (xv > tv) | ((xv == tv) & (j * kPer + e <= tt));
          hit |= ((((tk >> e) & 1u) == 0u) & reach) ? (1u << e) : 0u;
        }
        if (hit != 0u) {
          int slot = atomicAdd(&sCount, __popc(hit));
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            if (((hit >> e) & 1u) && slot < kMaxCand)  // the bound holds; the check is a backstop
              sCand[slot++] = make_key(value(x, e), static_cast<uint32_t>(j * kPer + e));
          }
        }
      }
    }
  }
  __syncthreads();

  float M = sM[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sM[i]);
  const float Msub = M == -INFINITY ? 0.f : M;
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) S += sS[i] * __builtin_amdgcn_exp2f(sM[i] - Msub);
  const float lse = (Msub + __log2f(S)) * kLn2;
  const float cbase_score = p < 0 ? 0.f : base_cum;
  const int C = sCount < kMaxCand ? sCount : kMaxCand;
  for (int i = tid; i < C; i += kThreads) {
    const uint64_t k = sCand[i];
    const int rank = keys_above(sCand, C, k);
    if (rank < w) {
      ws_score[cbase + rank] = cbase_score + (key_value(k) - lse);
      ws_tok[cbase + rank] = static_cast<int>(key_index(k));
    }
  }
  if (tid >= C && tid < w) {  // fewer allowed tokens than w
    ws_score[cbase + tid] = -INFINITY;
    ws_tok[cbase + tid] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void topw_select_kernel(int32_t* parent, int32_t* tok,
                                                               float* cum, int32_t* n_nodes,
                                                               int n_max, int w,
                                                               const float* ws_score,
                                                               const int32_t* ws_tok) {
  __shared__ uint64_t sCand[kTopwMaxW * kTopwMaxW];
  __shared__ int sCandT[kTopwMaxW * kTopwMaxW];
  __shared__ uint64_t sSurv[kThreads];
  __shared__ uint64_t sWmax[kWaves + 1];
  __shared__ uint64_t sTau;
  __shared__ int sCount, sSurvCount;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  // A thread holds one row's candidates (score, token), ranks 0 .. w-1.  A
  // candidate's index is row * w + rank: lower parent first (row = parent +
  // 1), then the row's own order.  Consecutive rows sit in different waves
  // (row = lane * kWaves + wave), so that every wave has rows and the
  // threshold's bound (the w-th best wave maximum) exists: with rows in the
  // first waves only, every head would be ranked exactly.
  static_assert(kThreads > kMaxNodes, "a thread for every row (root + n_max nodes)");
  const int row = (tid & 63) * kWaves + (tid >> 6);
  const int rr = row <= n_max ? row : n_max;
  const size_t rbase = (static_cast<size_t>(b) * (n_max + 1) + rr) * w;
  float sc[kTopwMaxW];
  int tk[kTopwMaxW];
#pragma unroll
  for (int k = 0; k < kTopwMaxW; ++k) {
    const int kk = k < w ? k : w - 1;
    sc[k] = ws_score[rbase + kk];
    tk[k] = ws_tok[rbase + kk];
  }
  int n = n_nodes[b];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const int room = n_max - n;
  const int take = w < room ? w : room;
  if (take <= 0) return;  // uniform
  if (tid == 0) sCount = 0;

  const bool row_ok = row <= n && tk[0] >= 0;
  const uint64_t head = row_ok ? make_key(sc[0], static_cast<uint32_t>(row * w)) : 0ull;
  const uint64_t tau = block_threshold(head, take, sSurv, sWmax, &sTau, &sSurvCount);
  if (head != 0 && head >= tau) {
    // the row's candidates that reach the threshold are a prefix of it
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kTopwMaxW; ++k)
      cnt += (k < w && tk[k] >= 0 && make_key(sc[k], row * w + k) >= tau) ? 1 : 0;
    int slot = atomicAdd(&sCount, cnt);
#pragma unroll
    for (int k = 0; k < kTopwMaxW; ++k) {
      if (k < cnt) {
        sCand[slot + k] = make_key(sc[k], row * w + k);
        sCandT[slot + k] = tk[k];
      }
    }
  }
  __syncthreads();
  const int C = sCount;
  const int appended = C < take ? C : take;
  for (int i = tid; i < C; i += kThreads) {
    const uint64_t k = sCand[i];
    const int rank = keys_above(sCand, C, k);
    if (rank < appended) {
      const size_t slot = static_cast<size_t>(b) * n_max + n + rank;
      parent[slot] = static_cast<int>(key_index(k)) / w - 1;
      tok[slot] = sCandT[i];
      cum[slot] = key_value(k);
    }
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
  const dim3 blk(kThreads);
  const bool bf = logit_dtype == TA_BF16;
  const int per = bf ? 8 : 4;
  const bool vec = V % per == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  auto rows = [&](auto kernel) {
    return launch(kernel, g1, blk, s, logits, parent, tok, cum, n_nodes, n_max, V, w, ws_score,
                  ws_tok);
  };
  const hipError_t e = bf ? (vec ? rows(topw_rows_kernel<true, true>) : rows(topw_rows_kernel<true, false>))
                          : (vec ? rows(topw_rows_kernel<false, true>) : rows(topw_rows_kernel<false, false>));
  if (e != hipSuccess) return e;
  return launch(topw_select_kernel, dim3(B), blk, s, parent, tok, cum, n_nodes, n_max, w, ws_score,
                ws_tok);
}

}  // namespace ta
