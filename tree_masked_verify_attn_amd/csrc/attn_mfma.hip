// bf16 tree-masked verify/expand attention on the gfx950 matrix cores.
//
// What it computes is the same as the generic kernel (SwiftSpec summary,
// Section 3.1.3 Figure 3 and Section 3.2; draft-length co-design article,
// key mechanism): for query row (node i, head h) softmax attention over the
// P prefix positions plus the tree positions of i's ancestors and itself,
// KV head h / G.  The G heads x query nodes of one KV head form up to 128
// rows, the dense [rows x d] . [d x tokens] products over the prefix run on
// MFMA, and only the tail tile that reaches the tree cache tests the
// per-row ancestor bitmask.
//
// Layout of the work (one work group = 4 waves of 64 lanes):
//  * grid = (sequence x KV head, split, row tile); a split is `chunk` KV
//    positions; a row tile is 32 x NRG query rows (NRG = 1..4 row groups).
//  * Each wave owns one 32-row group and a share of every LDS tile's tokens
//    (with NRG < 4 several waves share a row group and split the tile's
//    tokens; they merge their softmax states in LDS at the end).
//  * Per 32-token sub-tile a wave computes S^T = K . Q^T with
//    v_mfma_f32_32x32x16_bf16 (tokens are the M side): lane l then holds 16
//    scores of ONE query row (l % 32), so the row max and sum are in-lane
//    plus one permlane32 swap.  The output is accumulated transposed,
//    O^T = V^T . P^T: P^T is the MFMA B operand straight from registers
//    (tokens permuted consistently on both sides of the contraction), V^T
//    comes from the token-major LDS tile through ds_read_b64_tr_b16, and
//    every accumulator of lane l belongs to row l % 32, so the rescale after
//    a new running maximum needs no cross-lane traffic.  Rescaling is lazy:
//    the reference maximum only moves when a score exceeds it by 2^8.
//  * K/V tiles (64 or 128 positions) are staged through LDS with an XOR
//    swizzle of the 16-byte chunks that keeps both the K operand reads
//    (16 consecutive positions, same chunk) and the transposed V reads
//    (4 positions x 2 chunks) free of bank conflicts.  The next tile is
//    prefetched into registers while the current one is consumed.
//  * A split sequence leaves partial (max, sum, output) states in the
//    workspace; the combine launch (attn_merge.hip) finishes it.
#include "partial_f16.h"
#include "ta_device.h"

namespace ta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.f;  // log2 units: p may reach 2^8 before a rescale
constexpr float kLn2 = 0.69314718055994530942f;

// XOR swizzle of the 16-byte chunk index of LDS row t (see the header).
template <int D>
__device__ __forceinline__ int swz(int t) {
  const int h = ((t & 3) << 1) | ((t >> 2) & 1);
  return D == 128 ? (h | (((t >> 3) & 1) << 3)) : h;
}
template <int D>
__device__ __forceinline__ int lds_off(int t, int chunk) {  // bytes
  return t * (D * 2) + ((chunk ^ swz<D>(t)) << 4);
}

__device__ __forceinline__ float lane_swap32(float x) {
  // value of lane (l ^ 32)
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 63) < 32 ? r[1] : r[0]);
}

template <int D, int NRG>
struct Cfg {
  static constexpr int TT = NRG == 1 ? 128 : 64;           // KV positions per LDS tile
  static constexpr int SS = NRG == 1 ? 4 : (NRG == 2 ? 2 : 1);  // waves sharing a row group
  static constexpr int SUB = TT / (32 * SS);               // 32-position sub-tiles per wave
  static constexpr int CH = D / 8;                         // 16-byte chunks per row
  static constexpr int NLOAD = TT * CH / kThreads;         // 16-byte loads per thread (K, V each)
  static constexpr int KS = D / 16;                        // MFMA k-steps over d
  static constexpr int MB = D / 32;                        // 32-channel output blocks
  static constexpr int RPT = 32 * NRG;                     // rows per tile
  static constexpr int TILE_BYTES = TT * D * 2;            // one of K or V
  // cross-wave merge scratch: (SS-1) x NRG slots of [MB*16 + 2][64] floats
  static constexpr int MERGE_BYTES = (SS - 1) * NRG * (MB * 16 + 2) * 64 * 4;
  static constexpr int LDS_BYTES = 2 * TILE_BYTES > MERGE_BYTES ? 2 * TILE_BYTES : MERGE_BYTES;
};

template <int D, int NRG>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(AttnParams p) {
  using C = Cfg<D, NRG>;
  __shared__ __attribute__((aligned(16))) uint8_t sKV[C::LDS_BYTES];
  __shared__ uint64_t sAnc[kMaxNodes][kMaskWords];
  __shared__ int sJump[kMaxNodes];
  uint8_t* sK = sKV;
  uint8_t* sV = sKV + C::TILE_BYTES;

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
  const int lhi = lane >> 5;   // 0 for lanes 0..31, 1 for 32..63
  const int l32 = lane & 31;

  SeqBounds sb;
  if (!seq_bounds(p.prefix_len, p.n_nodes, b, p.n_max, p.T_cap, sb)) return;
  const int nsplit = (sb.T + p.chunk - 1) / p.chunk;
  if (split >= nsplit) return;
  const int t_begin = split * p.chunk;
  const int t_end = min(sb.T, t_begin + p.chunk);

  // This wave's row group and token share.
  const int rg = (NRG == 3) ? (wave < 3 ? wave : -1) : (wave % NRG);
  const int th = (NRG == 3) ? 0 : (wave / NRG);
  const int R = p.n_q * p.G;
  const int row_in_tile = (rg < 0 ? 0 : rg) * 32 + l32;
  const int grow = rtile * C::RPT + row_in_tile;
  int node = -1, slot = 0, g = 0;
  if (rg >= 0 && grow < R) {
    slot = grow / p.G;
    g = grow % p.G;
    node = p.expand ? sb.n - p.n_q + slot : slot;
    if (node < 0 || node >= sb.n) node = -1;
  }
  // The whole group may have no valid row (e.g. expand rows before node 0).
  if (!__syncthreads_or(node >= 0)) return;

  const bool has_tree = t_end > sb.P;
  if (has_tree) build_ancestor_masks(p.parent + static_cast<size_t>(b) * p.n_max, sb.n, sAnc, sJump);

  // Q^T operand (B side of S^T = K . Q^T): lane holds row l32, chunk 2*ks + lhi.
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const size_t qrow = ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * D;
  bf16x8 qreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (node >= 0) v = *reinterpret_cast<const u32x4*>(Q + qrow + (2 * ks + lhi) * 8);
    qreg[ks] = __builtin_bit_cast(bf16x8, v);
  }
  uint64_t anc[kMaskWords] = {0, 0, 0, 0};
  __syncthreads();  // ancestor masks ready
  if (has_tree && node >= 0) {
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) anc[w] = sAnc[node][w];
  }

  // ---- K/V tile staging -------------------------------------------------
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v);
  u32x4 rk[C::NLOAD], rv[C::NLOAD];
  auto load_tile = [&](int tb) {
#pragma unroll
    for (int i = 0; i < C::NLOAD; ++i) {
      const int e = tid + i * kThreads;
      const int t = e / C::CH, c = e % C::CH;
      const int tok = tb + t;
      if (tok < t_end) {
        const size_t off = kv_offset(p.block_table, p.block_size, p.max_blocks, p.num_blocks,
                                     p.T_cap, p.Hkv, D, b, tok, hkv) + c * 8;
        rk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kg + off));
        rv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vg + off));
      } else {
        rk[i] = u32x4{0u, 0u, 0u, 0u};
        rv[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::NLOAD; ++i) {
      const int e = tid + i * kThreads;
      const int t = e / C::CH, c = e % C::CH;
      const int o = lds_off<D>(t, c);
      *reinterpret_cast<u32x4*>(sK + o) = rk[i];
      *reinterpret_cast<u32x4*>(sV + o) = rv[i];
    }
  };

  // ---- running softmax state (row l32 of this wave's group) ---------------
  f32x16 acc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum, scaled log2 units
  float l_sum = 0.f;
  const float cs = p.scale_log2;
  const int lim = min(sb.P, t_end);  // positions below lim need no mask

  load_tile(t_begin);
  store_tile();
  __syncthreads();

  for (int tb = t_begin; tb < t_end; tb += C::TT) {
    const int next = tb + C::TT;
    if (next < t_end) load_tile(next);

    if (rg >= 0) {
#pragma unroll
      for (int s = 0; s < C::SUB; ++s) {
        const int lt0 = (th * C::SUB + s) * 32;  // first position of the sub-tile in the tile
        const int sub = tb + lt0;
        if (sub >= t_end) break;
        // S^T = K . Q^T  (M = 32 positions, N = 32 rows, K = d)
        f32x16 S;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(sK + lds_off<D>(lt0 + l32, 2 * ks + lhi));
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qreg[ks], S,
                                                      0, 0, 0);
        }
        // lane holds positions sub + 8*(r/4) + 4*lhi + r%4 of row l32
        if (sub + 32 > lim) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = sub + 8 * (r >> 2) + 4 * lhi + (r & 3);
            bool vis = t < t_end;
            if (vis && t >= sb.P) {
              const int j = t - sb.P;
              vis = (anc[j >> 6] >> (j & 63)) & 1ull;
            }
            if (!vis) S[r] = -INFINITY;
          }
        }
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = fmaxf(mx, lane_swap32(mx)) * cs;
        // lazy rescale: move the reference only when a score exceeds it by 2^8
        const bool bump = mx > m_ref + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(bump) != 0ull) {
          const float m_new = bump ? mx : m_ref;
          const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
          l_sum *= alpha;
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
          m_ref = m_new;
        }
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        float rs = 0.f;
        bf16x8 pk[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = exp2f(fmaf(S[r], cs, -m_use));
          rs += pr;
          pk[r >> 3][r & 7] = static_cast<__bf16>(pr);
        }
        l_sum += rs + lane_swap32(rs);
        // O^T += V^T . P^T  (M = 32 channels, N = 32 rows, K = 16 positions)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) {
            // 16-lane group: 4 positions x 16 channels, transposed on read
            const int gi = lane >> 4, j = lane & 15;
            const int d0 = 32 * mb + 16 * (gi & 1);
            const int trow = lt0 + 16 * kk + 4 * (gi >> 1) + (j >> 2);
            const int dd = d0 + 4 * (j & 3);
            const int o1 = lds_off<D>(trow, dd >> 3) + (dd & 7) * 2;
            const int o2 = lds_off<D>(trow + 8, dd >> 3) + (dd & 7) * 2;
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + o1));
            const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + o2));
            const u32x2 w1 = __builtin_bit_cast(u32x2, v1), w2 = __builtin_bit_cast(u32x2, v2);
            const u32x4 w = {w1[0], w1[1], w2[0], w2[1]};
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                              pk[kk], acc[mb], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
    if (next < t_end) store_tile();
    __syncthreads();
  }

  // ---- merge the waves that shared a row group (through LDS) --------------
  if (C::SS > 1) {
    float* scratch = reinterpret_cast<float*>(sKV);  // [(SS-1)*NRG][66][64] floats
    constexpr int kStride = (C::MB * 16 + 2) * 64;
    if (rg >= 0 && th > 0) {
      float* my = scratch + ((th - 1) * NRG + rg) * kStride;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) my[(mb * 16 + r) * 64 + lane] = acc[mb][r];
      my[(C::MB * 16) * 64 + lane] = m_ref;
      my[(C::MB * 16 + 1) * 64 + lane] = l_sum;
    }
    __syncthreads();
    if (rg >= 0 && th == 0) {
      float M = m_ref;
#pragma unroll
      for (int o = 1; o < C::SS; ++o)
        M = fmaxf(M, scratch[((o - 1) * NRG + rg) * kStride + (C::MB * 16) * 64 + lane]);
      const float a0 = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - M);
      l_sum *= a0;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] *= a0;
#pragma unroll
      for (int o = 1; o < C::SS; ++o) {
        const float* ot = scratch + ((o - 1) * NRG + rg) * kStride;
        const float mo = ot[(C::MB * 16) * 64 + lane];
        const float ao = (mo == -INFINITY) ? 0.f : exp2f(mo - M);
        l_sum = fmaf(ot[(C::MB * 16 + 1) * 64 + lane], ao, l_sum);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] = fmaf(ot[(mb * 16 + r) * 64 + lane], ao, acc[mb][r]);
      }
      m_ref = M;
    }
  }
  const bool owner = rg >= 0 && th == 0;  // holds the work group's state of its rows

  uint16_t* Out = static_cast<uint16_t*>(p.out);
  const size_t orow = ((static_cast<size_t>(b) * p.n_q + slot) * p.Hq + hkv * p.G + g) * D;
  const size_t lrow = (static_cast<size_t>(b) * p.Hq + hkv * p.G + g) * p.n_q + slot;

  if (nsplit == 1) {
    if (owner && node >= 0) {
      const float inv = 1.f / l_sum;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * mb + 8 * q4 + 4 * lhi;
          const uint32_t lo = f32_to_bf16_bits(acc[mb][4 * q4 + 0] * inv) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(acc[mb][4 * q4 + 1] * inv)) << 16);
          const uint32_t hi = f32_to_bf16_bits(acc[mb][4 * q4 + 2] * inv) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(acc[mb][4 * q4 + 3] * inv)) << 16);
          *reinterpret_cast<u32x2*>(Out + orow + d) = u32x2{lo, hi};
        }
      if (p.lse != nullptr && lhi == 0) p.lse[lrow] = (m_ref + log2f(l_sum)) * kLn2;
    }
    return;
  }

  // ---- publish the partial state for the combine launch --------------------
  const int tile_id = bh * p.n_row_tiles + rtile;
  const size_t part = static_cast<size_t>(tile_id) * p.n_split;
  if (owner) {  // wave-uniform: every lane takes part in the row maximum
    const size_t pr = (part + split) * C::RPT + row_in_tile;
    const int e = partial_exp(acc);
    store_partial_f16(acc, m_ref, l_sum, e, lhi, reinterpret_cast<uint16_t*>(p.ws_o) + pr * D,
                      reinterpret_cast<PartialRec*>(p.ws_ml) + pr);
  }
  // the combine launch (attn_merge.hip) finishes split sequences
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.B * p.Hkv, p.n_split, p.n_row_tiles);
  const dim3 block(kThreads);
  switch (p.rows_per_tile / 32) {
    case 1: return launch(attn_mfma_kernel<D, 1>, grid, block, s, p);
    case 2: return launch(attn_mfma_kernel<D, 2>, grid, block, s, p);
    case 3: return launch(attn_mfma_kernel<D, 3>, grid, block, s, p);
    case 4: return launch(attn_mfma_kernel<D, 4>, grid, block, s, p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t s) {
  if (p.d == 128) return launch_d<128>(p, s);
  if (p.d == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ta
