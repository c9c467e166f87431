// C ABI of libtreeattn: host-side validation, split planning and launches.
// Declarations and semantics: include/tree_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>

#include "ta_internal.h"
#include "tree_attn.h"

namespace ta {
namespace {
thread_local char g_last_error[256] = "";
}  // namespace
void set_last_error(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", where, hipGetErrorName(e),
                hipGetErrorString(e));
}
}  // namespace ta

namespace {

using ta::AttnParams;

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return TA_OK;
  ta::set_last_error(e, where);
  return TA_ERR_HIP;
}

int device_cu_count() {
  // Compute units of the current device (cached per device id).
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev] = cus;
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kGenericRows = 32;
constexpr int kMfmaRows = 128;  // query rows (G x nodes) per MFMA work group, at most

struct Plan {
  int kernel;         // 1 generic, 2 MFMA (register prefetch), 3 MFMA (LDS-DMA ring),
                      // 4 MFMA over balanced units (LDS-DMA ring across jobs)
  int rows_per_tile;
  int n_row_tiles;
  int chunk;
  int n_split;
  size_t ws_bytes;
};

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// tree_accept_reroot's workspace: the argmax per node, the copy of parent,
// then of prefix_len and of n_nodes (each on its own 256-byte boundary).
size_t accept_reroot_region(size_t bytes) { return (bytes + 255) / 256 * 256; }
size_t accept_reroot_ws_bytes(int B, int n_max) {
  const size_t rows = static_cast<size_t>(B) * n_max * sizeof(int32_t);
  const size_t seq = static_cast<size_t>(B) * sizeof(int32_t);
  return 2 * accept_reroot_region(rows) + 2 * accept_reroot_region(seq);
}

// Chooses the kernel, the row tiling and the split-KV chunk.  The automatic
// chunk gives about two work groups per compute unit, never below 256 KV
// positions per split (smaller chunks cost more in partial results than they
// gain in parallelism).
bool make_plan(int B, int n_q, int Hq, int Hkv, int d, int dtype, int T_cap, bool paged,
               const ta_attn_opts* opts, Plan& pl) {
  const int G = Hq / Hkv;
  const int R = n_q * G;
  int kernel = opts ? opts->kernel : 0;
  const bool mfma_ok = dtype == TA_BF16 && (d == 128 || d == 64);
  // Automatic: bf16 paged caches (the mixed-length serving layout) take the
  // units kernel, which gives every work group the same number of KV tiles
  // whatever the length mix; contiguous bf16 caches (one capacity, the
  // equal-length case) the streaming kernel; anything else the generic one.
  if (kernel == 0) {
    const long long tiles_max = static_cast<long long>(B) * Hkv *
                                ((n_q * G + kMfmaRows - 1) / kMfmaRows + 1) *
                                ((T_cap + 31) / 32 + ta::kUnitJobCost);
    const bool units_ok = paged && B <= ta::kUnitMaxSeqs && tiles_max < (1LL << 31);
    kernel = mfma_ok ? (units_ok ? 4 : 3) : 1;
  }
  if (kernel >= 2 && !mfma_ok) return false;
  if (kernel < 1 || kernel > 4) return false;
  pl.kernel = kernel;
  // Both MFMA kernels share one plan (so they need the same workspace): tiles
  // hold 32 x NRG rows (NRG = 1..4 row groups of 32).
  const bool mfma = kernel != 1;
  pl.rows_per_tile = mfma ? std::min(kMfmaRows, round_up(R, 32)) : kGenericRows;
  pl.n_row_tiles = (R + pl.rows_per_tile - 1) / pl.rows_per_tile;
  const long long items = static_cast<long long>(B) * Hkv * pl.n_row_tiles;
  if (kernel == 4) {
    // G work groups (two per compute unit, all resident) share the stream of
    // at most items * ceil(T_cap / 32) tiles; the stream positions are int.
    if (B > ta::kUnitMaxSeqs) return false;
    if (items * ((T_cap + 31) / 32 + ta::kUnitJobCost) >= (1LL << 31)) return false;
    const int groups = 2 * device_cu_count();
    pl.chunk = T_cap;
    pl.n_split = groups;
    const size_t slots = 2 * static_cast<size_t>(groups) * pl.rows_per_tile;
    pl.ws_bytes = slots * d * sizeof(float) + slots * 2 * sizeof(float) +
                  static_cast<size_t>(B) * 4 * sizeof(int32_t);
    return true;
  }
  int chunk = opts ? opts->chunk_tokens : 0;
  if (chunk < 0 || chunk % 64 != 0) return false;
  if (chunk == 0) {
    // A contiguous cache gives every sequence one capacity, the usual layout
    // for sequences of equal length: one split per resident work group (two
    // per compute unit).  A paged cache usually holds sequences of mixed
    // lengths, whose actual lengths only the device knows: four times as many
    // splits as resident groups, so that the hardware dispatcher balances
    // long and short sequences as groups finish.
    const long long want = (paged ? 8LL : 2LL) * device_cu_count();
    long long splits = items > 0 ? (want + items - 1) / items : 1;
    splits = std::max(1LL, splits);
    chunk = round_up(static_cast<int>((T_cap + splits - 1) / splits), 64);
    chunk = std::max(chunk, 256);
  }
  // MFMA tiles span 128 positions when a tile has a single row group.
  const int gran = (mfma && pl.rows_per_tile == 32) ? 128 : 64;
  if (chunk % gran != 0) chunk = round_up(chunk, gran);
  chunk = std::max(gran, std::min(chunk, round_up(std::max(T_cap, 1), gran)));
  pl.chunk = chunk;
  pl.n_split = (T_cap + chunk - 1) / chunk;
  if (pl.n_split < 1) pl.n_split = 1;
  // launch limits: splits and row tiles are grid y / z (at most 65535 each)
  if (pl.n_split > 65535 || pl.n_row_tiles > 65535) return false;
  const long long tiles = static_cast<long long>(B) * Hkv * pl.n_row_tiles;
  pl.ws_bytes = ta::attn_ws_bytes(static_cast<int>(tiles), pl.n_split, pl.rows_per_tile, d);
  return true;
}

int check_common(int B, int n_q, int n_max, int Hq, int Hkv, int d, int dtype, int T_cap) {
  if (B < 0 || n_q < 1 || n_max < 1 || Hq < 1 || Hkv < 1 || T_cap < 1) return TA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return TA_ERR_INVALID_ARG;
  if (dtype != TA_F32 && dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  return TA_OK;
}

int check_kv(const ta_kv& kv) {
  if (kv.k == nullptr || kv.v == nullptr || kv.T_cap < 1) return TA_ERR_INVALID_ARG;
  if (kv.block_table != nullptr) {
    if (kv.block_size < 1 || kv.max_blocks < 1 || kv.num_blocks < 1) return TA_ERR_INVALID_ARG;
    if (static_cast<long long>(kv.max_blocks) * kv.block_size < kv.T_cap)
      return TA_ERR_INVALID_ARG;
  }
  return TA_OK;
}

// tree_cache_reroot and its draft-side variant: the move launches (groups of
// layers), then the metadata launch (which also moves tok / cum when given).
int reroot_call(const ta_kv* kv_layers, int n_layers, int32_t* prefix_len, int32_t* parent,
                int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                const uint8_t* keep_subtree, int32_t* tok, float* cum, int B, int n_max, int Hkv,
                int d, int dtype, void* stream) {
  if (B < 0 || n_layers < 0 || n_max < 1 || Hkv < 1) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (dtype != TA_F32 && dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (prefix_len == nullptr || parent == nullptr || n_nodes == nullptr || path == nullptr ||
      path_len == nullptr || keep_subtree == nullptr || (n_layers > 0 && kv_layers == nullptr))
    return TA_ERR_INVALID_ARG;
  for (int i = 0; i < n_layers; ++i) {
    const int st = check_kv(kv_layers[i]);
    if (st != TA_OK) return st;
    if (!aligned16(kv_layers[i].k) || !aligned16(kv_layers[i].v)) return TA_ERR_INVALID_ARG;
  }
  if (B == 0) return TA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int row_bytes = d * (dtype == TA_BF16 ? 2 : 4);
  for (int l0 = 0; l0 < n_layers; l0 += ta::kRerootMaxLayersPerLaunch) {
    const int cnt = std::min(ta::kRerootMaxLayersPerLaunch, n_layers - l0);
    ta::RerootLayers L{};
    for (int i = 0; i < cnt; ++i) {
      const ta_kv& kv = kv_layers[l0 + i];
      L.l[i] = ta::RerootLayer{kv.k, kv.v, kv.block_table, kv.block_size, kv.max_blocks,
                               kv.num_blocks, kv.T_cap};
    }
    hipError_t e = ta::launch_reroot_move(L, cnt, prefix_len, parent, n_nodes, path, path_len,
                                          keep_subtree, B, n_max, Hkv, row_bytes, s);
    if (e != hipSuccess) return hip_status(e, "tree_cache_reroot move launch");
  }
  hipError_t e = ta::launch_reroot_meta(prefix_len, parent, n_nodes, path, path_len, keep_subtree,
                                        B, n_max, tok, cum, s);
  return hip_status(e, "tree_cache_reroot metadata launch");
}

}  // namespace

namespace ta {

int run_attention(const void* q, ta_kv kv, const int32_t* prefix_len, const int32_t* parent,
                  const int32_t* n_nodes, int B, int n_q, int n_max, int expand, int Hq, int Hkv,
                  int d, int dtype, float scale, void* out, float* lse, void* ws,
                  size_t ws_bytes, const ta_attn_opts* opts, void* stream,
                  ScratchFn scratch, const RopeArgs* rope) {
  int st = check_common(B, n_q, n_max, Hq, Hkv, d, dtype, kv.T_cap);
  if (st != TA_OK) return st;
  st = check_kv(kv);
  if (st != TA_OK) return st;
  if (q == nullptr || out == nullptr || prefix_len == nullptr || parent == nullptr ||
      n_nodes == nullptr)
    return TA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale != scale) return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  Plan pl;
  if (!make_plan(B, n_q, Hq, Hkv, d, dtype, kv.T_cap, kv.block_table != nullptr, opts, pl))
    return TA_ERR_UNSUPPORTED;
  if (pl.kernel != 1 && !(aligned16(q) && aligned16(out) && aligned16(kv.k) && aligned16(kv.v)))
    return TA_ERR_INVALID_ARG;
  // The streaming kernel keeps one split's paged block ids in LDS; when they do
  // not fit it hands the call to the other MFMA kernel (same plan, same workspace).
  if (pl.kernel == 3 && kv.block_table != nullptr &&
      pl.chunk / kv.block_size + 2 > ta::kStreamMaxSplitBlocks)
    pl.kernel = 2;
  if (scratch != nullptr && pl.ws_bytes > 0) {
    // the library's own scratch array stands in for the caller's workspace
    st = scratch(pl.ws_bytes, stream, &ws);
    if (st != TA_OK) return st;
    ws_bytes = pl.ws_bytes;
  }
  if (pl.ws_bytes > 0 && (ws == nullptr || ws_bytes < pl.ws_bytes || !aligned16(ws)))
    return TA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool fused_rope = false;
  if (rope != nullptr) {
    if (rope->k_new == nullptr || rope->v_new == nullptr || out == q || !(rope->base > 0.f) ||
        rope->base != rope->base || rope->base == INFINITY)
      return TA_ERR_INVALID_ARG;
    // Rotated on load by the streaming kernel when it serves the call; else the
    // RoPE append writes the rotated queries into `out`, which the attention
    // launch then reads as its queries (no kernel writes an output row that
    // another work group still reads as a query).
    fused_rope = pl.kernel == 3 && kv.block_table == nullptr &&
                 ta::stream_rope_fits(d, pl.rows_per_tile, Hq / Hkv) &&
                 aligned16(rope->k_new) && aligned16(rope->v_new);
    if (!fused_rope) {
      ta::RopeParams rp{};
      rp.q_in = q;
      rp.q_out = out;
      rp.k_new = rope->k_new;
      rp.v_new = rope->v_new;
      rp.k = kv.k;
      rp.v = kv.v;
      rp.block_table = kv.block_table;
      rp.block_size = kv.block_size;
      rp.max_blocks = kv.max_blocks;
      rp.num_blocks = kv.num_blocks;
      rp.T_cap = kv.T_cap;
      rp.prefix_len = prefix_len;
      rp.parent = parent;
      rp.n_nodes = n_nodes;
      rp.B = B;
      rp.n_q = n_q;
      rp.n_max = n_max;
      rp.Hq = Hq;
      rp.Hkv = Hkv;
      rp.d = d;
      rp.expand = expand;
      rp.base = rope->base;
      const hipError_t e = ta::launch_rope_append(rp, dtype, s);
      if (e != hipSuccess) return hip_status(e, "RoPE append launch");
      q = out;
    }
  }

  AttnParams p{};
  p.q = q;
  p.out = out;
  p.lse = lse;
  p.k = kv.k;
  p.v = kv.v;
  p.block_table = kv.block_table;
  p.block_size = kv.block_size;
  p.max_blocks = kv.max_blocks;
  p.num_blocks = kv.num_blocks;
  p.T_cap = kv.T_cap;
  p.prefix_len = prefix_len;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.B = B;
  p.n_max = n_max;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.G = Hq / Hkv;
  p.n_q = n_q;
  p.expand = expand;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.chunk = pl.chunk;
  p.n_split = pl.n_split;
  p.rows_per_tile = pl.rows_per_tile;
  p.n_row_tiles = pl.n_row_tiles;
  // The MFMA kernels leave half-precision partial states (d fp16 values and a
  // 16-byte record per row) in the space sized for fp32 ones (d + 2 floats).
  p.ws_f16 = pl.kernel >= 2 ? 1 : 0;
  const size_t o_bytes = p.ws_f16 ? sizeof(uint16_t) : sizeof(float);
  if (pl.kernel == 4) {
    const size_t slots = 2 * static_cast<size_t>(pl.n_split) * pl.rows_per_tile;
    uint8_t* base = static_cast<uint8_t*>(ws);
    p.ws_o = reinterpret_cast<float*>(base);
    p.ws_ml = reinterpret_cast<float*>(base + slots * d * o_bytes);
    p.ws_seq = reinterpret_cast<int32_t*>(base + slots * (d + 2) * sizeof(float));
  } else if (pl.ws_bytes > 0) {
    const int tiles = B * Hkv * pl.n_row_tiles;
    const size_t parts = static_cast<size_t>(tiles) * pl.n_split * pl.rows_per_tile;
    uint8_t* base = static_cast<uint8_t*>(ws);
    p.ws_o = reinterpret_cast<float*>(base);
    p.ws_ml = reinterpret_cast<float*>(base + parts * d * o_bytes);
  }
  if (fused_rope) {
    p.rope = 1;
    p.k_new = rope->k_new;
    p.v_new = rope->v_new;
    p.rope_base = rope->base;
  }
  hipError_t e;
  const char* where;
  if (pl.kernel == 4) {
    e = ta::launch_attn_units(p, s);
    where = "attention (units kernel) launch";
    if (e == hipSuccess) {
      e = ta::launch_attn_merge_units(p, s);
      where = "attention units combine launch";
    }
    return hip_status(e, where);
  }
  if (pl.kernel == 3) {
    e = ta::launch_attn_stream(p, s);
    where = "attention (streaming MFMA kernel) launch";
  } else if (pl.kernel == 2) {
    e = ta::launch_attn_mfma(p, s);
    where = "attention (MFMA kernel) launch";
  } else {
    e = ta::launch_attn_generic(p, dtype, s);
    where = "attention (generic kernel) launch";
  }
  if (e == hipSuccess && pl.n_split > 1) {
    e = ta::launch_attn_merge(p, dtype, s);
    where = "attention split combine launch";
  }
  return hip_status(e, where);
}

}  // namespace ta

extern "C" {

size_t tree_attn_workspace_bytes(int B, int n_q, int Hq, int Hkv, int d, int dtype, int T_cap,
                                 const ta_attn_opts* opts) {
  if (check_common(B, n_q, n_q, Hq, Hkv, d, dtype, T_cap) != TA_OK) return static_cast<size_t>(-1);
  if (B == 0) return 0;
  Plan pl;
  // enough for either layout's plan
  Plan pp;
  if (!make_plan(B, n_q, Hq, Hkv, d, dtype, T_cap, false, opts, pl) ||
      !make_plan(B, n_q, Hq, Hkv, d, dtype, T_cap, true, opts, pp))
    return static_cast<size_t>(-1);
  return std::max(pl.ws_bytes, pp.ws_bytes);
}

int tree_attn_verify(const void* q, ta_kv kv, const int32_t* prefix_len, const int32_t* parent,
                     const int32_t* n_nodes, int B, int n_max, int Hq, int Hkv, int d, int dtype,
                     float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                     const ta_attn_opts* opts, void* stream) {
  return ta::run_attention(q, kv, prefix_len, parent, n_nodes, B, n_max, n_max, 0, Hq, Hkv, d,
                           dtype, scale, out, lse, ws, ws_bytes, opts, stream, nullptr, nullptr);
}

int tree_attn_expand(const void* q, ta_kv kv, const int32_t* prefix_len, const int32_t* parent,
                     const int32_t* n_nodes, int B, int w, int n_max, int Hq, int Hkv, int d,
                     int dtype, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                     const ta_attn_opts* opts, void* stream) {
  if (w < 1 || w > n_max) return TA_ERR_INVALID_ARG;
  return ta::run_attention(q, kv, prefix_len, parent, n_nodes, B, w, n_max, 1, Hq, Hkv, d, dtype,
                           scale, out, lse, ws, ws_bytes, opts, stream, nullptr, nullptr);
}

int tree_attn_verify_rope(const void* q, const void* k_new, const void* v_new, ta_kv kv,
                          const int32_t* prefix_len, const int32_t* parent, const int32_t* n_nodes,
                          int B, int n_max, int Hq, int Hkv, int d, int dtype, float scale,
                          float base, void* out, float* lse, void* ws, size_t ws_bytes,
                          const ta_attn_opts* opts, void* stream) {
  const ta::RopeArgs r{k_new, v_new, base};
  return ta::run_attention(q, kv, prefix_len, parent, n_nodes, B, n_max, n_max, 0, Hq, Hkv, d,
                           dtype, scale, out, lse, ws, ws_bytes, opts, stream, nullptr, &r);
}

int tree_attn_expand_rope(const void* q, const void* k_new, const void* v_new, ta_kv kv,
                          const int32_t* prefix_len, const int32_t* parent, const int32_t* n_nodes,
                          int B, int w, int n_max, int Hq, int Hkv, int d, int dtype, float scale,
                          float base, void* out, float* lse, void* ws, size_t ws_bytes,
                          const ta_attn_opts* opts, void* stream) {
  if (w < 1 || w > n_max) return TA_ERR_INVALID_ARG;
  const ta::RopeArgs r{k_new, v_new, base};
  return ta::run_attention(q, kv, prefix_len, parent, n_nodes, B, w, n_max, 1, Hq, Hkv, d, dtype,
                           scale, out, lse, ws, ws_bytes, opts, stream, nullptr, &r);
}

int accept_greedy_path(const void* logits, int logit_dtype, const int32_t* parent,
                       const int32_t* tok, const int32_t* n_nodes, const int32_t* root_tok, int B,
                       int n_max, int V, int32_t* path, int32_t* path_len, int32_t* bonus,
                       void* stream) {
  if (B < 0 || n_max < 1 || V < 1) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (logit_dtype != TA_F32 && logit_dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (logits == nullptr || parent == nullptr || tok == nullptr || n_nodes == nullptr ||
      root_tok == nullptr || path == nullptr || path_len == nullptr || bonus == nullptr)
    return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  hipError_t e = ta::launch_accept(logits, logit_dtype, parent, tok, n_nodes, root_tok, B, n_max,
                                   V, path, path_len, bonus, static_cast<hipStream_t>(stream));
  return hip_status(e, "accept_greedy_path launch");
}

size_t accept_sampling_workspace_bytes(int B, int n_max) {
  if (B < 0 || n_max < 1 || n_max > TA_MAX_NODES) return static_cast<size_t>(-1);
  return ta::samp_ws_bytes(B, n_max);
}

int accept_sampling_path(const void* target_logits, const void* draft_logits, int logit_dtype,
                         const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
                         const int32_t* root_tok, const float* u_accept, const float* u_bonus,
                         float temperature, int B, int n_max, int V, int32_t* path,
                         int32_t* path_len, int32_t* bonus, void* ws, size_t ws_bytes,
                         void* stream) {
  if (B < 0 || n_max < 1 || V < 1) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (logit_dtype != TA_F32 && logit_dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (!(temperature > 0.f) || temperature == INFINITY) return TA_ERR_INVALID_ARG;
  // logits scale for the base-2 exponentials: log2(e) / T
  const float c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  if (!(c2 > 0.f) || c2 == INFINITY) return TA_ERR_INVALID_ARG;
  if (target_logits == nullptr || draft_logits == nullptr || parent == nullptr ||
      tok == nullptr || n_nodes == nullptr || root_tok == nullptr || u_accept == nullptr ||
      u_bonus == nullptr || path == nullptr || path_len == nullptr || bonus == nullptr)
    return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  if (ws == nullptr || ws_bytes < ta::samp_ws_bytes(B, n_max) || !aligned16(ws))
    return TA_ERR_WORKSPACE;
  hipError_t e = ta::launch_accept_sampling(target_logits, draft_logits, logit_dtype, parent, tok,
                                            n_nodes, root_tok, u_accept, u_bonus, c2, B, n_max,
                                            V, path, path_len, bonus, ws,
                                            static_cast<hipStream_t>(stream));
  return hip_status(e, "accept_sampling_path launch");
}

int tree_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new, ta_kv kv,
                     const int32_t* prefix_len, const int32_t* parent, const int32_t* n_nodes,
                     int B, int n_q, int n_max, int expand, int Hq, int Hkv, int d, int dtype,
                     float base, void* stream) {
  int st = check_common(B, n_q, n_max, Hq, Hkv, d, dtype, kv.T_cap);
  if (st != TA_OK) return st;
  st = check_kv(kv);
  if (st != TA_OK) return st;
  if (n_q > n_max || (expand != 0 && expand != 1)) return TA_ERR_INVALID_ARG;
  if (!(base > 0.f) || base != base || base == INFINITY) return TA_ERR_INVALID_ARG;
  if (q == nullptr || q_out == nullptr || k_new == nullptr || v_new == nullptr ||
      prefix_len == nullptr || parent == nullptr || n_nodes == nullptr)
    return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  ta::RopeParams p{};
  p.q_in = q;
  p.q_out = q_out;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k = kv.k;
  p.v = kv.v;
  p.block_table = kv.block_table;
  p.block_size = kv.block_size;
  p.max_blocks = kv.max_blocks;
  p.num_blocks = kv.num_blocks;
  p.T_cap = kv.T_cap;
  p.prefix_len = prefix_len;
  p.parent = parent;
  p.n_nodes = n_nodes;
  p.B = B;
  p.n_q = n_q;
  p.n_max = n_max;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.expand = expand;
  p.base = base;
  hipError_t e = ta::launch_rope_append(p, dtype, static_cast<hipStream_t>(stream));
  return hip_status(e, "tree_rope_append launch");
}

int tree_token_walk(const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
                    const int32_t* verified, const int32_t* verified_len, int B, int n_max,
                    int m_max, int32_t* path, int32_t* path_len, uint8_t* keep, void* stream) {
  if (B < 0 || n_max < 1 || m_max < 1) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (m_max > ta::kWalkMaxTokens) return TA_ERR_UNSUPPORTED;
  if (parent == nullptr || tok == nullptr || n_nodes == nullptr || verified == nullptr ||
      verified_len == nullptr || path == nullptr || path_len == nullptr || keep == nullptr)
    return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  hipError_t e = ta::launch_token_walk(parent, tok, n_nodes, verified, verified_len, B, n_max,
                                       m_max, path, path_len, keep,
                                       static_cast<hipStream_t>(stream));
  return hip_status(e, "tree_token_walk launch");
}

int tree_select_subtree(const float* cum, const int32_t* parent, const int32_t* tok,
                        const int32_t* n_nodes, int B, int n_max, int bs, int32_t* sel_node,
                        int32_t* sel_parent, int32_t* sel_tok, int32_t* sel_n, void* stream) {
  if (B < 0 || n_max < 1 || bs < 1 || bs > n_max) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (cum == nullptr || parent == nullptr || tok == nullptr || n_nodes == nullptr ||
      sel_node == nullptr || sel_parent == nullptr || sel_tok == nullptr || sel_n == nullptr)
    return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  hipError_t e = ta::launch_select_subtree(cum, parent, tok, n_nodes, B, n_max, bs, sel_node,
                                           sel_parent, sel_tok, sel_n,
                                           static_cast<hipStream_t>(stream));
  return hip_status(e, "tree_select_subtree launch");
}

int tree_cache_reroot(const ta_kv* kv_layers, int n_layers, int32_t* prefix_len, int32_t* parent,
                      int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                      const uint8_t* keep_subtree, int B, int n_max, int Hkv, int d, int dtype,
                      void* stream) {
  return reroot_call(kv_layers, n_layers, prefix_len, parent, n_nodes, path, path_len,
                     keep_subtree, nullptr, nullptr, B, n_max, Hkv, d, dtype, stream);
}

int tree_cache_reroot_draft(const ta_kv* kv_layers, int n_layers, int32_t* prefix_len,
                            int32_t* parent, int32_t* n_nodes, const int32_t* path,
                            const int32_t* path_len, const uint8_t* keep_subtree, int32_t* tok,
                            float* cum, int B, int n_max, int Hkv, int d, int dtype,
                            void* stream) {
  if (tok == nullptr) return TA_ERR_INVALID_ARG;
  return reroot_call(kv_layers, n_layers, prefix_len, parent, n_nodes, path, path_len,
                     keep_subtree, tok, cum, B, n_max, Hkv, d, dtype, stream);
}

size_t tree_accept_reroot_workspace_bytes(int B, int n_max) {
  if (B < 0 || n_max < 1 || n_max > TA_MAX_NODES) return static_cast<size_t>(-1);
  return accept_reroot_ws_bytes(B, n_max);
}

int tree_accept_reroot(const void* logits, int logit_dtype, const int32_t* tok,
                       const int32_t* root_tok, const ta_kv* kv_layers, int n_layers,
                       int32_t* prefix_len, int32_t* parent, int32_t* n_nodes,
                       const uint8_t* keep_subtree, int B, int n_max, int V, int Hkv, int d,
                       int dtype, int32_t* path, int32_t* path_len, int32_t* bonus, void* ws,
                       size_t ws_bytes, void* stream) {
  if (B < 0 || n_max < 1 || V < 1 || n_layers < 0 || Hkv < 1) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (logit_dtype != TA_F32 && logit_dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (dtype != TA_F32 && dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return TA_ERR_UNSUPPORTED;
  if (logits == nullptr || tok == nullptr || root_tok == nullptr || prefix_len == nullptr ||
      parent == nullptr || n_nodes == nullptr || keep_subtree == nullptr || path == nullptr ||
      path_len == nullptr || bonus == nullptr || (n_layers > 0 && kv_layers == nullptr))
    return TA_ERR_INVALID_ARG;
  for (int i = 0; i < n_layers; ++i) {
    const int st = check_kv(kv_layers[i]);
    if (st != TA_OK) return st;
    if (!aligned16(kv_layers[i].k) || !aligned16(kv_layers[i].v)) return TA_ERR_INVALID_ARG;
  }
  if (B == 0) return TA_OK;
  if (ws == nullptr || ws_bytes < accept_reroot_ws_bytes(B, n_max) || !aligned16(ws))
    return TA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const size_t rows = accept_reroot_region(static_cast<size_t>(B) * n_max * sizeof(int32_t));
  const size_t seq = accept_reroot_region(static_cast<size_t>(B) * sizeof(int32_t));
  int32_t* amax = reinterpret_cast<int32_t*>(w);
  ta::MetaSnapshot snap{prefix_len, parent, reinterpret_cast<int32_t*>(w + 2 * rows),
                        reinterpret_cast<int32_t*>(w + 2 * rows + seq),
                        reinterpret_cast<int32_t*>(w + rows)};
  hipError_t e = ta::launch_argmax(logits, logit_dtype, n_nodes, B, n_max, V, amax, snap, s);
  if (e != hipSuccess) return hip_status(e, "tree_accept_reroot argmax launch");
  const int row_bytes = d * (dtype == TA_BF16 ? 2 : 4);
  // Every launch takes the path itself from the snapshot; the first writes
  // the path and the new metadata out.
  int l0 = 0;
  do {
    const int cnt = std::min(ta::kRerootMaxLayersPerLaunch, n_layers - l0);
    ta::RerootLayers L{};
    for (int i = 0; i < cnt; ++i) {
      const ta_kv& kv = kv_layers[l0 + i];
      L.l[i] = ta::RerootLayer{kv.k, kv.v, kv.block_table, kv.block_size, kv.max_blocks,
                               kv.num_blocks, kv.T_cap};
    }
    e = ta::launch_accept_reroot(L, cnt, prefix_len, parent, n_nodes, snap, tok, root_tok, amax,
                                 keep_subtree, B, n_max, Hkv, row_bytes, path, path_len, bonus,
                                 l0 == 0 ? 1 : 0, s);
    if (e != hipSuccess) return hip_status(e, "tree_accept_reroot launch");
    l0 += cnt;
  } while (l0 < n_layers);
  return TA_OK;
}

size_t tree_expand_top_w_workspace_bytes(int B, int n_max, int w) {
  if (B < 0 || n_max < 1 || n_max > TA_MAX_NODES || w < 1 || w > ta::kTopwMaxW)
    return static_cast<size_t>(-1);
  return ta::topw_ws_bytes(B, n_max, w);
}

int tree_expand_top_w(const void* logits, int logit_dtype, int32_t* parent, int32_t* tok,
                      float* cum, int32_t* n_nodes, int B, int n_max, int V, int w, void* ws,
                      size_t ws_bytes, void* stream) {
  if (B < 0 || n_max < 1 || V < 1 || w < 1) return TA_ERR_INVALID_ARG;
  if (n_max > TA_MAX_NODES) return TA_ERR_TREE_TOO_LARGE;
  if (w > ta::kTopwMaxW || V > ta::kTopwMaxVocab) return TA_ERR_UNSUPPORTED;
  if (logit_dtype != TA_F32 && logit_dtype != TA_BF16) return TA_ERR_UNSUPPORTED;
  if (logits == nullptr || parent == nullptr || tok == nullptr || cum == nullptr ||
      n_nodes == nullptr)
    return TA_ERR_INVALID_ARG;
  if (B == 0) return TA_OK;
  if (ws == nullptr || ws_bytes < ta::topw_ws_bytes(B, n_max, w) || !aligned16(ws))
    return TA_ERR_WORKSPACE;
  hipError_t e = ta::launch_topw(logits, logit_dtype, parent, tok, cum, n_nodes, B, n_max, V, w,
                                 ws, static_cast<hipStream_t>(stream));
  return hip_status(e, "tree_expand_top_w launch");
}

const char* ta_status_string(int status) {
  switch (status) {
    case TA_OK: return "TA_OK";
    case TA_ERR_INVALID_ARG: return "TA_ERR_INVALID_ARG: invalid argument";
    case TA_ERR_UNSUPPORTED: return "TA_ERR_UNSUPPORTED: unsupported size or dtype";
    case TA_ERR_TREE_TOO_LARGE: return "TA_ERR_TREE_TOO_LARGE: more than 256 tree nodes";
    case TA_ERR_WORKSPACE: return "TA_ERR_WORKSPACE: workspace missing or too small";
    case TA_ERR_HIP: return "TA_ERR_HIP: HIP launch or runtime failure";
    case TA_ERR_SCRATCH:
      return "TA_ERR_SCRATCH: the call needs more than the 72 MiB scratch array of "
             "tree_attn_verify_noalloc";
    default: return "unknown ta_status";
  }
}

const char* ta_version(void) { return "0.1.0"; }

const char* ta_last_error(void) { return ta::g_last_error; }

}  // extern "C"
