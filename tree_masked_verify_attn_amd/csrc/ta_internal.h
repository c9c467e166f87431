// Internal declarations shared by the HIP translation units of libtreeattn.
// Public API: include/tree_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

#include "tree_attn.h"

namespace ta {

// Launches `kernel` and returns the status of this launch only (unlike
// hipGetLastError, which also reports errors left behind by other code).
template <typename Tuple, size_t... I>
inline hipError_t launch_tuple(const void* kernel, dim3 grid, dim3 block, hipStream_t s,
                               Tuple& vals, std::index_sequence<I...>) {
  void* ptrs[] = {static_cast<void*>(&std::get<I>(vals))..., nullptr};
  return hipLaunchKernel(kernel, grid, block, ptrs, 0, s);
}
template <typename... Params, typename... Args>
inline hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         Args&&... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  // converted to the kernel's own parameter types before their addresses are taken
  std::tuple<std::decay_t<Params>...> vals(std::forward<Args>(args)...);
  return launch_tuple(reinterpret_cast<const void*>(kernel), grid, block, s, vals,
                      std::index_sequence_for<Params...>{});
}

// Records the last HIP failure of the calling thread (read by ta_last_error).
void set_last_error(hipError_t e, const char* where);

// ---------------------------------------------------------------------------
// Plain-old-data parameter block of one attention launch (passed by value).
// ---------------------------------------------------------------------------
struct AttnParams {
  const void* q;
  void* out;
  float* lse;
  const void* k;
  const void* v;
  const int32_t* block_table;  // nullptr: contiguous layout
  int32_t block_size, max_blocks, num_blocks, T_cap;
  const int32_t* prefix_len;
  const int32_t* parent;
  const int32_t* n_nodes;
  int32_t B, n_max, Hq, Hkv, d, G;
  int32_t n_q;          // query rows per sequence in q/out (n_max or w)
  int32_t expand;       // 0: row r is node r; 1: row r is node n - n_q + r
  float scale_log2;     // softmax scale * log2(e): scores are kept in log2 units
  // split-KV plan
  int32_t chunk;        // KV tokens per split (multiple of 64)
  int32_t n_split;      // splits allocated per (b, kv head, row tile)
  int32_t rows_per_tile;
  int32_t n_row_tiles;
  // workspace (only when n_split > 1)
  float* ws_o;          // [tiles][n_split][rows_per_tile][d] unnormalised partial outputs
  float* ws_ml;         // [tiles][n_split][rows_per_tile][2]  running max (log2) and sum
  // ws_f16 = 1 (the bf16 MFMA kernels): ws_o holds the partial outputs in
  // half precision and ws_ml 16-byte records instead (layout in partial_f16.h)
  int32_t ws_f16;
  // units kernel only: n_split is its number of work groups G, ws_o / ws_ml
  // hold 2G slots of rows_per_tile rows, ws_seq one 16-byte record per
  // sequence (its stream start, the stream's length, and the P and n the
  // attention launch took)
  int32_t* ws_seq;
  // RoPE on load (streaming kernel only, contiguous caches): q holds the
  // un-rotated queries, k_new / v_new [B][n_q][Hkv][d] the new nodes' keys
  // (un-rotated) and values, which the kernel rotates, attends to and writes
  // to cache rows P + node (the work groups of row tile 0).
  const void* k_new;
  const void* v_new;
  float rope_base;
  int32_t rope;
};

// One attention call (tree_attn_verify / tree_attn_expand): validation,
// planning, launches.  With `scratch` set, the workspace arguments are
// ignored and scratch(bytes the plan needs, stream, &ws) supplies the buffer
// once the plan is known (only when the plan needs one).
typedef int (*ScratchFn)(size_t need, void* stream, void** ws);
// RoPE at tree positions as part of the call (tree_attn_*_rope): the new
// nodes' keys and values [B][n_q][Hkv][d] and the base.
struct RopeArgs {
  const void* k_new;
  const void* v_new;
  float base;
};
int run_attention(const void* q, ta_kv kv, const int32_t* prefix_len, const int32_t* parent,
                  const int32_t* n_nodes, int B, int n_q, int n_max, int expand, int Hq, int Hkv,
                  int d, int dtype, float scale, void* out, float* lse, void* ws,
                  size_t ws_bytes, const ta_attn_opts* opts, void* stream, ScratchFn scratch,
                  const RopeArgs* rope);

// Workspace layout: the partial outputs, then the (max, sum) pairs.  Returns
// the bytes needed for a plan (0 when there is a single split).
size_t attn_ws_bytes(int tiles, int n_split, int rows_per_tile, int d);

hipError_t launch_attn_generic(const AttnParams& p, int dtype, hipStream_t s);
// Second launch of a split call: combines the partial states into out / lse.
hipError_t launch_attn_merge(const AttnParams& p, int dtype, hipStream_t s);
hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t s);
// Streaming MFMA variant: a ring of four 32-position LDS stages.
hipError_t launch_attn_stream(const AttnParams& p, hipStream_t s);
// Whether the streaming kernel can rotate on load for these sizes (its
// cos/sin table of one row tile's query slots fits two ring stages).
bool stream_rope_fits(int d, int rows_per_tile, int G);
constexpr int kStreamMaxSplitBlocks = 512;  // paged: block ids of one split held in LDS
// Units kernel: every (sequence, row tile, KV head) job's tiles laid end to end,
// G equal ranges of them, one per work group; then a combine launch.
constexpr int kUnitMaxSeqs = 1024;
constexpr int kUnitJobCost = 6;  // stream units a job counts beyond its tiles
hipError_t launch_attn_units(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_merge_units(const AttnParams& p, hipStream_t s);

// Accept: argmax pass (writes a[i] into path) then the path pass.
// A copy of the tree metadata taken by the argmax launch (parent == nullptr:
// none), so that the launch after it can rewrite the live arrays while its
// other work groups still read the old values from the copy.
struct MetaSnapshot {
  const int32_t* prefix_len;
  const int32_t* parent;
  int32_t* prefix_len_out;  // [B]
  int32_t* n_nodes_out;     // [B]
  int32_t* parent_out;      // [B][n_max]
};
// argmax of every node's logits row (lowest index on ties) into out [B][n_max]
// (and the snapshot of the metadata).
hipError_t launch_argmax(const void* logits, int logit_dtype, const int32_t* n_nodes, int B,
                         int n_max, int V, int32_t* out, const MetaSnapshot& snap, hipStream_t s);
hipError_t launch_accept(const void* logits, int logit_dtype, const int32_t* parent,
                         const int32_t* tok, const int32_t* n_nodes, const int32_t* root_tok,
                         int B, int n_max, int V, int32_t* path, int32_t* path_len,
                         int32_t* bonus, hipStream_t s);

// Top-w expansion: a rows pass (per-row log-sum-exp and w best allowed
// tokens) then a select pass that appends the w best candidates.
constexpr int kTopwMaxW = 16;
constexpr int kTopwMaxVocab = 1 << 18;
size_t samp_ws_bytes(int B, int n_max);
hipError_t launch_accept_sampling(const void* tgt, const void* dft, int logit_dtype,
                                  const int32_t* parent, const int32_t* tok,
                                  const int32_t* n_nodes, const int32_t* root_tok,
                                  const float* u_accept, const float* u_bonus, float c2, int B,
                                  int n_max, int V, int32_t* path, int32_t* path_len,
                                  int32_t* bonus, void* ws, hipStream_t s);
size_t topw_ws_bytes(int B, int n_max, int w);
hipError_t launch_topw(const void* logits, int logit_dtype, int32_t* parent, int32_t* tok,
                       float* cum, int32_t* n_nodes, int B, int n_max, int V, int w, void* ws,
                       hipStream_t s);

// RoPE at tree positions (P - 1 + depth) of the query rows and the new nodes'
// keys, and the append of those keys and values to cache rows P + node.
struct RopeParams {
  const void* q_in;
  void* q_out;
  const void* k_new;
  const void* v_new;
  void* k;
  void* v;
  const int32_t* block_table;
  int32_t block_size, max_blocks, num_blocks, T_cap;
  const int32_t* prefix_len;
  const int32_t* parent;
  const int32_t* n_nodes;
  int32_t B, n_q, n_max, Hq, Hkv, d, expand;
  float base;
};
hipError_t launch_rope_append(const RopeParams& p, int dtype, hipStream_t s);

// Draft side of an iteration: the walk along the verified tokens (re-root
// path and keep flag) and the choice of the size-bs subtree to send.
constexpr int kWalkMaxTokens = 1024;
hipError_t launch_token_walk(const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
                             const int32_t* verified, const int32_t* verified_len, int B,
                             int n_max, int m_max, int32_t* path, int32_t* path_len,
                             uint8_t* keep, hipStream_t s);
hipError_t launch_select_subtree(const float* cum, const int32_t* parent, const int32_t* tok,
                                 const int32_t* n_nodes, int B, int n_max, int bs,
                                 int32_t* sel_node, int32_t* sel_parent, int32_t* sel_tok,
                                 int32_t* sel_n, hipStream_t s);

// Re-root: one launch per group of layers moves rows, then one updates metadata.
constexpr int kRerootMaxLayersPerLaunch = 32;
struct RerootLayer {
  void* k;
  void* v;
  const int32_t* block_table;
  int32_t block_size, max_blocks, num_blocks, T_cap;
};
struct RerootLayers {
  RerootLayer l[kRerootMaxLayersPerLaunch];
};
hipError_t launch_reroot_move(const RerootLayers& layers, int n_layers,
                              const int32_t* prefix_len, const int32_t* parent,
                              const int32_t* n_nodes, const int32_t* path,
                              const int32_t* path_len, const uint8_t* keep, int B, int n_max,
                              int Hkv, int row_bytes, hipStream_t s);
hipError_t launch_reroot_meta(int32_t* prefix_len, int32_t* parent, int32_t* n_nodes,
                              const int32_t* path, const int32_t* path_len, const uint8_t* keep,
                              int B, int n_max, int32_t* tok, float* cum, hipStream_t s);
// Greedy acceptance + re-root of a group of layers in one launch (see
// reroot.hip); amax holds the target's argmax per node (launch_argmax).
hipError_t launch_accept_reroot(const RerootLayers& layers, int n_layers, int32_t* prefix_len,
                                int32_t* parent, int32_t* n_nodes, const MetaSnapshot& snap,
                                const int32_t* tok, const int32_t* root_tok, const int32_t* amax,
                                const uint8_t* keep, int B, int n_max, int Hkv, int row_bytes,
                                int32_t* path, int32_t* path_len, int32_t* bonus, int first,
                                hipStream_t s);

}  // namespace ta
