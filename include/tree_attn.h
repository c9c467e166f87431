/*
 * tree_attn.h -- C ABI of the MI355X (gfx950) tree-masked verify/expand
 * attention library (libtreeattn.so).
 *
 * The operations follow the pages this library implements:
 *
 *   [SS]  "SwiftSpec summary -- Disaggregated Speculative Decoding"
 *   [DL]  "Draft-length co-design" article (speculative decoding with an AI
 *         model co-design for faster LLM inference)
 *   [MD]  "MineDraft notes" (batch parallelism)
 *
 * Conventions shared by every call
 * --------------------------------
 * Tree.  A draft tree holds one token per node; parent -> child means "the
 *   child's token follows the parent's" ([SS] Section 3.1).  Nodes are stored
 *   in topological order: -1 <= parent[b*n_max + i] < i.  parent = -1 marks a
 *   child of the root, and the root is the last token of the prefix cache.
 *   On the target side the root token itself is node 0 (parent[0] = -1,
 *   parent[i] >= 0 for i >= 1), so verifying 1 + D tokens means n = 1 + D
 *   query nodes ([DL] key mechanism).  At most TA_MAX_NODES nodes.
 *
 * KV cache.  One layer's keys and values ([SS] Section 3.2 invariant):
 *   positions 0 .. P-1 of a sequence hold the prefix cache (verified tokens),
 *   position P + i holds tree node i.  P = prefix_len[b] and the tree size
 *   n = n_nodes[b] live in device memory, so a whole step can be captured in
 *   a HIP graph without host synchronisation.
 *   - contiguous:  K, V are [B][T_cap][Hkv][d]
 *   - paged:       K, V are [num_blocks][block_size][Hkv][d]; position t of
 *                  sequence b is block block_table[b*max_blocks + t/block_size],
 *                  slot t % block_size ([MD] Section 5.3, vLLM KV blocks).
 *   Elements are fp32 or bf16 (TA_F32 / TA_BF16); d is 64 or 128.
 *
 * Grouped-query attention.  G = Hq / Hkv query heads share one KV head; query
 *   head h reads KV head h / G ([DL] key mechanism: G = query heads per KV
 *   head, G x (1 + D) query rows per KV head).
 *
 * Memory and errors.  Every array argument is a device pointer unless the
 *   comment says "host".  The caller allocates and owns everything, including
 *   the attention workspace; the library allocates nothing and keeps no state
 *   between calls.  Calls are asynchronous on `stream` (a hipStream_t; NULL
 *   is the default stream) and return a ta_status synchronously for problems
 *   the host can see (null pointers, unsupported sizes or dtypes, workspace
 *   too small, a failed launch).  Device-side preconditions (valid parent
 *   arrays, P + n <= T_cap, valid block ids, a root path in `path`, finite
 *   logits) are the caller's; when they are violated the results are
 *   unspecified, but the kernels clamp every index so that no access leaves
 *   the buffers described here.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TA_MAX_NODES 256   /* tree capacity per sequence (4 x 64-bit masks) */

typedef enum {
  TA_OK = 0,
  TA_ERR_INVALID_ARG = -1,     /* null pointer, negative size, Hq % Hkv != 0, ... */
  TA_ERR_UNSUPPORTED = -2,     /* d not in {64,128}, unknown dtype, ...          */
  TA_ERR_TREE_TOO_LARGE = -3,  /* n_max > TA_MAX_NODES                           */
  TA_ERR_WORKSPACE = -4,       /* workspace missing or smaller than required     */
  TA_ERR_HIP = -5,             /* a HIP runtime call or kernel launch failed     */
  TA_ERR_SCRATCH = -6          /* tree_attn_verify_noalloc: the call's plan needs
                                  more than TA_NOALLOC_SCRATCH_BYTES            */
} ta_status;

typedef enum { TA_F32 = 0, TA_BF16 = 1 } ta_dtype;

/* One layer's KV cache.  block_table == NULL selects the contiguous layout. */
typedef struct {
  void* k;                       /* keys   (layout above)                          */
  void* v;                       /* values (same layout as k)                      */
  const int32_t* block_table;    /* paged: [B][max_blocks] physical block ids      */
  int32_t block_size;            /* paged: tokens per block (> 0)                  */
  int32_t max_blocks;            /* paged: columns of block_table                  */
  int32_t num_blocks;            /* paged: blocks in the pool (ids are < this)     */
  int32_t T_cap;                 /* contiguous: tokens per sequence in k and v;
                                    paged: logical capacity, <= max_blocks*block_size */
} ta_kv;

/* Optional tuning/testing knobs for the attention calls (NULL = automatic). */
typedef struct {
  int32_t chunk_tokens;  /* KV tokens per split-KV work item, a multiple of 64; 0 = auto */
  int32_t kernel;        /* 0 = auto (bf16: 4 for paged caches, 3 for contiguous ones;
                            else 1); 1 = generic fp32-math kernel;
                            2 = bf16 MFMA kernel, register prefetch; 3 = bf16 MFMA kernel,
                            LDS-DMA ring and pipelined tiles (paged calls whose split spans
                            more than 510 blocks run on kernel 2); 4 = bf16 MFMA kernel over
                            balanced units: every job's KV tiles end to end, one equal range
                            per resident work group, the ring running across jobs (B <= 1024;
                            chunk_tokens is ignored) */
} ta_attn_opts;

/*
 * Workspace (bytes) needed by tree_attn_verify / tree_attn_expand for these
 * sizes, enough for the plan of a contiguous and of a paged cache alike.
 * n_q is n_max for verify and w for expand.  The workspace holds the split-KV
 * partial results (per split or work-group range and query row: running
 * maximum, sum and unnormalised output, the output in fp32 for the generic
 * kernel and in fp16 under a per-row power-of-two scale for the bf16 MFMA
 * kernels) that a second, combining launch of the same call reads, and for
 * kernel 4 a 16-byte record per sequence (its place in the work stream); its
 * contents need no initialisation and are meaningless between calls.  Calls
 * that overlap in time must not share a workspace.  Returns 0 when the plans
 * need none (kernels 1-3 without a split; ws may then be NULL), or
 * (size_t)-1 for invalid sizes.
 */
size_t tree_attn_workspace_bytes(int B, int n_q, int Hq, int Hkv, int d, int dtype, int T_cap,
                                 const ta_attn_opts* opts);

/*
 * Tree-masked verification attention ([SS] Section 3.1.2 Figure 2 target
 * side; [DL] key mechanism: the 1 + D drafted tokens are checked in one
 * pass).  Query rows are every tree node i < n_nodes[b]; row i attends to all
 * P prefix positions and to the tree positions of its ancestors and itself.
 *
 *   q      [B][n_max][Hq][d]  (dtype)  queries, already position-rotated
 *   out    [B][n_max][Hq][d]  (dtype)  softmax(scale*q.k^T restricted) . v,
 *                                      rounded to nearest-even for bf16
 *   lse    [B][Hq][n_max]     fp32     natural-log log-sum-exp of the scaled,
 *                                      masked scores (may be NULL)
 *   Rows i >= n_nodes[b] of out and lse are not written.
 *   The queries' own K/V must already sit at positions P + i.
 */
int tree_attn_verify(const void* q, ta_kv kv, const int32_t* prefix_len, const int32_t* parent,
                     const int32_t* n_nodes, int B, int n_max, int Hq, int Hkv, int d, int dtype,
                     float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                     const ta_attn_opts* opts, void* stream);

/*
 * Tree-masked expansion attention ([SS] Section 3.1.3 Figure 3: w new
 * leaves x (prefix + tree) non-square mask).  Query row r is tree node
 * n_nodes[b] - w + r (the w newest nodes, whose K/V are already appended);
 * rows with a negative node index are not written.
 *
 *   q, out [B][w][Hq][d] (dtype);  lse [B][Hq][w] fp32 (may be NULL)
 */
int tree_attn_expand(const void* q, ta_kv kv, const int32_t* prefix_len, const int32_t* parent,
                     const int32_t* n_nodes, int B, int w, int n_max, int Hq, int Hkv, int d,
                     int dtype, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                     const ta_attn_opts* opts, void* stream);

/*
 * Verification / expansion attention with the position embedding fused in
 * ([SS] Section 3.3: the masked-attention kernel takes RoPE; Section 3.2: a
 * node's KV is written once, where it was computed).  The same results, and
 * the same cache rows written, as tree_rope_append(q, q_rot, k_new, v_new, kv,
 * ...) followed by tree_attn_verify / tree_attn_expand on q_rot, in one call:
 *
 *   q             [B][n_q][Hq][d] (dtype) un-rotated queries (n_q = n_max for
 *                 verify, w for expand; slot s holds node s, or node
 *                 n_nodes[b] - w + s when expanding)
 *   k_new, v_new  [B][n_q][Hkv][d] (dtype) the same slots' un-rotated keys and
 *                 their values; the call rotates the keys to the nodes'
 *                 positions P - 1 + depth and writes keys and values to cache
 *                 rows P + node, as tree_rope_append does
 *   base          RoPE base (> 0, finite): channel pair (j, j + d/2) turns by
 *                 position * base^(-2j/d)
 *   everything else as for tree_attn_verify / tree_attn_expand (the same
 *   workspace size).
 *
 * bf16 contiguous caches with at most 64 query slots per 128-row tile (G >= 4
 * for 128 rows) run one launch that rotates the queries as it loads them,
 * stages the new nodes' rotated keys for its own tree tiles and has the work
 * groups of row tile 0 write the new rows.  Other calls run the RoPE append
 * (rotated queries into `out`) and then the attention launch on `out`.  `out`
 * must not alias q, k_new, v_new or the cache.
 */
int tree_attn_verify_rope(const void* q, const void* k_new, const void* v_new, ta_kv kv,
                          const int32_t* prefix_len, const int32_t* parent, const int32_t* n_nodes,
                          int B, int n_max, int Hq, int Hkv, int d, int dtype, float scale,
                          float base, void* out, float* lse, void* ws, size_t ws_bytes,
                          const ta_attn_opts* opts, void* stream);
int tree_attn_expand_rope(const void* q, const void* k_new, const void* v_new, ta_kv kv,
                          const int32_t* prefix_len, const int32_t* parent, const int32_t* n_nodes,
                          int B, int w, int n_max, int Hq, int Hkv, int d, int dtype, float scale,
                          float base, void* out, float* lse, void* ws, size_t ws_bytes,
                          const ta_attn_opts* opts, void* stream);

/*
 * Greedy longest accepted path ([DL] how speculative decoding works and the
 * Acceptance Length entry: accept up to the first mismatch, then the
 * target's own token; AL in [1, 1 + D]).
 *
 *   logits   [B][n_max][V]  fp32 or bf16 (logit_dtype); row i is the target's
 *                           distribution after node i
 *   tok      [B][n_max]     int32 draft token of each node
 *   root_tok [B]            int32 the target's token after the last prefix
 *                           token (on the target side: the root token, tok[0])
 *   path     [B][n_max]     int32 out: node ids of the accepted path from the
 *                           top of the tree, then -1
 *   path_len [B]            int32 out: its length (= AL on the target side)
 *   bonus    [B]            int32 out: the target's next token after the path
 *
 * a[i] = argmax of row i (lowest index on ties).  Node i is accepted when
 * every node u on its root path has tok[u] == (parent[u] < 0 ? root_tok :
 * a[parent[u]]).  The deepest accepted node wins (lowest index on ties);
 * bonus = a[best], or root_tok when nothing is accepted.
 */
int accept_greedy_path(const void* logits, int logit_dtype, const int32_t* parent,
                       const int32_t* tok, const int32_t* n_nodes, const int32_t* root_tok, int B,
                       int n_max, int V, int32_t* path, int32_t* path_len, int32_t* bonus,
                       void* stream);

/*
 * Evolving-tree-cache re-root with in-place KV compaction ([SS] Section 3.2,
 * Figure 4; Section 3.1.2 Figure 2).  For each sequence with k = path_len[b]
 * and path v_0 .. v_{k-1} (a root path of the tree):
 *   - rows P + v_j move to P + j (the verified nodes join the prefix);
 *   - if keep_subtree[b] and k > 0, the descendants of v_{k-1}, in their
 *     original order, move to P + k, P + k + 1, ...; their parents are
 *     renumbered and children of v_{k-1} get parent -1;
 *   - prefix_len[b] += k; n_nodes[b] = number of kept nodes; parent entries
 *     past it are set to -1.  k == 0 with keep is a no-op; k == 0 without
 *     keep drops the tree.
 * Every layer in kv_layers (a HOST array of n_layers descriptors, K and V,
 * all with the same dtype, Hkv and d) is compacted bit for bit; rows at or
 * past the new end are left unspecified.  prefix_len, parent and n_nodes are
 * updated in place after all layers have been moved.
 */
int tree_cache_reroot(const ta_kv* kv_layers, int n_layers, int32_t* prefix_len, int32_t* parent,
                      int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                      const uint8_t* keep_subtree, int B, int n_max, int Hkv, int d, int dtype,
                      void* stream);

/*
 * Draft-side re-root ([SS] Section 3.1.1 Algorithm 1: Re-root, then Select
 * on the re-rooted tree; Section 3.2 update procedure; Section 3.1.3: a
 * node's weight is the sum of values from the root down to it).  Exactly
 * tree_cache_reroot, and with the same node mapping the per-node arrays the
 * draft keeps beside its tree:
 *
 *   tok [B][n_max] int32 in/out: node tokens (required); kept node number r
 *            (in original order) takes the token of the node it was
 *   cum [B][n_max] fp32 in/out (may be NULL): cumulative log-probabilities
 *            (as tree_expand_top_w keeps them), re-based to the new root, the
 *            last verified node v: cum'[r] = cum[kept node r] - cum[v], one
 *            fp32 subtraction
 *
 * Entries at or past the new n_nodes[b] are set to -1 (tok) and -inf (cum).
 * k == 0 with keep changes nothing; k == 0 without keep, or a path whose
 * last node has no descendants, leaves no node.  The draft's next
 * tree_expand_top_w and tree_select_subtree then read a consistent tree.
 */
int tree_cache_reroot_draft(const ta_kv* kv_layers, int n_layers, int32_t* prefix_len,
                            int32_t* parent, int32_t* n_nodes, const int32_t* path,
                            const int32_t* path_len, const uint8_t* keep_subtree, int32_t* tok,
                            float* cum, int B, int n_max, int Hkv, int d, int dtype,
                            void* stream);

/*
 * accept_greedy_path followed by tree_cache_reroot on the path it finds, in
 * two launches instead of four: the same outputs and the same final caches
 * and metadata, bit for bit ([DL] Acceptance Length entry; [SS] Section 3.2,
 * Figure 4).  The target side's verify step ends with it.
 *
 *   logits, logit_dtype, tok, root_tok, V: as for accept_greedy_path
 *   kv_layers, n_layers, prefix_len, parent, n_nodes, keep_subtree, Hkv, d,
 *   dtype: as for tree_cache_reroot (prefix_len, parent, n_nodes in/out)
 *   path, path_len, bonus: outputs as for accept_greedy_path (the path
 *            before the re-root renumbers the nodes)
 *   ws       device workspace of tree_accept_reroot_workspace_bytes(B, n_max)
 *            bytes, 16-byte aligned: the argmax per node and a copy of
 *            prefix_len, parent and n_nodes.  Its contents need no
 *            initialisation and are meaningless between calls.  Calls that
 *            overlap in time must not share a workspace.
 *
 * The first launch takes every node's argmax and copies the metadata.  In
 * the second (one more per 32 layers past the first 32), every work group of
 * the re-root move finds the accepted path itself from the copy, and one
 * group per sequence writes the path and the new metadata.  Errors as for
 * the two calls, plus TA_ERR_WORKSPACE.
 */
size_t tree_accept_reroot_workspace_bytes(int B, int n_max);
int tree_accept_reroot(const void* logits, int logit_dtype, const int32_t* tok,
                       const int32_t* root_tok, const ta_kv* kv_layers, int n_layers,
                       int32_t* prefix_len, int32_t* parent, int32_t* n_nodes,
                       const uint8_t* keep_subtree, int B, int n_max, int V, int Hkv, int d,
                       int dtype, int32_t* path, int32_t* path_len, int32_t* bonus, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * Tree verification by speculative sampling, temperature > 0 ([MD] the
 * PEARL walkthrough: a rejected draft token is replaced by a draw from
 * norm(max(0, p - q)); [MD] experimental setup: sampling at temperature
 * 1.0; [SS] Section 3.1: the draft tree).
 *
 *   target_logits, draft_logits [B][n_max][V] fp32 or bf16 (logit_dtype):
 *            row i is the target's / the draft's distribution after node i
 *   parent, tok, n_nodes, root_tok: as for accept_greedy_path (device)
 *   u_accept [B][n_max] fp32: a uniform number in [0, 1) per node, used
 *            when that node is tested; u_bonus [B] fp32: one per sequence
 *            for the bonus draw (the caller draws them)
 *   path, path_len, bonus: outputs as for accept_greedy_path
 *
 * With p = softmax(target row / T) and q = softmax(draft row / T) at an
 * accepted node: the walk starts at the lowest-index node with parent -1
 * whose token is root_tok (none: path_len 0, bonus = root_tok); the node's
 * children are tried in index order against r (first p): child c with token
 * x is accepted when u_accept[c] * q(x) < r(x) and the walk moves to it; a
 * rejection sets r = norm(max(0, r - q)) (unchanged if that sums to 0).
 * When no child is accepted the bonus is the smallest token t whose running
 * sum of r exceeds u_bonus * sum(r).  Drawn this way, with the tree's
 * siblings independent draws from q, every emitted token follows the
 * target's distribution.  Arithmetic is fp32; logits must be finite;
 * 0 < temperature < inf.  ws holds accept_sampling_workspace_bytes bytes
 * (16-byte aligned; calls that overlap in time must not share it).  A node
 * with k rejected children costs k passes over its two rows (k steps per
 * element each).
 */
int accept_sampling_path(const void* target_logits, const void* draft_logits, int logit_dtype,
                         const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
                         const int32_t* root_tok, const float* u_accept, const float* u_bonus,
                         float temperature, int B, int n_max, int V, int32_t* path,
                         int32_t* path_len, int32_t* bonus, void* ws, size_t ws_bytes,
                         void* stream);

/* Workspace (bytes) for accept_sampling_path, or (size_t)-1 for invalid sizes. */
size_t accept_sampling_workspace_bytes(int B, int n_max);

/*
 * Maximum-likelihood draft-tree expansion step ([SS] Section 3.1.3: a node's
 * value is the log-softmax probability of its token under its parent's
 * distribution, its weight the sum of the values from the root down to it;
 * an expansion takes the w best new leaves).
 *
 *   logits   [B][n_max + 1][V] fp32 or bf16 (logit_dtype): row 0 is the draft
 *            distribution after the root (the last prefix token), row 1 + i
 *            the one after node i
 *   parent   [B][n_max] int32 in/out, tok [B][n_max] int32 in/out,
 *   cum      [B][n_max] fp32 in/out: weight (cumulative log-probability) of
 *            each node, which the caller keeps for the existing nodes
 *   n_nodes  [B] int32 in/out
 *
 * For each sequence with n = n_nodes[b] the candidates are the pairs (p, t)
 * with p in {-1 (root), 0 .. n-1} and t a token (0 <= t < V) that is not
 * already the token of a child of p.  Candidate (p, t) scores
 *     cum[p] + logits[b][p + 1][t] - log sum_v exp(logits[b][p + 1][v])
 * (cum[-1] = 0), computed in fp32.  The best min(w, n_max - n) candidates
 * (higher score first; ties: lower p, then higher logit, then lower t)
 * become nodes n, n+1, ...: parent, tok and cum are written there and
 * n_nodes[b] grows by their number.  Logits must be finite.  1 <= w <= 16,
 * V <= 262144; ws holds tree_expand_top_w_workspace_bytes bytes (no
 * initialisation needed; calls that overlap in time must not share it).
 */
int tree_expand_top_w(const void* logits, int logit_dtype, int32_t* parent, int32_t* tok,
                      float* cum, int32_t* n_nodes, int B, int n_max, int V, int w, void* ws,
                      size_t ws_bytes, void* stream);

/* Workspace (bytes) for tree_expand_top_w, or (size_t)-1 for invalid sizes. */
size_t tree_expand_top_w_workspace_bytes(int B, int n_max, int w);

/*
 * Rotary position embedding at tree positions and the KV append of the new
 * nodes ([SS] Section 3.3: the masked attention takes the position
 * embedding, RoPE; Section 3.2: a node's KV stays where it was computed).
 * Run before tree_attn_verify / tree_attn_expand, which take rotated Q and K.
 *
 *   q, q_out     [B][n_q][Hq][d]  query rows, un-rotated in, rotated out (may
 *                alias); slot s holds node s (expand = 0) or node
 *                n_nodes[b] - n_q + s (expand = 1)
 *   k_new, v_new [B][n_q][Hkv][d] the same slots' keys (un-rotated) and values
 *   kv           the cache: the rotated key and the value of the node in slot
 *                s go to row prefix_len[b] + node (layouts as for
 *                tree_attn_verify)
 *   prefix_len, parent, n_nodes: as for tree_attn_verify (device)
 *
 * Node i sits at position P - 1 + depth(i) (a child of the root at P, where P
 * = prefix_len[b]); channel pair (j, j + d/2), j < d/2, turns by position *
 * base^(-2j/d) ("rotate half").  Angles are reduced in double precision, the
 * rotation is done in fp32 and stored in dtype.  Slots without a node are not
 * written.  1 <= n_q <= n_max; base > 0.
 */
int tree_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new, ta_kv kv,
                     const int32_t* prefix_len, const int32_t* parent, const int32_t* n_nodes,
                     int B, int n_q, int n_max, int expand, int Hq, int Hkv, int d, int dtype,
                     float base, void* stream);

/*
 * Draft-side walk along the target's verified tokens ([SS] Section 3.1.1
 * Algorithm 1, Synchronize and Re-root; Section 3.2 update procedure;
 * Section 3.1.2 Figure 2).
 *
 *   parent [B][n_max], tok [B][n_max], n_nodes [B]: the draft tree
 *   verified [B][m_max] int32, verified_len [B] int32: the tokens the target
 *            verified after the root, in order (the bonus token included)
 *   path [B][n_max] int32 out, path_len [B] int32 out, keep [B] uint8 out
 *
 * From the root (parent -1), each verified token that is the token of a
 * child of the current node moves the walk to that child (the lowest index
 * among children with equal tokens); the walk stops at the first token that
 * no child carries.  path gets the matched nodes, path_len their number, and
 * keep = 1 when every verified token matched (the last one becomes the root
 * and its subtree stays), else 0 (a new tree starts; the tokens after the
 * match need the draft model).  The outputs are the path / path_len /
 * keep_subtree arguments of tree_cache_reroot.  1 <= m_max <= 1024;
 * verified_len is clamped to [0, m_max].  All pointers are device pointers.
 */
int tree_token_walk(const int32_t* parent, const int32_t* tok, const int32_t* n_nodes,
                    const int32_t* verified, const int32_t* verified_len, int B, int n_max,
                    int m_max, int32_t* path, int32_t* path_len, uint8_t* keep, void* stream);

/*
 * The subtree of bs nodes to send to the target ([SS] Section 3.1.1
 * Algorithm 1, Select: the most promising subtree of size bs).
 *
 *   cum [B][n_max] fp32: cumulative log-probability of each node (as
 *            tree_expand_top_w keeps it); parent, tok, n_nodes: the tree
 *   sel_node, sel_parent, sel_tok [B][bs] int32 out; sel_n [B] int32 out
 *
 * The min(bs, n) nodes of largest cum (ties: lower index; NaN ranks last)
 * are chosen.  When cum does not increase from a parent to its child (true of
 * cumulative log-probabilities) they form a subtree and maximise the sum of
 * exp(cum), the expected number of accepted tokens under the draft model.
 * They are written in node order: sel_node the node index, sel_parent the
 * position of its parent inside the selection (-1: child of the root; also
 * for a parent that was not chosen, which only scores rising along a path
 * cause), sel_tok its token; entries past sel_n[b] are -1 / -1 / 0.
 * 1 <= bs <= n_max.  All pointers are device pointers.
 */
int tree_select_subtree(const float* cum, const int32_t* parent, const int32_t* tok,
                        const int32_t* n_nodes, int B, int n_max, int bs, int32_t* sel_node,
                        int32_t* sel_parent, int32_t* sel_tok, int32_t* sel_n, void* stream);

/*
 * tree_attn_verify for callers that cannot allocate memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels, plan and results as tree_attn_verify, without the
 * workspace pair: the split-KV partial results go to a fixed device array of
 * TA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call there).  The call allocates nothing.  A call whose plan needs
 * more than that (tree_attn_workspace_bytes tells) returns TA_ERR_SCRATCH
 * before any launch; the automatic plans of calls with d <= 128 on a
 * 256-compute-unit MI355X need at most 68.2 MB.  Every call on one GPU shares
 * that GPU's array and it keeps the last call's contents (the kernels
 * initialise what they read), so calls that overlap in time on one GPU race:
 * order them on one stream.  `stream` must belong to the current device.
 */
#define TA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
int tree_attn_verify_noalloc(const void* q, ta_kv kv, const int32_t* prefix_len,
                             const int32_t* parent, const int32_t* n_nodes, int B, int n_max,
                             int Hq, int Hkv, int d, int dtype, float scale, void* out,
                             float* lse, const ta_attn_opts* opts, void* stream);

/* Human-readable name of a ta_status value (static string). */
const char* ta_status_string(int status);

/* Library version, e.g. "0.1.0" (static string). */
const char* ta_version(void);

/* The HIP error behind the calling thread's most recent TA_ERR_HIP, as
 * "<where>: <hip error name> (<description>)"; "" if there was none.  The
 * string is thread-local and valid until the thread's next failing call. */
const char* ta_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
