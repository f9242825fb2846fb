/*
 * hydra.h - C ABI of libhydra: one Hydra/Medusa draft-and-verify round on an
 * AMD Instinct MI355X (gfx950).
 *
 * A round has four stages, one entry point each:
 *   hydra_draft_heads      draft heads + per-head top-k, filling the candidate tree
 *                          (hydra_draft_heads_sketch: the same with two-layer
 *                          LayerNorm heads; hydra_draft_heads_attn: with
 *                          Hydra++ self-attention fusion)
 *   tree_build             final tree (identity or pruned), ancestor table
 *   tree_attention_verify  tree-masked attention over a paged KV prefix
 *                          (tree_rope / tree_rope_qk first rotate the tree Q/K rows at
 *                          positions prefix_len + depth; tree_decoder_layer
 *                          runs a whole target layer over the tree rows and
 *                          tree_verify_layers the target's whole forward pass:
 *                          embeddings, every layer, final norm)
 *   tree_accept            target vocabulary projection + acceptance walk
 *   tree_commit            kept branch into the paged KV cache, next root and h
 * plus host-side tree-plan builders, workspace-size queries and status strings.
 *
 * Sources (cited by page title and section):
 *   [HG] "Hydra Guide: Sequentially-Dependent Speculative AI" (AiFetchly blog)
 *   [SD] "Speculative Decoding" (thegustafson.com blog)
 *   [MH] "Medusa Heads" (Ultralytics glossary)
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host". The caller owns every
 *     buffer; the library allocates and frees nothing. Scratch memory comes
 *     from a caller-provided workspace `ws` of at least the size the matching
 *     *_workspace_size query returns (ws may be NULL when that size is 0).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream) and the call returns without synchronising. Faults inside
 *     kernels surface at the caller's next synchronisation.
 *   - Return value: HYDRA_OK (0) or a negative HYDRA_ERR_* code. On error no
 *     work has been enqueued (argument checks happen first) except for
 *     HYDRA_ERR_HIP, which reports a failed launch. hydra_last_error()
 *     returns a thread-local message describing the last failure.
 *   - Layouts are row-major and dense. dtype selects the element type of the
 *     activation and weight tensors: HYDRA_F32 (float) or HYDRA_BF16
 *     (bfloat16 bits in uint16). Logits, log-sum-exps and cumulative
 *     log-probabilities are always float32; token ids and indices int32.
 *     With HYDRA_BF16, OR-ing HYDRA_VOCAB_PACKED into dtype says that the
 *     vocabulary projection weights of the call (the heads' W2, W_t, the W
 *     of hydra_vocab_projection) are in the packed layout of
 *     hydra_pack_weight; every other tensor keeps its row-major layout.
 *     HYDRA_LAYER_PACKED (tree_decoder_layer, tree_verify_layers) says the
 *     same of the decoder layers' Wqkv, Wo, Wgu and Wd (each layer's matrix
 *     packed on its own; the norm gains stay plain).
 *   - Entry points are stateless and reentrant; calls that share a workspace
 *     must be ordered on one stream.
 */
#ifndef HYDRA_H
#define HYDRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYDRA_OK 0
#define HYDRA_ERR_INVALID (-1)     /* bad pointer, size or index */
#define HYDRA_ERR_UNSUPPORTED (-2) /* valid but unsupported shape or dtype */
#define HYDRA_ERR_WORKSPACE (-3)   /* workspace smaller than required */
#define HYDRA_ERR_HIP (-4)         /* a HIP launch failed */

#define HYDRA_F32 0
#define HYDRA_BF16 1
#define HYDRA_VOCAB_PACKED 0x100 /* dtype flag: vocabulary weights packed */
#define HYDRA_LAYER_PACKED 0x200 /* dtype flag: decoder layer weights packed */
/* dtype flag of hydra_draft_heads with folded embedding tables (emb_proj):
 * W1[k] is the packed [d, d] copy of W1_k[:, :d], the h half (hydra_pack_weight
 * of that contiguous half), the only part of W1 such a call reads. For callers
 * that stream the h halves at the packed layout's rate. */
#define HYDRA_W1H_PACKED 0x400

#define HYDRA_MAX_DEPTH 8     /* deepest tree (number of draft heads used) */
#define HYDRA_MAX_TOPK 16     /* widest fan-out of one node */
#define HYDRA_MAX_TREE 1024   /* nodes of a candidate tree before pruning */
#define HYDRA_MAX_VERIFY 256  /* rows of the tree that is verified */

/* Human-readable name of a status code (static string). */
const char* hydra_status_string(int code);
/* Message of the last failing call on this thread ("" if none). */
const char* hydra_last_error(void);
/* Version of this interface; bumps when a signature changes. */
int hydra_abi_version(void);

/* ------------------------------------------------------------------------
 * Tree plans (host only, no device work)
 *
 * A plan is the shape of a candidate tree, independent of token values, in
 * breadth-first order: node 0 is the root (the last known token, not yet in
 * the KV cache); parent[i] < i; the children of a node are contiguous and
 * sorted by rank, where rank is the entry of the parent's top-k list that the
 * child takes. All arrays are host int32 of length max_nodes (capacity).
 * Return value: number of nodes N (> 0), or a negative error code.
 * ---------------------------------------------------------------------- */

/* Cartesian tree from a branching vector b[0..K-1]: head k keeps its top-b_k
 * continuations of every node at depth k-1, giving sum_k prod_{j<=k} b_j
 * candidates plus the root ([HG] "Candidate Tree Construction"; [MH] "Tree
 * Attention und Akzeptanz", top-2 x top-3 = six candidates). */
int hydra_plan_cartesian(const int32_t* b, int K, int max_nodes,
                         int32_t* parent, int32_t* rank, int32_t* depth);

/* Static sparse tree of n_nodes rows, root included ([MH] "Tree Attention und
 * Akzeptanz": a 64-node sparse tree of the most accurate combinations). With no
 * accuracy statistics available, rank paths (r_1..r_d) with r_j < caps[j-1]
 * are ordered by (2^d * prod(r_j + 1), d, path) ascending and the first
 * n_nodes - 1 are kept. caps[0..K-1], K <= HYDRA_MAX_DEPTH. */
int hydra_plan_sparse(const int32_t* caps, int K, int n_nodes, int max_nodes,
                      int32_t* parent, int32_t* rank, int32_t* depth);

/* Head rows of a plan. Hydra (hydra = 1, [HG] "Candidate Tree Construction"):
 * head k runs once for every node at depth k-1 that has children, on
 * [h || e(token of that node)]. Medusa (hydra = 0, [MH] "Tree Attention und
 * Akzeptanz"): one row per depth serves every parent at that depth.
 * Outputs (host):
 *   node_row[N]          row whose top-k list gives node i's children, -1 if none
 *   row_node[R]          node a row conditions on (Hydra), -1 (Medusa)
 *   row_first[Dmax+1]    rows of head k (1-based) are [row_first[k-1], row_first[k])
 *   depth_first[Dmax+2]  nodes of depth k are [depth_first[k], depth_first[k+1])
 *   k_per_depth[Dmax]    top-k width head k needs (widest fan-out at depth k-1)
 * row_node needs capacity N; row_first/depth_first/k_per_depth capacity
 * HYDRA_MAX_DEPTH + 2. Returns R (number of rows) or a negative error code. */
int hydra_plan_rows(int N, const int32_t* parent, const int32_t* rank,
                    const int32_t* depth, int hydra, int32_t* node_row,
                    int32_t* row_node, int32_t* row_first, int32_t* depth_first,
                    int32_t* k_per_depth);

/* ------------------------------------------------------------------------
 * Packed weight layout for the streaming projections
 *
 * The vocabulary projections stream W once per call and are bound by HBM
 * reads. Row-major, the chip's concurrent reads of a K chunk are 512-byte
 * pieces 2K bytes apart (one per row); packed, every 16-row tile's chunk
 * of 256 columns is 8 KB in one place and chunk c of all tiles lies in one
 * contiguous range, so the reads of a chunk sweep contiguous memory (same
 * arithmetic, a layout of the same values). Layout: tiles of 16 rows (the
 * last one padded with zero rows), chunk-major: chunk c of tile t is 4096
 * bf16 at (c * ceil(N / 16) + t) * 4096; inside it, 32-column step s at
 * + 512 s, 8-column group g at + 128 g, row r at + 8 r (8 values of row
 * 16 t + r, columns 256 c + 32 s + 8 g ..).
 *
 * hydra_packed_weight_size: bytes of the packed copy of a bf16 W [N, K]
 * (0 when K % 256 != 0 or a size is not positive).
 * hydra_pack_weight: writes it; W and packed 16-byte aligned, not aliasing.
 * Errors: HYDRA_ERR_INVALID (sizes, null or aliasing pointers),
 * HYDRA_ERR_UNSUPPORTED (K % 256 != 0). No workspace.
 * ---------------------------------------------------------------------- */
size_t hydra_packed_weight_size(int N, int K);

int hydra_pack_weight(int N, int K, const void* W, void* packed, void* stream);

/* ------------------------------------------------------------------------
 * Stage 1: draft heads
 *
 * For every head row r of depth k (rows of head k) and sequence b:
 *   x   = h_b (Medusa)  or  [h_b || E[token of row_node[r]]] (Hydra)
 *   a   = W1_k x + b1_k
 *   u   = h_b + SiLU(a)   (residual = 1)   or   SiLU(a)   (residual = 0)
 *   z   = W2_k u                          -> head_logits[b, r, :]
 *   lse = log sum exp z                   -> head_lse[b, r]
 * ([MH] "So sagen die Köpfe voraus": SiLU layer with a residual connection and
 * a vocabulary projection; [HG] "1. Embedding Conditioning Mechanics": Hydra
 * heads read [h || e(x_parent)].) Every child c of a node served by row r
 * takes entry rank[c] of the row's top-k list (sorted by logit descending,
 * ties to the lower id) and cand_logp[c] = cand_logp[parent] + z[tok] - lse.
 * Heads run in depth order because Hydra head k needs depth k-1's tokens.
 * In bf16 mode u is stored as bfloat16 (round to nearest even); the
 * projections accumulate in float32.
 *
 * dtype        HYDRA_F32 or HYDRA_BF16 (h, emb, W1, b1, W2, head_hidden)
 * B, d, V      sequences, hidden size, vocabulary size
 * hydra        1: [h || e(parent)] input of width 2d; 0: Medusa, input h;
 *              2: full path ([HG] "2. Generalizing to Arbitrary Tree Depths"):
 *              head k reads [h || E[t_0] || ... || E[t_{k-1}]] of width
 *              (k + 1) d, t_j the token of the depth-j node on the path from
 *              the root to the expanded node (emb_proj is not used)
 * residual     1: u = h + SiLU(a); 0: u = SiLU(a)
 * h            [B, d]
 * root_tok     [B] int32, token of the root of each tree
 * emb          [V, d] embedding table (Hydra); ignored (may be NULL) for Medusa
 * emb_proj     NULL, or (Hydra, bf16) a host array of n_heads device pointers
 *              to float32 [V, d] tables from hydra_fold_embedding: table k-1
 *              holds W1_k[:, d:] E^T, the embedding half of head k's layer for
 *              every token. With them the embedding half is a row lookup
 *              instead of a pass over W1_k[:, d:] (the same sum, as the layer
 *              is linear in e), used when B <= 16; otherwise
 *              the tables are ignored.
 * n_heads      entries in W1/b1/W2 (>= Dmax)
 * W1, b1, W2   host arrays of n_heads device pointers: W1_k [d, in] (in = 2d
 *              Hydra, d Medusa, (k + 1) d full path), b1_k [d], W2_k [V, d];
 *              head k at index k-1
 * N, Dmax      plan nodes, plan depth
 * node_parent, node_rank, node_row   device int32 [N] (plan and hydra_plan_rows)
 * R, row_node  rows per sequence; device int32 [R]
 * row_first, depth_first, k_per_depth  host arrays from hydra_plan_rows
 * head_logits  out [B, R, V] float32
 * head_lse     out [B, R] float32
 * head_hidden  out [B, R, d] (dtype) or NULL
 * cand_tok     out [B, N] int32 (cand_tok[b, 0] = root_tok[b])
 * cand_logp    out [B, N] float32 (cand_logp[b, 0] = 0)
 * Supported: bf16 needs d % 256 == 0; k_per_depth[i] <= HYDRA_MAX_TOPK <= V.
 * ---------------------------------------------------------------------- */
size_t hydra_draft_heads_workspace_size(int dtype, int B, int d, int V, int hydra,
                                        int Dmax, const int32_t* row_first);

int hydra_draft_heads(int dtype, int B, int d, int V, int hydra, int residual,
                      const void* h, const int32_t* root_tok, const void* emb,
                      const float* const* emb_proj, int n_heads, const void* const* W1, const void* const* b1,
                      const void* const* W2, int N, int Dmax,
                      const int32_t* node_parent, const int32_t* node_rank,
                      const int32_t* node_row, int R, const int32_t* row_node,
                      const int32_t* row_first, const int32_t* depth_first,
                      const int32_t* k_per_depth, float* head_logits, float* head_lse,
                      void* head_hidden, int32_t* cand_tok, float* cand_logp,
                      void* ws, size_t ws_bytes, void* stream);

/* Stage 1 with the two-layer heads of [HG] "End-to-End Implementation" (its
 * HydraHeadLayer and HydraDraftEngine modules). Same tree expansion, outputs
 * and plan arguments as hydra_draft_heads (Hydra mode); only u differs:
 *   head 1:   u = LN_1(T(SiLU(Wa_1 h_b + ba_1)))
 *   head k>1: a = T(SiLU(Wa_k [h_b || E[token of row_node[r]]] + ba_k))
 *             u = LN_k(Wb_k a + bb_k)
 *   LN_k(x) = (x - mean) / sqrt(var + ln_eps) * ln_g_k + ln_b_k over the d
 *   values of a row (biased variance). T() rounds to dtype (the identity for
 *   float32); u is stored in dtype.
 * then z = W2_k u and everything after it as in hydra_draft_heads.
 *
 * hidden_dim   H, the width of a (1024 in the source)
 * Wa, ba       host arrays of n_heads device pointers: Wa_1 [d, d], ba_1 [d];
 *              Wa_k [H, 2d], ba_k [H] for k > 1
 * Wb, bb       host arrays of n_heads device pointers: Wb_k [d, H], bb_k [d]
 *              for k > 1 (entry 0 is not read and may be NULL)
 * ln_g, ln_b   host arrays of n_heads device pointers, [d] each
 * W2           host array of n_heads device pointers, W2_k [V, d]
 * ln_eps       LayerNorm epsilon (> 0; 1e-5 in the source)
 * Plan arguments as in hydra_draft_heads; head 1 must have one row (R's first
 * row, the root). Supported: d, H <= 8192, multiples of 4; bf16 needs d % 256 == 0 and
 * H % 256 == 0. Errors as in hydra_draft_heads. */
size_t hydra_draft_heads_sketch_workspace_size(int dtype, int B, int d, int V, int hidden_dim,
                                               int Dmax, const int32_t* row_first);

int hydra_draft_heads_sketch(int dtype, int B, int d, int V, int hidden_dim, const void* h,
                             const int32_t* root_tok, const void* emb, int n_heads,
                             const void* const* Wa, const void* const* ba, const void* const* Wb,
                             const void* const* bb, const void* const* ln_g, const void* const* ln_b,
                             const void* const* W2, float ln_eps, int N, int Dmax,
                             const int32_t* node_parent, const int32_t* node_rank,
                             const int32_t* node_row, int R, const int32_t* row_node,
                             const int32_t* row_first, const int32_t* depth_first,
                             const int32_t* k_per_depth, float* head_logits, float* head_lse,
                             void* head_hidden, int32_t* cand_tok, float* cand_logp,
                             void* ws, size_t ws_bytes, void* stream);

/* Stage 1 with Hydra++ self-attention fusion ([HG] "3. Hydra++: Enhanced
 * Architectures and Knowledge Distillation": one causal self-attention layer
 * over the candidate token embeddings). One layer shared by all heads, one
 * attention head, no biases: at the node a head row expands, with path
 * tokens t_0 .. t_{k-1} (root first) and x_j = emb[t_j],
 *   q = Wq x_{k-1},  K_j = Wk x_j,  V_j = Wv x_j   (j <= k - 1, float32)
 *   a = sum_j softmax_j(q . K_j / sqrt(d)) V_j     (stored in dtype)
 *   c = x_{k-1} + Wo a                             (stored in dtype)
 * and the one-layer Hydra head reads [h || c] in place of [h || e(parent)]:
 * u = h + SiLU(W1_k [h || c] + b1_k) (residual = 1), z = W2_k u; the tree
 * expansion, outputs and plan arguments are those of hydra_draft_heads
 * (Hydra mode). Each node's K/V is computed once, when its own row runs,
 * and kept in the workspace for its descendants.
 *
 * Wqkv     [3d, d] (dtype): rows of Wq, then Wk, then Wv
 * Wo       [d, d] (dtype)
 * W1, b1, W2, residual and the rest as in hydra_draft_heads (W1_k [d, 2d]).
 * Supported: d <= 8192; bf16 needs d % 256 == 0. Errors as in
 * hydra_draft_heads. */
size_t hydra_draft_heads_attn_workspace_size(int dtype, int B, int d, int V, int N, int Dmax,
                                             const int32_t* row_first);

int hydra_draft_heads_attn(int dtype, int B, int d, int V, int residual, const void* h,
                           const int32_t* root_tok, const void* emb, const void* Wqkv, const void* Wo,
                           int n_heads, const void* const* W1, const void* const* b1,
                           const void* const* W2, int N, int Dmax, const int32_t* node_parent,
                           const int32_t* node_rank, const int32_t* node_row, int R,
                           const int32_t* row_node, const int32_t* row_first, const int32_t* depth_first,
                           const int32_t* k_per_depth, float* head_logits, float* head_lse,
                           void* head_hidden, int32_t* cand_tok, float* cand_logp, void* ws,
                           size_t ws_bytes, void* stream);

/* Folded embedding table of one Hydra head, computed once per weight set:
 * out[t, n] = sum_j W1[n, d + j] * emb[t, j] for every token t, with W1 the
 * head's [d, 2d] first-layer weight ([HG] "1. Embedding Conditioning
 * Mechanics": the layer reads [h || e(x_parent)], so its e half depends on
 * the token alone). bf16 emb [V, d] and W1, float32 out [V, d] (caller-owned,
 * V * d * 4 bytes), float32 accumulation; needs d % 64 == 0. Errors:
 * HYDRA_ERR_UNSUPPORTED for float32 or other d, HYDRA_ERR_INVALID for bad
 * sizes or NULL pointers. */
int hydra_fold_embedding(int dtype, int V, int d, const void* emb, const void* W1, float* out,
                         void* stream);

/* Vocabulary projection used by the heads and the target:
 * Y[m, n] = sum_k X[m, k] * W[n, k], float32 accumulation and output.
 * X [M, K], W [N, K] (dtype), Y [M, N] float32. bf16 needs K % 256 == 0.
 * With k > 0 the same pass also leaves, in the workspace, per row and per
 * 64-column block of W, the block's largest logit (with its id) and
 * (max, sum exp); finish them with hydra_vocab_topk. k = 0: no workspace is
 * needed (ws may be NULL). 0 <= k <= HYDRA_MAX_TOPK, k <= N. */
size_t hydra_vocab_projection_workspace_size(int M, int N, int k);

int hydra_vocab_projection(int dtype, int M, int K, int N, int k, const void* X,
                           const void* W, float* Y, void* ws, size_t ws_bytes,
                           void* stream);

/* Row reductions of a projection made with k > 0, from its workspace and its
 * logits Y [M, N] (unchanged since the projection): lse[m] = log sum_n
 * exp(Y[m, n]) and the k largest logits of each row, sorted by value
 * descending, ties to the lower id ([HG] "Candidate Tree Construction": each
 * head keeps its top-b_k tokens). The top k are read from the k blocks with
 * the largest maxima, which hold them all.
 * lse [M] float32, ids [M, k] int32, vals [M, k] float32 (any may be NULL). */
int hydra_vocab_topk(int M, int N, int k, const float* Y, const void* ws, size_t ws_bytes,
                     float* lse, int32_t* ids, float* vals, void* stream);

/* ------------------------------------------------------------------------
 * Stage 2: tree build
 *
 * Turns the candidate tree into the tree that is verified. n_keep == N: the
 * candidate tree itself. n_keep < N (dense tree): keep the root and the best
 * n_keep - 1 candidates by (cand_logp descending, depth ascending, index
 * ascending) - closed under taking parents since log-probs are <= 0 - and
 * renumber the survivors breadth-first (by depth, new parent index, rank).
 * Also builds the ancestor table that replaces a dense tree mask
 * ([HG] "Tree Attention Matrix with Topology-Aware Causal Masking": node u
 * sees v iff v is an ancestor of u or v = u).
 *
 * node_parent, node_rank, node_depth, node_row  device int32 [N] plan
 * cand_tok, cand_logp   [B, N] from hydra_draft_heads
 * tok, parent, depth    out [B, n_keep] int32 (parent of the root = -1)
 * anc                   out [B, n_keep, Dmax+1] int32: node at depth j on the
 *                       path root -> u (u itself at depth(u)), -1 beyond
 * q_row                 out [B, n_keep] int32: head row that drafted the
 *                       node's children (node_row of its source), -1 if none
 * src                   out [B, n_keep] int32: index in the candidate tree
 * Limits: N <= HYDRA_MAX_TREE, n_keep <= min(N, HYDRA_MAX_VERIFY).
 * ---------------------------------------------------------------------- */
size_t tree_build_workspace_size(int B, int N, int n_keep);

int tree_build(int B, int N, int Dmax, const int32_t* node_parent,
               const int32_t* node_rank, const int32_t* node_depth,
               const int32_t* node_row, const int32_t* cand_tok,
               const float* cand_logp, int n_keep, int32_t* tok, int32_t* parent,
               int32_t* depth, int32_t* anc, int32_t* q_row, int32_t* src,
               void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Before attention: positions of the tree rows and their rotary embedding
 *
 * [SD] "Beyond draft models: Medusa": the candidates of one head stand at the
 * same future position; [HG] "Parallel Verification and Greedy Acceptance
 * Algorithm": accepting a depth-k node advances to position t + k. Tree row u
 * of sequence b stands at pos = prefix_len[b] + depth[b, u] (siblings share
 * it; the root is at prefix_len[b]), and
 *   out[b, u, h, i]       = x_i cos(a) - x_{i+D/2} sin(a)
 *   out[b, u, h, i + D/2] = x_{i+D/2} cos(a) + x_i sin(a),
 *   a = pos * theta^(-2i/D), i < D/2
 * (the half-split layout of the LLaMA family), computed in float64 and
 * rounded once to the storage type. Apply it to the tree Q and K rows (not V)
 * before tree_attention_verify; the cached prefix K rows were rotated at
 * their own positions when they were written (tree_commit copies rotated
 * rows, whose positions L + depth are the cache positions they land on).
 *
 * x, out        [B, N, H, D] (dtype); out may equal x (in place)
 * depth         [B, N] int32 from tree_build
 * prefix_len    [B] int32
 * theta         rotary base (> 1; 10000 in the LLaMA family)
 * Limits: D even. B = 0 is a no-op. No workspace.
 * ---------------------------------------------------------------------- */
int tree_rope(int dtype, int B, int N, int H, int D, const void* x, void* out,
              const int32_t* depth, const int32_t* prefix_len, float theta,
              void* stream);

/* tree_rope of the tree Q rows [B, N, Hq, D] and K rows [B, N, Hkv, D] in one
 * launch, each value exactly as tree_rope computes it (q_out may equal q and
 * k_out may equal k). Same limits and errors as tree_rope. */
int tree_rope_qk(int dtype, int B, int N, int Hq, int Hkv, int D, const void* q, void* q_out,
                 const void* k, void* k_out, const int32_t* depth, const int32_t* prefix_len, float theta,
                 void* stream);

/* ------------------------------------------------------------------------
 * Stage 3: tree-masked attention verify (one attention layer's share)
 *
 * The N tree rows are appended after each sequence's KV prefix; row u (query
 * head hq) attends to prefix positions [0, prefix_len[b]) and to the tree rows
 * in anc[b, u, :] (its ancestors and itself) ([HG] "Tree Attention Matrix with
 * Topology-Aware Causal Masking"; [MH] "Tree Attention und Akzeptanz"):
 *   s_j = scale * q_u . k_j,   o_u = sum_j softmax(s)_j v_j,
 * with query head hq reading key/value head hq / (Hq / Hkv).
 *
 * q                  [B, N, Hq, D]          (dtype)
 * k_tree, v_tree     [B, N, Hkv, D]         (dtype)
 * k_pages, v_pages   [n_pages, Hkv, page_size, D] (dtype); position p of
 *                    sequence b lives in page block_table[b, p / page_size],
 *                    slot p % page_size
 * block_table        [B, max_pages] int32 page ids
 * prefix_len         [B] int32; each sequence attends to its whole prefix,
 *                    clamped to max_pages * page_size; page ids must be
 *                    < n_pages (out-of-range ids contribute nothing)
 * max_prefix_len     the longest prefix the caller expects: it sizes the
 *                    split plan and the workspace only (each sequence cuts
 *                    its own prefix into the planned number of ranges), so a
 *                    longer prefix_len is still attended in full
 * anc                [B, N, Dmax+1] int32 from tree_build
 * depth              [B, N] int32 from tree_build
 * out                out [B, N, Hq, D] (dtype)
 * lse                out [B, N, Hq] float32 (natural log-sum-exp of the scaled
 *                    scores) or NULL
 * Limits: N <= HYDRA_MAX_VERIFY, D in {32, 64, 128}, Hq % Hkv == 0,
 * page_size in {16, 32, 64}, Dmax <= HYDRA_MAX_DEPTH.
 * ---------------------------------------------------------------------- */
size_t tree_attention_verify_workspace_size(int dtype, int B, int N, int Hq, int Hkv,
                                            int D, int max_prefix_len);

int tree_attention_verify(int dtype, int B, int N, int Hq, int Hkv, int D,
                          float scale, const void* q, const void* k_tree,
                          const void* v_tree, const void* k_pages,
                          const void* v_pages, int n_pages, int page_size,
                          const int32_t* block_table, int max_pages,
                          const int32_t* prefix_len, int max_prefix_len,
                          const int32_t* anc, const int32_t* depth, int Dmax,
                          void* out, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * The target's decoder layer over the tree rows (the verification pass)
 *
 * [SD] "Draft, then verify": the target scores every candidate in one
 * forward pass; [HG] "Tree Attention Matrix with Topology-Aware Causal
 * Masking": each row sees the prefix and its ancestors. One LLaMA pre-norm
 * layer (the pages' model family; the layer form is a reading):
 *   a = rms(x) g1;  [q | k | v] = a Wqkv^T;  q, k rotated at prefix_len + depth
 *   (as tree_rope);  o = tree-masked attention over this layer's paged prefix
 *   (as tree_attention_verify, scale 1/sqrt(D));  x1 = x + o Wo^T;
 *   b = rms(x1) g2;  [gate | up] = b Wgu^T;  x_out = x1 + (silu(gate) * up) Wd^T,
 * with rms(y) = y / sqrt(mean(y^2) + eps). a, q, k, v, o, x1, b, the gated
 * product and x_out are stored in dtype; products accumulate in float32.
 *
 * x              [B, N, d] (dtype) hidden states of the tree rows
 * ln1, ln2       [d] (dtype) norm gains
 * Wqkv           [(Hq + 2 Hkv) D, d] (dtype): Wq rows, then Wk, then Wv
 * Wo             [d, Hq D] (dtype)
 * Wgu            [2 F, d] (dtype): gate rows, then up rows
 * Wd             [d, F] (dtype)
 * k_pages ...    this layer's paged prefix, block table, lengths (as
 *                tree_attention_verify)
 * anc, depth     from tree_build
 * x_out          out [B, N, d] (dtype), must not alias x
 * k_tree, v_tree out [B, N, Hkv, D] (dtype): this layer's rotated keys and
 *                values of the tree rows (tree_commit's inputs for this layer)
 * Limits: those of tree_attention_verify; bf16 needs d, Hq D and F multiples
 * of 256. Workspace: tree_decoder_layer_workspace_size.
 * ---------------------------------------------------------------------- */
size_t tree_decoder_layer_workspace_size(int dtype, int B, int N, int d, int Hq,
                                         int Hkv, int D, int F,
                                         int max_prefix_len);

int tree_decoder_layer(int dtype, int B, int N, int d, int Hq, int Hkv, int D,
                       int F, const void* x, const void* ln1, const void* Wqkv,
                       const void* Wo, const void* ln2, const void* Wgu,
                       const void* Wd, float eps, float theta,
                       const void* k_pages, const void* v_pages, int n_pages,
                       int page_size, const int32_t* block_table, int max_pages,
                       const int32_t* prefix_len, int max_prefix_len,
                       const int32_t* anc, const int32_t* depth, int Dmax,
                       void* x_out, void* k_tree, void* v_tree, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The target's forward pass over the tree rows: every layer
 *
 * [SD] "Draft, then verify": one forward pass of the target scores every
 * candidate; [HG] "Tree Attention Matrix with Topology-Aware Causal
 * Masking": every layer's attention is tree-masked. The rows' input is the
 * embedding of their own token (the root row's is the root token); then
 * n_layers decoder layers as tree_decoder_layer, each over its own weights
 * and paged prefix; then the final norm h = rms(x) ln_f (stored in dtype).
 * h is what tree_accept takes as o (Z = W_t h) and tree_commit as hidden;
 * k_tree / v_tree are tree_commit's layer-stacked inputs.
 *
 * tok            [B, N] tree tokens (tree_build's tok); a token outside
 *                [0, V) reads a row of zeros
 * emb            [V, d] (dtype) token embeddings
 * ln1, ln2       [n_layers, d] (dtype)
 * Wqkv           [n_layers, (Hq + 2 Hkv) D, d] (dtype)
 * Wo             [n_layers, d, Hq D] (dtype)
 * Wgu            [n_layers, 2 F, d] (dtype)
 * Wd             [n_layers, d, F] (dtype)
 * ln_f           [d] (dtype) final norm gain
 * k_pages ...    [n_layers, n_pages, Hkv, page_size, D] (dtype), one block
 *                table and prefix length per sequence shared by the layers
 * h_out          out [B, N, d] (dtype)
 * k_tree, v_tree out [n_layers, B, N, Hkv, D] (dtype): every layer's rotated
 *                keys and values of the tree rows
 * Limits: those of tree_decoder_layer; emb and h_out 16-byte aligned.
 * Workspace: tree_verify_layers_workspace_size (two hidden-state buffers
 * plus one layer's). Errors as tree_decoder_layer.
 * ---------------------------------------------------------------------- */
size_t tree_verify_layers_workspace_size(int dtype, int B, int N, int d, int Hq,
                                         int Hkv, int D, int F,
                                         int max_prefix_len);

int tree_verify_layers(int dtype, int n_layers, int B, int N, int d, int Hq,
                       int Hkv, int D, int F, int V, const int32_t* tok,
                       const void* emb, const void* ln1, const void* Wqkv,
                       const void* Wo, const void* ln2, const void* Wgu,
                       const void* Wd, const void* ln_f, float eps, float theta,
                       const void* k_pages, const void* v_pages, int n_pages,
                       int page_size, const int32_t* block_table, int max_pages,
                       const int32_t* prefix_len, int max_prefix_len,
                       const int32_t* anc, const int32_t* depth, int Dmax,
                       void* h_out, void* k_tree, void* v_tree, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 4: acceptance
 *
 * Target logits Z[b, u, :] = W_t o[b, u, :] for every tree row (o flattened
 * over heads into the hidden size d), then one walk per sequence from the
 * root:
 *   mode 0, greedy ([HG] "Parallel Verification and Greedy Acceptance
 *     Algorithm"): y = arg max Z[u] (ties to the lower id); if a child of u
 *     carries y, accept it and continue there; otherwise stop and emit y as
 *     the bonus token.
 *   mode 1, rejection ([SD] "The acceptance criterion", "The correctness
 *     guarantee"): p = softmax(Z[u] / T), q = softmax(head_logits[q_row[u]] / T);
 *     children are tried in rank order, child c is accepted iff
 *     u_acc[c] * q(tok_c) < r(tok_c) where r starts at p and becomes
 *     norm(max(r - q, 0)) after each rejection; when u has no children or
 *     every child is rejected, one token is drawn from r by inverse CDF with
 *     u_res[u] (smallest id whose cumulative mass exceeds u_res * total). If
 *     a residual has no mass the previous r is kept.
 *   mode 2, typical ([MH] "Tree Attention und Akzeptanz": a candidate is
 *     kept when its target probability exceeds a threshold tied to the
 *     entropy; the longest accepted branch is kept; not distribution-exact):
 *     at parent u, p = softmax(Z[u] / T) and child c passes iff
 *     p(tok_c) > min(eps, delta * exp(-H(p))) (threshold form: a reading);
 *     the kept branch ends at the deepest node whose whole path passes (the
 *     smallest index among equally deep ones), and one token is drawn from
 *     p at its end by inverse CDF with u_res[end] (as in mode 1).
 * Outputs: n_accepted[b] = m accepted drafts; path[b, 0..m] tree rows from
 * the root, -1 after; out_tok[b, 0..m] the m accepted tokens then the bonus
 * or resampled token, -1 after.
 *
 * o                 [B, N, d] (dtype), d = Hq * D of the attention layer
 * W_t               [V, d] (dtype)
 * tok, parent       [B, N] int32 from tree_build (children sorted by rank)
 * q_row             [B, N] int32 from tree_build (mode 1)
 * head_logits       [B, R, V] float32 from hydra_draft_heads (mode 1)
 * u_acc, u_res      [B, N] float32 in [0, 1) (mode 1; mode 2 reads u_res)
 * temperature       T > 0 (modes 1 and 2)
 * eps, delta        typical-acceptance threshold parameters, >= 0 (mode 2)
 * target_logits     out [B, N, V] float32
 * n_accepted        out [B] int32
 * path, out_tok     out [B, Dmax+1] int32
 * ---------------------------------------------------------------------- */
size_t tree_accept_workspace_size(int mode, int B, int N, int V);

int tree_accept(int dtype, int mode, int B, int N, int d, int V, int Dmax,
                const void* o, const void* W_t, float temperature, float eps,
                float delta, const int32_t* tok, const int32_t* parent,
                const int32_t* q_row, const float* head_logits, int R,
                const float* u_acc,
                const float* u_res, float* target_logits, int32_t* n_accepted,
                int32_t* path, int32_t* out_tok, void* ws, size_t ws_bytes,
                void* stream);

/* tree_accept without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, outputs and kernels as tree_accept; the
 * scratch comes from a 32 MiB array the library holds on each GPU it runs on
 * (until the process ends) instead of ws. Calls whose
 * tree_accept_workspace_size(mode, B, N, V) exceeds 32 MiB return
 * HYDRA_ERR_WORKSPACE before anything is enqueued. The first call with a
 * device current looks up that device's array address (hipGetSymbolAddress);
 * make it outside graph capture. All calls on one GPU share its array: calls
 * that overlap in time on the same GPU (concurrent streams) race. Allocates
 * nothing. */
int tree_accept_noalloc(int dtype, int mode, int B, int N, int d, int V, int Dmax,
                        const void* o, const void* W_t, float temperature,
                        float eps, float delta, const int32_t* tok,
                        const int32_t* parent, const int32_t* q_row,
                        const float* head_logits, int R, const float* u_acc,
                        const float* u_res, float* target_logits,
                        int32_t* n_accepted, int32_t* path, int32_t* out_tok,
                        void* stream);

/* ------------------------------------------------------------------------
 * After acceptance: commit of the kept branch into the paged KV cache
 *
 * [HG] "Production Engineering and Training Best Practices" (tree KV-cache
 * items): tree K/V live in statically reserved blocks and rejected nodes are
 * rolled back without freeing memory; [SD] "The acceptance criterion": the
 * next round starts from the last accepted or resampled token; [MH] "Tree
 * Attention und Akzeptanz": the kept branch's last hidden state feeds the
 * heads next round. Per sequence b with L = prefix_len[b], m = n_accepted[b]:
 *   for j = 0..m: cache position L + j of every layer <- K/V of tree row
 *                 path[b, j] (the root, then the accepted drafts);
 *   next_prefix_len[b] = L + m + 1;  next_root_tok[b] = out_tok[b, m]
 *   (the bonus or resampled token, which is not cached);
 *   next_h[b] = hidden[b, path[b, m]] (when hidden is given).
 * Rejected rows are never written, and nothing is freed or cleared.
 *
 * k_tree, v_tree     [n_layers, B, N, Hkv, D] (dtype), tree rows of the
 *                    verify pass (tree_attention_verify's k_tree/v_tree
 *                    stacked over layers)
 * k_pages, v_pages   in/out [n_layers, n_pages, Hkv, page_size, D] (dtype);
 *                    one block_table for every layer (tree_attention_verify
 *                    layout per layer)
 * block_table        [B, max_pages] int32; the caller maps pages for
 *                    positions up to L + Dmax (a position whose page index is
 *                    >= max_pages or whose page id is outside [0, n_pages) is
 *                    skipped, never written out of bounds)
 * prefix_len         [B] int32
 * n_accepted, path, out_tok  [B], [B, Dmax+1], [B, Dmax+1] int32 from
 *                    tree_accept; a sequence with m outside [0, Dmax] or a
 *                    path row outside [0, N) commits nothing: its next length
 *                    is L, its next root -1 and its next_h row is untouched
 * hidden             [B, N, d] (dtype) per-row hidden state (the attention
 *                    output o of tree_accept) or NULL; then next_h is NULL
 * next_prefix_len    out [B] int32 (must not alias prefix_len)
 * next_root_tok      out [B] int32
 * next_h             out [B, d] (dtype) or NULL
 * Buffers of K/V and hidden states are 16-byte aligned; D % 8 == 0 and, with
 * hidden, d % 8 == 0. No workspace. B = 0 is a no-op.
 * ---------------------------------------------------------------------- */
int tree_commit(int dtype, int n_layers, int B, int N, int Hkv, int D, int Dmax,
                const void* k_tree, const void* v_tree, void* k_pages,
                void* v_pages, int n_pages, int page_size,
                const int32_t* block_table, int max_pages,
                const int32_t* prefix_len, const int32_t* n_accepted,
                const int32_t* path, const int32_t* out_tok, int d,
                const void* hidden, int32_t* next_prefix_len,
                int32_t* next_root_tok, void* next_h, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HYDRA_H */
