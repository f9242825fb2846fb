// Stage 1: draft heads, per-head top-k and candidate-tree fill.
//
// "Medusa Heads" (Ultralytics glossary), section "So sagen die Köpfe voraus":
// a head is one feed-forward layer with SiLU and a residual connection,
// followed by a vocabulary projection. "Hydra Guide: Sequentially-Dependent
// Speculative AI", sections "1. Embedding Conditioning Mechanics" and
// "Candidate Tree Construction": Hydra head k reads [h || e(x_parent)] and
// runs once per expanded node at depth k-1, keeping its top-b_k tokens.
//
// Per depth k (sequential: Hydra head k needs the tokens of depth k-1):
//   1. W1 over the rows: with few rows (bf16) the h half of every head's W1
//      runs once up front for all heads, and depth k streams only the
//      embedding half, adding the h half, b1, SiLU and the residual in its
//      epilogue (Medusa heads read h alone, so all their layers run in that
//      first launch); otherwise a split-K projection over the gathered rows
//      [h_b || E[token]] and a separate epilogue,
//   2. projection W2 -> head logits,
//   3. the W2 epilogue leaves per-block maxima and (max, sum exp) partials;
//      one workgroup per head row merges them into log-sum-exp and top-k and
//      fills every child that takes its token from that row.
#include "common.h"

namespace hydra {
namespace {

template <class T>
__global__ __launch_bounds__(256) void head_mlp_epilogue(int M, int d, int nsplit,
                                                         const float* __restrict__ part,
                                                         const T* __restrict__ b1,
                                                         const T* __restrict__ h, int P,
                                                         int residual, T* __restrict__ U,
                                                         T* __restrict__ hidden, RowMap map) {
  const size_t total = static_cast<size_t>(M) * d;
  for (size_t idx = blockIdx.x * 256ull + threadIdx.x; idx < total; idx += gridDim.x * 256ull) {
    const int m = static_cast<int>(idx / d);
    const int j = static_cast<int>(idx % d);
    // the (at most 16) split partials, every load issued before the first add
    float t[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < nsplit) t[s] = part[static_cast<size_t>(s) * total + idx];
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < nsplit) a += t[s];
    a += load_f(b1, j);
    const float act = a / (1.0f + expf(-a));  // SiLU(a) = a * sigmoid(a)
    const float u = residual ? load_f(h, static_cast<size_t>(m / P) * d + j) + act : act;
    store_f(U, idx, u);
    if (hidden) store_f(hidden, static_cast<size_t>(map(m)) * d + j, u);
  }
}

// Full-path input of the depth-k rows ([HG] "2. Generalizing to Arbitrary
// Tree Depths"): x = [h_b || E[t_0] || ... || E[t_{k-1}]], t_j the token of
// the depth-j node on the path from the root to the expanded node, copied
// into a contiguous [M, (k + 1) d] buffer for the split-K projection. One
// workgroup per (segment, row): segment j > 0 climbs k - j parent links from
// the expanded node (depth k - 1) to its depth-(j - 1) ancestor and copies
// that token's embedding row, 16 bytes per lane when rows allow it.
template <class T>
__global__ __launch_bounds__(256) void gather_path(int d, int k, int P, int r0, int N, int V, const T* __restrict__ h,
                                                   const T* __restrict__ emb, const int32_t* __restrict__ row_node,
                                                   const int32_t* __restrict__ parent,
                                                   const int32_t* __restrict__ root_tok,
                                                   const int32_t* __restrict__ tok, T* __restrict__ X) {
  const int seg = blockIdx.x, m = blockIdx.y;
  const int b = m / P;
  const T* src = h + static_cast<size_t>(b) * d;
  if (seg > 0) {
    int a = row_node[r0 + m % P];
    for (int s = 0; s < k - seg && a > 0; ++s) a = parent[a];
    int t = a <= 0 ? root_tok[b] : tok[static_cast<size_t>(b) * N + a];
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    src = emb + static_cast<size_t>(t) * d;
  }
  T* dst = X + (static_cast<size_t>(m) * (k + 1) + seg) * d;
  constexpr int kVec = 16 / sizeof(T);
  if (d % kVec == 0) {
    const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
    u32x4_t* d4 = reinterpret_cast<u32x4_t*>(dst);
    for (int i = threadIdx.x; i < d / kVec; i += 256) d4[i] = s4[i];
  } else {
    for (int i = threadIdx.x; i < d; i += 256) dst[i] = src[i];
  }
}

int w1_splits(int dtype, int in_dim, int d) {
  if (dtype == HYDRA_F32) return 1;
  // enough workgroups for 256 CUs: d / 64 row tiles times the splits
  int s = 1;
  while ((d / 64) * s < 512 && (in_dim / (s * 2)) % 256 == 0 && s < 16) s *= 2;
  return s;
}

}  // namespace
}  // namespace hydra

using namespace hydra;

namespace {
struct DraftWs {
  size_t part, u, a, keys, ms, x, total;
};
DraftWs draft_ws(int dtype, int B, int d, int V, int hydra_mode, int Dmax, const int32_t* row_first,
                 const int32_t* k_per_depth) {
  int maxP = 0;
  for (int k = 1; k <= Dmax; ++k) maxP = std::max(maxP, row_first[k] - row_first[k - 1]);
  const size_t M = static_cast<size_t>(B) * maxP;
  const size_t MU = std::max(M, static_cast<size_t>(B) * Dmax);  // Medusa keeps every head's u
  const int in_dim = hydra_mode ? 2 * d : d;
  const size_t esz = dtype == HYDRA_F32 ? 4 : 2;
  const size_t nwg = projection_nwg(V);
  DraftWs w;
  // full path (mode 2): up to 16 split-K partials and the gathered rows
  w.part = align_up((hydra_mode == 2 ? 16 : w1_splits(dtype, in_dim, d)) * M * d * sizeof(float), 256);
  w.x = hydra_mode == 2 ? align_up(M * (Dmax + 1) * d * esz, 256) : 0;
  w.u = align_up(MU * d * esz, 256);
  w.a = align_up(static_cast<size_t>(Dmax) * B * d * sizeof(float), 256);
  w.keys = align_up(M * nwg * sizeof(uint64_t), 256);
  w.ms = align_up(M * nwg * sizeof(float2), 256);
  w.total = w.part + w.u + w.a + w.keys + w.ms + w.x + 256;
  return w;
}
}  // namespace

extern "C" size_t hydra_draft_heads_workspace_size(int dtype, int B, int d, int V, int hydra_mode,
                                                   int Dmax, const int32_t* row_first) {
  if (B <= 0 || d <= 0 || V <= 0 || Dmax <= 0 || Dmax > HYDRA_MAX_DEPTH || !row_first) return 0;
  return draft_ws(dtype & ~(HYDRA_VOCAB_PACKED | HYDRA_W1H_PACKED), B, d, V, hydra_mode, Dmax, row_first,
                  nullptr).total;
}

extern "C" int hydra_draft_heads(int dtype, int B, int d, int V, int hydra_mode, int residual,
                                 const void* h, const int32_t* root_tok, const void* emb,
                                 const float* const* emb_proj, int n_heads, const void* const* W1, const void* const* b1,
                                 const void* const* W2, int N, int Dmax,
                                 const int32_t* node_parent, const int32_t* node_rank,
                                 const int32_t* node_row, int R, const int32_t* row_node,
                                 const int32_t* row_first, const int32_t* depth_first,
                                 const int32_t* k_per_depth, float* head_logits,
                                 float* head_lse, void* head_hidden, int32_t* cand_tok,
                                 float* cand_logp, void* ws, size_t ws_bytes, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int vpack = dtype & HYDRA_VOCAB_PACKED;  // packed vocabulary weights (hydra_pack_weight)
  const int w1hp = (dtype & HYDRA_W1H_PACKED) != 0;  // packed h halves of W1 (folded calls)
  dtype &= ~(HYDRA_VOCAB_PACKED | HYDRA_W1H_PACKED);
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "draft_heads: bad dtype %d", dtype);
  HY_CHECK(!vpack || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "draft_heads: packed vocabulary weights are bf16");
  HY_CHECK(B > 0 && d > 0 && V > 0, HYDRA_ERR_INVALID, "draft_heads: bad sizes B=%d d=%d V=%d", B, d, V);
  HY_CHECK(Dmax >= 1 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "draft_heads: Dmax=%d out of [1, %d]", Dmax, HYDRA_MAX_DEPTH);
  HY_CHECK(hydra_mode >= 0 && hydra_mode <= 2, HYDRA_ERR_INVALID, "draft_heads: hydra mode %d", hydra_mode);
  HY_CHECK(n_heads >= Dmax, HYDRA_ERR_INVALID, "draft_heads: n_heads=%d < Dmax=%d", n_heads, Dmax);
  HY_CHECK(N >= 2 && N <= HYDRA_MAX_TREE, HYDRA_ERR_INVALID, "draft_heads: N=%d out of [2, %d]", N, HYDRA_MAX_TREE);
  HY_CHECK(h && root_tok && W1 && b1 && W2 && node_parent && node_rank && node_row && row_first &&
               depth_first && k_per_depth && head_logits && head_lse && cand_tok && cand_logp,
           HYDRA_ERR_INVALID, "draft_heads: null pointer");
  HY_CHECK(!hydra_mode || (emb && row_node), HYDRA_ERR_INVALID, "draft_heads: Hydra mode needs emb and row_node");
  HY_CHECK(hydra_mode != 2 || (dtype == HYDRA_F32 || d % 256 == 0), HYDRA_ERR_UNSUPPORTED,
           "draft_heads: full-path bf16 needs d %% 256 == 0");
  HY_CHECK(dtype == HYDRA_F32 || d % 256 == 0, HYDRA_ERR_UNSUPPORTED, "draft_heads: bf16 needs d %% 256 == 0 (d=%d)", d);
  HY_CHECK(row_first[0] == 0 && row_first[Dmax] == R, HYDRA_ERR_INVALID, "draft_heads: row_first must span [0, R=%d)", R);
  HY_CHECK(depth_first[0] == 0 && depth_first[1] == 1 && depth_first[Dmax + 1] == N, HYDRA_ERR_INVALID,
           "draft_heads: depth_first must start 0, 1 and end at N=%d", N);
  for (int k = 1; k <= Dmax; ++k) {
    HY_CHECK(row_first[k] > row_first[k - 1], HYDRA_ERR_INVALID, "draft_heads: depth %d has no head rows", k);
    HY_CHECK(depth_first[k + 1] > depth_first[k], HYDRA_ERR_INVALID, "draft_heads: depth %d has no nodes", k);
    HY_CHECK(k_per_depth[k - 1] >= 1 && k_per_depth[k - 1] <= HYDRA_MAX_TOPK && k_per_depth[k - 1] <= V,
             HYDRA_ERR_UNSUPPORTED, "draft_heads: top-k %d at depth %d out of [1, %d]", k_per_depth[k - 1], k,
             HYDRA_MAX_TOPK);
    HY_CHECK(W1[k - 1] && b1[k - 1] && W2[k - 1], HYDRA_ERR_INVALID, "draft_heads: null weight of head %d", k);
    HY_CHECK(hydra_mode || row_first[k] - row_first[k - 1] == 1, HYDRA_ERR_INVALID,
             "draft_heads: Medusa mode has one row per depth");
    HY_CHECK(hydra_mode != 2 || static_cast<long long>(B) * (row_first[k] - row_first[k - 1]) <= 65535,
             HYDRA_ERR_UNSUPPORTED, "draft_heads: full path takes at most 65535 rows per depth");
  }
  const size_t need = hydra_draft_heads_workspace_size(dtype, B, d, V, hydra_mode, Dmax, row_first);
  HY_CHECK(ws_bytes >= need && (need == 0 || ws), HYDRA_ERR_WORKSPACE,
           "draft_heads: workspace %zu < required %zu", ws_bytes, need);

  int maxP = 0;
  for (int k = 1; k <= Dmax; ++k) maxP = std::max(maxP, row_first[k] - row_first[k - 1]);
  const size_t Mmax = static_cast<size_t>(B) * maxP;
  const size_t MU = std::max(Mmax, static_cast<size_t>(B) * Dmax);
  const int in_dim = hydra_mode ? 2 * d : d;
  const int ns = w1_splits(dtype, in_dim, d);
  const size_t esz = dtype == HYDRA_F32 ? 4 : 2;
  const int nwg = projection_nwg(V);
  const DraftWs wl = draft_ws(dtype, B, d, V, hydra_mode, Dmax, row_first, k_per_depth);
  Arena arena(ws, ws_bytes);
  float* part = arena.take<float>(wl.part / sizeof(float));
  char* U = arena.take<char>(MU * d * esz);
  float* Ah = arena.take<float>(static_cast<size_t>(Dmax) * B * d);
  uint64_t* tkeys = arena.take<uint64_t>(Mmax * nwg);
  float2* tms = arena.take<float2>(Mmax * nwg);
  char* Xp = hydra_mode == 2 ? arena.take<char>(wl.x) : nullptr;

  // Feed-forward layers. Medusa heads read h alone: with few rows all of
  // them run in one launch up front. Hydra head k >= 2 splits into the h
  // half, which runs inside the row merge of depth k - 1 (it does not depend
  // on that merge), and the embedding half, streamed at depth k. Otherwise
  // (head 1, many rows, float32) the whole layer runs per depth.
  const bf16_t* hb = static_cast<const bf16_t*>(h);
  // Folded embedding tables (Hydra, bf16, B <= 16): the embedding half of
  // head k's layer, W1[:, d:] e(token), is row `token` of emb_proj[k - 1],
  // so no depth streams W1[:, d:]. One launch up front runs head 1 (its h
  // half plus the root token's table row) and the h half of head 2 (slot 1
  // of Ah); the row merge of depth k then writes the rows of depth k + 1
  // from the tokens it picks, while its extra workgroups stream the h half of
  // head k + 2 into slot k + 1.
  const bool folded = hydra_mode == 1 && emb_proj && dtype == HYDRA_BF16 && d % 256 == 0 &&
                      mlp_fused_supported(dtype, B, d, d) && merge_ffn_supported(B, d, d);
  HY_CHECK(!w1hp || folded, HYDRA_ERR_UNSUPPORTED,
           "draft_heads: packed W1 h halves need the folded path (bf16 Hydra heads with tables, d %% 256 == 0)");
  if (folded) {
    for (int k = 1; k <= Dmax; ++k)
      HY_CHECK(emb_proj[k - 1], HYDRA_ERR_INVALID, "draft_heads: null folded embedding table of head %d", k);
    MlpArgs pre{};
    pre.M = B;
    pre.K = d;
    pre.d = d;
    pre.ldw = 2 * d;
    pre.wpacked = w1hp;
    pre.heads = Dmax >= 2 ? 2 : 1;
    pre.xs.x = h;
    pre.xs.ldx = d;
    pre.xs.mode = 0;
    pre.xs.V = V;
    pre.epi[0] = 3;
    pre.W[0] = static_cast<const bf16_t*>(W1[0]);
    pre.b1[0] = static_cast<const bf16_t*>(b1[0]);
    pre.Ef[0] = emb_proj[0];
    pre.etok = root_tok;
    pre.map[0] = RowMap{1, R, 0};
    if (Dmax >= 2) {
      pre.epi[1] = 0;
      pre.W[1] = static_cast<const bf16_t*>(W1[1]);
      pre.b1[1] = static_cast<const bf16_t*>(b1[1]);
    }
    pre.A = Ah;
    pre.h = hb;
    pre.P = 1;
    pre.residual = residual;
    pre.U = reinterpret_cast<bf16_t*>(U);
    pre.hidden = static_cast<bf16_t*>(head_hidden);
    const int rc = launch_mlp_fused(pre, stream);
    if (rc != HYDRA_OK) return rc;
  }
  bool split[HYDRA_MAX_DEPTH + 2] = {};
  if (hydra_mode == 1 && !folded)
    for (int k = 2; k <= Dmax; ++k)
      split[k] = mlp_fused_supported(dtype, B * (row_first[k] - row_first[k - 1]), d, d) &&
                 merge_ffn_supported(B, d, d);
  const bool medusa_once = !hydra_mode && mlp_fused_supported(dtype, B, d, d);
  if (medusa_once) {
    MlpArgs pre{};
    pre.M = B;
    pre.K = d;
    pre.d = d;
    pre.ldw = d;
    pre.heads = Dmax;
    pre.xs.x = h;
    pre.xs.ldx = d;
    pre.xs.mode = 0;
    pre.h = hb;
    pre.P = 1;
    pre.residual = residual;
    pre.U = reinterpret_cast<bf16_t*>(U);
    pre.hidden = static_cast<bf16_t*>(head_hidden);
    for (int k = 1; k <= Dmax; ++k) {
      pre.epi[k - 1] = 1;
      pre.W[k - 1] = static_cast<const bf16_t*>(W1[k - 1]);
      pre.b1[k - 1] = static_cast<const bf16_t*>(b1[k - 1]);
      pre.map[k - 1] = RowMap{1, R, row_first[k - 1]};
    }
    const int rc = launch_mlp_fused(pre, stream);
    if (rc != HYDRA_OK) return rc;
  }

  for (int k = 1; k <= Dmax; ++k) {
    const int P = row_first[k] - row_first[k - 1];
    const int r0 = row_first[k - 1];
    const int M = B * P;
    RowMap map{P, R, r0};
    // 1. W1 over [h || e(parent)] (Hydra) or h (Medusa)
    XSource xs{};
    xs.x = h;
    xs.ldx = d;
    xs.mode = hydra_mode ? 1 : 0;
    xs.emb = emb;
    xs.tok = cand_tok;
    xs.root_tok = root_tok;
    xs.V = V;
    xs.row_node = row_node;
    xs.ntree = N;
    xs.P = P;
    xs.r0 = r0;
    xs.d = d;
    int rc;
    const char* Uk = U;  // rows of this depth's u
    MlpArgs fa{};
    fa.M = M;
    fa.d = d;
    fa.heads = 1;
    fa.xs = xs;
    fa.h = hb;
    fa.P = P;
    fa.residual = residual;
    fa.U = reinterpret_cast<bf16_t*>(U);
    fa.hidden = static_cast<bf16_t*>(head_hidden);
    fa.map[0] = map;
    if (hydra_mode == 2) {
      // full path: gather [h || E[t_0] || ... || E[t_{k-1}]], split-K W1, epilogue
      const int width = (k + 1) * d;
      if (dtype == HYDRA_F32)
        gather_path<float><<<dim3(k + 1, M), 256, 0, stream>>>(
            d, k, P, r0, N, V, static_cast<const float*>(h), static_cast<const float*>(emb), row_node, node_parent,
            root_tok, cand_tok, reinterpret_cast<float*>(Xp));
      else
        gather_path<bf16_t><<<dim3(k + 1, M), 256, 0, stream>>>(d, k, P, r0, N, V, hb, static_cast<const bf16_t*>(emb),
                                                                row_node, node_parent, root_tok, cand_tok,
                                                                reinterpret_cast<bf16_t*>(Xp));
      HY_LAUNCH_CHECK("draft_heads: path gather");
      int nsp = 1;
      rc = launch_projection_parts(dtype, M, width, d, Xp, W1[k - 1], part, wl.part / sizeof(float), &nsp, stream);
      if (rc != HYDRA_OK) return rc;
      const size_t total = static_cast<size_t>(M) * d;
      const int grid = static_cast<int>(std::min<size_t>((total + 255) / 256, 4096));
      if (dtype == HYDRA_F32)
        head_mlp_epilogue<float><<<grid, 256, 0, stream>>>(
            M, d, nsp, part, static_cast<const float*>(b1[k - 1]), static_cast<const float*>(h), P, residual,
            reinterpret_cast<float*>(U), static_cast<float*>(head_hidden), map);
      else
        head_mlp_epilogue<bf16_t><<<grid, 256, 0, stream>>>(M, d, nsp, part, static_cast<const bf16_t*>(b1[k - 1]),
                                                            hb, P, residual, reinterpret_cast<bf16_t*>(U),
                                                            static_cast<bf16_t*>(head_hidden), map);
      HY_LAUNCH_CHECK("draft_heads: mlp epilogue");
    } else if (medusa_once) {
      Uk = U + static_cast<size_t>(k - 1) * B * d * esz;  // written by the all-heads launch
    } else if (folded) {
      // rows written by the launch up front (k = 1) or the previous merge
    } else if (split[k]) {
      // embedding half; the epilogue adds the h half (with b1), SiLU and the residual
      fa.K = d;
      fa.ldw = 2 * d;
      fa.epi[0] = 2;
      fa.xs.mode = 2;
      fa.W[0] = static_cast<const bf16_t*>(W1[k - 1]) + d;
      fa.A = Ah;
      rc = launch_mlp_fused(fa, stream);
      if (rc != HYDRA_OK) return rc;
    } else if (mlp_fused_supported(dtype, M, in_dim, d)) {
      // the whole layer: few rows, the waves of a workgroup split K
      if (!hydra_mode) fa.xs.mode = 0;
      fa.K = in_dim;
      fa.ldw = in_dim;
      fa.epi[0] = 1;
      fa.W[0] = static_cast<const bf16_t*>(W1[k - 1]);
      fa.b1[0] = static_cast<const bf16_t*>(b1[k - 1]);
      rc = launch_mlp_fused(fa, stream);
      if (rc != HYDRA_OK) return rc;
    } else {
      if (!hydra_mode) xs.mode = 0;  // Medusa: every row of sequence b is h_b (P = 1)
      rc = launch_projection(dtype, M, in_dim, d, xs, W1[k - 1], dtype == HYDRA_F32 ? part : nullptr,
                             RowMap{M, 0, 0}, d, ns, dtype == HYDRA_F32 ? nullptr : part,
                             TopkPartials{nullptr, nullptr}, stream);
      if (rc != HYDRA_OK) return rc;
      // epilogue: u = h + SiLU(sum + b1)
      const size_t total = static_cast<size_t>(M) * d;
      const int grid = static_cast<int>(std::min<size_t>((total + 255) / 256, 4096));
      const int nsum = dtype == HYDRA_F32 ? 1 : ns;
      if (dtype == HYDRA_F32) {
        head_mlp_epilogue<float><<<grid, 256, 0, stream>>>(
            M, d, nsum, part, static_cast<const float*>(b1[k - 1]), static_cast<const float*>(h), P, residual,
            reinterpret_cast<float*>(U), static_cast<float*>(head_hidden), map);
      } else {
        head_mlp_epilogue<bf16_t><<<grid, 256, 0, stream>>>(
            M, d, nsum, part, static_cast<const bf16_t*>(b1[k - 1]), hb, P, residual,
            reinterpret_cast<bf16_t*>(U), static_cast<bf16_t*>(head_hidden), map);
      }
      HY_LAUNCH_CHECK("draft_heads: mlp epilogue");
    }
    // 2. W2: head logits
    XSource xu{};
    xu.x = Uk;
    xu.ldx = d;
    xu.mode = 0;
    const int kk = k_per_depth[k - 1];
    rc = launch_projection(dtype | vpack, M, d, V, xu, W2[k - 1], head_logits, map, V, 1, nullptr,
                           TopkPartials{tkeys, tms}, stream);
    if (rc != HYDRA_OK) return rc;
    // 3. log-sum-exp, top-k, tree fill
    MergeArgs ma{};
    ma.M = M;
    ma.nwg = nwg;
    ma.k = kk;
    ma.keys = tkeys;
    ma.ms = tms;
    ma.Y = head_logits;
    ma.ldy = V;
    ma.V = V;
    ma.map = map;
    ma.lse = head_lse;
    ma.amax = nullptr;
    ma.P = P;
    ma.r0 = r0;
    ma.N = N;
    ma.node_lo = depth_first[k];
    ma.node_hi = depth_first[k + 1];
    ma.node_parent = node_parent;
    ma.node_rank = node_rank;
    ma.node_row = node_row;
    ma.root_tok = root_tok;
    ma.cand_tok = cand_tok;
    ma.cand_logp = cand_logp;
    if (folded && k < Dmax) {
      ma.Enext = emb_proj[k];
      ma.Anext = Ah + static_cast<size_t>(k) * B * d;
      ma.h = hb;
      ma.U = reinterpret_cast<bf16_t*>(U);
      ma.hidden = static_cast<bf16_t*>(head_hidden);
      ma.d = d;
      ma.R = R;
      ma.rn = row_first[k];
      ma.Pn = row_first[k + 1] - row_first[k];
      ma.residual = residual;
    }
    if (folded && k + 2 <= Dmax) {
      // h half of head k + 2 in the same launch, into slot k + 1 of Ah
      MlpArgs hf{};
      hf.M = B;
      hf.K = d;
      hf.d = d;
      hf.ldw = 2 * d;
      hf.wpacked = w1hp;
      hf.heads = 1;
      hf.xs.x = h;
      hf.xs.ldx = d;
      hf.xs.mode = 0;
      hf.W[0] = static_cast<const bf16_t*>(W1[k + 1]);
      hf.b1[0] = static_cast<const bf16_t*>(b1[k + 1]);
      hf.A = Ah + static_cast<size_t>(k + 1) * B * d;
      hf.P = 1;
      rc = launch_topk_merge(ma, stream, &hf);
    } else if (!folded && k < Dmax && split[k + 1]) {
      // h half of head k + 1 in the same launch: Ah = W1[:, :d] h + b1
      MlpArgs hf{};
      hf.M = B;
      hf.K = d;
      hf.d = d;
      hf.ldw = 2 * d;
      hf.heads = 1;
      hf.xs.x = h;
      hf.xs.ldx = d;
      hf.xs.mode = 0;
      hf.W[0] = static_cast<const bf16_t*>(W1[k]);
      hf.b1[0] = static_cast<const bf16_t*>(b1[k]);
      hf.A = Ah;
      hf.P = 1;
      rc = launch_topk_merge(ma, stream, &hf);
    } else {
      rc = launch_topk_merge(ma, stream);
    }
    if (rc != HYDRA_OK) return rc;
  }
  return HYDRA_OK;
}

extern "C" int hydra_fold_embedding(int dtype, int V, int d, const void* emb, const void* W1, float* out,
                                    void* stream_) {
  clear_error();
  HY_CHECK(dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "fold_embedding: bf16 only (dtype %d)", dtype);
  HY_CHECK(V > 0 && d > 0, HYDRA_ERR_INVALID, "fold_embedding: bad sizes V=%d d=%d", V, d);
  HY_CHECK(emb && W1 && out, HYDRA_ERR_INVALID, "fold_embedding: null pointer");
  HY_CHECK(gemm_supported(d), HYDRA_ERR_UNSUPPORTED, "fold_embedding: needs d %% 64 == 0 (d=%d)", d);
  // out[t][n] = sum_j W1[n][d + j] * emb[t][j]: the embedding half of the
  // Hydra layer for every token, one tiled product
  return launch_projection_gemm(V, d, d, static_cast<const bf16_t*>(emb), d, static_cast<const bf16_t*>(W1) + d,
                                2 * d, out, RowMap{V, 0, 0}, d, TopkPartials{nullptr, nullptr},
                                static_cast<hipStream_t>(stream_));
}
