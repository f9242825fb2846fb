// Stage 1 with Hydra++ self-attention fusion.
//
// "Hydra Guide: Sequentially-Dependent Speculative AI", section "3. Hydra++:
// Enhanced Architectures and Knowledge Distillation": the draft heads gain one
// light causal self-attention layer over the candidate token embeddings.
// Here (the pages give no more) one layer is shared by all heads: at an
// expanded node with path tokens t_0 .. t_{k-1} and x_j = e(t_j), the query
// is Wq x_{k-1}, the keys and values Wk x_j and Wv x_j over the path (causal:
// the node and its ancestors), and c = x_{k-1} + Wo softmax(q.K / sqrt(d)) V
// takes the place of e(parent) in the one-layer Hydra head,
// u = h + SiLU(W1 [h || c] + b1).
//
// Every node that is expanded gets a head row, and every ancestor of an
// expanded node was itself expanded at an earlier depth, so each node's key
// and value are computed once, when its own row runs, and kept in a per-node
// float32 cache for its descendants. Per depth k:
//   1. gather x_{k-1} = E[token] of each row's node,
//   2. one split-K product with [Wq; Wk; Wv] ([3d, d]),
//   3. path_scores / path_values: workgroups of 256 columns of a row sum the
//      partials, store the node's K/V and leave their share of the k dot
//      products; then each takes the row's softmax over the path and writes
//      its columns of the attention output a (rounded to the storage type),
//   4. Wo a, then c = x_{k-1} + Wo a written next to h as [h || c],
//   5. W1 over [h || c] and the head epilogue, then W2 and the merge of the
//      one-layer path.
#include "common.h"

namespace hydra {
namespace {

constexpr int kMaxWidth = 8192;  // d

template <class T>
__global__ __launch_bounds__(256) void gather_rows(int d, int P, int r0, int N, int V, const T* __restrict__ emb,
                                                   const int32_t* __restrict__ row_node,
                                                   const int32_t* __restrict__ root_tok,
                                                   const int32_t* __restrict__ tok, T* __restrict__ X) {
  const int m = blockIdx.x, b = m / P;
  const int node = row_node[r0 + m % P];
  int t = node <= 0 ? root_tok[b] : tok[static_cast<size_t>(b) * N + node];
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  const T* src = emb + static_cast<size_t>(t) * d;
  T* dst = X + static_cast<size_t>(m) * d;
  constexpr int kVec = 16 / sizeof(T);
  if (d % kVec == 0) {
    for (int i = threadIdx.x; i < d / kVec; i += 256)
      reinterpret_cast<u32x4_t*>(dst)[i] = reinterpret_cast<const u32x4_t*>(src)[i];
  } else {
    for (int i = threadIdx.x; i < d; i += 256) dst[i] = src[i];
  }
}

// sum of the ns (at most 16) split partials of element i, in split order,
// every load issued before the first add
__device__ __forceinline__ float sum_parts(const float* __restrict__ p, int ns, size_t stride, size_t i) {
  float t[16];
#pragma unroll
  for (int s = 0; s < 16; ++s)
    if (s < ns) t[s] = p[s * stride + i];
  float v = t[0];
#pragma unroll
  for (int s = 1; s < 16; ++s)
    if (s < ns) v += t[s];
  return v;
}

constexpr int kChunk = 256;  // columns per workgroup of the path attention

// The path attention in two launches over (column chunk, row) workgroups, so
// that a row's 3d partial sums and k cached keys and values are read by d/256
// CUs instead of one.
// Scores: sums the [Wq; Wk; Wv] partials ([ns][M][3d]) of this chunk, stores
// the node's K and V in the [B, N, d] float32 caches, and leaves this
// chunk's share of q . K_j for every path position in S[m][chunk][j]; the
// chunk-0 workgroup also leaves the path (root first) in path[m][j].
__global__ __launch_bounds__(kChunk) void path_scores(int d, int k, int P, int r0, int N, int ns, size_t stride,
                                                      const float* __restrict__ qkv,
                                                      const int32_t* __restrict__ row_node,
                                                      const int32_t* __restrict__ parent, float* __restrict__ Kc,
                                                      float* __restrict__ Vc, float* __restrict__ S,
                                                      int32_t* __restrict__ path) {
  __shared__ int anc[HYDRA_MAX_DEPTH + 1];
  __shared__ float red[kChunk / 64][HYDRA_MAX_DEPTH + 1];
  const int chunk = blockIdx.x, m = blockIdx.y, b = m / P;
  const int nchunk = gridDim.x;
  const int node = row_node[r0 + m % P];
  if (threadIdx.x == 0) {
    int a = node;
    for (int j = k - 1; j >= 0; --j) {
      anc[j] = a;
      a = a > 0 ? parent[a] : 0;
    }
  }
  const int c = chunk * kChunk + threadIdx.x;
  const bool on = c < d;
  const size_t row = static_cast<size_t>(m) * 3 * d;
  float q = 0.f, kv = 0.f;
  if (on) {
    q = sum_parts(qkv, ns, stride, row + c);
    kv = sum_parts(qkv, ns, stride, row + d + c);
    const float vv = sum_parts(qkv, ns, stride, row + 2 * d + c);
    const size_t nb = (static_cast<size_t>(b) * N + node) * d;
    Kc[nb + c] = kv;
    Vc[nb + c] = vv;
  }
  __syncthreads();
  if (chunk == 0 && threadIdx.x < k) path[m * (HYDRA_MAX_DEPTH + 1) + threadIdx.x] = anc[threadIdx.x];
#pragma unroll
  for (int j = 0; j <= HYDRA_MAX_DEPTH; ++j) {
    if (j < k) {  // uniform over the workgroup
      float t = 0.f;
      if (on) t = q * (j == k - 1 ? kv : Kc[(static_cast<size_t>(b) * N + anc[j]) * d + c]);
      t = wave_sum(t);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][j] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x < k) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kChunk / 64; ++w) t += red[w][threadIdx.x];
    S[(static_cast<size_t>(m) * nchunk + chunk) * (HYDRA_MAX_DEPTH + 1) + threadIdx.x] = t;
  }
}

// Values: the scores of the row (chunk shares summed in a fixed order, in
// float64), softmax over the path, and a = sum_j p_j V_j for this chunk.
template <class T>
__global__ __launch_bounds__(kChunk) void path_values(int d, int k, int N, int P, const float* __restrict__ S,
                                                      const int32_t* __restrict__ path,
                                                      const float* __restrict__ Vc, T* __restrict__ A) {
  __shared__ float p[HYDRA_MAX_DEPTH + 1];
  const int chunk = blockIdx.x, m = blockIdx.y, b = m / P;
  const int nchunk = gridDim.x;
  if (threadIdx.x < 64) {  // one wave: lane j < k sums position j's shares
    const int j = threadIdx.x;
    float sc = -INFINITY;
    if (j < k) {
      double t = 0.0;
      for (int ch = 0; ch < nchunk; ++ch) t += S[(static_cast<size_t>(m) * nchunk + ch) * (HYDRA_MAX_DEPTH + 1) + j];
      sc = static_cast<float>(t) / sqrtf(static_cast<float>(d));
    }
    const float mx = wave_max(sc);
    const float e = j < k ? expf(sc - mx) : 0.f;
    const float den = wave_sum(e);
    if (j < k) p[j] = e / den;
  }
  __syncthreads();
  const int c = chunk * kChunk + threadIdx.x;
  if (c >= d) return;
  const int32_t* pr = path + m * (HYDRA_MAX_DEPTH + 1);
  float a = 0.f;
#pragma unroll
  for (int j = 0; j <= HYDRA_MAX_DEPTH; ++j)
    if (j < k) a += p[j] * Vc[(static_cast<size_t>(b) * N + pr[j]) * d + c];
  store_f(A, static_cast<size_t>(m) * d + c, a);
}

// [h_b || c] with c = T(x + sum of the Wo partials), x the gathered e row
template <class T>
__global__ __launch_bounds__(256) void fuse_rows(int M, int d, int P, int ns, const float* __restrict__ part,
                                                 const T* __restrict__ X, const T* __restrict__ h,
                                                 T* __restrict__ X2) {
  const size_t total = static_cast<size_t>(M) * d;
  for (size_t idx = blockIdx.x * 256ull + threadIdx.x; idx < total; idx += gridDim.x * 256ull) {
    const int m = static_cast<int>(idx / d), j = static_cast<int>(idx % d);
    const float c = load_f(X, idx) + sum_parts(part, ns, total, idx);
    store_f(X2, static_cast<size_t>(m) * 2 * d + j, load_f(h, static_cast<size_t>(m / P) * d + j));
    store_f(X2, static_cast<size_t>(m) * 2 * d + d + j, c);
  }
}

// u = h + SiLU(sum + b1) (or SiLU alone) -> U[m] and hidden[map(m)]
template <class T>
__global__ __launch_bounds__(256) void head_epilogue(int M, int d, int P, int ns, const float* __restrict__ part,
                                                     const T* __restrict__ b1, const T* __restrict__ h, int residual,
                                                     T* __restrict__ U, T* __restrict__ hidden, RowMap map) {
  const size_t total = static_cast<size_t>(M) * d;
  for (size_t idx = blockIdx.x * 256ull + threadIdx.x; idx < total; idx += gridDim.x * 256ull) {
    const int m = static_cast<int>(idx / d), j = static_cast<int>(idx % d);
    const float a = sum_parts(part, ns, total, idx) + load_f(b1, j);
    const float act = a / (1.0f + expf(-a));
    const float u = residual ? load_f(h, static_cast<size_t>(m / P) * d + j) + act : act;
    store_f(U, idx, u);
    if (hidden) store_f(hidden, static_cast<size_t>(map(m)) * d + j, u);
  }
}

struct AttnWs {
  size_t part, x, a, x2, u, kc, vc, sc, path, keys, ms, total;
};
AttnWs attn_ws(int dtype, int B, int d, int V, int N, int Dmax, const int32_t* row_first) {
  int maxP = 0;
  for (int k = 1; k <= Dmax; ++k) maxP = std::max(maxP, row_first[k] - row_first[k - 1]);
  const size_t M = static_cast<size_t>(B) * maxP;
  const size_t esz = dtype == HYDRA_F32 ? 4 : 2;
  const size_t nwg = projection_nwg(V);
  AttnWs w;
  w.part = align_up(16 * M * 3 * d * sizeof(float), 256);
  w.x = align_up(M * d * esz, 256);
  w.a = align_up(M * d * esz, 256);
  w.x2 = align_up(M * 2 * d * esz, 256);
  w.u = align_up(M * d * esz, 256);
  w.kc = align_up(static_cast<size_t>(B) * N * d * sizeof(float), 256);
  w.vc = w.kc;
  w.sc = align_up(M * ((d + kChunk - 1) / kChunk) * (HYDRA_MAX_DEPTH + 1) * sizeof(float), 256);
  w.path = align_up(M * (HYDRA_MAX_DEPTH + 1) * sizeof(int32_t), 256);
  w.keys = align_up(M * nwg * sizeof(uint64_t), 256);
  w.ms = align_up(M * nwg * sizeof(float2), 256);
  w.total = w.part + w.x + w.a + w.x2 + w.u + w.kc + w.vc + w.sc + w.path + w.keys + w.ms + 256;
  return w;
}

bool M_ok(int B, int Dmax, const int32_t* row_first) {
  for (int k = 1; k <= Dmax; ++k)
    if (static_cast<long long>(B) * (row_first[k] - row_first[k - 1]) > 65535) return false;
  return true;
}

int grid_for(size_t total) { return static_cast<int>(std::min<size_t>((total + 255) / 256, 4096)); }

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" size_t hydra_draft_heads_attn_workspace_size(int dtype, int B, int d, int V, int N, int Dmax,
                                                        const int32_t* row_first) {
  if (B <= 0 || d <= 0 || V <= 0 || N <= 0 || Dmax <= 0 || Dmax > HYDRA_MAX_DEPTH || !row_first) return 0;
  return attn_ws(dtype & ~HYDRA_VOCAB_PACKED, B, d, V, N, Dmax, row_first).total;
}

extern "C" int hydra_draft_heads_attn(int dtype, int B, int d, int V, int residual, const void* h,
                                      const int32_t* root_tok, const void* emb, const void* Wqkv, const void* Wo,
                                      int n_heads, const void* const* W1, const void* const* b1,
                                      const void* const* W2, int N, int Dmax, const int32_t* node_parent,
                                      const int32_t* node_rank, const int32_t* node_row, int R,
                                      const int32_t* row_node, const int32_t* row_first, const int32_t* depth_first,
                                      const int32_t* k_per_depth, float* head_logits, float* head_lse,
                                      void* head_hidden, int32_t* cand_tok, float* cand_logp, void* ws,
                                      size_t ws_bytes, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int vpack = dtype & HYDRA_VOCAB_PACKED;  // packed vocabulary weights (hydra_pack_weight)
  dtype &= ~HYDRA_VOCAB_PACKED;
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "draft_heads_attn: bad dtype %d", dtype);
  HY_CHECK(!vpack || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "draft_heads_attn: packed vocabulary weights are bf16");
  HY_CHECK(B > 0 && d > 0 && V > 0, HYDRA_ERR_INVALID, "draft_heads_attn: bad sizes B=%d d=%d V=%d", B, d, V);
  HY_CHECK(d <= kMaxWidth, HYDRA_ERR_UNSUPPORTED, "draft_heads_attn: d=%d > %d", d, kMaxWidth);
  HY_CHECK(dtype == HYDRA_F32 || d % 256 == 0, HYDRA_ERR_UNSUPPORTED, "draft_heads_attn: bf16 needs d %% 256 == 0");
  HY_CHECK(Dmax >= 1 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "draft_heads_attn: Dmax=%d out of [1, %d]", Dmax,
           HYDRA_MAX_DEPTH);
  HY_CHECK(n_heads >= Dmax, HYDRA_ERR_INVALID, "draft_heads_attn: n_heads=%d < Dmax=%d", n_heads, Dmax);
  HY_CHECK(N >= 2 && N <= HYDRA_MAX_TREE, HYDRA_ERR_INVALID, "draft_heads_attn: N=%d out of [2, %d]", N,
           HYDRA_MAX_TREE);
  HY_CHECK(h && root_tok && emb && Wqkv && Wo && W1 && b1 && W2 && node_parent && node_rank && node_row &&
               row_node && row_first && depth_first && k_per_depth && head_logits && head_lse && cand_tok &&
               cand_logp,
           HYDRA_ERR_INVALID, "draft_heads_attn: null pointer");
  HY_CHECK(row_first[0] == 0 && row_first[Dmax] == R, HYDRA_ERR_INVALID,
           "draft_heads_attn: row_first must span [0, R=%d)", R);
  HY_CHECK(depth_first[0] == 0 && depth_first[1] == 1 && depth_first[Dmax + 1] == N, HYDRA_ERR_INVALID,
           "draft_heads_attn: depth_first must start 0, 1 and end at N=%d", N);
  for (int k = 1; k <= Dmax; ++k) {
    HY_CHECK(row_first[k] > row_first[k - 1], HYDRA_ERR_INVALID, "draft_heads_attn: depth %d has no head rows", k);
    HY_CHECK(depth_first[k + 1] > depth_first[k], HYDRA_ERR_INVALID, "draft_heads_attn: depth %d has no nodes", k);
    HY_CHECK(k_per_depth[k - 1] >= 1 && k_per_depth[k - 1] <= HYDRA_MAX_TOPK && k_per_depth[k - 1] <= V,
             HYDRA_ERR_UNSUPPORTED, "draft_heads_attn: top-k %d at depth %d out of [1, %d]", k_per_depth[k - 1], k,
             HYDRA_MAX_TOPK);
    HY_CHECK(W1[k - 1] && b1[k - 1] && W2[k - 1], HYDRA_ERR_INVALID, "draft_heads_attn: null weight of head %d", k);
  }
  HY_CHECK(M_ok(B, Dmax, row_first), HYDRA_ERR_UNSUPPORTED, "draft_heads_attn: more than 65535 rows at one depth");
  const size_t need = hydra_draft_heads_attn_workspace_size(dtype, B, d, V, N, Dmax, row_first);
  HY_CHECK(ws && ws_bytes >= need, HYDRA_ERR_WORKSPACE, "draft_heads_attn: workspace %zu < required %zu", ws_bytes,
           need);

  const AttnWs wl = attn_ws(dtype, B, d, V, N, Dmax, row_first);
  Arena arena(ws, ws_bytes);
  float* part = arena.take<float>(wl.part / sizeof(float));
  char* X = arena.take<char>(wl.x);
  char* Ab = arena.take<char>(wl.a);
  char* X2 = arena.take<char>(wl.x2);
  char* U = arena.take<char>(wl.u);
  float* Kc = arena.take<float>(wl.kc / sizeof(float));
  float* Vc = arena.take<float>(wl.vc / sizeof(float));
  float* Sc = arena.take<float>(wl.sc / sizeof(float));
  int32_t* pathb = arena.take<int32_t>(wl.path / sizeof(int32_t));
  uint64_t* tkeys = arena.take<uint64_t>(wl.keys / sizeof(uint64_t));
  float2* tms = arena.take<float2>(wl.ms / sizeof(float2));
  const size_t pf = wl.part / sizeof(float);
  const bool f32 = dtype == HYDRA_F32;

  for (int k = 1; k <= Dmax; ++k) {
    const int P = row_first[k] - row_first[k - 1];
    const int r0 = row_first[k - 1];
    const int M = B * P;
    const RowMap map{P, R, r0};
    int ns = 1, rc;
    // 1-2. x_{k-1} and its query, key and value
    if (f32)
      gather_rows<float><<<M, 256, 0, stream>>>(d, P, r0, N, V, static_cast<const float*>(emb), row_node, root_tok,
                                                cand_tok, reinterpret_cast<float*>(X));
    else
      gather_rows<bf16_t><<<M, 256, 0, stream>>>(d, P, r0, N, V, static_cast<const bf16_t*>(emb), row_node, root_tok,
                                                 cand_tok, reinterpret_cast<bf16_t*>(X));
    HY_LAUNCH_CHECK("draft_heads_attn: gather");
    rc = launch_projection_parts(dtype, M, d, 3 * d, X, Wqkv, part, pf, &ns, stream);
    if (rc != HYDRA_OK) return rc;
    // 3. causal attention over the path
    const size_t stride = static_cast<size_t>(M) * 3 * d;
    const dim3 grid((d + kChunk - 1) / kChunk, M);
    path_scores<<<grid, kChunk, 0, stream>>>(d, k, P, r0, N, ns, stride, part, row_node, node_parent, Kc, Vc, Sc, pathb);
    HY_LAUNCH_CHECK("draft_heads_attn: path scores");
    if (f32)
      path_values<float><<<grid, kChunk, 0, stream>>>(d, k, N, P, Sc, pathb, Vc, reinterpret_cast<float*>(Ab));
    else
      path_values<bf16_t><<<grid, kChunk, 0, stream>>>(d, k, N, P, Sc, pathb, Vc, reinterpret_cast<bf16_t*>(Ab));
    HY_LAUNCH_CHECK("draft_heads_attn: path values");
    // 4. c = x + Wo a, next to h
    rc = launch_projection_parts(dtype, M, d, d, Ab, Wo, part, pf, &ns, stream);
    if (rc != HYDRA_OK) return rc;
    const size_t total = static_cast<size_t>(M) * d;
    if (f32)
      fuse_rows<float><<<grid_for(total), 256, 0, stream>>>(M, d, P, ns, part, reinterpret_cast<const float*>(X),
                                                            static_cast<const float*>(h), reinterpret_cast<float*>(X2));
    else
      fuse_rows<bf16_t><<<grid_for(total), 256, 0, stream>>>(M, d, P, ns, part, reinterpret_cast<const bf16_t*>(X),
                                                             static_cast<const bf16_t*>(h),
                                                             reinterpret_cast<bf16_t*>(X2));
    HY_LAUNCH_CHECK("draft_heads_attn: fuse");
    // 5. the one-layer head over [h || c]
    rc = launch_projection_parts(dtype, M, 2 * d, d, X2, W1[k - 1], part, pf, &ns, stream);
    if (rc != HYDRA_OK) return rc;
    if (f32)
      head_epilogue<float><<<grid_for(total), 256, 0, stream>>>(
          M, d, P, ns, part, static_cast<const float*>(b1[k - 1]), static_cast<const float*>(h), residual,
          reinterpret_cast<float*>(U), static_cast<float*>(head_hidden), map);
    else
      head_epilogue<bf16_t><<<grid_for(total), 256, 0, stream>>>(
          M, d, P, ns, part, static_cast<const bf16_t*>(b1[k - 1]), static_cast<const bf16_t*>(h), residual,
          reinterpret_cast<bf16_t*>(U), static_cast<bf16_t*>(head_hidden), map);
    HY_LAUNCH_CHECK("draft_heads_attn: head epilogue");
    XSource xu{};
    xu.x = U;
    xu.ldx = d;
    xu.mode = 0;
    rc = launch_projection(dtype | vpack, M, d, V, xu, W2[k - 1], head_logits, map, V, 1, nullptr, TopkPartials{tkeys, tms},
                           stream);
    if (rc != HYDRA_OK) return rc;
    MergeArgs ma{};
    ma.M = M;
    ma.nwg = projection_nwg(V);
    ma.k = k_per_depth[k - 1];
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
    rc = launch_topk_merge(ma, stream);
    if (rc != HYDRA_OK) return rc;
  }
  return HYDRA_OK;
}
