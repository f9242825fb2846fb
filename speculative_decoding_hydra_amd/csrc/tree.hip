// Stage 2: the tree that is verified, and its ancestor table.
//
// "Hydra Guide: Sequentially-Dependent Speculative AI", section "Tree
// Attention Matrix with Topology-Aware Causal Masking": node u may attend to
// node v iff v is an ancestor of u or v = u. Instead of a dense N x N mask the
// verify pass reads anc[u][j], the node at depth j on the path root -> u.
//
// Dense trees ("Medusa Heads", section "Tree Attention und Akzeptanz": 64-node
// sparse vs 256-node dense trees) are pruned to n_keep rows: the root plus the
// best n_keep - 1 candidates by (cumulative log-prob descending, depth
// ascending, index ascending). Log-probs are <= 0, so a child never outranks
// its parent and the kept set is closed under parents. Survivors keep their
// relative breadth-first order, which is the order by (depth, new parent
// index, rank), so renumbering is a stable compaction.
#include "common.h"

namespace hydra {
namespace {

constexpr int kBuildThreads = 1024;

__global__ __launch_bounds__(kBuildThreads) void tree_build_kernel(
    int N, int Dmax, const int32_t* __restrict__ node_parent, const int32_t* __restrict__ node_rank,
    const int32_t* __restrict__ node_depth, const int32_t* __restrict__ node_row,
    const int32_t* __restrict__ cand_tok, const float* __restrict__ cand_logp, int n_keep,
    int32_t* __restrict__ tok, int32_t* __restrict__ parent, int32_t* __restrict__ depth,
    int32_t* __restrict__ anc, int32_t* __restrict__ q_row, int32_t* __restrict__ src) {
  __shared__ float s_lp[HYDRA_MAX_TREE];
  __shared__ int s_dep[HYDRA_MAX_TREE];
  __shared__ int s_new[HYDRA_MAX_TREE];
  __shared__ int s_src[HYDRA_MAX_VERIFY];
  __shared__ int s_par[HYDRA_MAX_VERIFY];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* ct = cand_tok + static_cast<size_t>(b) * N;
  const float* cl = cand_logp + static_cast<size_t>(b) * N;

  for (int i = tid; i < N; i += kBuildThreads) {
    s_lp[i] = cl[i];
    s_dep[i] = node_depth[i];
  }
  __syncthreads();
  if (n_keep >= N) {
    for (int i = tid; i < N; i += kBuildThreads) s_new[i] = i;
  } else {
    for (int i = tid; i < N; i += kBuildThreads) {
      int keep = 1;
      if (i > 0) {
        const float li = s_lp[i];
        const int di = s_dep[i];
        int ahead = 0;
        for (int j = 1; j < N; ++j) {
          const float lj = s_lp[j];
          const int dj = s_dep[j];
          ahead += (lj > li) || (lj == li && (dj < di || (dj == di && j < i)));
        }
        keep = ahead < n_keep - 1;
      }
      s_new[i] = keep;
    }
    __syncthreads();
    if (tid == 0) {
      int c = 0;
      for (int i = 0; i < N; ++i) s_new[i] = s_new[i] ? c++ : -1;
    }
  }
  __syncthreads();
  const int nk = n_keep < N ? n_keep : N;
  for (int i = tid; i < N; i += kBuildThreads) {
    const int ni = s_new[i];
    if (ni >= 0 && ni < nk) s_src[ni] = i;
  }
  __syncthreads();
  for (int u = tid; u < nk; u += kBuildThreads) {
    const int i = s_src[u];
    const int p = node_parent[i];
    const int pn = p >= 0 ? s_new[p] : -1;
    const size_t o = static_cast<size_t>(b) * nk + u;
    tok[o] = ct[i];
    parent[o] = pn;
    depth[o] = s_dep[i];
    q_row[o] = node_row[i];
    src[o] = i;
    s_par[u] = pn;
  }
  __syncthreads();
  for (int u = tid; u < nk; u += kBuildThreads) {
    int32_t* a = anc + (static_cast<size_t>(b) * nk + u) * (Dmax + 1);
    const int du = s_dep[s_src[u]];
    for (int j = 0; j <= Dmax; ++j) a[j] = -1;
    int v = u;
    for (int j = du < Dmax ? du : Dmax; j >= 0 && v >= 0; --j) {
      a[j] = v;
      v = s_par[v];
    }
  }
}

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" size_t tree_build_workspace_size(int B, int N, int n_keep) {
  (void)B;
  (void)N;
  (void)n_keep;
  return 0;
}

extern "C" int tree_build(int B, int N, int Dmax, const int32_t* node_parent,
                          const int32_t* node_rank, const int32_t* node_depth,
                          const int32_t* node_row, const int32_t* cand_tok,
                          const float* cand_logp, int n_keep, int32_t* tok, int32_t* parent,
                          int32_t* depth, int32_t* anc, int32_t* q_row, int32_t* src, void* ws,
                          size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  clear_error();
  HY_CHECK(B > 0, HYDRA_ERR_INVALID, "tree_build: B=%d", B);
  HY_CHECK(N >= 1 && N <= HYDRA_MAX_TREE, HYDRA_ERR_INVALID, "tree_build: N=%d out of [1, %d]", N, HYDRA_MAX_TREE);
  HY_CHECK(Dmax >= 1 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "tree_build: Dmax=%d out of [1, %d]", Dmax,
           HYDRA_MAX_DEPTH);
  HY_CHECK(n_keep >= 1 && n_keep <= N && n_keep <= HYDRA_MAX_VERIFY, HYDRA_ERR_INVALID,
           "tree_build: n_keep=%d out of [1, min(N=%d, %d)]", n_keep, N, HYDRA_MAX_VERIFY);
  HY_CHECK(node_parent && node_rank && node_depth && node_row && cand_tok && cand_logp && tok && parent &&
               depth && anc && q_row && src,
           HYDRA_ERR_INVALID, "tree_build: null pointer");
  tree_build_kernel<<<B, kBuildThreads, 0, static_cast<hipStream_t>(stream)>>>(
      N, Dmax, node_parent, node_rank, node_depth, node_row, cand_tok, cand_logp, n_keep, tok, parent, depth,
      anc, q_row, src);
  HY_LAUNCH_CHECK("tree_build");
  return HYDRA_OK;
}
