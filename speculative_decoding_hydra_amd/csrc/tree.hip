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
  __shared__ int s_wave[kBuildThreads / 64];
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
    // rank of candidate i among 1..N-1 by (log-prob desc, depth asc, index
    // asc): kRankSplit adjacent threads count the candidates ahead of it,
    // each over every kRankSplit-th entry of the list
    constexpr int kRankSplit = 4;
    static_assert(64 % kRankSplit == 0, "a candidate's threads share a wave");
    for (int base = 0; base < N; base += kBuildThreads / kRankSplit) {
      const int i = base + tid / kRankSplit, part = tid % kRankSplit;
      int ahead = 0;
      if (i < N && i > 0) {
        const float li = s_lp[i];
        const int di = s_dep[i];
        for (int j = 1 + part; j < N; j += kRankSplit) {
          const float lj = s_lp[j];
          const int dj = s_dep[j];
          ahead += (lj > li) || (lj == li && (dj < di || (dj == di && j < i)));
        }
      }
      // the kRankSplit partial counts of a candidate sit in adjacent lanes
#pragma unroll
      for (int o = 1; o < kRankSplit; o <<= 1) ahead += __shfl_xor(ahead, o);
      if (i < N && part == 0) s_new[i] = i == 0 || ahead < n_keep - 1;
    }
    __syncthreads();
    // stable compaction: new index = number of kept candidates before i
    // (wave ballot, per-wave counts, then their prefix)
    const int lane = tid & 63, wave = tid >> 6;
    int total = 0;
    for (int base = 0; base < N; base += kBuildThreads) {
      const int i = base + tid;
      const bool keep = i < N && s_new[i] != 0;
      const uint64_t ballot = __ballot(keep);
      if (lane == 0) s_wave[wave] = __popcll(ballot);
      __syncthreads();
      int before = total;
      for (int w = 0; w < wave; ++w) before += s_wave[w];
      for (int w = 0; w < kBuildThreads / 64; ++w) total += s_wave[w];
      before += __popcll(ballot & ((uint64_t(1) << lane) - 1));
      __syncthreads();
      if (i < N) s_new[i] = keep ? before : -1;
    }
  }
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
