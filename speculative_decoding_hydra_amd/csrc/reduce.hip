// Vocabulary-wide row reductions of the draft heads and the target:
// log-sum-exp, sorted top-k ("Hydra Guide: Sequentially-Dependent Speculative
// AI", section "Candidate Tree Construction": head k keeps its top-b_k
// tokens) and arg max (section "Parallel Verification and Greedy Acceptance
// Algorithm"). Ties go to the lower token id.
//
// The projection epilogue leaves, for every row and every 64-column
// workgroup, that workgroup's sorted top-k and (max, sum exp(z - max)); the
// global top-k of a row is the top-k of the union of those lists. One
// workgroup per row merges them, then fills the candidate tree: every child
// that takes its token from this row gets entry rank of the list and the
// cumulative log-probability of its parent plus z[token] - lse.
#include "common.h"

namespace hydra {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;

// k-way merge of the per-workgroup lists (each sorted, k entries): thread t
// owns lists t, t + 256, ... (at most L) and holds them whole in registers;
// k rounds of a block-wide max over the list heads, the owner of the winning
// head pops it. No loads happen during the rounds.
template <int KL, int L>
__global__ __launch_bounds__(kMergeThreads) void topk_kway_kernel(MergeArgs a) {
  __shared__ uint64_t s_best[2][kMergeWaves];
  __shared__ float wm[kMergeWaves], wsum[kMergeWaves];
  __shared__ uint64_t top[KL];
  __shared__ float s_lse;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k;
  const uint64_t* keys = a.keys + static_cast<size_t>(i) * a.nwg * k;
  const float2* ms = a.ms + static_cast<size_t>(i) * a.nwg;

  uint64_t lst[L][KL];
  float2 p[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int w = tid + j * kMergeThreads;
    const int wc = w < a.nwg ? w : 0;
    p[j] = ms[wc];
#pragma unroll
    for (int e = 0; e < KL; ++e) lst[j][e] = keys[static_cast<size_t>(wc) * k + (e < k ? e : 0)];
    if (w >= a.nwg) p[j].x = -INFINITY;
#pragma unroll
    for (int e = 0; e < KL; ++e)
      if (w >= a.nwg || e >= k) lst[j][e] = 0;
  }
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int j = 0; j < L; ++j) {
    if (p[j].x == -INFINITY) continue;
    const float nm = fmaxf(m, p[j].x);
    s = (m == -INFINITY ? 0.f : s * expf(m - nm)) + p[j].y * expf(p[j].x - nm);
    m = nm;
  }
  wave_ms(m, s);
  if (lane == 0) {
    wm[wave] = m;
    wsum[wave] = s;
  }
  for (int r = 0; r < k; ++r) {
    uint64_t best = lst[0][0];
#pragma unroll
    for (int j = 1; j < L; ++j) best = lst[j][0] > best ? lst[j][0] : best;
    best = wave_max_u64(best);
    if (lane == 0) s_best[r & 1][wave] = best;
    __syncthreads();
    uint64_t g = s_best[r & 1][0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) g = s_best[r & 1][w] > g ? s_best[r & 1][w] : g;
    if (tid == 0) top[r] = g;
    // keys are unique, so exactly one list head equals the winner
#pragma unroll
    for (int j = 0; j < L; ++j) {
      if (g != 0 && lst[j][0] == g) {
#pragma unroll
        for (int e = 0; e < KL - 1; ++e) lst[j][e] = lst[j][e + 1];
        lst[j][KL - 1] = 0;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, wm[w]);
    float S = 0.f;
    for (int w = 0; w < kMergeWaves; ++w)
      if (wm[w] != -INFINITY) S += wsum[w] * expf(wm[w] - M);
    s_lse = M + logf(S);
    if (a.lse) a.lse[a.map(i)] = s_lse;
    if (a.amax) a.amax[i] = key_id(top[0]);
  }
  if (tid < k) {
    if (a.topk_ids) a.topk_ids[static_cast<size_t>(i) * k + tid] = key_id(top[tid]);
    if (a.topk_vals) a.topk_vals[static_cast<size_t>(i) * k + tid] = key_value(top[tid]);
  }
  __syncthreads();
  if (a.node_hi <= a.node_lo) return;
  const float lse = s_lse;
  const int b = i / a.P;
  const int r = a.r0 + i % a.P;
  const size_t base = static_cast<size_t>(b) * a.N;
  if (r == 0 && tid == 0) {
    a.cand_tok[base] = a.root_tok[b];
    a.cand_logp[base] = 0.f;
  }
  for (int c = a.node_lo + tid; c < a.node_hi; c += kMergeThreads) {
    const int pp = a.node_parent[c];
    if (pp < 0 || a.node_row[pp] != r) continue;
    const int rk = a.node_rank[c];
    if (rk < 0 || rk >= k) continue;
    const uint64_t key = top[rk];
    const float plogp = pp == 0 ? 0.f : a.cand_logp[base + pp];
    a.cand_tok[base + c] = key_id(key);
    a.cand_logp[base + c] = plogp + (key_value(key) - lse);
  }
}

template <int KL>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(MergeArgs a) {
  constexpr int BATCH = 8;  // keys in flight per thread
  __shared__ uint64_t wtop[kMergeWaves][KL];
  __shared__ float wm[kMergeWaves], wsum[kMergeWaves];
  __shared__ uint64_t top[KL];
  __shared__ float s_lse;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k;
  const uint64_t* keys = a.keys + static_cast<size_t>(i) * a.nwg * k;
  const float2* ms = a.ms + static_cast<size_t>(i) * a.nwg;

  float m = -INFINITY, s = 0.f;
  for (int w0 = 0; w0 < a.nwg; w0 += kMergeThreads * BATCH) {
    float2 p[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int w = w0 + j * kMergeThreads + tid;
      p[j] = ms[w < a.nwg ? w : 0];
      if (w >= a.nwg) p[j].x = -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (p[j].x == -INFINITY) continue;
      const float nm = fmaxf(m, p[j].x);
      s = (m == -INFINITY ? 0.f : s * expf(m - nm)) + p[j].y * expf(p[j].x - nm);
      m = nm;
    }
  }
  uint64_t l[KL];
#pragma unroll
  for (int j = 0; j < KL; ++j) l[j] = 0;
  const int total = a.nwg * k;
  for (int e0 = 0; e0 < total; e0 += kMergeThreads * BATCH) {
    uint64_t c[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int e = e0 + j * kMergeThreads + tid;
      c[j] = keys[e < total ? e : 0];
      if (e >= total) c[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) list_insert<KL>(l, c[j]);
  }

  wave_ms(m, s);
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_u64(l[0]);
    if (l[0] == best && best != 0) list_pop<KL>(l);
    if (lane == 0) wtop[wave][j] = best;
  }
  if (lane == 0) {
    wm[wave] = m;
    wsum[wave] = s;
  }
  __syncthreads();
  if (wave == 0) {
    int ptr = 0;
    for (int j = 0; j < k; ++j) {
      const uint64_t cand = (lane < kMergeWaves && ptr < k) ? wtop[lane][ptr] : 0;
      const uint64_t best = wave_max_u64(cand);
      if (lane < kMergeWaves && cand == best && best != 0) ++ptr;
      if (lane == 0) top[j] = best;
    }
    if (lane == 0) {
      float M = -INFINITY;
      for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, wm[w]);
      float S = 0.f;
      for (int w = 0; w < kMergeWaves; ++w)
        if (wm[w] != -INFINITY) S += wsum[w] * expf(wm[w] - M);
      s_lse = M + logf(S);
      if (a.lse) a.lse[a.map(i)] = s_lse;
      if (a.amax) a.amax[i] = key_id(top[0]);
    }
    if (lane < k) {
      if (a.topk_ids) a.topk_ids[static_cast<size_t>(i) * k + lane] = key_id(top[lane]);
      if (a.topk_vals) a.topk_vals[static_cast<size_t>(i) * k + lane] = key_value(top[lane]);
    }
  }
  __syncthreads();
  if (a.node_hi <= a.node_lo) return;
  const float lse = s_lse;
  const int b = i / a.P;
  const int r = a.r0 + i % a.P;
  const size_t base = static_cast<size_t>(b) * a.N;
  if (r == 0 && tid == 0) {
    a.cand_tok[base] = a.root_tok[b];
    a.cand_logp[base] = 0.f;
  }
  for (int c = a.node_lo + tid; c < a.node_hi; c += kMergeThreads) {
    const int p = a.node_parent[c];
    if (p < 0 || a.node_row[p] != r) continue;
    const int rk = a.node_rank[c];
    if (rk < 0 || rk >= k) continue;
    const uint64_t key = top[rk];
    const float plogp = p == 0 ? 0.f : a.cand_logp[base + p];
    a.cand_tok[base + c] = key_id(key);
    a.cand_logp[base + c] = plogp + (key_value(key) - lse);
  }
}

}  // namespace

int launch_topk_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.M <= 0) return HYDRA_OK;
  if (a.k < 1 || a.k > HYDRA_MAX_TOPK) {
    set_error("top-k merge: k=%d out of [1, %d]", a.k, HYDRA_MAX_TOPK);
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (a.nwg <= 2 * kMergeThreads) {
    if (a.k == 1) topk_kway_kernel<1, 2><<<a.M, kMergeThreads, 0, stream>>>(a);
    else if (a.k <= 4) topk_kway_kernel<4, 2><<<a.M, kMergeThreads, 0, stream>>>(a);
    else topk_kway_kernel<HYDRA_MAX_TOPK, 2><<<a.M, kMergeThreads, 0, stream>>>(a);
  } else if (a.k == 1) {
    topk_merge_kernel<1><<<a.M, kMergeThreads, 0, stream>>>(a);
  } else if (a.k <= 4) {
    topk_merge_kernel<4><<<a.M, kMergeThreads, 0, stream>>>(a);
  } else {
    topk_merge_kernel<HYDRA_MAX_TOPK><<<a.M, kMergeThreads, 0, stream>>>(a);
  }
  HY_LAUNCH_CHECK("top-k merge");
  return HYDRA_OK;
}

}  // namespace hydra
