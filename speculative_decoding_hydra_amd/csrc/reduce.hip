// Vocabulary-wide row reductions of the draft heads and the target:
// log-sum-exp, sorted top-k ("Hydra Guide: Sequentially-Dependent Speculative
// AI", section "Candidate Tree Construction": head k keeps its top-b_k
// tokens) and arg max (section "Parallel Verification and Greedy Acceptance
// Algorithm"). Ties go to the lower token id.
//
// The projection epilogue leaves, for every row and every 64-column block,
// the block's largest key and (max, sum exp(z - max)). A workgroup finishes a
// row: it combines the (max, sum) pairs into the log-sum-exp, picks the k
// blocks with the largest maxima and takes the top k of their 64 k logits.
// That is exact: a key in any other block is below its block's maximum,
// which is below k distinct block maxima, so it cannot rank among the first
// k. Keys are unique (value, then id), so the order is total. Each selection
// runs as k rounds of a wave-wide max in every wave, then one wave ranks the
// waves' winners by counting. The workgroup then fills the candidate tree:
// every child that takes its token from this row gets entry rank of the list
// and the cumulative log-probability of its parent plus z[token] - lse.
#include "ffn.h"
#include "walk.h"

namespace hydra {
namespace {

constexpr int kMergeWaves = 4;
constexpr int kMergeThreads = kMergeWaves * 64;

// k rounds of a wave-wide max over the lanes' sorted lists; lane 0 writes
// the winners to out[0..k)
template <int LL>
__device__ __forceinline__ void wave_top_k(uint64_t (&l)[LL], int k, uint64_t* out, int lane) {
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_u64(l[0]);
    if (l[0] == best && best != 0) list_pop<LL>(l);
    if (lane == 0) out[j] = best;
  }
}

// wave 0: the k largest of the waves' winner lists cand[0 .. kMergeWaves * k)
// by rank counting (keys are unique, zero entries are padding). With fewer
// than k nonzero candidates the remaining entries of top are 0.
__device__ __forceinline__ void rank_top_k(const uint64_t* cand, int k, uint64_t* top, int lane) {
  const int n = kMergeWaves * k;  // <= 64
  const uint64_t mine = lane < n ? cand[lane] : 0;
  int rank = 0;
  for (int c = 0; c < n; ++c) rank += cand[c] > mine ? 1 : 0;
  if (lane < k) top[lane] = 0;  // same wave, so these stores land before the ones below
  if (lane < n && mine != 0 && rank < k) top[rank] = mine;
}

// Next-depth Hydra feed-forward rows from the folded embedding table:
// u = h[b] + SiLU(Anext[b] + Enext[token]) for the nu queued children of
// this row. Workgroup g of the row's ng takes columns [g d / ng, (g + 1) d / ng)
// in chunks of 256; in a chunk thread t covers the 4 columns 4 (t % 64) of
// children t / 64, t / 64 + 4, ... so every thread has at most KL / 4 rows,
// and all of its table loads are in flight before the first is used.
template <int KL>
__device__ __forceinline__ void next_rows(const MergeArgs& a, int b, int g, int nu, const int* urow,
                                          const int* utok) {
  constexpr int IPT = KL < 4 ? 1 : KL / 4;  // rows per thread
  if (nu == 0) return;
  const int d = a.d;
  const int cw = d / a.ng;
  const int e0 = threadIdx.x >> 6;
  int tk[IPT], m[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int e = e0 + 4 * j < nu ? e0 + 4 * j : nu - 1;  // past nu: repeat the last child, never stored
    const int t = utok[e];
    tk[j] = t < 0 ? 0 : (t >= a.V ? a.V - 1 : t);
    m[j] = urow[e];
  }
  for (int c0 = g * cw + (threadIdx.x & 63) * 4; c0 < (g + 1) * cw; c0 += 256) {
    float4 ev[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) ev[j] = *reinterpret_cast<const float4*>(a.Enext + static_cast<size_t>(tk[j]) * d + c0);
    const float4 ah = *reinterpret_cast<const float4*>(a.Anext + static_cast<size_t>(b) * d + c0);
    const u32x2_t hv = *reinterpret_cast<const u32x2_t*>(a.h + static_cast<size_t>(b) * d + c0);
    const float hf[4] = {bf16_to_f32(static_cast<bf16_t>(hv.x & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(hv.x >> 16)),
                         bf16_to_f32(static_cast<bf16_t>(hv.y & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(hv.y >> 16))};
    const float af[4] = {ah.x, ah.y, ah.z, ah.w};
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      if (e0 + 4 * j >= nu) continue;  // not break: the loop unrolls fully and ev stays in registers
      const float evf[4] = {ev[j].x, ev[j].y, ev[j].z, ev[j].w};
      bf16_t out[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = af[q] + evf[q];
        // SiLU(v) = v * sigmoid(v) with the hardware exp2 and reciprocal:
        // a few float32 ulp, far below the bf16 rounding that follows
        const float act = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
        out[q] = f32_to_bf16(a.residual ? hf[q] + act : act);
      }
      const u32x2_t packed{static_cast<uint32_t>(out[0]) | (static_cast<uint32_t>(out[1]) << 16),
                           static_cast<uint32_t>(out[2]) | (static_cast<uint32_t>(out[3]) << 16)};
      *reinterpret_cast<u32x2_t*>(a.U + static_cast<size_t>(m[j]) * d + c0) = packed;
      if (a.hidden) {
        const int hr = (m[j] / a.Pn) * a.R + a.rn + m[j] % a.Pn;
        *reinterpret_cast<u32x2_t*>(a.hidden + static_cast<size_t>(hr) * d + c0) = packed;
      }
    }
  }
}

// KL: list capacity (>= k); LL: per-thread list of block maxima (holds all of
// a thread's slots when nwg <= 256 * LL, else LL = KL keeps its top KL)
// g: which of the row's ng workgroups this is; all select the same top k,
// workgroup 0 writes the row's results and each writes its share of the
// next-depth rows.
template <int KL, int LL>
__device__ __forceinline__ void merge_row(const MergeArgs& a, int i, int g) {
  __shared__ uint64_t s_cand[kMergeWaves * KL];
  __shared__ uint64_t s_top[KL];
  __shared__ float s_m[kMergeWaves], s_s[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k;
  const uint64_t* keys = a.keys + static_cast<size_t>(i) * a.nwg;
  const bool want_lse = a.ms != nullptr;
  const float2* ms = a.ms + (want_lse ? static_cast<size_t>(i) * a.nwg : 0);

  // 1. (max, sum exp) of the row; per thread its block maxima, sorted
  float m = -INFINITY, s = 0.f;
  uint64_t l[LL];
#pragma unroll
  for (int j = 0; j < LL; ++j) l[j] = 0;
  for (int w0 = 0; w0 < a.nwg; w0 += kMergeThreads * LL) {
    uint64_t c[LL];
    float2 p[LL];
#pragma unroll
    for (int j = 0; j < LL; ++j) {
      const int w = w0 + j * kMergeThreads + tid;
      const int wc = w < a.nwg ? w : 0;
      c[j] = keys[wc];
      p[j] = want_lse ? ms[wc] : make_float2(-INFINITY, 0.f);
      if (w >= a.nwg) {
        c[j] = 0;
        p[j].x = -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < LL; ++j) {
      ms_combine(m, s, p[j].x, p[j].y);
      list_insert<LL>(l, c[j]);
    }
  }
  wave_ms(m, s);
  if (lane == 0) {
    s_m[wave] = m;
    s_s[wave] = s;
  }
  // 2. the k largest block maxima
  wave_top_k<LL>(l, k, s_cand + wave * k, lane);
  __syncthreads();
  if (wave == 0) rank_top_k(s_cand, k, s_top, lane);
  __syncthreads();

  // 3. the top k of those blocks' logits (for k = 1 the largest maximum is
  // it). The k-th largest block maximum T is a lower bound for the k-th
  // largest logit (the k maxima are k keys >= T), so only keys >= T are
  // candidates: usually little more than the maxima themselves. They are
  // collected in LDS and ranked by counting.
  if (KL > 1 && k > 1) {
    constexpr int BPW = (KL + kMergeWaves - 1) / kMergeWaves;  // blocks per wave
    __shared__ uint64_t s_c[KL * kProjRowsPerWG];
    __shared__ int s_nc;
    const float* y = a.Y + static_cast<size_t>(a.map(i)) * a.ldy;
    const uint64_t T = s_top[k - 1];
    if (tid == 0) s_nc = 0;
    float v[BPW];
    int col[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int e = wave + j * kMergeWaves;
      const uint64_t t = s_top[e < k ? e : 0];
      col[j] = (key_id(t) / kProjRowsPerWG) * kProjRowsPerWG + lane;
      const bool ok = e < k && t != 0 && col[j] >= 0 && col[j] < a.V;
      v[j] = y[ok ? col[j] : 0];
      if (!ok) col[j] = -1;
    }
    __syncthreads();  // s_nc cleared, every read of s_top above done
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const uint64_t key = col[j] >= 0 ? topk_key(v[j], col[j]) : 0;
      if (key != 0 && key >= T) s_c[atomicAdd(&s_nc, 1)] = key;
    }
    if (tid < k) s_top[tid] = 0;
    __syncthreads();
    const int n = s_nc;
    for (int c = tid; c < n; c += kMergeThreads) {
      const uint64_t mine = s_c[c];
      int rank = 0;
      for (int o = 0; o < n; ++o) rank += s_c[o] > mine ? 1 : 0;
      if (rank < k) s_top[rank] = mine;
    }
    __syncthreads();
  }

  const bool fold = a.Enext != nullptr;  // uniform over the launch
  __shared__ int s_nu;
  __shared__ int s_urow[KL], s_utok[KL];
  const int b = i / a.P;
  if (wave == 0) {  // one wave writes the row
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, s_m[w]);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w)
      if (s_m[w] != -INFINITY) S += s_s[w] * expf(s_m[w] - M);
    const float lse = M + logf(S);
    const bool writer = g == 0;
    if (lane == 0) {
      if (writer && a.lse) a.lse[a.map(i)] = lse;
      if (writer && a.amax) a.amax[i] = key_id(s_top[0]);
      s_nu = 0;
    }
    if (writer && lane < k) {
      const uint64_t mine = s_top[lane];
      if (a.topk_ids) a.topk_ids[static_cast<size_t>(i) * k + lane] = key_id(mine);
      if (a.topk_vals) a.topk_vals[static_cast<size_t>(i) * k + lane] = key_value(mine);
    }
    if (a.node_hi > a.node_lo) {
      const int r = a.r0 + i % a.P;
      const size_t base = static_cast<size_t>(b) * a.N;
      if (writer && r == 0 && lane == 0) {
        a.cand_tok[base] = a.root_tok[b];
        a.cand_logp[base] = 0.f;
      }
      for (int c = a.node_lo + lane; c < a.node_hi; c += 64) {
        const int pp = a.node_parent[c];
        if (pp < 0 || a.node_row[pp] != r) continue;
        const int rk = a.node_rank[c];
        if (rk < 0 || rk >= k) continue;
        const uint64_t key = s_top[rk];
        if (writer) {
          const float plogp = pp == 0 ? 0.f : a.cand_logp[base + pp];
          a.cand_tok[base + c] = key_id(key);
          a.cand_logp[base + c] = plogp + (key_value(key) - lse);
        }
        const int nr = fold ? a.node_row[c] - a.rn : -1;
        if (nr >= 0 && nr < a.Pn) {  // c is expanded at the next depth: queue its feed-forward row
          const int e = atomicAdd(&s_nu, 1);  // one parent per row, so e < k <= KL
          if (e < KL) {
            s_urow[e] = b * a.Pn + nr;
            s_utok[e] = key_id(key);
          }
        }
      }
    }
  }
  if (a.walk_count) {  // uniform over the launch
    // the last of sequence wb's rows to finish walks its tree: the release
    // fence publishes this row's arg max before the count, the acquire fence
    // of the last one makes every row's visible (across the XCDs' L2s)
    __shared__ int s_last;
    const int wb = i / a.N;
    if (tid == 0) {
      __threadfence();
      s_last = atomicAdd(&a.walk_count[wb], 1) == a.N - 1;
    }
    __syncthreads();
    if (s_last && wave == 0) {
      __threadfence();
      greedy_walk_seq(wb, a.N, a.wDmax, a.amax, a.wtok, a.wparent, a.n_accepted, a.path, a.out_tok);
    }
    return;
  }
  if (!fold) return;
  __syncthreads();
  next_rows<KL>(a, b, g, s_nu < KL ? s_nu : KL, s_urow, s_utok);
}

template <int KL, int LL>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(MergeArgs a) {
  merge_row<KL, LL>(a, blockIdx.x / a.ng, blockIdx.x % a.ng);
}

// The same rows, plus the h half of the next Hydra head in workgroups
// M .. M + d / 16: that feed-forward stream does not depend on this merge, so
// it fills the otherwise idle chip while the merge runs.
template <int KL, int LL, int PF>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_ffn_kernel(MergeArgs a, MlpArgs f) {
  const int nm = a.M * a.ng;
  if (static_cast<int>(blockIdx.x) < nm) {
    merge_row<KL, LL>(a, blockIdx.x / a.ng, blockIdx.x % a.ng);
  } else {
    mlp_tile<1, PF, kMergeWaves>(f, blockIdx.x - nm, 0);
  }
}

template <int KL, int LL>
void launch_ll(const MergeArgs& a, const MlpArgs* f, hipStream_t stream) {
  const int nm = a.M * a.ng;
  if (!f) {
    topk_merge_kernel<KL, LL><<<nm, kMergeThreads, 0, stream>>>(a);
  } else if ((f->K / kMergeWaves / 32) % 8 == 0) {
    topk_merge_ffn_kernel<KL, LL, 8><<<nm + f->d / 16, kMergeThreads, 0, stream>>>(a, *f);
  } else {
    topk_merge_ffn_kernel<KL, LL, 1><<<nm + f->d / 16, kMergeThreads, 0, stream>>>(a, *f);
  }
}

template <int KL>
void launch_kl(const MergeArgs& a, const MlpArgs* f, hipStream_t stream) {
  if (a.nwg <= 2 * kMergeThreads) launch_ll<KL, (KL < 2 ? KL : 2)>(a, f, stream);
  else if (a.nwg <= 4 * kMergeThreads) launch_ll<KL, (KL < 4 ? KL : 4)>(a, f, stream);
  else launch_ll<KL, KL>(a, f, stream);
}

}  // namespace

bool merge_ffn_supported(int M, int K, int d) {
  return M >= 1 && M <= 16 && K % (kMergeWaves * 32) == 0 && d % 16 == 0;
}

int launch_topk_merge(const MergeArgs& args, hipStream_t stream, const MlpArgs* ffn) {
  if (args.M <= 0) return HYDRA_OK;
  MergeArgs a = args;
  // next-depth rows: up to one workgroup per 256 columns per row, about 512
  // workgroups in all (each repeats the row's top-k), dividing d / 256
  a.ng = 1;
  if (a.Enext && a.d >= 256) {
    const int q = a.d / 256;
    a.ng = std::max(1, std::min(q, 512 / a.M));
    while (q % a.ng) --a.ng;
  }
  if (a.k < 1 || a.k > HYDRA_MAX_TOPK) {
    set_error("top-k merge: k=%d out of [1, %d]", a.k, HYDRA_MAX_TOPK);
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (!a.ms && (a.lse || a.node_hi > a.node_lo)) {
    set_error("top-k merge: log-sum-exp and tree fill need the (max, sum exp) partials");
    return HYDRA_ERR_INVALID;
  }
  if (a.Enext && (a.d % (256 * a.ng) != 0 || !a.Anext || !a.h || !a.U || a.Pn < 1)) {
    set_error("top-k merge: next-depth rows need d %% %d == 0 (d=%d) and their buffers", 256 * a.ng, a.d);
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (a.walk_count && (a.k != 1 || !a.amax || a.N < 1 || a.Enext)) {
    set_error("top-k merge: the greedy walk needs k = 1, the arg maxes and no next-depth rows");
    return HYDRA_ERR_INVALID;
  }
  if (a.k > 1 && !a.Y) {
    set_error("top-k merge: k=%d needs the logits", a.k);
    return HYDRA_ERR_INVALID;
  }
  if (ffn && (ffn->heads != 1 || ffn->epi[0] != 0 || !merge_ffn_supported(ffn->M, ffn->K, ffn->d))) {
    set_error("top-k merge: unsupported feed-forward work (M=%d K=%d)", ffn->M, ffn->K);
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (a.k == 1) launch_kl<1>(a, ffn, stream);
  else if (a.k <= 4) launch_kl<4>(a, ffn, stream);
  else if (a.k <= 8) launch_kl<8>(a, ffn, stream);
  else launch_kl<HYDRA_MAX_TOPK>(a, ffn, stream);
  HY_LAUNCH_CHECK("top-k merge");
  return HYDRA_OK;
}

}  // namespace hydra
