// Stage 1 with the two-layer heads of the Hydra guide's implementation sketch.
//
// "Hydra Guide: Sequentially-Dependent Speculative AI", section "End-to-End
// Implementation" (the HydraHeadLayer and HydraDraftEngine modules): head 1
// maps h through Linear(d, d), SiLU and LayerNorm(d); head k >= 2 fuses
// [h || e(x_parent)] through Linear(2d, H), SiLU, Linear(H, d) and
// LayerNorm(d) (H = 1024 there); every head ends in its own bias-free
// vocabulary projection, and candidates expand head by head from each
// parent's top-k exactly as with the one-layer heads.
//
// Per depth k the rows are few (one per expanded node), so each Linear is a
// weight stream: the split-K projection kernels write float32 partials and a
// row kernel finishes them (partials + bias, SiLU, LayerNorm), one workgroup
// per row (1024 threads, 16-byte loads of every partial at once) holding the
// row in LDS between the statistics and the output. The
// vocabulary projection and the merge (log-sum-exp, top-k, tree fill) are the
// one-layer path's.
#include "common.h"

namespace hydra {
namespace {

constexpr int kSketchThreads = 1024;
constexpr int kSketchMaxWidth = 8192;  // row held in LDS: 32 KB of float32

__device__ __forceinline__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  __syncthreads();  // red may still be read by the previous sum
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kSketchThreads / 64; ++w) t += red[w];
  return t;
}

template <class T>
__device__ __forceinline__ float round_to(float v);
template <>
__device__ __forceinline__ float round_to<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float round_to<bf16_t>(float v) {
  return bf16_to_f32(f32_to_bf16(v));
}

template <class T>
__device__ __forceinline__ float finish(float v, const T* bias, int j, int act) {
  v += load_f(bias, j);
  return act ? round_to<T>(v / (1.0f + expf(-v))) : v;
}

template <class T>
__device__ __forceinline__ void store4(T* p, size_t i, float4 v) {
  store_f(p, i, v.x);
  store_f(p, i + 1, v.y);
  store_f(p, i + 2, v.z);
  store_f(p, i + 3, v.w);
}

// Row m of width W (W % 4 == 0): v = sum of the ns partials (stride floats
// apart) + bias; with act, v = T(SiLU(v)); with g, v = (v - mean) /
// sqrt(var + eps) * g + beta over the row (biased variance). T(v) goes to
// out[m] and, with hidden, to hidden[map(m)]. Rows are few (one per expanded
// node), so a workgroup of 1024 threads takes a row: every thread issues the
// 16-byte loads of its columns from all partials at once.
template <class T>
__global__ __launch_bounds__(kSketchThreads) void sketch_rows(int W, int ns, size_t stride,
                                                              const float* __restrict__ part,
                                                              const T* __restrict__ bias, int act,
                                                              const T* __restrict__ g, const T* __restrict__ beta,
                                                              float eps, T* __restrict__ out,
                                                              T* __restrict__ hidden, RowMap map) {
  extern __shared__ float4 row[];
  __shared__ double red[kSketchThreads / 64];
  const int m = blockIdx.x;
  const int W4 = W / 4;
  const size_t base = static_cast<size_t>(m) * W;
  float s = 0.f;
  for (int c = threadIdx.x; c < W4; c += kSketchThreads) {
    float4 v = *reinterpret_cast<const float4*>(part + base + 4 * c);
    for (int t = 1; t < ns; ++t) {
      const float4 q = *reinterpret_cast<const float4*>(part + t * stride + base + 4 * c);
      v.x += q.x;
      v.y += q.y;
      v.z += q.z;
      v.w += q.w;
    }
    v.x = finish(v.x, bias, 4 * c, act);
    v.y = finish(v.y, bias, 4 * c + 1, act);
    v.z = finish(v.z, bias, 4 * c + 2, act);
    v.w = finish(v.w, bias, 4 * c + 3, act);
    row[c] = v;  // each thread reads back only its own columns
    s += (v.x + v.y) + (v.z + v.w);
  }
  T* hrow = hidden ? hidden + static_cast<size_t>(map(m)) * W : nullptr;
  if (!g) {
    for (int c = threadIdx.x; c < W4; c += kSketchThreads) {
      store4(out, base + 4 * c, row[c]);
      if (hrow) store4(hrow, 4 * c, row[c]);
    }
    return;
  }
  const float mean = static_cast<float>(block_sum_d(s, red) / W);
  float q = 0.f;
  for (int c = threadIdx.x; c < W4; c += kSketchThreads) {
    const float4 v = row[c];
    q += (v.x - mean) * (v.x - mean) + (v.y - mean) * (v.y - mean) + (v.z - mean) * (v.z - mean) +
         (v.w - mean) * (v.w - mean);
  }
  const float rstd = static_cast<float>(1.0 / sqrt(block_sum_d(q, red) / W + eps));
  for (int c = threadIdx.x; c < W4; c += kSketchThreads) {
    const float4 v = row[c];
    const int j = 4 * c;
    const float4 y = make_float4((v.x - mean) * rstd * load_f(g, j) + load_f(beta, j),
                                 (v.y - mean) * rstd * load_f(g, j + 1) + load_f(beta, j + 1),
                                 (v.z - mean) * rstd * load_f(g, j + 2) + load_f(beta, j + 2),
                                 (v.w - mean) * rstd * load_f(g, j + 3) + load_f(beta, j + 3));
    store4(out, base + j, y);
    if (hrow) store4(hrow, j, y);
  }
}

template <class T>
void launch_rows(int M, int W, int ns, const float* part, const void* bias, int act, const void* g,
                 const void* beta, float eps, void* out, void* hidden, RowMap map, hipStream_t stream) {
  sketch_rows<T><<<M, kSketchThreads, W * sizeof(float), stream>>>(
      W, ns, static_cast<size_t>(M) * W, part, static_cast<const T*>(bias), act, static_cast<const T*>(g),
      static_cast<const T*>(beta), eps, static_cast<T*>(out), static_cast<T*>(hidden), map);
}

int rows(int dtype, int M, int W, int ns, const float* part, const void* bias, int act, const void* g,
         const void* beta, float eps, void* out, void* hidden, RowMap map, hipStream_t stream) {
  if (dtype == HYDRA_F32)
    launch_rows<float>(M, W, ns, part, bias, act, g, beta, eps, out, hidden, map, stream);
  else
    launch_rows<bf16_t>(M, W, ns, part, bias, act, g, beta, eps, out, hidden, map, stream);
  HY_LAUNCH_CHECK("draft_heads_sketch: row epilogue");
  return HYDRA_OK;
}

// split of K for the gathered [h || e] rows: about 512 workgroups of 64
// output columns, every K range a multiple of 256
int gather_splits(int dtype, int M, int K, int N) {
  if (dtype == HYDRA_F32) return 1;
  const int wg = (N + 63) / 64 * ((M + 255) / 256);
  int s = 1;
  while (s < 16 && wg * s < 512 && (K / 256) % (s * 2) == 0) s *= 2;
  return s;
}

struct SketchWs {
  size_t part, a, u, keys, ms, total;
};
SketchWs sketch_ws(int dtype, int B, int d, int V, int hid, int Dmax, const int32_t* row_first) {
  int maxP = 0;
  for (int k = 1; k <= Dmax; ++k) maxP = std::max(maxP, row_first[k] - row_first[k - 1]);
  const size_t M = static_cast<size_t>(B) * maxP;
  const size_t esz = dtype == HYDRA_F32 ? 4 : 2;
  const size_t nwg = projection_nwg(V);
  SketchWs w;
  w.part = align_up(16 * M * std::max(d, hid) * sizeof(float), 256);
  w.a = align_up(M * hid * esz, 256);
  w.u = align_up(M * d * esz, 256);
  w.keys = align_up(M * nwg * sizeof(uint64_t), 256);
  w.ms = align_up(M * nwg * sizeof(float2), 256);
  w.total = w.part + w.a + w.u + w.keys + w.ms + 256;
  return w;
}

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" size_t hydra_draft_heads_sketch_workspace_size(int dtype, int B, int d, int V, int hidden_dim, int Dmax,
                                                          const int32_t* row_first) {
  if (B <= 0 || d <= 0 || V <= 0 || hidden_dim <= 0 || Dmax <= 0 || Dmax > HYDRA_MAX_DEPTH || !row_first) return 0;
  return sketch_ws(dtype & ~HYDRA_VOCAB_PACKED, B, d, V, hidden_dim, Dmax, row_first).total;
}

extern "C" int hydra_draft_heads_sketch(int dtype, int B, int d, int V, int hidden_dim, const void* h,
                                        const int32_t* root_tok, const void* emb, int n_heads,
                                        const void* const* Wa, const void* const* ba, const void* const* Wb,
                                        const void* const* bb, const void* const* ln_g, const void* const* ln_b,
                                        const void* const* W2, float ln_eps, int N, int Dmax,
                                        const int32_t* node_parent, const int32_t* node_rank,
                                        const int32_t* node_row, int R, const int32_t* row_node,
                                        const int32_t* row_first, const int32_t* depth_first,
                                        const int32_t* k_per_depth, float* head_logits, float* head_lse,
                                        void* head_hidden, int32_t* cand_tok, float* cand_logp, void* ws,
                                        size_t ws_bytes, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int hid = hidden_dim;
  const int vpack = dtype & HYDRA_VOCAB_PACKED;  // packed vocabulary weights (hydra_pack_weight)
  dtype &= ~HYDRA_VOCAB_PACKED;
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "draft_heads_sketch: bad dtype %d", dtype);
  HY_CHECK(!vpack || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "draft_heads_sketch: packed vocabulary weights are bf16");
  HY_CHECK(B > 0 && d > 0 && V > 0 && hid > 0, HYDRA_ERR_INVALID,
           "draft_heads_sketch: bad sizes B=%d d=%d V=%d hidden=%d", B, d, V, hid);
  HY_CHECK(d <= kSketchMaxWidth && hid <= kSketchMaxWidth, HYDRA_ERR_UNSUPPORTED,
           "draft_heads_sketch: d=%d and hidden=%d must be <= %d", d, hid, kSketchMaxWidth);
  HY_CHECK(d % 4 == 0 && hid % 4 == 0, HYDRA_ERR_UNSUPPORTED,
           "draft_heads_sketch: d and hidden must be multiples of 4 (d=%d hidden=%d)", d, hid);
  HY_CHECK(dtype == HYDRA_F32 || (d % 256 == 0 && hid % 256 == 0), HYDRA_ERR_UNSUPPORTED,
           "draft_heads_sketch: bf16 needs d and hidden multiples of 256 (d=%d hidden=%d)", d, hid);
  HY_CHECK(ln_eps > 0.f, HYDRA_ERR_INVALID, "draft_heads_sketch: LayerNorm eps must be > 0");
  HY_CHECK(Dmax >= 1 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "draft_heads_sketch: Dmax=%d out of [1, %d]", Dmax,
           HYDRA_MAX_DEPTH);
  HY_CHECK(n_heads >= Dmax, HYDRA_ERR_INVALID, "draft_heads_sketch: n_heads=%d < Dmax=%d", n_heads, Dmax);
  HY_CHECK(N >= 2 && N <= HYDRA_MAX_TREE, HYDRA_ERR_INVALID, "draft_heads_sketch: N=%d out of [2, %d]", N,
           HYDRA_MAX_TREE);
  HY_CHECK(h && root_tok && emb && Wa && ba && Wb && bb && ln_g && ln_b && W2 && node_parent && node_rank &&
               node_row && row_node && row_first && depth_first && k_per_depth && head_logits && head_lse &&
               cand_tok && cand_logp,
           HYDRA_ERR_INVALID, "draft_heads_sketch: null pointer");
  HY_CHECK(row_first[0] == 0 && row_first[Dmax] == R, HYDRA_ERR_INVALID,
           "draft_heads_sketch: row_first must span [0, R=%d)", R);
  HY_CHECK(row_first[1] == 1, HYDRA_ERR_INVALID, "draft_heads_sketch: head 1 has one row (the root)");
  HY_CHECK(depth_first[0] == 0 && depth_first[1] == 1 && depth_first[Dmax + 1] == N, HYDRA_ERR_INVALID,
           "draft_heads_sketch: depth_first must start 0, 1 and end at N=%d", N);
  for (int k = 1; k <= Dmax; ++k) {
    HY_CHECK(row_first[k] > row_first[k - 1], HYDRA_ERR_INVALID, "draft_heads_sketch: depth %d has no head rows", k);
    HY_CHECK(depth_first[k + 1] > depth_first[k], HYDRA_ERR_INVALID, "draft_heads_sketch: depth %d has no nodes", k);
    HY_CHECK(k_per_depth[k - 1] >= 1 && k_per_depth[k - 1] <= HYDRA_MAX_TOPK && k_per_depth[k - 1] <= V,
             HYDRA_ERR_UNSUPPORTED, "draft_heads_sketch: top-k %d at depth %d out of [1, %d]", k_per_depth[k - 1],
             k, HYDRA_MAX_TOPK);
    HY_CHECK(Wa[k - 1] && ba[k - 1] && ln_g[k - 1] && ln_b[k - 1] && W2[k - 1] &&
                 (k == 1 || (Wb[k - 1] && bb[k - 1])),
             HYDRA_ERR_INVALID, "draft_heads_sketch: null weight of head %d", k);
  }
  const size_t need = hydra_draft_heads_sketch_workspace_size(dtype, B, d, V, hid, Dmax, row_first);
  HY_CHECK(ws && ws_bytes >= need, HYDRA_ERR_WORKSPACE, "draft_heads_sketch: workspace %zu < required %zu",
           ws_bytes, need);

  const SketchWs wl = sketch_ws(dtype, B, d, V, hid, Dmax, row_first);
  const size_t esz = dtype == HYDRA_F32 ? 4 : 2;
  const int nwg = projection_nwg(V);
  Arena arena(ws, ws_bytes);
  float* part = arena.take<float>(wl.part / sizeof(float));
  char* A = arena.take<char>(wl.a);
  char* U = arena.take<char>(wl.u);
  uint64_t* tkeys = arena.take<uint64_t>(wl.keys / sizeof(uint64_t));
  float2* tms = arena.take<float2>(wl.ms / sizeof(float2));
  const size_t part_floats = wl.part / sizeof(float);

  for (int k = 1; k <= Dmax; ++k) {
    const int P = row_first[k] - row_first[k - 1];
    const int r0 = row_first[k - 1];
    const int M = B * P;
    const RowMap map{P, R, r0};
    int ns = 1, rc;
    if (k == 1) {
      // u = LayerNorm(T(SiLU(Wa h + ba))), one row per sequence
      rc = launch_projection_parts(dtype, M, d, d, h, Wa[0], part, part_floats, &ns, stream);
      if (rc != HYDRA_OK) return rc;
      rc = rows(dtype, M, d, ns, part, ba[0], 1, ln_g[0], ln_b[0], ln_eps, U, head_hidden, map, stream);
      if (rc != HYDRA_OK) return rc;
    } else {
      // a = T(SiLU(Wa [h || e(parent)] + ba)) over the gathered rows
      XSource xs{};
      xs.x = h;
      xs.ldx = d;
      xs.mode = 1;
      xs.emb = emb;
      xs.tok = cand_tok;
      xs.root_tok = root_tok;
      xs.V = V;
      xs.row_node = row_node;
      xs.ntree = N;
      xs.P = P;
      xs.r0 = r0;
      xs.d = d;
      ns = gather_splits(dtype, M, 2 * d, hid);
      rc = launch_projection(dtype, M, 2 * d, hid, xs, Wa[k - 1], dtype == HYDRA_F32 ? part : nullptr,
                             RowMap{M, 0, 0}, hid, ns, dtype == HYDRA_F32 ? nullptr : part,
                             TopkPartials{nullptr, nullptr}, stream);
      if (rc != HYDRA_OK) return rc;
      rc = rows(dtype, M, hid, ns, part, ba[k - 1], 1, nullptr, nullptr, ln_eps, A, nullptr, RowMap{M, 0, 0},
                stream);
      if (rc != HYDRA_OK) return rc;
      // u = LayerNorm(Wb a + bb)
      rc = launch_projection_parts(dtype, M, hid, d, A, Wb[k - 1], part, part_floats, &ns, stream);
      if (rc != HYDRA_OK) return rc;
      rc = rows(dtype, M, d, ns, part, bb[k - 1], 0, ln_g[k - 1], ln_b[k - 1], ln_eps, U, head_hidden, map, stream);
      if (rc != HYDRA_OK) return rc;
    }
    // head logits with the fused row partials, then log-sum-exp, top-k and tree fill
    XSource xu{};
    xu.x = U;
    xu.ldx = d;
    xu.mode = 0;
    rc = launch_projection(dtype | vpack, M, d, V, xu, W2[k - 1], head_logits, map, V, 1, nullptr,
                           TopkPartials{tkeys, tms}, stream);
    if (rc != HYDRA_OK) return rc;
    MergeArgs ma{};
    ma.M = M;
    ma.nwg = nwg;
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
