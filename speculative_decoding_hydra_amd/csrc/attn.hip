// Stage 3: tree-masked attention verify over a paged KV prefix.
//
// "Hydra Guide: Sequentially-Dependent Speculative AI", section "Tree
// Attention Matrix with Topology-Aware Causal Masking", and "Medusa Heads",
// section "Tree Attention und Akzeptanz": the tree rows are appended after the
// prefix; row u sees every prefix position and the tree rows that are its
// ancestors or itself. "Speculative Decoding", section "The core asymmetry":
// verifying k rows costs about as much as a prompt of length k, so all tree
// rows share one pass over the KV prefix.
//
// gfx950 design (bf16, D = 128):
//   * grid = (prefix splits + 1) x (query tiles of 64 rows) x (sequence, KV
//     head). Query rows of a KV head are (node u, query head g) pairs, so GQA
//     packs the G query heads into the same tile.
//   * per 64-key tile, K is staged in LDS row-major and V transposed, both
//     shared by the 4 waves (16 query rows each);
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 puts each query in one lane
//     column, so the online-softmax statistics need only two cross-lane steps
//     and the probabilities are already laid out as the B operand of
//     O^T = V^T . P^T (the token order inside a 32-key step is permuted
//     identically on both operands);
//   * the extra split holds the tree rows: the mask comes from the ancestor
//     table (v visible to u iff anc[u][depth v] == v), no dense mask;
//   * splits write unnormalised partials; a combine kernel merges them with
//     their log-sum-exps and rounds the output to bf16.
#include "common.h"

namespace hydra {
namespace {

constexpr int kKT = 64;  // keys per tile
constexpr int kMaxSplitPages = 1024;  // page ids one split stages in LDS

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

template <int D>
__global__ __launch_bounds__(256) void attn_split_mfma(
    int B, int N, int Hq, int Hkv, float scale_log2, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k_tree, const bf16_t* __restrict__ v_tree,
    const bf16_t* __restrict__ k_pages, const bf16_t* __restrict__ v_pages, int n_pages,
    int page_size, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ anc,
    const int32_t* __restrict__ depth, int Dmax, int nsplit, int lsplit, int NQ, int NQpad,
    float* __restrict__ opart, float* __restrict__ mpart, float* __restrict__ lpart) {
  static_assert(D == 128, "tile mapping assumes D = 128");
  constexpr int KROW = D + 8;    // K row in LDS (bf16), 16-byte pad
  constexpr int VROW = kKT + 4;  // V^T row in LDS (bf16), 8-byte pad
  constexpr int DJ = D / 32;
  constexpr int DD = D / 16;
  __shared__ __align__(16) bf16_t klds[kKT * KROW];
  __shared__ __align__(16) bf16_t vlds[D * VROW];
  __shared__ bool s_ok[kKT];
  __shared__ int s_dep[kKT];                              // depth of each tree key of the tile
  __shared__ int s_pages[kMaxSplitPages];                 // page ids of this split
  __shared__ int s_anc[64][HYDRA_MAX_DEPTH + 1];          // ancestor rows of the 64 query rows

  const int split = blockIdx.x;
  const bool tree_part = split == nsplit;
  const int qtile = blockIdx.y;
  const int b = blockIdx.z / Hkv;
  const int hkv = blockIdx.z % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, lq = lane & 15;

  const int qi = qtile * 64 + wave * 16 + lq;
  const bool qvalid = qi < NQ;
  const int u = qvalid ? qi / G : 0;
  const int gq = qi % G;
  bf16x8_t qreg[DJ];
  {
    const bf16_t* qp = q + ((static_cast<size_t>(b) * N + u) * Hq + hkv * G + gq) * D + 8 * g;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      const u32x4_t v = qvalid ? *reinterpret_cast<const u32x4_t*>(qp + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
      qreg[j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  int L = prefix_len[b];
  const int cap = max_pages * page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int t_begin, t_end;
  if (tree_part) {
    t_begin = 0;
    t_end = N;
  } else {
    t_begin = split * lsplit;
    t_end = min(L, t_begin + lsplit);
  }
  const int32_t* dep_b = depth + static_cast<size_t>(b) * N;
  const int wrow_q = wave * 16 + lq;  // this lane's query row inside the tile
  if (tree_part) {
    for (int e = tid; e < 64 * (Dmax + 1); e += 256) {
      const int r = e / (Dmax + 1), j = e % (Dmax + 1);
      const int qr = qtile * 64 + r;
      s_anc[r][j] = qr < NQ ? anc[(static_cast<size_t>(b) * N + qr / G) * (Dmax + 1) + j] : -1;
    }
  } else {
    const int p0 = t_begin / page_size;
    const int np = t_end > t_begin ? (t_end - 1) / page_size - p0 + 1 : 0;
    for (int e = tid; e < np; e += 256) s_pages[e] = block_table[static_cast<size_t>(b) * max_pages + p0 + e];
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t oacc[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) oacc[dd] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // loader mapping: 4 consecutive keys x 8 dims per thread
  const int tg = tid >> 4;          // key group 0..15
  const int dc = tid & 15;          // 8-dim chunk 0..15
  const int tl = 4 * tg;

  u32x4_t kv[4], vv[4];
  int kvalid = 0;  // keys of this thread's group of 4 that exist (range and page)
  // Registers of the next tile: 4 keys x 8 dims of K and of V per thread.
  // Loads are unconditional (invalid keys re-read a valid row and are masked
  // through s_ok), so the compiler can keep them in flight across the tile.
  auto load_tile = [&](int t0) {
    const int tk = t0 + tl;
    int valid = tk < t_end ? min(4, t_end - tk) : 0;
    const bf16_t* kb;
    const bf16_t* vb;
    int stride;
    if (tree_part) {
      const int tc = tk < N ? tk : 0;
      const size_t off = ((static_cast<size_t>(b) * N + tc) * Hkv + hkv) * D + dc * 8;
      kb = k_tree + off;
      vb = v_tree + off;
      stride = Hkv * D;
    } else {
      const int tc = tk < t_end ? tk : t_begin;
      int pg = s_pages[tc / page_size - t_begin / page_size];
      if (pg < 0 || pg >= n_pages) {
        pg = 0;
        valid = 0;
      }
      const size_t off = ((static_cast<size_t>(pg) * Hkv + hkv) * page_size + tc % page_size) * D + dc * 8;
      kb = k_pages + off;
      vb = v_pages + off;
      stride = D;
    }
    kvalid = valid;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t o = j < valid ? static_cast<size_t>(j) * stride : 0;
      kv[j] = *reinterpret_cast<const u32x4_t*>(kb + o);
      vv[j] = *reinterpret_cast<const u32x4_t*>(vb + o);
    }
  };
  if (t_begin < t_end) load_tile(t_begin);

  for (int t0 = t_begin; t0 < t_end; t0 += kKT) {
    __syncthreads();  // previous tile fully consumed
    if (dc == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s_ok[tl + j] = j < kvalid;
        if (tree_part) s_dep[tl + j] = j < kvalid ? dep_b[t0 + tl + j] : -1;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4_t*>(&klds[(tl + j) * KROW + dc * 8]) = kv[j];
    {
      typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;
      const u16x8 a0 = __builtin_bit_cast(u16x8, vv[0]);
      const u16x8 a1 = __builtin_bit_cast(u16x8, vv[1]);
      const u16x8 a2 = __builtin_bit_cast(u16x8, vv[2]);
      const u16x8 a3 = __builtin_bit_cast(u16x8, vv[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x2_t w;
        w.x = pack2(a0[e], a1[e]);
        w.y = pack2(a2[e], a3[e]);
        *reinterpret_cast<u32x2_t*>(&vlds[(dc * 8 + e) * VROW + tl]) = w;
      }
    }
    __syncthreads();
    if (t0 + kKT < t_end) load_tile(t0 + kKT);  // next tile in flight during this one

    // S^T tile: lane holds keys 16 tt + 4 g + i for query column lq
    f32x4_t sacc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      sacc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&klds[(16 * tt + lq) * KROW + 32 * j + 8 * g]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qreg[j],
                                                          sacc[tt], 0, 0, 0);
      }
    }
    float sv[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * tt + 4 * g + i;
        bool ok = s_ok[16 * tt + 4 * g + i];
        if (tree_part) {
          const int dv = s_dep[16 * tt + 4 * g + i];
          ok = ok && dv >= 0 && dv <= Dmax && s_anc[wrow_q][dv] == t;
        }
        const float s = ok ? sacc[tt][i] * scale_log2 : -INFINITY;
        sv[tt][i] = s;
        mt = fmaxf(mt, s);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sv[tt][i] - m_use);
        sv[tt][i] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) oacc[dd] *= alpha;

    // P^T operands: slots 0..3 = keys 32 ks + 4 g + i, slots 4..7 = keys 32 ks + 16 + 4 g + i
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<__bf16>(sv[2 * ks][i]);
        pb[4 + i] = static_cast<__bf16>(sv[2 * ks + 1][i]);
      }
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) {
        const bf16_t* vr = &vlds[(16 * dd + lq) * VROW + 32 * ks + 4 * g];
        u32x4_t a;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + 16);
        a.x = lo.x;
        a.y = lo.y;
        a.z = hi.x;
        a.w = hi.y;
        oacc[dd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), pb, oacc[dd],
                                                          0, 0, 0);
      }
    }
  }

  if (qvalid) {
    const size_t row = (static_cast<size_t>(split * B + b) * Hkv + hkv) * NQpad + qi;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd)
      *reinterpret_cast<float4*>(opart + row * D + 16 * dd + 4 * g) =
          make_float4(oacc[dd][0], oacc[dd][1], oacc[dd][2], oacc[dd][3]);
    if (g == 0) {
      mpart[row] = m_run;
      lpart[row] = l_run;
    }
  }
}

// Merge the splits of one (sequence, KV head, query row). D / 4 lanes per row,
// four dims per lane, so a wave merges 64 * 4 / D rows at once.
template <class T>
__global__ __launch_bounds__(256) void attn_combine(int B, int N, int Hq, int Hkv, int D, int nparts,
                                                    int NQ, int NQpad, const float* __restrict__ opart,
                                                    const float* __restrict__ mpart,
                                                    const float* __restrict__ lpart, T* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int lpr = D / 4;  // lanes per row
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const int row = tid / lpr;  // over B * Hkv * NQ
  const int c = tid % lpr;
  if (row >= B * Hkv * NQ) return;
  const int qi = row % NQ;
  const int bh = row / NQ;
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int G = Hq / Hkv;
  const int u = qi / G, hq = hkv * G + qi % G;
  const size_t stride = static_cast<size_t>(B) * Hkv * NQpad;
  const size_t r0 = (static_cast<size_t>(b) * Hkv + hkv) * NQpad + qi;
  float M = -INFINITY;
  for (int s = 0; s < nparts; ++s) M = fmaxf(M, mpart[r0 + s * stride]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float Lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nparts; ++s) {
    const size_t r = r0 + s * stride;
    const float w = exp2f(mpart[r] - Mu);
    Lsum += lpart[r] * w;
    const float4 o = *reinterpret_cast<const float4*>(opart + r * D + 4 * c);
    acc.x += o.x * w;
    acc.y += o.y * w;
    acc.z += o.z * w;
    acc.w += o.w * w;
  }
  const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
  T* o = out + ((static_cast<size_t>(b) * N + u) * Hq + hq) * D + 4 * c;
  store_f(o, 0, acc.x * inv);
  store_f(o, 1, acc.y * inv);
  store_f(o, 2, acc.z * inv);
  store_f(o, 3, acc.w * inv);
  if (lse && c == 0) lse[(static_cast<size_t>(b) * N + u) * Hq + hq] = (Mu + log2f(Lsum)) * 0.69314718055994531f;
}

// Generic path (float32, or D other than 128): one wave per (b, u, hq),
// online softmax over chunks of 64 keys, lanes over keys then over D.
template <class T>
__global__ __launch_bounds__(64) void attn_simple(int B, int N, int Hq, int Hkv, int D, float scale,
                                                  const T* __restrict__ q, const T* __restrict__ k_tree,
                                                  const T* __restrict__ v_tree, const T* __restrict__ k_pages,
                                                  const T* __restrict__ v_pages, int n_pages, int page_size,
                                                  const int32_t* __restrict__ block_table, int max_pages,
                                                  const int32_t* __restrict__ prefix_len,
                                                  const int32_t* __restrict__ anc, int Dmax, T* __restrict__ out,
                                                  float* __restrict__ lse) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  __shared__ const T* vrow[64];
  const int lane = threadIdx.x;
  const int idx = blockIdx.x;  // (b, u, hq)
  const int hq = idx % Hq;
  const int u = (idx / Hq) % N;
  const int b = idx / (Hq * N);
  const int hkv = hq / (Hq / Hkv);
  const T* qp = q + ((static_cast<size_t>(b) * N + u) * Hq + hq) * D;
  for (int d = lane; d < D; d += 64) qs[d] = load_f(qp, d) * scale;
  __syncthreads();
  int L = prefix_len[b];
  const int cap = max_pages * page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int32_t* au = anc + (static_cast<size_t>(b) * N + u) * (Dmax + 1);
  int n_anc = 0;
  while (n_anc <= Dmax && au[n_anc] >= 0) ++n_anc;
  const int total = L + n_anc;
  float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c0 = 0; c0 < total; c0 += 64) {
    const int j = c0 + lane;
    float s = -INFINITY;
    const T* kr = nullptr;
    const T* vr = nullptr;
    if (j < L) {
      const int pg = block_table[static_cast<size_t>(b) * max_pages + j / page_size];
      if (pg >= 0 && pg < n_pages) {
        const size_t off = ((static_cast<size_t>(pg) * Hkv + hkv) * page_size + j % page_size) * D;
        kr = k_pages + off;
        vr = v_pages + off;
      }
    } else if (j < total) {
      const int v = au[j - L];
      const size_t off = ((static_cast<size_t>(b) * N + v) * Hkv + hkv) * D;
      kr = k_tree + off;
      vr = v_tree + off;
    }
    if (kr) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], load_f(kr, d), acc);
      s = acc;
    }
    const float mt = wave_max(s);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    const float p = kr ? expf(s - m_use) : 0.f;
    const float psum = wave_sum(p);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    o0 *= alpha;
    o1 *= alpha;
    ps[lane] = p;
    vrow[lane] = vr;
    __syncthreads();
    const int cnt = min(64, total - c0);
    for (int t = 0; t < cnt; ++t) {
      const T* r = vrow[t];
      if (!r) continue;
      const float w = ps[t];
      if (lane < D) o0 = fmaf(w, load_f(r, lane), o0);
      if (lane + 64 < D) o1 = fmaf(w, load_f(r, lane + 64), o1);
    }
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  T* op = out + ((static_cast<size_t>(b) * N + u) * Hq + hq) * D;
  if (lane < D) store_f(op, lane, o0 * inv);
  if (lane + 64 < D) store_f(op, lane + 64, o1 * inv);
  if (lse && lane == 0) lse[(static_cast<size_t>(b) * N + u) * Hq + hq] = m_run + logf(l_run);
}

struct SplitPlan {
  int nsplit, lsplit, qtiles, NQ, NQpad;
};

SplitPlan plan_splits(int B, int N, int Hq, int Hkv, int max_prefix_len) {
  SplitPlan p;
  p.NQ = N * (Hq / Hkv);
  p.qtiles = (p.NQ + 63) / 64;
  p.NQpad = p.qtiles * 64;
  const int base = B * Hkv * p.qtiles;
  const int Lr = max_prefix_len > 0 ? max_prefix_len : 0;
  int want = (512 + base - 1) / base;            // workgroups for 256 CUs, twice over
  int maxs = (Lr + 255) / 256;                   // at least 4 key tiles per split
  int s = want < maxs ? want : maxs;
  if (s < 1) s = 1;
  int ls = (Lr + s - 1) / s;
  ls = (ls + kKT - 1) / kKT * kKT;
  const int lcap = (kMaxSplitPages - 1) * 16;  // pages of a split must fit in LDS (page_size >= 16)
  if (ls > lcap) ls = lcap / kKT * kKT;
  if (ls < kKT) ls = kKT;
  p.lsplit = ls;
  p.nsplit = Lr > 0 ? (Lr + ls - 1) / ls : 0;
  return p;
}

bool use_mfma(int dtype, int D) { return dtype == HYDRA_BF16 && D == 128; }

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" size_t tree_attention_verify_workspace_size(int dtype, int B, int N, int Hq, int Hkv, int D,
                                                       int max_prefix_len) {
  if (!use_mfma(dtype, D) || B <= 0 || N <= 0 || Hkv <= 0 || Hq <= 0) return 0;
  const SplitPlan p = plan_splits(B, N, Hq, Hkv, max_prefix_len);
  const size_t rows = static_cast<size_t>(p.nsplit + 1) * B * Hkv * p.NQpad;
  return align_up(rows * D * sizeof(float), 256) + 2 * align_up(rows * sizeof(float), 256) + 256;
}

extern "C" int tree_attention_verify(int dtype, int B, int N, int Hq, int Hkv, int D, float scale,
                                     const void* q, const void* k_tree, const void* v_tree,
                                     const void* k_pages, const void* v_pages, int n_pages, int page_size,
                                     const int32_t* block_table, int max_pages, const int32_t* prefix_len,
                                     int max_prefix_len, const int32_t* anc, const int32_t* depth, int Dmax,
                                     void* out, float* lse, void* ws, size_t ws_bytes, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "tree_attention: bad dtype %d", dtype);
  HY_CHECK(B > 0 && N > 0 && Hq > 0 && Hkv > 0, HYDRA_ERR_INVALID, "tree_attention: bad sizes B=%d N=%d Hq=%d Hkv=%d",
           B, N, Hq, Hkv);
  HY_CHECK(N <= HYDRA_MAX_VERIFY, HYDRA_ERR_INVALID, "tree_attention: N=%d > %d", N, HYDRA_MAX_VERIFY);
  HY_CHECK(Hq % Hkv == 0, HYDRA_ERR_INVALID, "tree_attention: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  HY_CHECK(D == 32 || D == 64 || D == 128, HYDRA_ERR_UNSUPPORTED, "tree_attention: D=%d not in {32, 64, 128}", D);
  HY_CHECK(page_size == 16 || page_size == 32 || page_size == 64, HYDRA_ERR_UNSUPPORTED,
           "tree_attention: page_size=%d not in {16, 32, 64}", page_size);
  HY_CHECK(Dmax >= 1 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "tree_attention: Dmax=%d", Dmax);
  HY_CHECK(max_prefix_len >= 0 && max_prefix_len <= max_pages * page_size, HYDRA_ERR_INVALID,
           "tree_attention: max_prefix_len=%d exceeds max_pages*page_size=%d", max_prefix_len,
           max_pages * page_size);
  HY_CHECK(n_pages >= 0 && max_pages >= 1, HYDRA_ERR_INVALID, "tree_attention: n_pages=%d max_pages=%d", n_pages,
           max_pages);
  HY_CHECK(q && k_tree && v_tree && block_table && prefix_len && anc && depth && out, HYDRA_ERR_INVALID,
           "tree_attention: null pointer");
  HY_CHECK(n_pages == 0 || (k_pages && v_pages), HYDRA_ERR_INVALID, "tree_attention: null page pool");
  HY_CHECK(max_prefix_len == 0 || n_pages >= 1, HYDRA_ERR_INVALID,
           "tree_attention: a prefix of %d tokens needs a page pool", max_prefix_len);
  const size_t need = tree_attention_verify_workspace_size(dtype, B, N, Hq, Hkv, D, max_prefix_len);
  HY_CHECK(ws_bytes >= need && (need == 0 || ws), HYDRA_ERR_WORKSPACE, "tree_attention: workspace %zu < %zu",
           ws_bytes, need);

  if (!use_mfma(dtype, D)) {
    const int grid = B * N * Hq;
    if (dtype == HYDRA_F32) {
      attn_simple<float><<<grid, 64, 0, stream>>>(
          B, N, Hq, Hkv, D, scale, static_cast<const float*>(q), static_cast<const float*>(k_tree),
          static_cast<const float*>(v_tree), static_cast<const float*>(k_pages), static_cast<const float*>(v_pages),
          n_pages, page_size, block_table, max_pages, prefix_len, anc, Dmax, static_cast<float*>(out), lse);
    } else {
      attn_simple<bf16_t><<<grid, 64, 0, stream>>>(
          B, N, Hq, Hkv, D, scale, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_tree),
          static_cast<const bf16_t*>(v_tree), static_cast<const bf16_t*>(k_pages),
          static_cast<const bf16_t*>(v_pages), n_pages, page_size, block_table, max_pages, prefix_len, anc, Dmax,
          static_cast<bf16_t*>(out), lse);
    }
    HY_LAUNCH_CHECK("tree_attention(simple)");
    return HYDRA_OK;
  }

  const SplitPlan p = plan_splits(B, N, Hq, Hkv, max_prefix_len);
  const int nparts = p.nsplit + 1;
  const size_t rows = static_cast<size_t>(nparts) * B * Hkv * p.NQpad;
  Arena arena(ws, ws_bytes);
  float* opart = arena.take<float>(rows * D);
  float* mpart = arena.take<float>(rows);
  float* lpart = arena.take<float>(rows);
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(nparts, p.qtiles, B * Hkv);
  attn_split_mfma<128><<<grid, 256, 0, stream>>>(
      B, N, Hq, Hkv, scale_log2, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_tree),
      static_cast<const bf16_t*>(v_tree), static_cast<const bf16_t*>(k_pages), static_cast<const bf16_t*>(v_pages),
      n_pages, page_size, block_table, max_pages, prefix_len, anc, depth, Dmax, p.nsplit, p.lsplit, p.NQ, p.NQpad,
      opart, mpart, lpart);
  HY_LAUNCH_CHECK("tree_attention(split)");
  const long long cthreads = static_cast<long long>(B) * Hkv * p.NQ * (D / 4);
  attn_combine<bf16_t><<<static_cast<int>((cthreads + 255) / 256), 256, 0, stream>>>(B, N, Hq, Hkv, D, nparts, p.NQ, p.NQpad, opart, mpart,
                                                           lpart, static_cast<bf16_t*>(out), lse);
  HY_LAUNCH_CHECK("tree_attention(combine)");
  return HYDRA_OK;
}
