// One decoder layer of the target over every tree row (the verification pass).
//
// "Speculative Decoding", section "Draft, then verify": the target scores
// all candidates in one forward pass; "Hydra Guide: Sequentially-Dependent
// Speculative AI", section "Tree Attention Matrix with Topology-Aware Causal
// Masking": each row sees the prefix and its own ancestors. The layer is the
// LLaMA pre-norm block of the pages' models (Vicuna, LLaMA-2):
//   a = rms(x) g1;  q, k, v = a Wq^T, a Wk^T, a Wv^T;  q, k rotated at L + depth;
//   o = tree attention;  x1 = x + o Wo^T;
//   b = rms(x1) g2;  x2 = x1 + (silu(b Wg^T) * (b Wu^T)) Wd^T.
//
// At decode shapes the rows are few (64 per sequence) and the layer streams
// its weights once (404 MB at the 7B shape), so every product is the
// bandwidth-bound projection kernel (one launch for Q, K and V together, one
// for the gate and up rows together); the elementwise and row-wise steps
// between them (norms, rotation, SwiGLU, residuals) are small kernels over
// M x d values. Activations are stored in the layer's dtype at the same
// points as the reference arithmetic: a, q, k, v (before and after the
// rotation), o, x1, b, the gated product and x2.
#include "common.h"

extern "C" size_t tree_attention_verify_workspace_size(int dtype, int B, int N, int Hq, int Hkv, int D,
                                                       int max_prefix_len);
extern "C" int tree_attention_verify(int dtype, int B, int N, int Hq, int Hkv, int D, float scale, const void* q,
                                     const void* k_tree, const void* v_tree, const void* k_pages,
                                     const void* v_pages, int n_pages, int page_size, const int32_t* block_table,
                                     int max_pages, const int32_t* prefix_len, int max_prefix_len,
                                     const int32_t* anc, const int32_t* depth, int Dmax, void* out, float* lse,
                                     void* ws, size_t ws_bytes, void* stream);

namespace hydra {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ T cv(float v);
template <>
__device__ __forceinline__ float cv<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ bf16_t cv<bf16_t>(float v) {
  return f32_to_bf16(v);
}

// v rounded to T and back
template <typename T>
__device__ __forceinline__ float rt(float v);
template <>
__device__ __forceinline__ float rt<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float rt<bf16_t>(float v) {
  return bf16_to_f32(f32_to_bf16(v));
}

// sum of the ns (at most 16) split-K partials of element i (stride floats
// apart), in split order; the bound is fixed so that every load is issued
// before the first add
__device__ __forceinline__ float psum(const float* __restrict__ p, int ns, size_t stride, size_t i) {
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
constexpr int kNormThreads = 256;

// One workgroup per row. With add: x1 = T(x + add) is stored first and
// normalised; without: x itself. out = T(x1 / sqrt(mean(x1^2) + eps) * g).
template <typename T>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_rows(int d, float eps, const T* __restrict__ x,
                                                             const float* __restrict__ add, int ns, size_t stride,
                                                             T* __restrict__ x1, const T* __restrict__ g,
                                                             T* __restrict__ out) {
  __shared__ float red[kNormThreads / 64];
  const size_t row = blockIdx.x;
  const T* xr = x + row * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += kNormThreads) {
    float v = ld<T>(xr, i);
    if (add) {
      v = rt<T>(v + psum(add, ns, stride, row * d + i));
      x1[row * d + i] = cv<T>(v);
    }
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
  const float inv = rsqrtf(tot / d + eps);
  for (int i = threadIdx.x; i < d; i += kNormThreads) {
    const float v = add ? ld<T>(x1, row * d + i) : ld<T>(xr, i);
    out[row * d + i] = cv<T>(v * inv * ld<T>(g, i));
  }
}

// bf16 rows with d % 8 == 0 and d <= 8 * kNormThreads * VPT, at most NSM
// partials: every thread keeps its (up to VPT) 8-value chunks in registers
// between the two passes, with 16-byte loads and stores, and issues all its
// loads (the row, then every partial) before the first sum, so the partials
// cost one memory round trip rather than one per split (the 7B round through
// 32 layers, two norms each over four partials: 4.70 -> 4.60 ms); same
// arithmetic, in the same order, as rmsnorm_rows
template <int VPT, int NSM>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_rows_bf16(int d, float eps, const bf16_t* __restrict__ x,
                                                                  const float* __restrict__ add, int ns,
                                                                  size_t stride, bf16_t* __restrict__ x1,
                                                                  const bf16_t* __restrict__ g,
                                                                  bf16_t* __restrict__ out) {
  __shared__ float red[kNormThreads / 64];
  const size_t row = blockIdx.x;
  const int nch = d / 8;
  float v[VPT][8];
  u32x4_t raw[VPT];
  float4 pa[VPT][NSM][2];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int c = threadIdx.x + j * kNormThreads;
    if (c >= nch) continue;
    raw[j] = *reinterpret_cast<const u32x4_t*>(x + row * d + c * 8);
    if (add) {
#pragma unroll
      for (int q = 0; q < NSM; ++q)
        if (q < ns) {
          pa[j][q][0] = *reinterpret_cast<const float4*>(add + q * stride + row * d + c * 8);
          pa[j][q][1] = *reinterpret_cast<const float4*>(add + q * stride + row * d + c * 8 + 4);
        }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int c = threadIdx.x + j * kNormThreads;
    if (c >= nch) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[j][2 * e] = bf16_to_f32(static_cast<bf16_t>(raw[j][e] & 0xffffu));
      v[j][2 * e + 1] = bf16_to_f32(static_cast<bf16_t>(raw[j][e] >> 16));
    }
    if (add) {
      float4 a0 = pa[j][0][0], a1 = pa[j][0][1];
#pragma unroll
      for (int q = 1; q < NSM; ++q)
        if (q < ns) {
          a0.x += pa[j][q][0].x;
          a0.y += pa[j][q][0].y;
          a0.z += pa[j][q][0].z;
          a0.w += pa[j][q][0].w;
          a1.x += pa[j][q][1].x;
          a1.y += pa[j][q][1].y;
          a1.z += pa[j][q][1].z;
          a1.w += pa[j][q][1].w;
        }
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      u32x4_t packed;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = rt<bf16_t>(v[j][e] + av[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        packed[e] = static_cast<uint32_t>(f32_to_bf16(v[j][2 * e])) |
                    (static_cast<uint32_t>(f32_to_bf16(v[j][2 * e + 1])) << 16);
      *reinterpret_cast<u32x4_t*>(x1 + row * d + c * 8) = packed;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
  const float inv = rsqrtf(tot / d + eps);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int c = threadIdx.x + j * kNormThreads;
    if (c >= nch) continue;
    const u32x4_t graw = *reinterpret_cast<const u32x4_t*>(g + c * 8);
    u32x4_t packed;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g0 = bf16_to_f32(static_cast<bf16_t>(graw[e] & 0xffffu));
      const float g1 = bf16_to_f32(static_cast<bf16_t>(graw[e] >> 16));
      packed[e] = static_cast<uint32_t>(f32_to_bf16(v[j][2 * e] * inv * g0)) |
                  (static_cast<uint32_t>(f32_to_bf16(v[j][2 * e + 1] * inv * g1)) << 16);
    }
    *reinterpret_cast<u32x4_t*>(out + row * d + c * 8) = packed;
  }
}

template <typename T>
void launch_norm(int M, int d, float eps, const T* x, const float* add, int ns, T* x1, const T* g, T* out,
                 hipStream_t stream) {
  const size_t stride = static_cast<size_t>(M) * d;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int nsa = add ? ns : 1;
    if (d % 8 == 0 && d <= 8 * kNormThreads * 2 && nsa <= 4) {
      rmsnorm_rows_bf16<2, 4><<<M, kNormThreads, 0, stream>>>(d, eps, x, add, ns, stride, x1, g, out);
      return;
    }
    if (d % 8 == 0 && d <= 8 * kNormThreads * 4 && nsa <= 4) {
      rmsnorm_rows_bf16<4, 4><<<M, kNormThreads, 0, stream>>>(d, eps, x, add, ns, stride, x1, g, out);
      return;
    }
    if (d % 8 == 0 && d <= 8 * kNormThreads * 4 && nsa <= 8) {
      rmsnorm_rows_bf16<4, 8><<<M, kNormThreads, 0, stream>>>(d, eps, x, add, ns, stride, x1, g, out);
      return;
    }
  }
  rmsnorm_rows<T><<<M, kNormThreads, 0, stream>>>(d, eps, x, add, ns, stride, x1, g, out);
}

// Q, K, V out of the fused projection [M][(Hq + 2 Hkv) D] (float32): each
// value rounded to T, Q and K rotated at prefix_len + depth (float64 angles)
// and rounded again. One thread per (row, head, pair).
template <typename T>
__global__ __launch_bounds__(256) void qkv_rope(long long pairs, int N, int Hq, int Hkv, int D, double log_theta,
                                                const float* __restrict__ qkv, int ns, size_t stride,
                                                const int32_t* __restrict__ depth,
                                                const int32_t* __restrict__ prefix_len, T* __restrict__ q,
                                                T* __restrict__ k, T* __restrict__ v) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= pairs) return;
  const int half = D / 2, H = Hq + 2 * Hkv;
  const int i = static_cast<int>(t % half);
  const long long rh = t / half;
  const int h = static_cast<int>(rh % H);
  const long long m = rh / H;  // row = b * N + u
  const size_t src = static_cast<size_t>(m) * H * D + static_cast<size_t>(h) * D;
  const double a = rt<T>(psum(qkv, ns, stride, src + i)), b = rt<T>(psum(qkv, ns, stride, src + i + half));
  if (h >= Hq + Hkv) {  // V: no rotation
    T* dst = v + (static_cast<size_t>(m) * Hkv + (h - Hq - Hkv)) * D;
    dst[i] = cv<T>(static_cast<float>(a));
    dst[i + half] = cv<T>(static_cast<float>(b));
    return;
  }
  const int bseq = static_cast<int>(m / N);
  const double pos = static_cast<double>(prefix_len[bseq]) + static_cast<double>(depth[m]);
  double s, c;
  sincos(pos * exp(-2.0 * i / D * log_theta), &s, &c);
  T* dst = h < Hq ? q + (static_cast<size_t>(m) * Hq + h) * D : k + (static_cast<size_t>(m) * Hkv + (h - Hq)) * D;
  dst[i] = cv<T>(static_cast<float>(a * c - b * s));
  dst[i + half] = cv<T>(static_cast<float>(b * c + a * s));
}

// g = T(silu(gate) * up) from the fused projection [M][2F] (gate columns first)
template <typename T>
__global__ __launch_bounds__(256) void swiglu_rows(long long n, int F, const float* __restrict__ gu, int ns,
                                                   size_t stride, T* __restrict__ g) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n) return;
  const long long m = t / F;
  const int j = static_cast<int>(t % F);
  const float gate = psum(gu, ns, stride, static_cast<size_t>(m) * 2 * F + j);
  const float up = psum(gu, ns, stride, static_cast<size_t>(m) * 2 * F + F + j);
  g[t] = cv<T>(gate / (1.0f + expf(-gate)) * up);
}

// out = T(x + add)
template <typename T>
__global__ __launch_bounds__(256) void residual_add(long long n, const T* __restrict__ x,
                                                    const float* __restrict__ add, int ns,
                                                    T* __restrict__ out) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t < n) out[t] = cv<T>(ld<T>(x, t) + psum(add, ns, static_cast<size_t>(n), t));
}

struct LayerWs {
  size_t a, acc, q, o, x1, g, attn, total;
};

LayerWs layer_ws(int dtype, int B, int N, int d, int Hq, int Hkv, int D, int F, int max_prefix_len) {
  LayerWs w{};
  const size_t M = static_cast<size_t>(B) * N, esz = dtype == HYDRA_F32 ? 4 : 2;
  // split-K partials: up to 8 for the d-wide products (few output tiles)
  const size_t accn = std::max({M * (Hq + 2 * Hkv) * D * 2, M * 2 * F * 2, 8 * M * static_cast<size_t>(d)});
  w.a = align_up(M * d * esz, 256);
  w.acc = align_up(accn * 4, 256);
  w.q = align_up(M * Hq * D * esz, 256);
  w.o = w.q;
  w.x1 = w.a;
  w.g = align_up(M * F * esz, 256);
  w.attn = align_up(tree_attention_verify_workspace_size(dtype, B, N, Hq, Hkv, D, max_prefix_len), 256);
  w.total = w.a + w.acc + w.q + w.o + w.x1 + w.g + w.attn + 256 * 8;
  return w;
}

// The layer's scratch, carved from its workspace in one fixed order (the
// forward pass reads x1 and acc of the layer before after it returns)
template <typename T>
struct LayerBufs {
  T* a;
  float* acc;
  T* q;
  T* o;
  T* x1;
  T* g;
  void* attn;
};

template <typename T>
LayerBufs<T> layer_bufs(const LayerWs& w, void* ws, size_t ws_bytes) {
  Arena arena(ws, ws_bytes);
  LayerBufs<T> b;
  b.a = arena.take<T>(w.a / sizeof(T));
  b.acc = arena.take<float>(w.acc / 4);
  b.q = arena.take<T>(w.q / sizeof(T));
  b.o = arena.take<T>(w.o / sizeof(T));
  b.x1 = arena.take<T>(w.x1 / sizeof(T));
  b.g = arena.take<T>(w.g / sizeof(T));
  b.attn = arena.take<char>(w.attn);
  return b;
}

// wflag: HYDRA_LAYER_PACKED when Wqkv, Wo, Wgu and Wd are packed.
// Chaining (the forward pass through several layers): with in_ns > 0 the
// layer's input is not materialised yet; it is x1 + the in_ns down-product
// partials of the layer before (both still in this workspace), and the first
// norm adds them, stores the sum to x_store and normalises it in one launch.
// With out_ns the layer leaves its own residual the same way (x1 and the
// partials in the workspace, their count in *out_ns) instead of writing x_out.
template <typename T>
int run_layer(int dtype, int wflag, int B, int N, int d, int Hq, int Hkv, int D, int F, const T* x, const T* ln1,
              const T* Wqkv, const T* Wo, const T* ln2, const T* Wgu, const T* Wd, float eps, float theta,
              const void* k_pages, const void* v_pages, int n_pages, int page_size, const int32_t* block_table,
              int max_pages, const int32_t* prefix_len, int max_prefix_len, const int32_t* anc,
              const int32_t* depth, int Dmax, T* x_out, T* k_tree, T* v_tree, void* ws, size_t ws_bytes,
              hipStream_t stream, int in_ns = 0, T* x_store = nullptr, int* out_ns = nullptr) {
  const LayerWs w = layer_ws(dtype, B, N, d, Hq, Hkv, D, F, max_prefix_len);
  const LayerBufs<T> buf = layer_bufs<T>(w, ws, ws_bytes);
  T* a = buf.a;
  float* acc = buf.acc;
  T* q = buf.q;
  T* o = buf.o;
  T* x1 = buf.x1;
  T* g = buf.g;
  const int M = B * N;
  int ns = 1;  // split-K partials of the last product
  auto proj = [&](int K, int Nout, const T* X, const T* W) {
    return launch_projection_parts(dtype | wflag, M, K, Nout, X, W, acc, w.acc / 4, &ns, stream);
  };
  auto blocks = [](long long n) { return static_cast<unsigned>((n + 255) / 256); };
  // a = rms(x) g1 (chained: x = x1 + partials of the layer before, stored first)
  const T* xin = x;
  if (in_ns > 0) {
    launch_norm<T>(M, d, eps, x1, acc, in_ns, x_store, ln1, a, stream);
    xin = x_store;
  } else {
    launch_norm<T>(M, d, eps, x, nullptr, 1, nullptr, ln1, a, stream);
  }
  HY_LAUNCH_CHECK("decoder layer: norm 1");
  // q, k, v (one product), rotated
  int rc = proj(d, (Hq + 2 * Hkv) * D, a, Wqkv);
  if (rc != HYDRA_OK) return rc;
  const long long pairs = static_cast<long long>(M) * (Hq + 2 * Hkv) * (D / 2);
  qkv_rope<T><<<blocks(pairs), 256, 0, stream>>>(pairs, N, Hq, Hkv, D, log(static_cast<double>(theta)), acc, ns,
                                                  static_cast<size_t>(M) * (Hq + 2 * Hkv) * D, depth, prefix_len, q,
                                                  k_tree, v_tree);
  HY_LAUNCH_CHECK("decoder layer: q/k/v");
  rc = tree_attention_verify(dtype, B, N, Hq, Hkv, D, 1.0f / sqrtf(static_cast<float>(D)), q, k_tree, v_tree,
                             k_pages, v_pages, n_pages, page_size, block_table, max_pages, prefix_len,
                             max_prefix_len, anc, depth, Dmax, o, nullptr, buf.attn, w.attn, stream);
  if (rc != HYDRA_OK) return rc;
  // x1 = x + o Wo^T;  b = rms(x1) g2 (into a)
  rc = proj(Hq * D, d, o, Wo);
  if (rc != HYDRA_OK) return rc;
  launch_norm<T>(M, d, eps, xin, acc, ns, x1, ln2, a, stream);
  HY_LAUNCH_CHECK("decoder layer: norm 2");
  // g = silu(b Wg^T) * (b Wu^T): one gated launch (bf16, up to 64 rows), else
  // the product's partials and an elementwise pass;  x2 = x1 + g Wd^T
  if (projection_glu_supported(dtype | wflag, M, d, F)) {
    rc = launch_projection_glu(dtype | wflag, M, d, F, a, Wgu, reinterpret_cast<bf16_t*>(g), stream);
    if (rc != HYDRA_OK) return rc;
  } else {
    rc = proj(d, 2 * F, a, Wgu);
    if (rc != HYDRA_OK) return rc;
    const long long gn = static_cast<long long>(M) * F;
    swiglu_rows<T><<<blocks(gn), 256, 0, stream>>>(gn, F, acc, ns, static_cast<size_t>(M) * 2 * F, g);
    HY_LAUNCH_CHECK("decoder layer: swiglu");
  }
  rc = proj(F, d, g, Wd);
  if (rc != HYDRA_OK) return rc;
  if (out_ns) {
    *out_ns = ns;  // the next norm adds x1 and these partials
    return HYDRA_OK;
  }
  const long long xn = static_cast<long long>(M) * d;
  residual_add<T><<<blocks(xn), 256, 0, stream>>>(xn, x1, acc, ns, x_out);
  HY_LAUNCH_CHECK("decoder layer: residual");
  return HYDRA_OK;
}

// out[r] = emb[tok[r]]: the tree rows' input to the first layer; a token
// outside [0, V) gives a row of zeros. 16-byte copies when d allows.
template <typename T>
__global__ __launch_bounds__(256) void embed_rows(int d, int V, const int32_t* __restrict__ tok,
                                                  const T* __restrict__ emb, T* __restrict__ out) {
  const size_t row = blockIdx.x;
  const int t = tok[row];
  const bool ok = t >= 0 && t < V;
  const T* src = emb + static_cast<size_t>(ok ? t : 0) * d;
  T* dst = out + row * d;
  constexpr int per = 16 / sizeof(T);
  if (d % per == 0) {
    for (int c = threadIdx.x; c < d / per; c += 256) {
      const u32x4_t v = ok ? *reinterpret_cast<const u32x4_t*>(src + c * per) : u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(dst + c * per) = v;
    }
  } else {
    for (int i = threadIdx.x; i < d; i += 256) dst[i] = ok ? src[i] : cv<T>(0.f);
  }
}

struct VerifyWs {
  LayerWs layer;
  size_t x, total;
};

VerifyWs verify_ws(int dtype, int B, int N, int d, int Hq, int Hkv, int D, int F, int max_prefix_len) {
  VerifyWs w{};
  w.layer = layer_ws(dtype, B, N, d, Hq, Hkv, D, F, max_prefix_len);
  w.x = align_up(static_cast<size_t>(B) * N * d * (dtype == HYDRA_F32 ? 4 : 2), 256);
  w.total = w.layer.total + 2 * w.x + 256;
  return w;
}

// embeddings -> n_layers decoder layers (layer-stacked weights, pools and
// tree K/V) -> final norm; the hidden states ping-pong between two buffers
template <typename T>
int run_verify(int dtype, int wflag, int n_layers, int B, int N, int d, int Hq, int Hkv, int D, int F, int V,
               const int32_t* tok, const T* emb, const T* ln1, const T* Wqkv, const T* Wo, const T* ln2,
               const T* Wgu, const T* Wd, const T* ln_f, float eps, float theta, const T* k_pages,
               const T* v_pages, int n_pages, int page_size, const int32_t* block_table, int max_pages,
               const int32_t* prefix_len, int max_prefix_len, const int32_t* anc, const int32_t* depth, int Dmax,
               T* h_out, T* k_tree, T* v_tree, void* ws, size_t ws_bytes, hipStream_t stream) {
  const VerifyWs w = verify_ws(dtype, B, N, d, Hq, Hkv, D, F, max_prefix_len);
  Arena arena(ws, ws_bytes);
  T* cur = arena.take<T>(w.x / sizeof(T));
  T* nxt = arena.take<T>(w.x / sizeof(T));
  void* lws = arena.take<char>(w.layer.total);
  const size_t M = static_cast<size_t>(B) * N;
  embed_rows<T><<<static_cast<unsigned>(M), 256, 0, stream>>>(d, V, tok, emb, cur);
  HY_LAUNCH_CHECK("verify layers: embeddings");
  const size_t sqkv = static_cast<size_t>(Hq + 2 * Hkv) * D * d, so = static_cast<size_t>(d) * Hq * D;
  const size_t sgu = 2 * static_cast<size_t>(F) * d, sd = static_cast<size_t>(d) * F;
  const size_t skv = M * Hkv * D, spool = static_cast<size_t>(n_pages) * Hkv * page_size * D;
  // each layer leaves its residual in the workspace (x1 + down partials);
  // the next layer's first norm, and at the end the final norm, adds it and
  // stores the sum, so no launch of its own materialises a layer's output
  int ns = 0;
  for (int l = 0; l < n_layers; ++l) {
    const int rc = run_layer<T>(dtype, wflag, B, N, d, Hq, Hkv, D, F, cur, ln1 + l * static_cast<size_t>(d),
                                Wqkv + l * sqkv, Wo + l * so, ln2 + l * static_cast<size_t>(d), Wgu + l * sgu,
                                Wd + l * sd, eps, theta, k_pages + l * spool, v_pages + l * spool, n_pages,
                                page_size, block_table, max_pages, prefix_len, max_prefix_len, anc, depth, Dmax,
                                nullptr, k_tree + l * skv, v_tree + l * skv, lws, w.layer.total, stream, ns, cur,
                                &ns);
    if (rc != HYDRA_OK) return rc;
  }
  const LayerBufs<T> lb = layer_bufs<T>(w.layer, lws, w.layer.total);
  launch_norm<T>(static_cast<int>(M), d, eps, lb.x1, lb.acc, ns, nxt, ln_f, h_out, stream);
  HY_LAUNCH_CHECK("verify layers: final norm");
  return HYDRA_OK;
}

}  // namespace
}  // namespace hydra

extern "C" size_t tree_decoder_layer_workspace_size(int dtype, int B, int N, int d, int Hq, int Hkv, int D, int F,
                                                    int max_prefix_len) {
  if (B <= 0 || N <= 0 || d <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || F <= 0) return 0;
  return hydra::layer_ws(dtype & ~HYDRA_LAYER_PACKED, B, N, d, Hq, Hkv, D, F, max_prefix_len).total;
}

extern "C" int tree_decoder_layer(int dtype, int B, int N, int d, int Hq, int Hkv, int D, int F, const void* x,
                                  const void* ln1, const void* Wqkv, const void* Wo, const void* ln2,
                                  const void* Wgu, const void* Wd, float eps, float theta, const void* k_pages,
                                  const void* v_pages, int n_pages, int page_size, const int32_t* block_table,
                                  int max_pages, const int32_t* prefix_len, int max_prefix_len, const int32_t* anc,
                                  const int32_t* depth, int Dmax, void* x_out, void* k_tree, void* v_tree, void* ws,
                                  size_t ws_bytes, void* stream_) {
  using namespace hydra;
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int wflag = dtype & HYDRA_LAYER_PACKED;  // packed layer weights (hydra_pack_weight)
  dtype &= ~HYDRA_LAYER_PACKED;
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "decoder_layer: bad dtype %d", dtype);
  HY_CHECK(!wflag || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "decoder_layer: packed weights are bf16");
  HY_CHECK(B >= 0 && N >= 1 && d >= 1 && Hq >= 1 && Hkv >= 1 && D >= 2 && D % 2 == 0 && F >= 1 && Hq % Hkv == 0,
           HYDRA_ERR_INVALID, "decoder_layer: bad sizes B=%d N=%d d=%d Hq=%d Hkv=%d D=%d F=%d", B, N, d, Hq, Hkv, D,
           F);
  HY_CHECK(eps > 0.f && theta > 1.f, HYDRA_ERR_INVALID, "decoder_layer: eps must be > 0 and theta > 1");
  if (B == 0) return HYDRA_OK;
  HY_CHECK(x && ln1 && Wqkv && Wo && ln2 && Wgu && Wd && k_pages && v_pages && block_table && prefix_len && anc &&
               depth && x_out && k_tree && v_tree,
           HYDRA_ERR_INVALID, "decoder_layer: null pointer");
  HY_CHECK(x_out != x, HYDRA_ERR_INVALID, "decoder_layer: x_out must not alias x");
  HY_CHECK(dtype == HYDRA_F32 || (d % 256 == 0 && (Hq * D) % 256 == 0 && F % 256 == 0), HYDRA_ERR_UNSUPPORTED,
           "decoder_layer: bf16 needs d, Hq*D and F multiples of 256 (d=%d Hq*D=%d F=%d)", d, Hq * D, F);
  const size_t need = tree_decoder_layer_workspace_size(dtype, B, N, d, Hq, Hkv, D, F, max_prefix_len);
  HY_CHECK(ws && ws_bytes >= need, HYDRA_ERR_WORKSPACE, "decoder_layer: workspace %zu < %zu", ws_bytes, need);
  if (dtype == HYDRA_F32)
    return run_layer<float>(dtype, wflag, B, N, d, Hq, Hkv, D, F, static_cast<const float*>(x),
                            static_cast<const float*>(ln1), static_cast<const float*>(Wqkv),
                            static_cast<const float*>(Wo), static_cast<const float*>(ln2),
                            static_cast<const float*>(Wgu), static_cast<const float*>(Wd), eps, theta, k_pages,
                            v_pages, n_pages, page_size, block_table, max_pages, prefix_len, max_prefix_len, anc,
                            depth, Dmax, static_cast<float*>(x_out), static_cast<float*>(k_tree),
                            static_cast<float*>(v_tree), ws, ws_bytes, stream);
  return run_layer<bf16_t>(dtype, wflag, B, N, d, Hq, Hkv, D, F, static_cast<const bf16_t*>(x),
                           static_cast<const bf16_t*>(ln1), static_cast<const bf16_t*>(Wqkv),
                           static_cast<const bf16_t*>(Wo), static_cast<const bf16_t*>(ln2),
                           static_cast<const bf16_t*>(Wgu), static_cast<const bf16_t*>(Wd), eps, theta, k_pages,
                           v_pages, n_pages, page_size, block_table, max_pages, prefix_len, max_prefix_len, anc,
                           depth, Dmax, static_cast<bf16_t*>(x_out), static_cast<bf16_t*>(k_tree),
                           static_cast<bf16_t*>(v_tree), ws, ws_bytes, stream);
}

extern "C" size_t tree_verify_layers_workspace_size(int dtype, int B, int N, int d, int Hq, int Hkv, int D, int F,
                                                    int max_prefix_len) {
  if (B <= 0 || N <= 0 || d <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || F <= 0) return 0;
  return hydra::verify_ws(dtype & ~HYDRA_LAYER_PACKED, B, N, d, Hq, Hkv, D, F, max_prefix_len).total;
}

extern "C" int tree_verify_layers(int dtype, int n_layers, int B, int N, int d, int Hq, int Hkv, int D, int F, int V,
                                  const int32_t* tok, const void* emb, const void* ln1, const void* Wqkv,
                                  const void* Wo, const void* ln2, const void* Wgu, const void* Wd,
                                  const void* ln_f, float eps, float theta, const void* k_pages,
                                  const void* v_pages, int n_pages, int page_size, const int32_t* block_table,
                                  int max_pages, const int32_t* prefix_len, int max_prefix_len, const int32_t* anc,
                                  const int32_t* depth, int Dmax, void* h_out, void* k_tree, void* v_tree, void* ws,
                                  size_t ws_bytes, void* stream_) {
  using namespace hydra;
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int wflag = dtype & HYDRA_LAYER_PACKED;  // packed layer weights (hydra_pack_weight, layer by layer)
  dtype &= ~HYDRA_LAYER_PACKED;
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "verify_layers: bad dtype %d", dtype);
  HY_CHECK(!wflag || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "verify_layers: packed weights are bf16");
  HY_CHECK(n_layers >= 1 && B >= 0 && N >= 1 && d >= 1 && Hq >= 1 && Hkv >= 1 && D >= 2 && D % 2 == 0 && F >= 1 &&
               Hq % Hkv == 0 && V >= 1,
           HYDRA_ERR_INVALID, "verify_layers: bad sizes layers=%d B=%d N=%d d=%d Hq=%d Hkv=%d D=%d F=%d V=%d",
           n_layers, B, N, d, Hq, Hkv, D, F, V);
  HY_CHECK(eps > 0.f && theta > 1.f, HYDRA_ERR_INVALID, "verify_layers: eps must be > 0 and theta > 1");
  if (B == 0) return HYDRA_OK;
  HY_CHECK(tok && emb && ln1 && Wqkv && Wo && ln2 && Wgu && Wd && ln_f && k_pages && v_pages && block_table &&
               prefix_len && anc && depth && h_out && k_tree && v_tree,
           HYDRA_ERR_INVALID, "verify_layers: null pointer");
  HY_CHECK(dtype == HYDRA_F32 || (d % 256 == 0 && (Hq * D) % 256 == 0 && F % 256 == 0), HYDRA_ERR_UNSUPPORTED,
           "verify_layers: bf16 needs d, Hq*D and F multiples of 256 (d=%d Hq*D=%d F=%d)", d, Hq * D, F);
  const size_t need = tree_verify_layers_workspace_size(dtype, B, N, d, Hq, Hkv, D, F, max_prefix_len);
  HY_CHECK(ws && ws_bytes >= need, HYDRA_ERR_WORKSPACE, "verify_layers: workspace %zu < %zu", ws_bytes, need);
  if (dtype == HYDRA_F32)
    return run_verify<float>(
        dtype, wflag, n_layers, B, N, d, Hq, Hkv, D, F, V, tok, static_cast<const float*>(emb),
        static_cast<const float*>(ln1), static_cast<const float*>(Wqkv), static_cast<const float*>(Wo),
        static_cast<const float*>(ln2), static_cast<const float*>(Wgu), static_cast<const float*>(Wd),
        static_cast<const float*>(ln_f), eps, theta, static_cast<const float*>(k_pages),
        static_cast<const float*>(v_pages), n_pages, page_size, block_table, max_pages, prefix_len, max_prefix_len,
        anc, depth, Dmax, static_cast<float*>(h_out), static_cast<float*>(k_tree), static_cast<float*>(v_tree), ws,
        ws_bytes, stream);
  return run_verify<bf16_t>(
      dtype, wflag, n_layers, B, N, d, Hq, Hkv, D, F, V, tok, static_cast<const bf16_t*>(emb),
      static_cast<const bf16_t*>(ln1), static_cast<const bf16_t*>(Wqkv), static_cast<const bf16_t*>(Wo),
      static_cast<const bf16_t*>(ln2), static_cast<const bf16_t*>(Wgu), static_cast<const bf16_t*>(Wd),
      static_cast<const bf16_t*>(ln_f), eps, theta, static_cast<const bf16_t*>(k_pages),
      static_cast<const bf16_t*>(v_pages), n_pages, page_size, block_table, max_pages, prefix_len, max_prefix_len, anc,
      depth, Dmax, static_cast<bf16_t*>(h_out), static_cast<bf16_t*>(k_tree), static_cast<bf16_t*>(v_tree), ws,
      ws_bytes, stream);
}
