// Positions of the tree rows and their rotary embedding, before attention.
//
// "Speculative Decoding", section "Beyond draft models: Medusa": the
// candidates of one head stand at the same future position; "Hydra Guide:
// Sequentially-Dependent Speculative AI", section "Parallel Verification and
// Greedy Acceptance Algorithm": accepting a depth-k node advances to position
// t + k. So tree row u of sequence b sits at position prefix_len[b] +
// depth[b, u] (siblings share it), and each root-to-node branch reads as an
// ordinary sequence at consecutive positions. The rotation is the half-split
// layout of the LLaMA family: dimension i pairs with i + D/2 and turns by
// pos * theta^(-2i/D).
//
// The work is B * N * H * D/2 independent pairs: one thread per pair, angles
// and their sine and cosine in float64 (positions reach 10^4 and more, where
// a float32 angle loses three decimal digits), the rotation in float64 and
// one rounding to the storage type.
#include "common.h"

namespace hydra {
namespace {

template <typename T>
__device__ __forceinline__ double to_d(T v);
template <>
__device__ __forceinline__ double to_d<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ double to_d<bf16_t>(bf16_t v) {
  return bf16_to_f32(v);
}
template <typename T>
__device__ __forceinline__ T from_d(double v);
template <>
__device__ __forceinline__ float from_d<float>(double v) {
  return static_cast<float>(v);
}
template <>
__device__ __forceinline__ bf16_t from_d<bf16_t>(double v) {
  return f32_to_bf16(static_cast<float>(v));
}

template <typename T>
__device__ __forceinline__ void rope_pair(long long t, int N, int H, int D, const T* x, T* out,
                                          const int32_t* __restrict__ depth, const int32_t* __restrict__ prefix_len,
                                          double log_theta) {
  const int half = D / 2;
  const int i = static_cast<int>(t % half);
  const long long row = t / half;  // (b, u, h)
  const long long bu = row / H;
  const int b = static_cast<int>(bu / N);
  const double pos = static_cast<double>(prefix_len[b]) + static_cast<double>(depth[bu]);
  const double ang = pos * exp(-2.0 * i / D * log_theta);
  double s, c;
  sincos(ang, &s, &c);
  const size_t base = static_cast<size_t>(row) * D;
  const double a = to_d<T>(x[base + i]), v = to_d<T>(x[base + i + half]);
  out[base + i] = from_d<T>(a * c - v * s);
  out[base + i + half] = from_d<T>(v * c + a * s);
}

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(long long pairs, int N, int H, int D, const T* x,
                                                   T* out, const int32_t* __restrict__ depth,
                                                   const int32_t* __restrict__ prefix_len, double log_theta) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t < pairs) rope_pair<T>(t, N, H, D, x, out, depth, prefix_len, log_theta);
}

// Q and K of the tree rows in one launch: the first qpairs threads rotate Q
// (Hq heads), the rest K (Hkv heads), each exactly as rope_kernel does
template <typename T>
__global__ __launch_bounds__(256) void rope_qk_kernel(long long qpairs, long long pairs, int N, int Hq, int Hkv,
                                                      int D, const T* q, T* q_out, const T* k, T* k_out,
                                                      const int32_t* __restrict__ depth,
                                                      const int32_t* __restrict__ prefix_len, double log_theta) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t < qpairs)
    rope_pair<T>(t, N, Hq, D, q, q_out, depth, prefix_len, log_theta);
  else if (t < pairs)
    rope_pair<T>(t - qpairs, N, Hkv, D, k, k_out, depth, prefix_len, log_theta);
}

}  // namespace
}  // namespace hydra

extern "C" int tree_rope(int dtype, int B, int N, int H, int D, const void* x, void* out, const int32_t* depth,
                         const int32_t* prefix_len, float theta, void* stream) {
  using namespace hydra;
  clear_error();
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "tree_rope: bad dtype %d", dtype);
  HY_CHECK(B >= 0 && N >= 1 && H >= 1 && D >= 2 && D % 2 == 0, HYDRA_ERR_INVALID,
           "tree_rope: bad sizes B=%d N=%d H=%d D=%d (D even)", B, N, H, D);
  HY_CHECK(theta > 1.f, HYDRA_ERR_INVALID, "tree_rope: theta must be > 1 (got %g)", static_cast<double>(theta));
  if (B == 0) return HYDRA_OK;
  HY_CHECK(x && out && depth && prefix_len, HYDRA_ERR_INVALID, "tree_rope: null pointer");
  const long long pairs = static_cast<long long>(B) * N * H * (D / 2);
  const long long blocks = (pairs + 255) / 256;
  HY_CHECK(blocks <= 0x7fffffffll, HYDRA_ERR_UNSUPPORTED, "tree_rope: %lld pairs is too many", pairs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double lt = log(static_cast<double>(theta));
  if (dtype == HYDRA_F32)
    rope_kernel<float><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        pairs, N, H, D, static_cast<const float*>(x), static_cast<float*>(out), depth, prefix_len, lt);
  else
    rope_kernel<bf16_t><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        pairs, N, H, D, static_cast<const bf16_t*>(x), static_cast<bf16_t*>(out), depth, prefix_len, lt);
  HY_LAUNCH_CHECK("tree_rope");
  return HYDRA_OK;
}

extern "C" int tree_rope_qk(int dtype, int B, int N, int Hq, int Hkv, int D, const void* q, void* q_out,
                            const void* k, void* k_out, const int32_t* depth, const int32_t* prefix_len, float theta,
                            void* stream) {
  using namespace hydra;
  clear_error();
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "tree_rope_qk: bad dtype %d", dtype);
  HY_CHECK(B >= 0 && N >= 1 && Hq >= 1 && Hkv >= 1 && D >= 2 && D % 2 == 0, HYDRA_ERR_INVALID,
           "tree_rope_qk: bad sizes B=%d N=%d Hq=%d Hkv=%d D=%d (D even)", B, N, Hq, Hkv, D);
  HY_CHECK(theta > 1.f, HYDRA_ERR_INVALID, "tree_rope_qk: theta must be > 1 (got %g)", static_cast<double>(theta));
  if (B == 0) return HYDRA_OK;
  HY_CHECK(q && q_out && k && k_out && depth && prefix_len, HYDRA_ERR_INVALID, "tree_rope_qk: null pointer");
  const long long qpairs = static_cast<long long>(B) * N * Hq * (D / 2);
  const long long pairs = qpairs + static_cast<long long>(B) * N * Hkv * (D / 2);
  const long long blocks = (pairs + 255) / 256;
  HY_CHECK(blocks <= 0x7fffffffll, HYDRA_ERR_UNSUPPORTED, "tree_rope_qk: %lld pairs is too many", pairs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double lt = log(static_cast<double>(theta));
  if (dtype == HYDRA_F32)
    rope_qk_kernel<float><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        qpairs, pairs, N, Hq, Hkv, D, static_cast<const float*>(q), static_cast<float*>(q_out),
        static_cast<const float*>(k), static_cast<float*>(k_out), depth, prefix_len, lt);
  else
    rope_qk_kernel<bf16_t><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
        qpairs, pairs, N, Hq, Hkv, D, static_cast<const bf16_t*>(q), static_cast<bf16_t*>(q_out),
        static_cast<const bf16_t*>(k), static_cast<bf16_t*>(k_out), depth, prefix_len, lt);
  HY_LAUNCH_CHECK("tree_rope_qk");
  return HYDRA_OK;
}
