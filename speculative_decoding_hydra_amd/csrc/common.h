// Internal helpers shared by the libhydra HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <string>

#include "../../include/hydra.h"

namespace hydra {

// ---------------------------------------------------------------- errors

void set_error(const char* fmt, ...);
void clear_error();

#define HY_CHECK(cond, code, ...)            \
  do {                                       \
    if (!(cond)) {                           \
      ::hydra::set_error(__VA_ARGS__);       \
      return (code);                         \
    }                                        \
  } while (0)

#define HY_LAUNCH_CHECK(what)                                             \
  do {                                                                    \
    hipError_t e_ = hipGetLastError();                                    \
    if (e_ != hipSuccess) {                                               \
      ::hydra::set_error("%s: launch failed: %s", what, hipGetErrorString(e_)); \
      return HYDRA_ERR_HIP;                                               \
    }                                                                     \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bump allocator over a caller-provided workspace.
struct Arena {
  char* base;
  size_t cap, used;
  Arena(void* p, size_t n) : base(static_cast<char*>(p)), cap(n), used(0) {}
  template <class T>
  T* take(size_t count) {
    size_t off = align_up(used, 256);
    used = off + count * sizeof(T);
    return reinterpret_cast<T*>(base + off);
  }
  bool ok() const { return used <= cap; }
};

// ------------------------------------------------------------ bf16 bits

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <class T>
__device__ __forceinline__ float load_f(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<bf16_t>(const bf16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

template <class T>
__device__ __forceinline__ void store_f(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void store_f<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_f<bf16_t>(bf16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// Orderable key for (value descending, id ascending) selection: a larger key
// means a larger value, and for equal values a smaller id.
__device__ __forceinline__ uint64_t topk_key(float v, int id) {
  uint32_t b = __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(b) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(id));
}
__device__ __forceinline__ float key_value(uint64_t k) {
  uint32_t b = static_cast<uint32_t>(k >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}
__device__ __forceinline__ int key_id(uint64_t k) {
  return static_cast<int>(~static_cast<uint32_t>(k & 0xFFFFFFFFu));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ------------------------------------------------------- shared kernels

// Y[M, N] (float32) = X[M, K] . W[N, K]^T for the two dtypes; out row of
// X row m is (m / P) * S + O + m % P, split-K partials when nsplit > 1.
struct RowMap {
  int P, S, O;
  __device__ __forceinline__ int operator()(int m) const { return (m / P) * S + O + (m % P); }
};

// Source of the rows of X: contiguous, or the Hydra head input gathered on the
// fly as [h_b || E[token]] where b = m / P.
struct XSource {
  const void* x;        // contiguous [M, ldx] (mode 0) or h [B, d] (mode 1)
  int ldx;
  const void* emb;      // mode 1: [V, d]
  const int32_t* tok;   // mode 1: cand_tok [B, ntree]
  const int32_t* root_tok;  // mode 1: [B], the token of node 0
  const int32_t* row_node;  // mode 1: [R]; node whose token conditions row (b, r0 + m % P)
  int ntree, P, r0, d, V;
  int mode;
};

int launch_projection(int dtype, int M, int K, int N, XSource xs, const void* W,
                      float* Y, RowMap map, int ldy, int nsplit, float* part,
                      hipStream_t stream);

}  // namespace hydra
