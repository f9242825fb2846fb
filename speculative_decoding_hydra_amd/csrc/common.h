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
// 16-byte register vector; native vector types keep arrays of them in VGPRs
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

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

// ----------------------------------------------- DPP cross-lane reductions
// DPP moves are VALU instructions, so a reduction over G lanes costs
// log2(G) short dependent steps instead of LDS-routed shuffles. The patterns
// below combine lanes within groups of 2, 4, 8 and 16 (quad swaps, then the
// half-row and row mirrors); every lane of a group ends with the result.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane j <-> 7 - j within 8
constexpr int kDppMirror = 0x140;      // lane j <-> 15 - j within 16

// (every lane reads a valid source under these patterns, so the old value,
// 0 here, is never kept; 0 lets the compiler fuse the move into an integer max)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __uint_as_float(dpp32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = dpp32<CTRL>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp32<CTRL>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// max of a 32-bit word over aligned groups of G lanes (G in 1, 2, 4, 8, 16)
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (G >= 2) v = max(v, dpp32<kDppXor1>(v));
  if constexpr (G >= 4) v = max(v, dpp32<kDppXor2>(v));
  if constexpr (G >= 8) v = max(v, dpp32<kDppHalfMirror>(v));
  if constexpr (G >= 16) v = max(v, dpp32<kDppMirror>(v));
  return v;
}

// max of a key over aligned groups of G lanes: the value word first, then
// the id word among the lanes that hold that value (32-bit steps are single
// DPP-fused VALU operations; a 64-bit compare-and-select is several)
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32);
  const uint32_t mh = group_max_u32<G>(hi);
  const uint32_t ml = group_max_u32<G>(hi == mh ? static_cast<uint32_t>(v) : 0u);
  return (static_cast<uint64_t>(mh) << 32) | ml;
}

// (max, sum exp(x - max)) pairs combined over aligned groups of G lanes
__device__ __forceinline__ void ms_combine(float& m, float& s, float om, float os) {
  const float nm = fmaxf(m, om);
  s = (m == -INFINITY ? 0.f : s * expf(m - nm)) + (om == -INFINITY ? 0.f : os * expf(om - nm));
  m = nm;
}
template <int G>
__device__ __forceinline__ void group_ms(float& m, float& s) {
  if constexpr (G >= 2) ms_combine(m, s, dppf<kDppXor1>(m), dppf<kDppXor1>(s));
  if constexpr (G >= 4) ms_combine(m, s, dppf<kDppXor2>(m), dppf<kDppXor2>(s));
  if constexpr (G >= 8) ms_combine(m, s, dppf<kDppHalfMirror>(m), dppf<kDppHalfMirror>(s));
  if constexpr (G >= 16) ms_combine(m, s, dppf<kDppMirror>(m), dppf<kDppMirror>(s));
}

// (max, sum exp) over the whole wave, returned in every lane
__device__ __forceinline__ void wave_ms(float& m, float& s) {
  group_ms<16>(m, s);
  float rm = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(m), 0));
  float rs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s), 0));
#pragma unroll
  for (int row = 1; row < 4; ++row)
    ms_combine(rm, rs, __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(m), row * 16)),
               __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s), row * 16)));
  m = rm;
  s = rs;
}

// max of a 32-bit word over the whole wave, returned in every lane: rows of
// 16 by DPP, then the row pairs and the two halves by the gfx950 row-swap
// moves (VALU, no round trip through scalar registers)
__device__ __forceinline__ uint32_t max_swapped(uint32_t v, bool half32) {
  const auto a = half32 ? __builtin_amdgcn_permlane32_swap(v, v, false, false)
                        : __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(a[0], a[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return max_swapped(max_swapped(group_max_u32<16>(v), false), true);
}
// max of a key over the whole wave (value word, then id word), in every lane
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? static_cast<uint32_t>(v) : 0u);
  return (static_cast<uint64_t>(mh) << 32) | ml;
}

// Insert key x into a descending list of length K held in registers.
template <int K>
__device__ __forceinline__ void list_insert(uint64_t (&l)[K], uint64_t x) {
  if (x <= l[K - 1]) return;
#pragma unroll
  for (int j = K - 1; j > 0; --j) {
    const uint64_t prev = l[j - 1];
    l[j] = prev < x ? prev : (l[j] < x ? x : l[j]);
  }
  l[0] = l[0] < x ? x : l[0];
}

// Drop the head of a descending register list.
template <int K>
__device__ __forceinline__ void list_pop(uint64_t (&l)[K]) {
#pragma unroll
  for (int j = 0; j < K - 1; ++j) l[j] = l[j + 1];
  l[K - 1] = 0;
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
// Mode 2 (feed-forward kernel only): the embedding row E[token] alone.
struct XSource {
  const void* x;        // contiguous [M, ldx] (mode 0) or h [B, d] (mode 1)
  int ldx;
  const void* emb;      // modes 1, 2: [V, d]
  const int32_t* tok;   // modes 1, 2: cand_tok [B, ntree]
  const int32_t* root_tok;  // modes 1, 2: [B], the token of node 0
  const int32_t* row_node;  // modes 1, 2: [R]; node whose token conditions row (b, r0 + m % P)
  int ntree, P, r0, d, V;
  int mode;
};

// Optional fused row reduction of a projection: for every row and every
// 64-column block, the block's largest key (topk_key order) and (max, sum
// exp(z - max)) over its columns. keys == nullptr disables it.
struct TopkPartials {
  uint64_t* keys;  // [M][nwg]
  float2* ms;      // [M][nwg], or nullptr when no log-sum-exp is wanted
  int* clear;      // optional: the launch also zeroes clear[0 .. nclear) (nclear <= 256)
  int nclear;
};

// Packed weight layout (hydra_pack_weight): W [N][K] bf16 as 16-row tiles
// and 256-column chunks, chunk-major: chunk c of tile t is 8 KB at
// (c * ntiles + t) * 4096 elements; inside it, 32-column step s, then
// 8-column group g, then row r (16 bytes each), which is the operand order
// of v_mfma_f32_16x16x32_bf16 (lane 16 g + r holds row r, columns 8 g ..).
// Rows past N in the last tile are zeros. Element offset of the 16-byte
// piece holding row n, columns k .. k + 7 (k % 8 == 0):
constexpr int kPackChunk = 256;
__host__ __device__ inline size_t packed_piece(int n, int k, int N) {
  const size_t ntiles = static_cast<size_t>((N + 15) / 16);
  return ((static_cast<size_t>(k >> 8) * ntiles + (n >> 4)) * 8 + ((k & 255) >> 5)) * 512 +
         static_cast<size_t>(((k & 31) >> 3) * 16 + (n & 15)) * 8;
}

constexpr int kProjRowsPerWG = 64;
__host__ __device__ inline int projection_nwg(int N) { return (N + kProjRowsPerWG - 1) / kProjRowsPerWG; }

int launch_projection(int dtype, int M, int K, int N, XSource xs, const void* W, float* Y,
                      RowMap map, int ldy, int nsplit, float* part, TopkPartials tp,
                      hipStream_t stream);

// Tiled matrix-core projection for many contiguous rows (bf16, K % 64 == 0),
// same outputs and partials as launch_projection; row n of W starts at
// W + n * ldw, or ldw < 0: W is in the packed layout (K % 256 == 0).
bool gemm_supported(int K);
int launch_projection_gemm(int M, int K, int N, const bf16_t* X, int ldx, const bf16_t* W, int ldw, float* Y,
                           RowMap map, int ldy, TopkPartials tp, hipStream_t stream);
constexpr int kGemmMinRows = 65;  // from here on the tiled kernel beats the streaming one
// Split K for products with few output tiles: workgroups (blockIdx.y = s)
// take K range [s kper, min((s + 1) kper, K)) and write part + s * M * N
// (row-major [M][N]); kper % 64 == 0. The caller sums the nsplit partials.
int launch_projection_gemm_split(int M, int K, int N, const bf16_t* X, const bf16_t* W, int ldw, float* part, int nsplit,
                                 int kper, hipStream_t stream);
int gemm_workgroups(int M, int N);
// Y or its split-K partials for the decoder layer's products: picks the
// kernel by M and a split of K that gives the chip enough workgroups; writes
// nsplit partials part[s][M][N] (float32) and returns nsplit (>= 1).
int launch_projection_parts(int dtype, int M, int K, int N, const void* X, const void* W, float* part,
                            size_t part_floats, int* nsplit, hipStream_t stream);

// The decoder layer's gated feed-forward input g[m][j] = silu(gate) * up in
// one launch: W [2F][K] holds the gate rows, then the up rows (bf16, packed
// with HYDRA_LAYER_PACKED in dtype); X [M][K] contiguous; g_out [M][F] bf16.
// Same arithmetic as a product followed by the elementwise step.
bool projection_glu_supported(int dtype, int M, int K, int F);
int launch_projection_glu(int dtype, int M, int K, int F, const void* X, const void* W, bf16_t* g_out,
                          hipStream_t stream);

// Finish the fused row reduction: log-sum-exp and sorted top-k of each row,
// then either the candidate-tree fill (draft heads) or the arg max. The top-k
// is taken from the finished logits Y of the k blocks with the largest
// maxima (no key outside those blocks can rank among the first k).
struct MergeArgs {
  int M, nwg, k;
  const uint64_t* keys;
  const float2* ms;     // nullptr: no log-sum-exp (lse must be nullptr too)
  const float* Y;       // logits, row m at Y + map(m) * ldy, V columns
  int ldy, V;
  RowMap map;           // launch row -> output row (logits and head_lse)
  float* lse;           // [out rows] or nullptr
  int32_t* amax;        // [M] arg max or nullptr
  int32_t* topk_ids;    // [M][k] or nullptr
  float* topk_vals;     // [M][k] or nullptr
  // tree fill (draft heads); node_hi <= node_lo disables it
  int P, r0, N, node_lo, node_hi;
  const int32_t* node_parent;
  const int32_t* node_rank;
  const int32_t* node_row;
  const int32_t* root_tok;
  int32_t* cand_tok;
  float* cand_logp;
  // Hydra feed-forward rows of the next depth from the folded embedding
  // table: every filled child c with node_row[c] >= 0 gets
  //   u = h[b] + SiLU(Anext[b] + Enext[token of c])  (SiLU(...) alone without
  // the residual), stored as bf16 in U[b * Pn + node_row[c] - rn] and
  // hidden[b * R + node_row[c]]. Enext == nullptr disables it; needs d % 256 == 0.
  const float* Enext;   // [V][d]
  const float* Anext;   // [B][d], b1 included
  const bf16_t* h;      // [B][d]
  bf16_t* U;
  bf16_t* hidden;       // or nullptr
  int d, R, rn, Pn, residual;
  int ng;               // workgroups per row (set by the launcher)
  // greedy walk (k = 1, rows = B sequences x N tree rows, row i of sequence
  // i / N): the last row of a sequence to finish walks its tree from the arg
  // maxes. walk_count [B] must be zero when the launch starts (the projection
  // launch before it clears it).
  int* walk_count;      // nullptr disables it
  const int32_t* wtok;
  const int32_t* wparent;
  int wDmax;
  int32_t* n_accepted;
  int32_t* path;
  int32_t* out_tok;
};

// Feed-forward layer of the draft heads for few rows (bf16), for up to
// HYDRA_MAX_DEPTH heads at once (blockIdx.y selects the head), with b = m / P:
//   epi 0: A[y][m] = X_m . W[y]^T + b1[y]                  (float32)
//   epi 1: U[y][m] = h[b] + SiLU(X_m . W[y]^T + b1[y])      (bf16)
//   epi 2: U[m]    = h[b] + SiLU(X_m . W[0]^T + A[b])
//   epi 3: U[y][m] = h[b] + SiLU(X_m . W[y]^T + b1[y] + Ef[y][etok[b]])
// (without the residual, SiLU(...) alone); U rows are also written to
// hidden[map[y](m)] when hidden is set. W[y] points at the first used column
// of a [d, ldw] matrix and K columns are read.
struct MlpArgs {
  int M, K, d, ldw, heads;
  int wpacked;  // W[y] is a packed [d, K] matrix (hydra_pack_weight), ldw unused
  int epi[HYDRA_MAX_DEPTH];
  XSource xs;
  const bf16_t* W[HYDRA_MAX_DEPTH];
  const bf16_t* b1[HYDRA_MAX_DEPTH];
  const float* Ef[HYDRA_MAX_DEPTH];  // epi 3: folded embedding table [V][d]
  const int32_t* etok;               // epi 3: token of sequence b (clamped to [0, xs.V))
  float* A;
  const bf16_t* h;
  int P, residual;
  bf16_t* U;
  bf16_t* hidden;
  RowMap map[HYDRA_MAX_DEPTH];
};
bool mlp_fused_supported(int dtype, int M, int K, int d);
int launch_mlp_fused(const MlpArgs& a, hipStream_t stream);

// Row merge; with ffn (one head, epi 0, M <= 16 rows) the same launch also
// runs that feed-forward pass in extra workgroups.
bool merge_ffn_supported(int M, int K, int d);
int launch_topk_merge(const MergeArgs& a, hipStream_t stream, const MlpArgs* ffn = nullptr);

}  // namespace hydra
