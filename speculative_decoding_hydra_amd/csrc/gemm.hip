// Vocabulary projection for many rows: Y[m, n] = sum_k X[m, k] * W[n, k].
//
// With hundreds of rows (the target projection over every tree row of a
// 16-sequence batch: M = 1024, 268 GFLOP against 262 MB of W) the projection
// is bound by the matrix cores, not by HBM ("Parallel Verification and Greedy
// Acceptance Algorithm" in "Hydra Guide: Sequentially-Dependent Speculative
// AI": the target scores every tree row in one pass). From 65 rows on it also
// beats the streaming kernel. Design for gfx950:
//   * a workgroup computes a BN (n) x 256 (m) tile; its 8 waves hold
//     BN / 2 (n) x 64 (m) each in v_mfma_f32_16x16x32_bf16 accumulators, so
//     every operand read from LDS feeds 4 or BN / 32 MFMAs; BN = 256, or 128
//     when one m tile covers M (twice the workgroups for 65-256 rows);
//   * K advances in chunks of 64 held in NS LDS stages (two at BN = 256,
//     three at BN = 128), filled straight from global memory by DMA
//     (global_load_lds_dwordx4, no staging registers) NS - 1 chunks ahead;
//     one barrier per chunk; the operand reads are instructions the compiler
//     does not track, so it does not wait for the fills in flight before
//     them (measured at 1024 rows: 349-356 us against 355-369 us for the
//     same kernel staging through registers);
//   * workgroups are ordered so that the four m tiles of one n tile run on
//     the same XCD back to back and share that W tile in its L2;
//   * the epilogue writes Y and, per row and 64-column block, the largest key
//     and optionally (max, sum exp), the same partials as the streaming
//     projection leaves for the row merge.
#include <type_traits>

#include "common.h"

namespace hydra {
namespace {

constexpr int GBM = 256, GBK = 64;  // m tile and K chunk; the n tile BN is 256 or 128
// LDS rows are GBK bf16 (128 bytes) with the 16-byte chunk c of row r stored
// at position c ^ (r % 8): the MFMA operand reads (16 rows at one chunk per
// 16 lanes) then hit distinct banks, which padded rows do not achieve on gfx950
constexpr int GROW = GBK;
__device__ __forceinline__ int swz(int r, int c) { return r * GROW + ((c ^ (r & 7)) << 3); }
constexpr int GTHREADS = 512;

struct GemmArgs {
  int M, K, N, ldx, ldw, ldy, mtiles, ntiles;
  int kper;         // split K: workgroups with blockIdx.y = s take K range [s kper, (s + 1) kper)
  size_t ystride;   // ... and write Y + s * ystride
  const bf16_t* X;
  const bf16_t* W;
  float* Y;
  RowMap map;
  TopkPartials tp;
};

// combine a key over the four lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ uint64_t col_max_key(uint64_t v) {
  auto sw = [](uint64_t x, bool half32) {
    const uint32_t lo = static_cast<uint32_t>(x), hi = static_cast<uint32_t>(x >> 32);
    if (half32) {
      auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      const uint64_t p = (static_cast<uint64_t>(b[0]) << 32) | a[0];
      const uint64_t q = (static_cast<uint64_t>(b[1]) << 32) | a[1];
      return p > q ? p : q;
    }
    auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const uint64_t p = (static_cast<uint64_t>(b[0]) << 32) | a[0];
    const uint64_t q = (static_cast<uint64_t>(b[1]) << 32) | a[1];
    return p > q ? p : q;
  };
  return sw(sw(v, false), true);
}

__device__ __forceinline__ void col_ms(float& m, float& s) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  // (a[0], b[0]) and (a[1], b[1]) are this lane's pair and its partner's, in some order
  float m0 = __uint_as_float(a[0]), s0 = __uint_as_float(b[0]);
  ms_combine(m0, s0, __uint_as_float(a[1]), __uint_as_float(b[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m0), false, false);
  auto d = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s0), false, false);
  m = __uint_as_float(c[0]);
  s = __uint_as_float(d[0]);
  ms_combine(m, s, __uint_as_float(c[1]), __uint_as_float(d[1]));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16-byte LDS read issued as an instruction the compiler does not track: it
// would otherwise wait for every DMA fill still in flight (the chunks ahead)
// before the read. Its value is threaded through the s_waitcnt that follows
// (wait_lds), so nothing reads it earlier.
template <int OFF>
__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// 32-bit LDS address of a pointer into a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// f(integral_constant<int, I>) for I = I0 .. N - 1, unrolled
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// NS LDS stages of one K chunk each (W tile rows, then X tile rows), filled
// by DMA (global_load_lds_dwordx4) NS - 1 chunks ahead of use. (A 4-wave
// variant with 128 x 128 wave tiles and operand reads double-buffered across
// k steps took 435 us at 1024 rows: its accumulators fill the AGPRs and the
// compiler shuttles them through VGPRs inside the loop.)
template <int BN, int NS>
__global__ __launch_bounds__(GTHREADS, 1) void proj_gemm_kernel(GemmArgs a) {
  constexpr int WN = BN / 2;               // n columns per wave
  constexpr int NI = WN / 16;              // 16-column MFMA tiles per wave
  constexpr int ROWS = BN + GBM;           // LDS rows per stage (W, then X)
  constexpr int STAGE = ROWS * GROW;       // bf16 elements per stage
  constexpr int GROUPS = ROWS / 8 / 8;     // 8-row DMA groups per wave and chunk
  __shared__ __align__(16) bf16_t lds[NS * STAGE];
  // XCD-aware order: workgroup b runs on XCD b % 8; slot s = b / 8 there
  // covers m tile s % mtiles of n tile (s / mtiles) * 8 + b % 8
  const int bx = blockIdx.x;
  const int slot = bx >> 3;
  const int ntile = (slot / a.mtiles) * 8 + (bx & 7);
  const int mtile = slot % a.mtiles;
  if (ntile >= a.ntiles) return;  // whole workgroup: no barrier is pending
  const int n0 = ntile * BN, m0 = mtile * GBM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (a.tp.clear && bx == 0 && tid < a.tp.nclear) a.tp.clear[tid] = 0;
  const int kb = static_cast<int>(blockIdx.y) * a.kper;
  const int klen = a.K - kb < a.kper ? a.K - kb : a.kper;
  const int wn = wave & 1, wm = wave >> 1;  // 2 x 4 waves: WN n x 64 m each

  // DMA: lane l of a wave's 8-row group lands at row 8 g + l / 8, position l %
  // 8 of its row, which holds the row's 16-byte chunk (l % 8) ^ (row % 8)
  const int drow = lane >> 3, dchunk = (lane & 7) ^ drow;
  const bf16_t* src[GROUPS];
  int srow[GROUPS];
  bool isw[GROUPS];
#pragma unroll
  for (int j = 0; j < GROUPS; ++j) {
    const int r = 8 * (wave + 8 * j) + drow;  // stage row
    isw[j] = r < BN;
    if (r < BN) {
      const int n = n0 + r < a.N ? n0 + r : a.N - 1;  // rows past the end re-read the last row
      srow[j] = n;
      src[j] = a.ldw < 0 ? a.W : a.W + static_cast<size_t>(n) * a.ldw + kb + dchunk * 8;
    } else {
      const int m = m0 + r - BN < a.M ? m0 + r - BN : 0;
      srow[j] = m;
      src[j] = a.X + static_cast<size_t>(m) * a.ldx + kb + dchunk * 8;
    }
  }
  bf16_t* const lds0 = lds;
  auto issue = [&](int st, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < GROUPS; ++j) {
      const bf16_t* g = a.ldw < 0 && isw[j] ? src[j] + packed_piece(srow[j], kb + k0 + dchunk * 8, a.N) : src[j] + k0;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(g), (lds_void_t*)(lds0 + st * STAGE + (wave + 8 * j) * 8 * GROW),
                                       16, 0, 0);
    }
  };

  f32x4_t acc[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // operand rows differ by multiples of 16, so the swizzle depends on the
  // lane alone: k step s reads chunk 4 s + lane / 16 at position (4 s + lane
  // / 16) ^ (lane % 8)
  const int c0 = (lane >> 4) ^ (lane & 7);
  const uint32_t base = lds_addr(lds);
  const uint32_t arow0 = base + ((wn * WN + (lane & 15)) * GROW + c0 * 8) * 2;
  const uint32_t arow1 = base + ((wn * WN + (lane & 15)) * GROW + (c0 ^ 4) * 8) * 2;
  const uint32_t brow0 = base + ((BN + wm * 64 + (lane & 15)) * GROW + c0 * 8) * 2;
  const uint32_t brow1 = base + ((BN + wm * 64 + (lane & 15)) * GROW + (c0 ^ 4) * 8) * 2;

  const int nk = klen / GBK;
#pragma unroll
  for (int p = 0; p + 1 < NS; ++p)
    if (p < nk) issue(p, p * GBK);
  for (int c = 0; c < nk; ++c) {
    const int st = c % NS;
    // this wave's fills of chunk c have landed (those of the chunks after it
    // may still be in flight), then every wave's have and every wave is done
    // with chunk c - 1, whose stage takes chunk c + NS - 1
    if (c + NS - 2 < nk) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * GROUPS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("s_barrier" ::: "memory");
    if (c + NS - 1 < nk) issue((c + NS - 1) % NS, (c + NS - 1) * GBK);
    const uint32_t so = static_cast<uint32_t>(st * STAGE * 2);
    static_for<0, GBK / 32>([&](auto KS) __attribute__((always_inline)) {
      constexpr int ks = decltype(KS)::value;
      const uint32_t ab = (ks == 0 ? arow0 : arow1) + so, bb = (ks == 0 ? brow0 : brow1) + so;
      u32x4_t bv[4], av[NI];
      static_for<0, 4>([&](auto J) __attribute__((always_inline)) {
        bv[decltype(J)::value] = lds_read16<decltype(J)::value * 16 * GROW * 2>(bb);
      });
      static_for<0, NI>([&](auto I) __attribute__((always_inline)) {
        av[decltype(I)::value] = lds_read16<decltype(I)::value * 16 * GROW * 2>(ab);
      });
      if constexpr (NI == 8) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(bv[0]), "+v"(bv[1]), "+v"(bv[2]), "+v"(bv[3]), "+v"(av[0]), "+v"(av[1]), "+v"(av[2]),
                       "+v"(av[3]), "+v"(av[4]), "+v"(av[5]), "+v"(av[6]), "+v"(av[7]));
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(bv[0]), "+v"(bv[1]), "+v"(bv[2]), "+v"(bv[3]), "+v"(av[0]), "+v"(av[1]), "+v"(av[2]),
                       "+v"(av[3]));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[i]),
                                                              __builtin_bit_cast(bf16x8_t, bv[j]), acc[i][j], 0, 0, 0);
    });
  }

  // D[n][m]: lane holds n = 16 i + 4 (lane / 16) + e, m = 16 j + lane % 16 of the wave tile
  const int nb = n0 + wn * WN + (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 64 + j * 16 + (lane & 15);
    const bool mok = m < a.M;
    float* dst = a.Y + blockIdx.y * a.ystride + static_cast<size_t>(a.map(mok ? m : 0)) * a.ldy;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = nb + i * 16;
      if (!mok) continue;
      if (n + 3 < a.N && (a.ldy & 3) == 0) {
        *reinterpret_cast<float4*>(dst + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[n + e] = acc[i][j][e];
      }
    }
    if (!a.tp.keys) continue;
    // WN / 64 column blocks of 64 per wave: i = 4 bb .. 4 bb + 3
#pragma unroll
    for (int bb = 0; bb < WN / 64; ++bb) {
      float mx = -INFINITY;
      uint64_t best = 0;
#pragma unroll
      for (int i = 4 * bb; i < 4 * bb + 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = nb + i * 16 + e;
          const float v = n < a.N ? acc[i][j][e] : -INFINITY;
          mx = fmaxf(mx, v);
          const uint64_t key = n < a.N ? topk_key(v, n) : 0;
          best = key > best ? key : best;
        }
      best = col_max_key(best);
      const int col0 = n0 + wn * WN + bb * kProjRowsPerWG;
      const size_t slot_i = static_cast<size_t>(m) * projection_nwg(a.N) + col0 / kProjRowsPerWG;
      const bool writer = mok && (lane >> 4) == 0 && col0 < a.N;
      if (writer) a.tp.keys[slot_i] = best;
      if (a.tp.ms) {
        float s = 0.f;
#pragma unroll
        for (int i = 4 * bb; i < 4 * bb + 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = nb + i * 16 + e;
            if (n < a.N) s += expf(acc[i][j][e] - mx);
          }
        col_ms(mx, s);
        if (writer) a.tp.ms[slot_i] = make_float2(mx, s);
      }
    }
  }
}

}  // namespace

bool gemm_supported(int K) { return K % GBK == 0; }

int launch_projection_gemm(int M, int K, int N, const bf16_t* X, int ldx, const bf16_t* W, int ldw, float* Y,
                           RowMap map, int ldy, TopkPartials tp, hipStream_t stream) {
  GemmArgs a{};
  a.M = M;
  a.K = K;
  a.N = N;
  a.ldx = ldx;
  a.ldw = ldw;
  a.ldy = ldy;
  a.mtiles = (M + GBM - 1) / GBM;
  // one m tile: 128-column n tiles, so twice as many workgroups cover the chip
  const int bn = a.mtiles == 1 ? 128 : 256;
  a.ntiles = (N + bn - 1) / bn;
  a.X = X;
  a.W = W;
  a.Y = Y;
  a.map = map;
  a.tp = tp;
  a.kper = K;
  a.ystride = 0;
  const int slots = (a.ntiles + 7) / 8 * a.mtiles;  // per XCD
  if (bn == 128) proj_gemm_kernel<128, 3><<<slots * 8, GTHREADS, 0, stream>>>(a);
  else proj_gemm_kernel<256, 2><<<slots * 8, GTHREADS, 0, stream>>>(a);
  HY_LAUNCH_CHECK("projection(gemm)");
  return HYDRA_OK;
}

int launch_projection_gemm_split(int M, int K, int N, const bf16_t* X, const bf16_t* W, int ldw, float* part, int nsplit,
                                 int kper, hipStream_t stream) {
  GemmArgs a{};
  a.M = M;
  a.K = K;
  a.N = N;
  a.ldx = K;
  a.ldw = ldw;  // < 0: packed
  a.ldy = N;
  a.mtiles = (M + GBM - 1) / GBM;
  const int bn = a.mtiles == 1 ? 128 : 256;
  a.ntiles = (N + bn - 1) / bn;
  a.X = X;
  a.W = W;
  a.Y = part;
  a.map = RowMap{M, 0, 0};
  a.tp = TopkPartials{nullptr, nullptr};
  a.kper = kper;
  a.ystride = static_cast<size_t>(M) * N;
  const int slots = (a.ntiles + 7) / 8 * a.mtiles;
  const dim3 grid(slots * 8, nsplit);
  if (bn == 128) proj_gemm_kernel<128, 3><<<grid, GTHREADS, 0, stream>>>(a);
  else proj_gemm_kernel<256, 2><<<grid, GTHREADS, 0, stream>>>(a);
  HY_LAUNCH_CHECK("projection(gemm, split K)");
  return HYDRA_OK;
}

int gemm_workgroups(int M, int N) {
  const int mt = (M + GBM - 1) / GBM, bn = mt == 1 ? 128 : 256;
  return mt * ((N + bn - 1) / bn);
}

}  // namespace hydra
