// Vocabulary / MLP projections: Y[m, n] = sum_k X[m, k] * W[n, k].
//
// These are the draft heads' two layers ("Medusa Heads", section "So sagen die
// Köpfe voraus": a feed-forward layer then a vocabulary projection; "Hydra
// Guide", section "1. Embedding Conditioning Mechanics": the Hydra layer reads
// [h || e(x_parent)]) and the target vocabulary projection of the verify pass.
//
// At decode shapes M (tree rows) is 1..256 while W is 67-524 MB, so the kernel
// is bound by streaming W from HBM. Design for gfx950:
//   * each wave owns 16 rows of W and streams them with 16-byte loads straight
//     into registers (the MFMA A operand), PF K-chunks ahead of use, so every
//     wave keeps 16 KB of W in flight;
//   * the matching chunk of X (all M rows, padded to 16 * MT) is staged once
//     per workgroup in LDS and read as the B operand;
//   * v_mfma_f32_16x16x32_bf16 does the contraction with float32 accumulation;
//   * split-K over grid.y gives enough workgroups when N is small (W1: N = d);
//   * optional fused epilogue: per row and workgroup, the top-k of the
//     workgroup's 64 columns and (max, sum exp) over them, so the vocabulary
//     reductions need no second pass over the logits.
#include <type_traits>

#include "common.h"

namespace hydra {

namespace {

struct ProjArgs {
  int M, K, N;
  XSource xs;
  const bf16_t* W;
  float* Y;
  RowMap map;
  int ldy, kper, m_base;
  float* part;
  TopkPartials tp;
  int wpacked;  // W in the packed layout (packed_piece) rather than row-major [N][K]
  // gated product (glu_F > 0; bf16, WV = 2 G waves, no split, no top-k): W
  // holds gate rows [0, F) then up rows [F, 2F); workgroup b streams gate
  // rows 16 G b .. 16 G b + 16 G - 1 (waves 0 .. G - 1) and the same up rows
  // (waves G .. 2 G - 1) and writes glu_out[m][j] = bf16(silu(gate) * up)
  // instead of Y
  int glu_F;
  bf16_t* glu_out;
};

// REM: the K range need not be a multiple of PF * KC (a multiple of KC is
// enough); the chunks past its end are skipped and their loads clamped
template <int MT, int KC, int PF, int WV, bool SPLIT, bool TOPK, bool REM = false>
__global__ __launch_bounds__(64 * WV) void proj_bf16_kernel(ProjArgs a) {
  constexpr int NT = 64 * WV;      // threads
  constexpr int RPW = 16 * WV;     // rows of W per workgroup (one 16-row tile per wave)
  constexpr int MP = MT * 16;
  constexpr int LDS_ROW = KC + 8;  // 16-byte pad: rows land on different banks
  constexpr int STEPS = KC / 32;
  constexpr int VPR = KC / 8;      // 16-byte vectors per LDS row
  constexpr int XV = (MP * VPR + NT - 1) / NT;  // X vectors per thread and chunk
  constexpr bool XG = (MP * VPR) % NT != 0;      // ... the last one only for some threads
  constexpr int TROW = RPW + 1;    // epilogue tile row (floats)
  constexpr int XLDS = (TOPK && TROW * 2 > LDS_ROW) ? MP * TROW * 2 : MP * LDS_ROW;  // bf16 elements
  static_assert(!TOPK || RPW % kProjRowsPerWG == 0, "partials come in 64-column blocks");
  __shared__ __align__(16) bf16_t xlds[XLDS];

  const XSource& xs = a.xs;
  const int M = a.M, K = a.K, N = a.N, m_base = a.m_base;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // this wave's 16 rows of W; a wave whose rows lie past the end (the last
  // workgroup of a launch whose row count is no multiple of RPW) streams the
  // last tile again and stores nothing
  constexpr int G = WV / 2;  // gated product: gate (and up) row groups per workgroup
  int n_base;
  bool idle;
  if (a.glu_F > 0) {
    const int col = 16 * G * static_cast<int>(blockIdx.x) + 16 * (wave < G ? wave : wave - G);
    idle = col >= a.glu_F;
    const int c = idle ? a.glu_F - 16 : col;
    n_base = wave < G ? c : a.glu_F + c;
  } else {
    n_base = static_cast<int>(blockIdx.x) * RPW + wave * 16;
    idle = n_base >= N;
    if (idle) n_base = (N - 1) / 16 * 16;
  }
  int k_begin, k_end;
  if (a.kper > 0) {
    k_begin = blockIdx.y * a.kper;
    k_end = REM && k_begin + a.kper > a.K ? a.K : k_begin + a.kper;  // REM: the last split may be short
  } else {  // balanced: -kper splits of whole chunks, sizes differing by at most one chunk
    const int nsp = -a.kper, nch = a.K / KC;
    k_begin = static_cast<int>(static_cast<long>(blockIdx.y) * nch / nsp) * KC;
    k_end = static_cast<int>(static_cast<long>(blockIdx.y + 1) * nch / nsp) * KC;
  }
  const int K0 = xs.mode == 0 ? K : xs.d;
  if (TOPK && a.tp.clear && blockIdx.x == 0 && blockIdx.y == 0 && tid < a.tp.nclear) a.tp.clear[tid] = 0;

  // this lane's 16 bytes of W at column k (a multiple of 32) lie at
  // wp + (k / 256) * wcs + (k % 256 / 32) * wss: row-major, wp is the row
  // (rows past N re-read row N - 1) and the strides are 256 and 32 columns;
  // packed, wp is the lane's piece in the first 256-column chunk of its tile
  // (tile rows past N are zeros) and the strides are a chunk of all tiles and
  // one 1 KB step
  // packed weights reach this kernel with at most 64 rows (from 65 rows on,
  // contiguous X goes to the tiled kernel), so larger tiles leave it out
  const bool packed = MT <= 4 && a.wpacked != 0;
  const bf16_t* wp = packed ? a.W + static_cast<size_t>(n_base / 16) * kPackChunk * 16 + lane * 8
                            : a.W + static_cast<size_t>(min(n_base + (lane & 15), N - 1)) * K + (lane >> 4) * 8;
  const size_t wcs = packed ? static_cast<size_t>((N + 15) / 16) * kPackChunk * 16 : kPackChunk;
  const int wss = packed ? 512 : 32;
  auto wat = [wp, wcs, wss](int k) { return wp + (static_cast<size_t>(k >> 8) * wcs + ((k & 255) >> 5) * wss); };

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t wbuf[PF][STEPS];
  u32x4_t xbuf[XV];
  // This thread's X rows, fixed for the whole K range. Pointers come straight
  // from the kernel arguments (global address space); rows past M read row 0,
  // whose outputs are never stored, so every load below is unconditional.
  const bf16_t* xp0[XV];
  const bf16_t* xp1[XV];
  int xo[XV];
#pragma unroll
  for (int v = 0; v < XV; ++v) {
    const int idx = XG && tid + v * NT >= MP * VPR ? tid : tid + v * NT;  // (unused past the chunk)
    const int r = idx / VPR;
    const int c = (idx % VPR) * 8;
    xo[v] = r * LDS_ROW + c;
    const int m = m_base + r < M ? m_base + r : 0;
    if (xs.mode == 0) {
      xp0[v] = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(m) * xs.ldx + c;
      xp1[v] = xp0[v];
    } else {
      const int b = m / xs.P;
      const int node = xs.row_node[xs.r0 + m % xs.P];
      int t = node == 0 ? xs.root_tok[b] : xs.tok[static_cast<size_t>(b) * xs.ntree + node];
      t = t < 0 ? 0 : (t >= xs.V ? xs.V - 1 : t);
      xp0[v] = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(b) * xs.d + c;
      xp1[v] = static_cast<const bf16_t*>(xs.emb) + static_cast<size_t>(t) * xs.d - xs.d + c;
    }
  }

  // prologue: PF chunks of W in flight, the first X chunk in registers. W
  // is read once per launch: its loads are nontemporal (streamed past the
  // caches), about 9% more bandwidth than plain loads on this layout.
  // (the launcher guarantees PF * KC divides the K range of the workgroup,
  // or REM)
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int kp = REM && k_begin + p * KC > k_end - KC ? k_end - KC : k_begin + p * KC;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) wbuf[p][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wat(kp + s * 32)));
  }
  const bool xlast = !XG || tid + (XV - 1) * NT < MP * VPR;  // this thread stages an X vector in slot XV - 1
#pragma unroll
  for (int v = 0; v < XV; ++v)
    if (v + 1 < XV || xlast) xbuf[v] = *reinterpret_cast<const u32x4_t*>((k_begin < K0 ? xp0[v] : xp1[v]) + k_begin);

  const int k_last = k_end - KC;  // past-the-end prefetches re-read the last chunk
  // whole groups of PF chunks
  const int k_main = REM ? k_begin + (k_end - k_begin) / (PF * KC) * (PF * KC) : k_end;
  for (int kc0 = k_begin; kc0 < k_main; kc0 += PF * KC) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int kc = kc0 + p * KC;
      __syncthreads();
#pragma unroll
      for (int v = 0; v < XV; ++v)
        if (v + 1 < XV || xlast) *reinterpret_cast<u32x4_t*>(&xlds[xo[v]]) = xbuf[v];
      __syncthreads();
      const int kx = kc < k_last ? kc + KC : kc;
#pragma unroll
      for (int v = 0; v < XV; ++v)
        if (v + 1 < XV || xlast) xbuf[v] = *reinterpret_cast<const u32x4_t*>((kx < K0 ? xp0[v] : xp1[v]) + kx);
      const int kn = kc + PF * KC <= k_last ? kc + PF * KC : k_last;
      // B operands double-buffered: step s + 1's LDS reads are in flight
      // while step s's MFMAs run
      const bf16_t* xrow = &xlds[(lane & 15) * LDS_ROW + (lane >> 4) * 8];
      u32x4_t bq[2][MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) bq[0][t] = *reinterpret_cast<const u32x4_t*>(xrow + t * 16 * LDS_ROW);
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        if (s + 1 < STEPS) {
#pragma unroll
          for (int t = 0; t < MT; ++t)
            bq[(s + 1) & 1][t] = *reinterpret_cast<const u32x4_t*>(xrow + t * 16 * LDS_ROW + (s + 1) * 32);
        }
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wbuf[p][s]);
        wbuf[p][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wat(kn + s * 32)));
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[s & 1][t]), acc[t],
                                                          0, 0, 0);
      }
    }
  }
  if constexpr (REM) {
    // REM: up to PF - 1 chunks after the whole groups, their W already in
    // wbuf[0 ..]; the same steps as one pass of the loop above (kept out of
    // the loop, whose body carries no branch: a branch around the chunk there
    // costs about 18% at K = 11008, and a lambda shared with the loop made
    // the compiler drain every load at the loop's back edge)
    auto chunk = [&](const int p, const int kc) __attribute__((always_inline)) {
      __syncthreads();
#pragma unroll
      for (int v = 0; v < XV; ++v)
        if (v + 1 < XV || xlast) *reinterpret_cast<u32x4_t*>(&xlds[xo[v]]) = xbuf[v];
      __syncthreads();
      const int kx = kc < k_last ? kc + KC : kc;
#pragma unroll
      for (int v = 0; v < XV; ++v)
        if (v + 1 < XV || xlast) xbuf[v] = *reinterpret_cast<const u32x4_t*>((kx < K0 ? xp0[v] : xp1[v]) + kx);
      const int kn = kc + PF * KC <= k_last ? kc + PF * KC : k_last;
      // B operands double-buffered: step s + 1's LDS reads are in flight
      // while step s's MFMAs run
      const bf16_t* xrow = &xlds[(lane & 15) * LDS_ROW + (lane >> 4) * 8];
      u32x4_t bq[2][MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) bq[0][t] = *reinterpret_cast<const u32x4_t*>(xrow + t * 16 * LDS_ROW);
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        if (s + 1 < STEPS) {
#pragma unroll
          for (int t = 0; t < MT; ++t)
            bq[(s + 1) & 1][t] = *reinterpret_cast<const u32x4_t*>(xrow + t * 16 * LDS_ROW + (s + 1) * 32);
        }
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wbuf[p][s]);
        wbuf[p][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wat(kn + s * 32)));
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[s & 1][t]), acc[t],
                                                          0, 0, 0);
      }
    };
#pragma unroll
    for (int p = 0; p + 1 < PF; ++p)
      if (k_main + p * KC < k_end) chunk(p, k_main + p * KC);
  }

  if constexpr (!SPLIT && !TOPK && WV % 2 == 0 && MT <= 4) {
   if (a.glu_F > 0) {
    // the up values through LDS (MP rows x 16 G columns, padded), then waves
    // 0 .. G - 1 finish their gate columns; same expression as swiglu_rows
    constexpr int UR = 16 * G + 1;
    static_assert(MP * UR * 4 <= XLDS * 2, "the up tile fits the X staging area");
    float* upt = reinterpret_cast<float*>(xlds);
    __syncthreads();  // every wave is done with the last X chunk
    if (wave >= G) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          upt[(t * 16 + (lane & 15)) * UR + 16 * (wave - G) + 4 * (lane >> 4) + i] = acc[t][i];
    }
    __syncthreads();
    if (wave < G) {
      const int jl = 16 * wave + 4 * (lane >> 4);
      const int j0 = 16 * G * static_cast<int>(blockIdx.x) + jl;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int ml = t * 16 + (lane & 15), m = m_base + ml;
        if (m >= M || j0 >= a.glu_F) continue;
        uint32_t w2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float gate = acc[t][2 * h + e], up = upt[ml * UR + jl + 2 * h + e];
            packed |= static_cast<uint32_t>(f32_to_bf16(gate / (1.0f + expf(-gate)) * up)) << (16 * e);
          }
          w2[h] = packed;
        }
        *reinterpret_cast<uint2*>(a.glu_out + static_cast<size_t>(m) * a.glu_F + j0) = make_uint2(w2[0], w2[1]);
      }
    }
    return;
   }
  }

  // D[n][m]: lane holds n = 4 * (lane / 16) + i, m = lane % 16 of each tile.
  const int n0 = n_base + (lane >> 4) * 4;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m_base + t * 16 + (lane & 15);
    if (m >= M || idle) continue;
    float* dst;
    if constexpr (SPLIT) {
      dst = a.part + (static_cast<size_t>(blockIdx.y) * M + m) * N;
    } else {
      dst = a.Y + static_cast<size_t>(a.map(m)) * a.ldy;
    }
    if (n0 + 3 < N && (N & 3) == 0 && (SPLIT || (a.ldy & 3) == 0)) {
      *reinterpret_cast<float4*>(dst + n0) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n0 + i < N) dst[n0 + i] = acc[t][i];
    }
  }

  if constexpr (TOPK) {
    // the workgroup's [MP x RPW] tile through LDS; every 64-column block gets
    // its own partial slot, handled by 256 threads (TPR per row)
    constexpr int TPR = 256 / MP;
    constexpr int VPT = kProjRowsPerWG / TPR;
    float* tile = reinterpret_cast<float*>(xlds);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nl = wave * 16 + (lane >> 4) * 4 + i;
        tile[(t * 16 + (lane & 15)) * TROW + nl] =
            static_cast<int>(blockIdx.x) * RPW + nl < N ? acc[t][i] : -INFINITY;
      }
    __syncthreads();
    const int blk = tid / 256;  // 64-column block of this thread
    const int t2 = tid % 256;
    const int mloc = t2 / TPR, sub = t2 % TPR;
    const int m = m_base + mloc;
    const int col0 = static_cast<int>(blockIdx.x) * RPW + blk * kProjRowsPerWG;
    // rows past M skip the work (a row's TPR threads share one wave)
    if (m < M && col0 < N) {
      float mx = -INFINITY;
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int nl = blk * kProjRowsPerWG + sub + j * TPR;
        const float v = tile[mloc * TROW + nl];
        mx = fmaxf(mx, v);
        const uint64_t key = v == -INFINITY ? 0 : topk_key(v, static_cast<int>(blockIdx.x) * RPW + nl);
        best = key > best ? key : best;
      }
      // combine the TPR threads of the row (an aligned lane group of one wave)
      best = group_max_u64<TPR>(best);
      const size_t slot = static_cast<size_t>(m) * projection_nwg(N) + col0 / kProjRowsPerWG;
      if (sub == 0) a.tp.keys[slot] = best;
      if (a.tp.ms) {  // (max, sum exp) only when the row's log-sum-exp is wanted
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          const float v = tile[mloc * TROW + blk * kProjRowsPerWG + sub + j * TPR];
          if (v != -INFINITY) s += expf(v - mx);
        }
        group_ms<TPR>(mx, s);
        if (sub == 0) a.tp.ms[slot] = make_float2(mx, s);
      }
    }
  }
}

// float32 path (correctness-sized workloads): one wave per output column n,
// lanes split K, a wave reduction per row.
__global__ __launch_bounds__(256) void proj_f32_kernel(int M, int K, int N, XSource xs,
                                                       const float* __restrict__ W,
                                                       float* __restrict__ Y, RowMap map,
                                                       int ldy) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* wr = W + static_cast<size_t>(n) * K;
  const int K0 = xs.mode == 0 ? K : xs.d;
  for (int m = 0; m < M; ++m) {
    const float* p0;
    const float* p1;
    if (xs.mode == 0) {
      p0 = static_cast<const float*>(xs.x) + static_cast<size_t>(m) * xs.ldx;
      p1 = p0;
    } else {
      const int b = m / xs.P;
      const int node = xs.row_node[xs.r0 + m % xs.P];
      int t = node == 0 ? xs.root_tok[b] : xs.tok[static_cast<size_t>(b) * xs.ntree + node];
      t = t < 0 ? 0 : (t >= xs.V ? xs.V - 1 : t);
      p0 = static_cast<const float*>(xs.x) + static_cast<size_t>(b) * xs.d;
      p1 = static_cast<const float*>(xs.emb) + static_cast<size_t>(t) * xs.d - xs.d;
    }
    float s = 0.f;
    for (int k = lane; k < K; k += 64) s = fmaf(wr[k], k < K0 ? p0[k] : p1[k], s);
    s = wave_sum(s);
    if (lane == 0) Y[static_cast<size_t>(map(m)) * ldy + n] = s;
  }
}

// Row-reduction partials of finished float32 logits, in the same layout the
// fused epilogue writes: one wave per (row, 64-column slice).
__global__ __launch_bounds__(64) void logits_partials(int M, int N, const float* __restrict__ Y, RowMap map,
                                                      int ldy, TopkPartials tp) {
  const int m = blockIdx.y, w = blockIdx.x, lane = threadIdx.x;
  if (tp.clear && m == 0 && w == 0)
    for (int c = lane; c < tp.nclear; c += 64) tp.clear[c] = 0;
  const int n = w * kProjRowsPerWG + lane;
  const float v = n < N ? Y[static_cast<size_t>(map(m)) * ldy + n] : -INFINITY;
  const float mx = wave_max(v);
  const float s = wave_sum(v == -INFINITY ? 0.f : expf(v - mx));
  const uint64_t best = wave_max_u64(n < N ? topk_key(v, n) : 0);
  if (lane == 0) {
    const size_t slot = static_cast<size_t>(m) * gridDim.x + w;
    tp.keys[slot] = best;
    if (tp.ms) tp.ms[slot] = make_float2(mx, s);
  }
}

template <int MT, int PF, bool TOPK, bool REM = false>
void launch_bf16_pf(const ProjArgs& a, int nsplit, hipStream_t stream) {
  constexpr int KC = MT <= 4 ? 256 : (MT <= 8 ? 128 : 64);
  // split-K launches (partials) and direct launches are separate instances;
  // with 8+ row tiles, 8-wave workgroups share each staged X chunk twice as
  // far; at 4 row tiles (64 rows) 4-wave workgroups, twice as many, measured
  // faster (7B decoder layer 155 -> 152 us, 64 x 22016 product 49 -> 46.5 us)
  if (a.part) {
    dim3 grid((a.N + 63) / 64, nsplit);
    proj_bf16_kernel<MT, KC, PF, 4, true, false, REM><<<grid, 256, 0, stream>>>(a);
  } else if constexpr (MT >= 8) {
    dim3 grid((a.N + 127) / 128, 1);
    proj_bf16_kernel<MT, KC, PF, 8, false, TOPK, REM><<<grid, 512, 0, stream>>>(a);
  } else {
    dim3 grid((a.N + 63) / 64, 1);
    proj_bf16_kernel<MT, KC, PF, 4, false, TOPK, REM><<<grid, 256, 0, stream>>>(a);
  }
}

template <int MT, bool TOPK>
int launch_bf16(const ProjArgs& a, int nsplit, hipStream_t stream) {
  constexpr int KC = MT <= 4 ? 256 : (MT <= 8 ? 128 : 64);
  constexpr int PF = MT <= 4 ? 2 : (MT <= 8 ? 4 : 8);
  // the shortest K range of a workgroup, and whether every range is a whole
  // number of PF-chunk groups
  int kmin;
  bool whole;
  if (a.kper > 0) {
    kmin = std::min(a.kper, a.K - (nsplit - 1) * a.kper);
    whole = a.K % a.kper == 0 && a.kper % (PF * KC) == 0;
  } else {  // balanced split ranges
    const int nch = a.K / KC, ns = -a.kper;
    kmin = nch / ns * KC;
    whole = nch % ns == 0 && (nch / ns) % PF == 0;
  }
  const bool ragged = a.kper > 0 ? a.K % a.kper != 0 : (a.K / KC) % -a.kper != 0;
  if (whole) {
    launch_bf16_pf<MT, PF, TOPK>(a, nsplit, stream);
  } else if (kmin > PF * KC) {
    launch_bf16_pf<MT, PF, TOPK, true>(a, nsplit, stream);  // e.g. K = 11008: 43 chunks of 256
  } else if (ragged || kmin % KC != 0) {
    launch_bf16_pf<MT, 1, TOPK, true>(a, nsplit, stream);
  } else {
    launch_bf16_pf<MT, 1, TOPK>(a, nsplit, stream);  // K range of 256 .. PF*KC-256
  }
  HY_LAUNCH_CHECK("projection(bf16)");
  return HYDRA_OK;
}

template <bool TOPK>
int launch_bf16_mt(int mc, const ProjArgs& a, int nsplit, hipStream_t stream) {
  if (mc <= 16) return launch_bf16<1, TOPK>(a, nsplit, stream);
  if (mc <= 32) return launch_bf16<2, TOPK>(a, nsplit, stream);
  if (mc <= 64) return launch_bf16<4, TOPK>(a, nsplit, stream);
  if (mc <= 128) return launch_bf16<8, TOPK>(a, nsplit, stream);
  return launch_bf16<16, TOPK>(a, nsplit, stream);
}

// Gate column groups (16 columns each) per workgroup of the gated product,
// which has 2 G waves. Measured on MI355X (64 rows, K = 4096, packed
// weights): a CU streams its share at about the same rate with 4 waves as
// with 8, and markedly slower with fewer, so a launch of at least 4-wave
// workgroups takes as long as its busiest CU: with G = 2, 344 workgroups (F
// = 11008) took 43-45 us against 26.6 for 256 (F = 8192) and 49.7 for 512
// (F = 16384); G = 3 (230 workgroups, none doubled up on a CU) takes 37 us
// and G = 4 (172 workgroups) 47 us.
// The plan takes the G that leaves the busiest CU the fewest groups.
int plan_glu(int F) {
  const int pairs = F / 16;
  int best = 2;
  long best_cost = 1L << 62;
  for (const int g : {2, 3}) {
    const long cost = ((pairs + g - 1) / g + 255) / 256 * g;  // groups on the busiest CU
    if (cost < best_cost) {
      best = g;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace

// Launch Y = X . W^T. With nsplit > 1 (bf16 only) writes float32 partials
// part[split][m][n] instead of Y. M is processed in chunks of up to 256 rows.
int launch_projection(int dtype, int M, int K, int N, XSource xs, const void* W, float* Y, RowMap map,
                      int ldy, int nsplit, float* part, TopkPartials tp, hipStream_t stream) {
  const int wpacked = (dtype & HYDRA_VOCAB_PACKED) != 0;
  dtype &= ~HYDRA_VOCAB_PACKED;
  if (M <= 0 || N <= 0) return HYDRA_OK;
  if (wpacked && (dtype != HYDRA_BF16 || K % kPackChunk != 0)) {
    set_error("projection: packed weights are bf16 with K %% %d == 0 (K=%d)", kPackChunk, K);
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (tp.keys && (part || nsplit != 1)) {
    set_error("projection: the fused row reduction needs no split-K");
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (dtype == HYDRA_F32) {
    if (nsplit != 1) {
      set_error("projection: split-K is bf16 only");
      return HYDRA_ERR_UNSUPPORTED;
    }
    proj_f32_kernel<<<(N + 3) / 4, 256, 0, stream>>>(M, K, N, xs, static_cast<const float*>(W), Y, map, ldy);
    HY_LAUNCH_CHECK("projection(f32)");
    if (tp.keys) {
      logits_partials<<<dim3(projection_nwg(N), M), 64, 0, stream>>>(M, N, Y, map, ldy, tp);
      HY_LAUNCH_CHECK("projection(f32) partials");
    }
    return HYDRA_OK;
  }
  if (K % 256 != 0 || K % nsplit != 0 || (K / nsplit) % 256 != 0) {
    set_error("projection: bf16 needs K %% 256 == 0 per split (K=%d, splits=%d)", K, nsplit);
    return HYDRA_ERR_UNSUPPORTED;
  }
  if (M >= kGemmMinRows && nsplit == 1 && xs.mode == 0 && gemm_supported(K))
    return launch_projection_gemm(M, K, N, static_cast<const bf16_t*>(xs.x), xs.ldx, static_cast<const bf16_t*>(W),
                                  wpacked ? -1 : K, Y, map, ldy, tp, stream);
  if (wpacked && (M > 64 || xs.mode != 0 || nsplit != 1)) {
    set_error("projection: packed weights take contiguous rows without split K (M=%d)", M);
    return HYDRA_ERR_UNSUPPORTED;
  }
  ProjArgs a{M, K, N, xs, static_cast<const bf16_t*>(W), Y, map, ldy, K / nsplit, 0, part, tp, wpacked, 0, nullptr};
  for (int m0 = 0; m0 < M; m0 += 256) {
    const int mc = M - m0 < 256 ? M - m0 : 256;
    a.m_base = m0;
    const int rc =
        tp.keys ? launch_bf16_mt<true>(mc, a, nsplit, stream) : launch_bf16_mt<false>(mc, a, nsplit, stream);
    if (rc != HYDRA_OK) return rc;
  }
  return HYDRA_OK;
}

int launch_projection_parts(int dtype, int M, int K, int N, const void* X, const void* W, float* part,
                            size_t part_floats, int* nsplit, hipStream_t stream) {
  *nsplit = 1;
  const int wpacked = (dtype & HYDRA_LAYER_PACKED) != 0;  // W in the packed layout
  dtype &= ~HYDRA_LAYER_PACKED;
  if (wpacked && (dtype != HYDRA_BF16 || K % kPackChunk != 0)) {
    set_error("projection: packed weights are bf16 with K %% %d == 0 (K=%d)", kPackChunk, K);
    return HYDRA_ERR_UNSUPPORTED;
  }
  XSource xs{};
  xs.x = X;
  xs.ldx = K;
  xs.mode = 0;
  if (M <= 0 || N <= 0) return HYDRA_OK;
  const size_t mn = static_cast<size_t>(M) * N;
  const int cap = static_cast<int>(std::min<size_t>(16, std::max<size_t>(1, part_floats / mn)));
  if (dtype == HYDRA_F32 || K % 256 != 0)
    return launch_projection(dtype, M, K, N, xs, W, part, RowMap{M, 0, 0}, N, 1, nullptr,
                             TopkPartials{nullptr, nullptr}, stream);
  if (M >= kGemmMinRows && gemm_supported(K)) {
    // about one workgroup per CU, each K range at least 512 long
    const int wg = gemm_workgroups(M, N);
    int ns = std::max(1, std::min({cap, 8, (256 + wg - 1) / wg, K / 512}));
    const int kper = (K / 64 + ns - 1) / ns * 64;
    ns = (K + kper - 1) / kper;
    *nsplit = ns;
    return launch_projection_gemm_split(M, K, N, static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W),
                                        wpacked ? -1 : K, part,
                                        ns, kper, stream);
  }
  // streaming kernel: 64 output columns per workgroup and split; about one
  // workgroup per CU, each K range a multiple of 256 (measured on MI355X:
  // the 7B decoder layer takes 177 us with 256 workgroups, 188 with 512 and
  // 190 with 1024; the 70B layer is the same for all three)
  // (measured on MI355X at 64 rows, where every workgroup also stages a
  // 64-row X chunk per weight chunk: a CU holding two workgroups of a launch
  // gains nothing, so the count is rounded down: the 7B Q/K/V product takes
  // 24.7 us in 192 workgroups, 26.9 in 384; at 16 rows and fewer it is
  // rounded up)
  const int wg = (N + 63) / 64 * ((M + 255) / 256);
  const int per_cu = M > 32 ? std::max(1, 256 / wg) : (256 + wg - 1) / wg;
  const int ns = std::max(1, std::min({cap, 16, per_cu, K / 256}));
  *nsplit = ns;
  if (ns == 1)
    return launch_projection(dtype | (wpacked ? HYDRA_VOCAB_PACKED : 0), M, K, N, xs, W, part, RowMap{M, 0, 0}, N,
                             1, nullptr, TopkPartials{nullptr, nullptr}, stream);
  // split s takes chunks [s * nch / ns, (s + 1) * nch / ns) of the nch
  // 256-column chunks of K (a negative kper asks the kernel for this)
  ProjArgs a{M, K, N, xs, static_cast<const bf16_t*>(W), nullptr, RowMap{M, 0, 0}, N, -ns, 0, part,
             TopkPartials{nullptr, nullptr}, wpacked, 0, nullptr};
  for (int m0 = 0; m0 < M; m0 += 256) {
    const int mc = M - m0 < 256 ? M - m0 : 256;
    a.m_base = m0;
    const int rc = launch_bf16_mt<false>(mc, a, ns, stream);
    if (rc != HYDRA_OK) return rc;
  }
  return HYDRA_OK;
}

bool projection_glu_supported(int dtype, int M, int K, int F) {
  dtype &= ~HYDRA_LAYER_PACKED;
  return dtype == HYDRA_BF16 && M >= 1 && M <= 64 && K % kPackChunk == 0 && F % 16 == 0;
}

int launch_projection_glu(int dtype, int M, int K, int F, const void* X, const void* W, bf16_t* g_out,
                          hipStream_t stream) {
  const int wpacked = (dtype & HYDRA_LAYER_PACKED) != 0;
  if (!projection_glu_supported(dtype, M, K, F)) {
    set_error("projection: the gated product needs bf16, 1..64 rows, K %% 256 == 0, F %% 16 == 0");
    return HYDRA_ERR_UNSUPPORTED;
  }
  const int G = plan_glu(F);
  XSource xs{};
  xs.x = X;
  xs.ldx = K;
  xs.mode = 0;
  ProjArgs a{M, K, 2 * F, xs, static_cast<const bf16_t*>(W), nullptr, RowMap{M, 0, 0}, 2 * F, K, 0, nullptr,
             TopkPartials{nullptr, nullptr}, wpacked, F, g_out};
  const dim3 grid((F / 16 + G - 1) / G, 1);
  auto go = [&](auto MTC, auto GC) {
    constexpr int MT = decltype(MTC)::value, WV = 2 * decltype(GC)::value;
    if (K % (2 * kPackChunk) == 0)
      proj_bf16_kernel<MT, 256, 2, WV, false, false, false><<<grid, 64 * WV, 0, stream>>>(a);
    else if (K > 2 * kPackChunk)
      proj_bf16_kernel<MT, 256, 2, WV, false, false, true><<<grid, 64 * WV, 0, stream>>>(a);
    else
      proj_bf16_kernel<MT, 256, 1, WV, false, false, false><<<grid, 64 * WV, 0, stream>>>(a);
  };
  auto go_g = [&](auto MTC) {
    if (G == 3) go(MTC, std::integral_constant<int, 3>{});
    else go(MTC, std::integral_constant<int, 2>{});
  };
  if (M <= 16) go_g(std::integral_constant<int, 1>{});
  else if (M <= 32) go_g(std::integral_constant<int, 2>{});
  else go_g(std::integral_constant<int, 4>{});
  HY_LAUNCH_CHECK("projection(gated)");
  return HYDRA_OK;
}

}  // namespace hydra

namespace hydra {
namespace {

// one thread per 16-byte piece of the packed layout, in output order: reads
// row n, columns k .. k + 7 of W (zeros for rows past N)
__global__ __launch_bounds__(256) void pack_weight_kernel(int N, int K, const bf16_t* __restrict__ W,
                                                          bf16_t* __restrict__ out, size_t pieces) {
  const size_t p = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (p >= pieces) return;
  const size_t ntiles = static_cast<size_t>((N + 15) / 16);
  const int r = static_cast<int>(p & 15), g = static_cast<int>((p >> 4) & 3), s = static_cast<int>((p >> 6) & 7);
  const size_t ct = p >> 9;  // chunk * ntiles + tile
  const int t = static_cast<int>(ct % ntiles), c = static_cast<int>(ct / ntiles);
  const int n = t * 16 + r, k = c * kPackChunk + s * 32 + g * 8;
  u32x4_t v{0u, 0u, 0u, 0u};
  if (n < N) v = *reinterpret_cast<const u32x4_t*>(W + static_cast<size_t>(n) * K + k);
  *reinterpret_cast<u32x4_t*>(out + p * 8) = v;
}

}  // namespace
}  // namespace hydra

extern "C" size_t hydra_packed_weight_size(int N, int K) {
  if (N <= 0 || K <= 0 || K % hydra::kPackChunk != 0) return 0;
  return static_cast<size_t>((N + 15) / 16) * 16 * K * 2;
}

extern "C" int hydra_pack_weight(int N, int K, const void* W, void* packed, void* stream) {
  using namespace hydra;
  clear_error();
  HY_CHECK(N > 0 && K > 0, HYDRA_ERR_INVALID, "pack_weight: bad sizes N=%d K=%d", N, K);
  HY_CHECK(K % kPackChunk == 0, HYDRA_ERR_UNSUPPORTED, "pack_weight: needs K %% %d == 0 (K=%d)", kPackChunk, K);
  HY_CHECK(W && packed, HYDRA_ERR_INVALID, "pack_weight: null pointer");
  HY_CHECK(W != packed, HYDRA_ERR_INVALID, "pack_weight: packed must not alias W");
  const size_t pieces = hydra_packed_weight_size(N, K) / 16;
  pack_weight_kernel<<<static_cast<unsigned>((pieces + 255) / 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      N, K, static_cast<const bf16_t*>(W), static_cast<bf16_t*>(packed), pieces);
  HY_LAUNCH_CHECK("pack_weight");
  return HYDRA_OK;
}

namespace {
struct VocabWs {
  size_t keys, ms, total;
};
VocabWs vocab_ws(int M, int N, int k) {
  VocabWs w{0, 0, 0};
  if (M <= 0 || N <= 0 || k <= 0) return w;
  const size_t slots = static_cast<size_t>(M) * hydra::projection_nwg(N);
  w.keys = hydra::align_up(slots * sizeof(uint64_t), 256);
  w.ms = hydra::align_up(slots * sizeof(float2), 256);
  w.total = w.keys + w.ms + 256;
  return w;
}
}  // namespace

extern "C" size_t hydra_vocab_projection_workspace_size(int M, int N, int k) { return vocab_ws(M, N, k).total; }

extern "C" int hydra_vocab_projection(int dtype, int M, int K, int N, int k, const void* X, const void* W,
                                      float* Y, void* ws, size_t ws_bytes, void* stream) {
  using namespace hydra;
  clear_error();
  const int vpack = dtype & HYDRA_VOCAB_PACKED;  // packed vocabulary weights (hydra_pack_weight)
  dtype &= ~HYDRA_VOCAB_PACKED;
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "vocab_projection: bad dtype %d", dtype);
  HY_CHECK(!vpack || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "vocab_projection: packed vocabulary weights are bf16");
  HY_CHECK(M >= 0 && K > 0 && N > 0, HYDRA_ERR_INVALID, "vocab_projection: bad sizes M=%d K=%d N=%d", M, K, N);
  HY_CHECK(k >= 0 && k <= HYDRA_MAX_TOPK && k <= N, HYDRA_ERR_INVALID, "vocab_projection: k=%d out of [0, %d]", k,
           HYDRA_MAX_TOPK);
  HY_CHECK(M == 0 || (X && W && Y), HYDRA_ERR_INVALID, "vocab_projection: null pointer");
  HY_CHECK(dtype == HYDRA_F32 || K % 256 == 0, HYDRA_ERR_UNSUPPORTED,
           "vocab_projection: bf16 needs K %% 256 == 0 (K=%d)", K);
  const VocabWs w = vocab_ws(M, N, k);
  HY_CHECK(ws_bytes >= w.total && (w.total == 0 || ws), HYDRA_ERR_WORKSPACE,
           "vocab_projection: workspace %zu < %zu", ws_bytes, w.total);
  TopkPartials tp{nullptr, nullptr};
  if (k > 0) {
    Arena arena(ws, ws_bytes);
    tp.keys = arena.take<uint64_t>(w.keys / sizeof(uint64_t));
    tp.ms = arena.take<float2>(w.ms / sizeof(float2));
  }
  XSource xs{};
  xs.x = X;
  xs.ldx = K;
  xs.mode = 0;
  RowMap map{M > 0 ? M : 1, 0, 0};
  return launch_projection(dtype | vpack, M, K, N, xs, W, Y, map, N, 1, nullptr, tp, static_cast<hipStream_t>(stream));
}

extern "C" int hydra_vocab_topk(int M, int N, int k, const float* Y, const void* ws, size_t ws_bytes, float* lse,
                                int32_t* ids, float* vals, void* stream) {
  using namespace hydra;
  clear_error();
  HY_CHECK(M >= 0 && N > 0 && k >= 1 && k <= HYDRA_MAX_TOPK && k <= N, HYDRA_ERR_INVALID,
           "vocab_topk: bad sizes M=%d N=%d k=%d", M, N, k);
  const VocabWs w = vocab_ws(M, N, k);
  HY_CHECK(ws_bytes >= w.total && (w.total == 0 || ws), HYDRA_ERR_WORKSPACE, "vocab_topk: workspace %zu < %zu",
           ws_bytes, w.total);
  if (M == 0) return HYDRA_OK;
  HY_CHECK(Y, HYDRA_ERR_INVALID, "vocab_topk: null logits");
  Arena arena(const_cast<void*>(ws), ws_bytes);
  MergeArgs ma{};
  ma.M = M;
  ma.nwg = projection_nwg(N);
  ma.k = k;
  ma.keys = arena.take<uint64_t>(w.keys / sizeof(uint64_t));
  ma.ms = arena.take<float2>(w.ms / sizeof(float2));
  ma.Y = Y;
  ma.ldy = N;
  ma.V = N;
  ma.map = RowMap{M, 0, 0};
  ma.lse = lse;
  ma.topk_ids = ids;
  ma.topk_vals = vals;
  ma.P = 1;
  return launch_topk_merge(ma, static_cast<hipStream_t>(stream));
}
