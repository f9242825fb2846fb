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
//     into registers (the MFMA A operand), one K-chunk ahead of use;
//   * the matching chunk of X (all M rows, padded to 16 * MT) is staged once
//     per workgroup in LDS and read as the B operand;
//   * v_mfma_f32_16x16x32_bf16 does the contraction with float32 accumulation;
//   * split-K over grid.y gives enough workgroups when N is small (W1: N = d).
#include "common.h"

namespace hydra {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWG = 16 * kWaves;

struct RowPtrs {
  const bf16_t* p0;  // segment for k < K0
  const bf16_t* p1;  // segment for k >= K0 (pre-offset by -K0)
};

template <int MT, int KC, bool SPLIT>
__global__ __launch_bounds__(256) void proj_bf16_kernel(int M, int K, int N, XSource xs,
                                                        const bf16_t* __restrict__ W,
                                                        float* __restrict__ Y, RowMap map,
                                                        int ldy, int kper, int m_base,
                                                        float* __restrict__ part) {
  constexpr int MP = MT * 16;
  constexpr int LDS_ROW = KC + 8;  // 16-byte pad: rows land on different banks
  constexpr int STEPS = KC / 32;
  constexpr int VPR = KC / 8;      // 16-byte vectors per LDS row
  constexpr int XV = (MP * VPR + 255) / 256;
  __shared__ __align__(16) bf16_t xlds[MP * LDS_ROW];
  __shared__ RowPtrs rows[MP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_base = blockIdx.x * kRowsPerWG + wave * 16;
  const int k_begin = blockIdx.y * kper;
  const int k_end = k_begin + kper;
  const int K0 = xs.mode == 0 ? K : xs.d;

  if (tid < MP) {
    const int m = m_base + tid;
    RowPtrs rp{nullptr, nullptr};
    if (m < M) {
      if (xs.mode == 0) {
        rp.p0 = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(m) * xs.ldx;
        rp.p1 = rp.p0;
      } else {
        const int b = m / xs.P;
        const int node = xs.row_node[xs.r0 + m % xs.P];
        int t = node == 0 ? xs.root_tok[b] : xs.tok[static_cast<size_t>(b) * xs.ntree + node];
        t = t < 0 ? 0 : (t >= xs.V ? xs.V - 1 : t);
        rp.p0 = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(b) * xs.d;
        rp.p1 = static_cast<const bf16_t*>(xs.emb) + static_cast<size_t>(t) * xs.d - xs.d;
      }
    }
    rows[tid] = rp;
  }
  __syncthreads();

  const int wrow = min(n_base + (lane & 15), N - 1);
  const bf16_t* wp = W + static_cast<size_t>(wrow) * K + (lane >> 4) * 8;

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 wbuf[STEPS];
  uint4 xbuf[XV];

  auto load_x = [&](int kc) {
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int idx = tid + v * 256;
      const int r = idx / VPR;
      const int c = (idx % VPR) * 8;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r < MP && m_base + r < M) {
        const bf16_t* base = kc < K0 ? rows[r].p0 : rows[r].p1;
        val = *reinterpret_cast<const uint4*>(base + kc + c);
      }
      xbuf[v] = val;
    }
  };
  auto store_x = [&]() {
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int idx = tid + v * 256;
      const int r = idx / VPR;
      const int c = (idx % VPR) * 8;
      if (r < MP) *reinterpret_cast<uint4*>(&xlds[r * LDS_ROW + c]) = xbuf[v];
    }
  };

  load_x(k_begin);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) wbuf[s] = *reinterpret_cast<const uint4*>(wp + k_begin + s * 32);

  for (int kc = k_begin; kc < k_end; kc += KC) {
    __syncthreads();
    store_x();
    __syncthreads();
    const int kn = kc + KC;
    const bool more = kn < k_end;
    if (more) load_x(kn);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, wbuf[s]);
      if (more) wbuf[s] = *reinterpret_cast<const uint4*>(wp + kn + s * 32);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 bv = *reinterpret_cast<const uint4*>(
            &xlds[(t * 16 + (lane & 15)) * LDS_ROW + s * 32 + (lane >> 4) * 8]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv),
                                                        acc[t], 0, 0, 0);
      }
    }
  }

  // D[n][m]: lane holds n = 4 * (lane / 16) + i, m = lane % 16 of each tile.
  const int n0 = n_base + (lane >> 4) * 4;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m_base + t * 16 + (lane & 15);
    if (m >= M) continue;
    float* dst;
    if constexpr (SPLIT) {
      dst = part + (static_cast<size_t>(blockIdx.y) * M + m) * N;
    } else {
      dst = Y + static_cast<size_t>(map(m)) * ldy;
    }
    if (n0 + 3 < N && (N & 3) == 0 && (SPLIT || (ldy & 3) == 0)) {
      *reinterpret_cast<float4*>(dst + n0) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n0 + i < N) dst[n0 + i] = acc[t][i];
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

template <int MT>
int launch_bf16(int M, int K, int N, XSource xs, const void* W, float* Y, RowMap map, int ldy,
                int nsplit, float* part, int m_base, hipStream_t stream) {
  constexpr int KC = MT <= 4 ? 256 : (MT <= 8 ? 128 : 64);
  const int kper = K / nsplit;
  dim3 grid((N + kRowsPerWG - 1) / kRowsPerWG, nsplit);
  // split-K launches (partials) and direct launches are separate instances
  if (part) {
    proj_bf16_kernel<MT, KC, true><<<grid, 256, 0, stream>>>(
        M, K, N, xs, static_cast<const bf16_t*>(W), Y, map, ldy, kper, m_base, part);
  } else {
    proj_bf16_kernel<MT, KC, false><<<grid, 256, 0, stream>>>(
        M, K, N, xs, static_cast<const bf16_t*>(W), Y, map, ldy, kper, m_base, part);
  }
  HY_LAUNCH_CHECK("projection(bf16)");
  return HYDRA_OK;
}

}  // namespace

// Launch Y = X . W^T. With nsplit > 1 (bf16 only) writes float32 partials
// part[split][m][n] instead of Y. M is processed in chunks of up to 256 rows.
int launch_projection(int dtype, int M, int K, int N, XSource xs, const void* W, float* Y,
                      RowMap map, int ldy, int nsplit, float* part, hipStream_t stream) {
  if (M <= 0 || N <= 0) return HYDRA_OK;
  if (dtype == HYDRA_F32) {
    if (nsplit != 1) {
      set_error("projection: split-K is bf16 only");
      return HYDRA_ERR_UNSUPPORTED;
    }
    proj_f32_kernel<<<(N + 3) / 4, 256, 0, stream>>>(M, K, N, xs, static_cast<const float*>(W),
                                                     Y, map, ldy);
    HY_LAUNCH_CHECK("projection(f32)");
    return HYDRA_OK;
  }
  if (K % 256 != 0 || (K / nsplit) % 256 != 0 || K % nsplit != 0) {
    set_error("projection: bf16 needs K %% 256 == 0 per split (K=%d, splits=%d)", K, nsplit);
    return HYDRA_ERR_UNSUPPORTED;
  }
  for (int m0 = 0; m0 < M; m0 += 256) {
    const int mc = M - m0 < 256 ? M - m0 : 256;
    int rc;
    if (mc <= 16) rc = launch_bf16<1>(M, K, N, xs, W, Y, map, ldy, nsplit, part, m0, stream);
    else if (mc <= 32) rc = launch_bf16<2>(M, K, N, xs, W, Y, map, ldy, nsplit, part, m0, stream);
    else if (mc <= 64) rc = launch_bf16<4>(M, K, N, xs, W, Y, map, ldy, nsplit, part, m0, stream);
    else if (mc <= 128) rc = launch_bf16<8>(M, K, N, xs, W, Y, map, ldy, nsplit, part, m0, stream);
    else rc = launch_bf16<16>(M, K, N, xs, W, Y, map, ldy, nsplit, part, m0, stream);
    if (rc != HYDRA_OK) return rc;
  }
  return HYDRA_OK;
}

}  // namespace hydra

extern "C" int hydra_vocab_projection(int dtype, int M, int K, int N, const void* X,
                                      const void* W, float* Y, void* stream) {
  using namespace hydra;
  clear_error();
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "vocab_projection: bad dtype %d", dtype);
  HY_CHECK(M >= 0 && K > 0 && N > 0, HYDRA_ERR_INVALID, "vocab_projection: bad sizes M=%d K=%d N=%d", M, K, N);
  HY_CHECK(M == 0 || (X && W && Y), HYDRA_ERR_INVALID, "vocab_projection: null pointer");
  HY_CHECK(dtype == HYDRA_F32 || K % 256 == 0, HYDRA_ERR_UNSUPPORTED,
           "vocab_projection: bf16 needs K %% 256 == 0 (K=%d)", K);
  XSource xs{};
  xs.x = X;
  xs.ldx = K;
  xs.mode = 0;
  RowMap map{M > 0 ? M : 1, 0, 0};
  return launch_projection(dtype, M, K, N, xs, W, Y, map, N, 1, nullptr,
                           static_cast<hipStream_t>(stream));
}
