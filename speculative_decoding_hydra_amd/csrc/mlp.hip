// The draft heads' feed-forward layer for few rows, in one kernel:
//   a = W1 x + b1,  u = h + SiLU(a)  (or SiLU(a)),  stored as bf16.
// ("Medusa Heads", section "So sagen die Köpfe voraus": one SiLU layer with a
// residual connection; "Hydra Guide", section "1. Embedding Conditioning
// Mechanics": the Hydra layer reads [h || e(x_parent)].)
//
// W1 is [d, in] with d = 4096..8192, while the rows are few (one per expanded
// node, B * P <= 32). Tiling N in 64-row workgroups leaves too few
// workgroups, and split-K over the grid needs a second pass. Here a
// workgroup owns 16 rows of W1 and its 16 waves split K: each wave streams
// its K range of the 16 rows (the MFMA A operand) and reads the matching X
// slice straight from L2 (the B operand), with PF steps in flight. The waves'
// partial tiles meet in LDS and are summed in a fixed order, so the result is
// deterministic, then bias, SiLU and the residual are applied and u is
// rounded to bf16, all before the workgroup ends.
#include "common.h"

namespace hydra {
namespace {

constexpr int kMlpWaves = 16;

template <int MT, int PF>
__global__ __launch_bounds__(kMlpWaves * 64) void mlp_fused_kernel(MlpArgs a) {
  __shared__ f32x4_t red[kMlpWaves][MT][64];
  const XSource& xs = a.xs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int kw = a.K / kMlpWaves;
  const int kb = wave * kw;
  const int steps = kw / 32;
  const int K0 = xs.mode == 0 ? a.K : xs.d;  // a wave's K range never straddles K0

  const bf16_t* wp = a.W1 + static_cast<size_t>(n0 + (lane & 15)) * a.K + kb + (lane >> 4) * 8;
  const bf16_t* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int mr = t * 16 + (lane & 15);
    const int m = mr < a.M ? mr : 0;  // padded rows read row 0, never stored
    const bf16_t* p0;
    const bf16_t* p1;
    if (xs.mode == 0) {
      p0 = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(m) * xs.ldx;
      p1 = p0;
    } else {
      const int b = m / xs.P;
      const int node = xs.row_node[xs.r0 + m % xs.P];
      int tk = node == 0 ? xs.root_tok[b] : xs.tok[static_cast<size_t>(b) * xs.ntree + node];
      tk = tk < 0 ? 0 : (tk >= xs.V ? xs.V - 1 : tk);
      p0 = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(b) * xs.d;
      p1 = static_cast<const bf16_t*>(xs.emb) + static_cast<size_t>(tk) * xs.d - xs.d;
    }
    xp[t] = (kb < K0 ? p0 : p1) + kb + (lane >> 4) * 8;
  }

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t wr[PF], xr[PF][MT];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    wr[p] = *reinterpret_cast<const u32x4_t*>(wp + p * 32);
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[p][t] = *reinterpret_cast<const u32x4_t*>(xp[t] + p * 32);
  }
  const int last = steps - 1;
  for (int s0 = 0; s0 < steps; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int sn = s0 + p + PF <= last ? s0 + p + PF : last;  // past the end: re-read the last step
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wr[p]);
      wr[p] = *reinterpret_cast<const u32x4_t*>(wp + sn * 32);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, xr[p][t]);
        xr[p][t] = *reinterpret_cast<const u32x4_t*>(xp[t] + sn * 32);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  // D[n][m]: lane holds n = n0 + 4 * (lane / 16) + i, m = 16 t + lane % 16
  const int nb = n0 + (lane >> 4) * 4;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    f32x4_t sum = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < kMlpWaves; ++w) sum += red[w][t][lane];
    const int m = t * 16 + (lane & 15);
    if (m >= a.M) continue;
    const int b = m / a.P;
    bf16_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = sum[i] + bf16_to_f32(a.b1[nb + i]);
      const float act = v / (1.0f + expf(-v));  // SiLU(v) = v * sigmoid(v)
      const float u = a.residual ? bf16_to_f32(a.h[static_cast<size_t>(b) * a.d + nb + i]) + act : act;
      out[i] = f32_to_bf16(u);
    }
    const u32x2_t packed{static_cast<uint32_t>(out[0]) | (static_cast<uint32_t>(out[1]) << 16),
                         static_cast<uint32_t>(out[2]) | (static_cast<uint32_t>(out[3]) << 16)};
    *reinterpret_cast<u32x2_t*>(a.U + static_cast<size_t>(m) * a.d + nb) = packed;
    if (a.hidden) *reinterpret_cast<u32x2_t*>(a.hidden + static_cast<size_t>(a.map(m)) * a.d + nb) = packed;
  }
}

template <int MT>
void launch_mt(const MlpArgs& a, hipStream_t stream) {
  const int steps = a.K / kMlpWaves / 32;
  if (steps % 8 == 0) {
    mlp_fused_kernel<MT, 8><<<a.d / 16, kMlpWaves * 64, 0, stream>>>(a);
  } else {
    mlp_fused_kernel<MT, 1><<<a.d / 16, kMlpWaves * 64, 0, stream>>>(a);
  }
}

}  // namespace

bool mlp_fused_supported(int dtype, int M, int K, int d) {
  return dtype == HYDRA_BF16 && M >= 1 && M <= 32 && K % (kMlpWaves * 32) == 0 && d % 16 == 0;
}

int launch_mlp_fused(const MlpArgs& a, hipStream_t stream) {
  if (a.M <= 16) launch_mt<1>(a, stream);
  else launch_mt<2>(a, stream);
  HY_LAUNCH_CHECK("draft_heads: fused mlp");
  return HYDRA_OK;
}

}  // namespace hydra
