// Few-row feed-forward tile of the draft heads, shared by its own kernel and
// by the row-merge kernel, which runs the next head's h half in the same
// launch. A workgroup of NWV waves owns 16 output rows (tile) of head y; the
// waves split K, the epilogue runs on wave 0 (see MlpArgs).
#pragma once

#include "common.h"

namespace hydra {

template <int MT, int PF, int NWV>
__device__ __forceinline__ void mlp_tile(const MlpArgs& a, int tile, int y) {
  __shared__ f32x4_t red[NWV][MT][64];
  const XSource& xs = a.xs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = tile * 16;
  const int kw = a.K / NWV;
  const int kb = wave * kw;
  const int steps = kw / 32;
  const int K0 = xs.mode == 1 ? xs.d : a.K;  // mode 1: h below K0, the embedding above

  // this lane's 16 bytes of W at step s (32 columns each): row-major, row n0
  // + lane % 16 at column kb + 32 s + 8 (lane / 16); packed, the same piece
  // is lane 8 * lane of the 1 KB block of 32-column group q = kb / 32 + s of
  // tile n0 / 16 (packed_piece), so a wave reads 1 KB contiguous per step
  const bf16_t* wp = a.W[y] + static_cast<size_t>(n0 + (lane & 15)) * a.ldw + kb + (lane >> 4) * 8;
  const size_t ptiles = static_cast<size_t>((a.d + 15) / 16);
  auto wat = [&](int s) __attribute__((always_inline)) -> const bf16_t* {
    if (!a.wpacked) return wp + s * 32;
    const int q = (kb >> 5) + s;
    return a.W[y] + ((static_cast<size_t>(q >> 3) * ptiles + tile) * 8 + (q & 7)) * 512 + lane * 8;
  };
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
      const bf16_t* e = static_cast<const bf16_t*>(xs.emb) + static_cast<size_t>(tk) * xs.d;
      if (xs.mode == 1) {
        p0 = static_cast<const bf16_t*>(xs.x) + static_cast<size_t>(b) * xs.d;
        p1 = e - xs.d;
      } else {
        p0 = e;
        p1 = e;
      }
    }
    xp[t] = (kb < K0 ? p0 : p1) + kb + (lane >> 4) * 8;
  }

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t wr[PF], xr[PF][MT];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    wr[p] = *reinterpret_cast<const u32x4_t*>(wat(p));
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[p][t] = *reinterpret_cast<const u32x4_t*>(xp[t] + p * 32);
  }
  const int last = steps - 1;
  for (int s0 = 0; s0 < steps; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int sn = s0 + p + PF <= last ? s0 + p + PF : last;  // past the end: re-read the last step
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wr[p]);
      wr[p] = *reinterpret_cast<const u32x4_t*>(wat(sn));
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
  const int epi = a.epi[y];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    f32x4_t sum = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) sum += red[w][t][lane];
    const int m = t * 16 + (lane & 15);
    if (m >= a.M) continue;
    const int b = m / a.P;
    if (epi == 0) {
      float4 o;
      o.x = sum[0] + bf16_to_f32(a.b1[y][nb + 0]);
      o.y = sum[1] + bf16_to_f32(a.b1[y][nb + 1]);
      o.z = sum[2] + bf16_to_f32(a.b1[y][nb + 2]);
      o.w = sum[3] + bf16_to_f32(a.b1[y][nb + 3]);
      *reinterpret_cast<float4*>(a.A + (static_cast<size_t>(y) * a.M + m) * a.d + nb) = o;
      continue;
    }
    float4 add;
    if (epi == 2) {
      add = *reinterpret_cast<const float4*>(a.A + static_cast<size_t>(b) * a.d + nb);
    } else {
      add = make_float4(bf16_to_f32(a.b1[y][nb + 0]), bf16_to_f32(a.b1[y][nb + 1]), bf16_to_f32(a.b1[y][nb + 2]),
                        bf16_to_f32(a.b1[y][nb + 3]));
      if (epi == 3) {  // + the folded embedding half W1[:, d:] e(token)
        int tk = a.etok[b];
        tk = tk < 0 ? 0 : (tk >= a.xs.V ? a.xs.V - 1 : tk);
        const float4 e = *reinterpret_cast<const float4*>(a.Ef[y] + static_cast<size_t>(tk) * a.d + nb);
        add.x += e.x;
        add.y += e.y;
        add.z += e.z;
        add.w += e.w;
      }
    }
    const float addv[4] = {add.x, add.y, add.z, add.w};
    bf16_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = sum[i] + addv[i];
      const float act = v / (1.0f + expf(-v));  // SiLU(v) = v * sigmoid(v)
      const float u = a.residual ? bf16_to_f32(a.h[static_cast<size_t>(b) * a.d + nb + i]) + act : act;
      out[i] = f32_to_bf16(u);
    }
    const u32x2_t packed{static_cast<uint32_t>(out[0]) | (static_cast<uint32_t>(out[1]) << 16),
                         static_cast<uint32_t>(out[2]) | (static_cast<uint32_t>(out[3]) << 16)};
    *reinterpret_cast<u32x2_t*>(a.U + (static_cast<size_t>(y) * a.M + m) * a.d + nb) = packed;
    if (a.hidden) *reinterpret_cast<u32x2_t*>(a.hidden + static_cast<size_t>(a.map[y](m)) * a.d + nb) = packed;
  }
}

// The feed-forward tile needs K split evenly into 32-column steps per wave.
inline bool mlp_tile_fits(int K, int nwv) { return K % (nwv * 32) == 0; }

}  // namespace hydra
