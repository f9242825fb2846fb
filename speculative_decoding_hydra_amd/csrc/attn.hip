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
//   * grid = (prefix splits + 1) x (query tiles) x (sequence, KV head). Query
//     rows of a KV head are (node u, query head g) pairs, so GQA packs the G
//     query heads into the same tile. A workgroup of NW waves holds 16 NW
//     query rows (one 16-row MFMA tile per wave): with up to 256 rows per
//     workgroup every tree node of a KV head shares each K/V byte it streams.
//   * per tile of NW * 16 keys, K is staged in LDS row-major and V
//     transposed, both shared by all waves; the next tile (the next two for
//     small workgroups) is in flight in registers while one is consumed;
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

#include <type_traits>

namespace hydra {
namespace {

constexpr int kMaxSplitPages = 1024;  // page ids one split stages in LDS

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query column
// of an S^T tile): the gfx950 row swaps hand every lane its partner's value
// in a VALU step
__device__ __forceinline__ float col_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The running offset of a row moves only when a tile's maximum exceeds it by
// more than this (log2 units): probabilities stay below 2^8, and most tiles
// skip rescaling the accumulators.
constexpr float kRescaleSlack = 8.f;

// NW waves of RT 16-row query tiles each (16 NW RT query rows); a thread
// loads KPT keys x 8 dims of K and V, so a tile holds 4 NW KPT keys; PD tiles
// in flight. With RT = 2 every K and V^T operand read from LDS feeds two
// MFMAs. The prefix splits stream whole tiles without any mask and finish
// with at most one masked tile; the tree split masks every score with the
// ancestor test.
template <int NW, int RT, int PD, int KPT>
__global__ __launch_bounds__(NW * 64, 2) void attn_split_mfma(
    int B, int N, int Hq, int Hkv, float scale_log2, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k_tree, const bf16_t* __restrict__ v_tree,
    const bf16_t* __restrict__ k_pages, const bf16_t* __restrict__ v_pages, int n_pages,
    int page_shift, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ anc,
    const int32_t* __restrict__ depth, int Dmax, int nsplit, int lsplit, int NQ, int NQpad,
    float* __restrict__ opart, float* __restrict__ mpart, float* __restrict__ lpart) {
  constexpr int D = 128;
  constexpr int NT = NW * 64;
  constexpr int QR = NW * RT * 16;   // query rows per workgroup
  constexpr int TK = NT / 16 * KPT;  // keys per tile
  // K rows in LDS are 256 bytes with the 16-byte chunk c of key r at position
  // c ^ 2 (r % 8): the 16-row operand reads then hit distinct banks (padded
  // rows cost a two-way conflict on gfx950). V^T rows are TK + 4 bf16 with
  // column groups of 4 XOR-ed by (row / 8) % 16, which spreads the transposing
  // writes (16 rows 8 apart per instruction) over the banks.
  constexpr int KROW = D;
  constexpr int VROW = TK + 4;
  constexpr int DJ = D / 32;
  constexpr int DD = D / 16;
  static_assert(TK % 64 == 0, "tiles hold whole 64-key steps");
  __shared__ __align__(16) bf16_t klds[TK * KROW];
  __shared__ __align__(16) bf16_t vlds[D * VROW];
  __shared__ __align__(16) uint8_t s_ok[TK];              // key of the tile exists (range and page)
  __shared__ __align__(16) int s_dep[TK];                 // depth of each tree key of the tile
  __shared__ int s_pages[kMaxSplitPages];                 // page ids of this split
  __shared__ int s_anc[QR][HYDRA_MAX_DEPTH + 1];          // ancestor rows of the workgroup's query rows

  const int split = blockIdx.x;
  const bool tree_part = split == nsplit;
  const int qtile = blockIdx.y;
  const int b = blockIdx.z / Hkv;
  const int hkv = blockIdx.z % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, lq = lane & 15;
  const int kx = (lq & 7) << 1;  // K chunk swizzle of this lane's key rows
  const int page_size = 1 << page_shift;

  int wrow[RT];  // this lane's query rows inside the workgroup
  bf16x8_t qreg[RT][DJ];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    wrow[r] = (wave * RT + r) * 16 + lq;
    const int qi = qtile * QR + wrow[r];
    const bool qvalid = qi < NQ;
    const int u = qvalid ? qi / G : 0;
    const int gq = qi % G;
    const bf16_t* qp = q + ((static_cast<size_t>(b) * N + u) * Hq + hkv * G + gq) * D + 8 * g;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      const u32x4_t v = qvalid ? *reinterpret_cast<const u32x4_t*>(qp + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
      qreg[r][j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  int L = prefix_len[b];
  const int cap = max_pages << page_shift;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int t_begin = tree_part ? 0 : split * lsplit;
  const int t_end = tree_part ? N : min(L, t_begin + lsplit);
  const int p0 = t_begin >> page_shift;
  const int32_t* dep_b = depth + static_cast<size_t>(b) * N;
  int pages_bad = 0;
  if (tree_part) {
    for (int e = tid; e < QR * (Dmax + 1); e += NT) {
      const int rr = e / (Dmax + 1), j = e % (Dmax + 1);
      const int qr = qtile * QR + rr;
      s_anc[rr][j] = qr < NQ ? anc[(static_cast<size_t>(b) * N + qr / G) * (Dmax + 1) + j] : -1;
    }
  } else {
    const int np = t_end > t_begin ? ((t_end - 1) >> page_shift) - p0 + 1 : 0;
    for (int e = tid; e < np; e += NT) {
      const int pg = block_table[static_cast<size_t>(b) * max_pages + p0 + e];
      s_pages[e] = pg;
      pages_bad |= pg < 0 || pg >= n_pages;
    }
  }
  __syncthreads();
  // every page of the split valid: whole tiles then need no mask
  const bool pages_ok = __syncthreads_or(pages_bad) == 0;

  float m_run[RT], l_run[RT];
  f32x4_t oacc[RT][DD];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) oacc[r][dd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // loader mapping: KPT consecutive keys (one page, page_size >= 16) x 8 dims
  const int tg = tid >> 4;  // key group 0 .. NT / 16 - 1
  const int dc = tid & 15;  // 8-dim chunk 0..15
  const int tl = KPT * tg;
  const size_t page_stride = static_cast<size_t>(Hkv) << (page_shift + 7);  // Hkv * page_size * D
  const size_t head_off = (static_cast<size_t>(hkv) << (page_shift + 7)) + dc * 8;
  const size_t tree_off = (static_cast<size_t>(b) * N * Hkv + hkv) * D + dc * 8;

  u32x4_t kv[PD][KPT], vv[PD][KPT];
  int kvalid[PD];
  // Registers of a coming tile: KPT keys x 8 dims of K and of V per thread.
  // Loads are unconditional (invalid keys re-read a valid row and are masked
  // through s_ok), so the compiler can keep them in flight across the tile.
  auto load_tile = [&](auto SLOT, auto WHOLE, int t0) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    constexpr bool whole = decltype(WHOLE)::value;
    const int tk = t0 + tl;
    const bf16_t* kb;
    const bf16_t* vb;
    size_t stride;
    int valid = KPT;
    if (!whole) valid = tk < t_end ? min(KPT, t_end - tk) : 0;
    if (tree_part) {
      const int tc = valid > 0 ? tk : 0;
      const size_t off = tree_off + static_cast<size_t>(tc) * Hkv * D;
      kb = k_tree + off;
      vb = v_tree + off;
      stride = static_cast<size_t>(Hkv) * D;
    } else {
      const int tc = valid > 0 ? tk : t_begin;
      int pg = s_pages[(tc >> page_shift) - p0];
      if (!whole && (pg < 0 || pg >= n_pages)) {
        pg = 0;
        valid = 0;
      }
      const size_t off = pg * page_stride + head_off + (static_cast<size_t>(tc & (page_size - 1)) << 7);
      kb = k_pages + off;
      vb = v_pages + off;
      stride = D;
    }
    kvalid[sl] = valid;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const size_t o = whole || j < valid ? j * stride : 0;
      kv[sl][j] = *reinterpret_cast<const u32x4_t*>(kb + o);
      vv[sl][j] = *reinterpret_cast<const u32x4_t*>(vb + o);
    }
  };

  // one 64-key step of a staged tile: S^T, online softmax, P.V. MASKED reads
  // key validity (and in the tree split the ancestor test) per score.
  auto step = [&](auto MASKED, int c0, int t0) __attribute__((always_inline)) {
    constexpr bool masked = decltype(MASKED)::value;
    // S^T tiles: lane holds keys c0 + 16 tt + 4 g + i for query column lq
    f32x4_t sacc[RT][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int r = 0; r < RT; ++r) sacc[r][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&klds[(c0 + 16 * tt + lq) * KROW + (((4 * j + g) ^ kx) << 3)]);
#pragma unroll
        for (int r = 0; r < RT; ++r)
          sacc[r][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qreg[r][j],
                                                               sacc[r][tt], 0, 0, 0);
      }
    }
    uint32_t okb[RT];  // bit 4 tt + i: score (tt, i) of row tile r is visible
    if constexpr (masked) {
      uint32_t base = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&s_ok[c0 + 16 * tt + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) base |= ((w >> (8 * i)) & 1u) << (4 * tt + i);
      }
#pragma unroll
      for (int r = 0; r < RT; ++r) okb[r] = base;
      if (tree_part) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int4 d4 = *reinterpret_cast<const int4*>(&s_dep[c0 + 16 * tt + 4 * g]);
          const int dvs[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int dv = dvs[i];
            const int dvc = dv < 0 ? 0 : (dv > Dmax ? Dmax : dv);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              const bool vis = dv == dvc && s_anc[wrow[r]][dvc] == t0 + c0 + 16 * tt + 4 * g + i;
              okb[r] &= vis ? ~0u : ~(1u << (4 * tt + i));
            }
          }
        }
      }
    }
    bf16x8_t pb[RT][2];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      // raw scores; the scale (> 0) is folded into the exponent below
      float mt = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (masked) sacc[r][tt][i] = (okb[r] >> (4 * tt + i)) & 1u ? sacc[r][tt][i] : -INFINITY;
          mt = fmaxf(mt, sacc[r][tt][i]);
        }
      }
      mt = col_max(mt) * scale_log2;
      const bool grow = mt > m_run[r] + kRescaleSlack;
      const float m_new = grow ? fmaxf(m_run[r], mt) : m_run[r];
      if (__any(grow)) {  // wave-uniform: rescale only when an offset moved
        const float alpha = m_new == m_run[r] ? 1.f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
        l_run[r] *= alpha;
#pragma unroll
        for (int dd = 0; dd < DD; ++dd) oacc[r][dd] *= alpha;
        m_run[r] = m_new;
      }
      const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
      float sv[4][4];
      float ps = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[r][tt][i], scale_log2, neg_m));
          sv[tt][i] = pe;
          ps += pe;
        }
      l_run[r] += col_sum(ps);
      // P^T operands: slots 0..3 = keys 32 ks + 4 g + i, slots 4..7 = keys 32 ks + 16 + 4 g + i
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[r][ks][i] = static_cast<__bf16>(sv[2 * ks][i]);
          pb[r][ks][4 + i] = static_cast<__bf16>(sv[2 * ks + 1][i]);
        }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) {
        const int vrow = 16 * dd + lq;
        const int vx = ((vrow >> 3) & 15) << 2;
        const int col = c0 + 32 * ks + 4 * g;
        u32x4_t a;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(&vlds[vrow * VROW + (col ^ vx)]);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(&vlds[vrow * VROW + ((col + 16) ^ vx)]);
        a.x = lo.x;
        a.y = lo.y;
        a.z = hi.x;
        a.w = hi.y;
#pragma unroll
        for (int r = 0; r < RT; ++r)
          oacc[r][dd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), pb[r][ks],
                                                               oacc[r][dd], 0, 0, 0);
      }
    }
  };

  // one tile: stage slot SLOT in LDS (with the validity / depth bytes unless
  // WHOLE), refill the slot PD tiles ahead, then its 64-key steps
  auto process = [&](auto SLOT, auto WHOLE, int t0) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    constexpr bool whole = decltype(WHOLE)::value;
    __syncthreads();  // previous tile fully consumed
    if (!whole && dc == 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        s_ok[tl + j] = j < kvalid[sl];
        if (tree_part) s_dep[tl + j] = j < kvalid[sl] ? dep_b[t0 + tl + j] : -1;
      }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      *reinterpret_cast<u32x4_t*>(&klds[(tl + j) * KROW + ((dc ^ (((tl + j) & 7) << 1)) << 3)]) = kv[sl][j];
    {
      typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;
      u16x8 a[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) a[j] = __builtin_bit_cast(u16x8, vv[sl][j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (KPT == 4) {
          u32x2_t w;
          w.x = pack2(a[0][e], a[1][e]);
          w.y = pack2(a[2][e], a[3][e]);
          *reinterpret_cast<u32x2_t*>(&vlds[(dc * 8 + e) * VROW + (tl ^ ((dc & 15) << 2))]) = w;
        } else {
          *reinterpret_cast<uint32_t*>(&vlds[(dc * 8 + e) * VROW + (tl ^ ((dc & 15) << 2))]) =
              pack2(a[0][e], a[1][e]);
        }
      }
    }
    __syncthreads();
    const int tn = t0 + PD * TK;
    if (tn < t_end) {
      // the refill is whole too when it lies entirely inside a clean split
      if (whole && tn + TK <= t_end) load_tile(SLOT, std::true_type{}, tn);
      else load_tile(SLOT, std::false_type{}, tn);
    }
    for (int c = 0; c < TK / 64; ++c) step(std::integral_constant<bool, !whole>{}, 64 * c, t0);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, PD - 1>;
  using Whole = std::true_type;
  using Part = std::false_type;
  // whole prefix tiles over valid pages run unmasked in a loop of their own
  // (pairs of them when two are in flight), the rest masked
  const int ntiles = t_end > t_begin ? (t_end - t_begin + TK - 1) / TK : 0;
  const int nwhole = tree_part || !pages_ok ? 0 : (t_end - t_begin) / TK / PD * PD;
  if (ntiles > 0) {
    if (nwhole > 0) load_tile(S0{}, Whole{}, t_begin);
    else load_tile(S0{}, Part{}, t_begin);
  }
  if (PD > 1 && ntiles > 1) {
    if (nwhole > 1) load_tile(S1{}, Whole{}, t_begin + TK);
    else load_tile(S1{}, Part{}, t_begin + TK);
  }
  int it = 0;
  for (; it < nwhole; it += PD) {
    process(S0{}, Whole{}, t_begin + it * TK);
    if (PD > 1) process(S1{}, Whole{}, t_begin + (it + 1) * TK);
  }
  for (; it < ntiles; it += PD) {
    process(S0{}, Part{}, t_begin + it * TK);
    if (PD > 1 && it + 1 < ntiles) process(S1{}, Part{}, t_begin + (it + 1) * TK);
  }

#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int qi = qtile * QR + wrow[r];
    if (qi < NQ) {
      const size_t row = (static_cast<size_t>(split * B + b) * Hkv + hkv) * NQpad + qi;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd)
        *reinterpret_cast<float4*>(opart + row * D + 16 * dd + 4 * g) =
            make_float4(oacc[r][dd][0], oacc[r][dd][1], oacc[r][dd][2], oacc[r][dd][3]);
      if (g == 0) {
        mpart[row] = m_run[r];
        lpart[row] = l_run[r];
      }
    }
  }
}

// Merge the splits of one (sequence, KV head, query row). D / 4 lanes per row,
// four dims per lane, so a wave merges 64 * 4 / D rows at once; the parts are
// read in batches of CB so their loads overlap.
template <class T>
__global__ __launch_bounds__(256) void attn_combine(int B, int N, int Hq, int Hkv, int D, int nparts,
                                                    int NQ, int NQpad, const float* __restrict__ opart,
                                                    const float* __restrict__ mpart,
                                                    const float* __restrict__ lpart, T* __restrict__ out,
                                                    float* __restrict__ lse) {
  constexpr int CB = 8;
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
  for (int s0 = 0; s0 < nparts; s0 += CB) {
    float mv[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) mv[j] = s0 + j < nparts ? mpart[r0 + (s0 + j) * stride] : -INFINITY;
#pragma unroll
    for (int j = 0; j < CB; ++j) M = fmaxf(M, mv[j]);
  }
  const float Mu = M == -INFINITY ? 0.f : M;
  float Lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nparts; s0 += CB) {
    float mv[CB], lv[CB];
    float4 ov[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int sp = s0 + j < nparts ? s0 + j : s0;  // past the end: re-read a valid part, weight 0
      const size_t r = r0 + sp * stride;
      mv[j] = mpart[r];
      lv[j] = lpart[r];
      ov[j] = *reinterpret_cast<const float4*>(opart + r * D + 4 * c);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float w = s0 + j < nparts ? exp2f(mv[j] - Mu) : 0.f;
      Lsum += lv[j] * w;
      acc.x += ov[j].x * w;
      acc.y += ov[j].y * w;
      acc.z += ov[j].z * w;
      acc.w += ov[j].w * w;
    }
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
  int qr, nsplit, lsplit, qtiles, NQ, NQpad;
};

// Query rows per workgroup from the query rows of a KV head (up to 256 rows
// share one K/V stream), then prefix splits: enough workgroups to fill the
// chip, each split at least four tiles long and short enough that ragged
// batches balance.
SplitPlan plan_splits(int B, int N, int Hq, int Hkv, int max_prefix_len) {
  SplitPlan p;
  p.NQ = N * (Hq / Hkv);
  p.qr = p.NQ <= 64 ? 64 : (p.NQ <= 128 ? 128 : 256);
  const int TK = p.qr == 128 ? 128 : 64;  // keys per tile of the chosen kernel
  p.qtiles = (p.NQ + p.qr - 1) / p.qr;
  p.NQpad = p.qtiles * p.qr;
  const int base = B * Hkv * p.qtiles;
  const int Lr = max_prefix_len > 0 ? max_prefix_len : 0;
  const int target = p.qr == 64 ? 512 : 256;
  int s = target / base - 1;  // the tree split takes one slot
  const int maxs = (Lr + 4 * TK - 1) / (4 * TK);
  if (s > maxs) s = maxs;
  const int mins = (Lr + 16 * TK - 1) / (16 * TK);
  if (s < mins) s = mins;
  if (s < 1) s = 1;
  int ls = (Lr + s - 1) / s;
  ls = (ls + TK - 1) / TK * TK;
  const int lcap = (kMaxSplitPages - 1) * 16;  // pages of a split must fit in LDS (page_size >= 16)
  if (ls > lcap) ls = lcap / TK * TK;
  if (ls < TK) ls = TK;
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
  const int page_shift = page_size == 16 ? 4 : (page_size == 32 ? 5 : 6);
  dim3 grid(nparts, p.qtiles, B * Hkv);
#define HY_ATTN_ARGS                                                                                           \
  B, N, Hq, Hkv, scale_log2, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_tree),               \
      static_cast<const bf16_t*>(v_tree), static_cast<const bf16_t*>(k_pages), static_cast<const bf16_t*>(v_pages), \
      n_pages, page_shift, block_table, max_pages, prefix_len, anc, depth, Dmax, p.nsplit, p.lsplit, p.NQ, p.NQpad, \
      opart, mpart, lpart
  if (p.qr == 64) attn_split_mfma<4, 1, 2, 4><<<grid, 256, 0, stream>>>(HY_ATTN_ARGS);
  else if (p.qr == 128) attn_split_mfma<8, 1, 1, 4><<<grid, 512, 0, stream>>>(HY_ATTN_ARGS);
  else attn_split_mfma<8, 2, 1, 2><<<grid, 512, 0, stream>>>(HY_ATTN_ARGS);
#undef HY_ATTN_ARGS
  HY_LAUNCH_CHECK("tree_attention(split)");
  const long long cthreads = static_cast<long long>(B) * Hkv * p.NQ * (D / 4);
  attn_combine<bf16_t><<<static_cast<int>((cthreads + 255) / 256), 256, 0, stream>>>(B, N, Hq, Hkv, D, nparts, p.NQ, p.NQpad, opart, mpart,
                                                           lpart, static_cast<bf16_t*>(out), lse);
  HY_LAUNCH_CHECK("tree_attention(combine)");
  return HYDRA_OK;
}
