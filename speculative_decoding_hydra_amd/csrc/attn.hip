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
// gfx950 design (bf16, D = 128). The query rows of a KV head are (node u,
// query head g) pairs, so GQA packs the G query heads into the same tile.
// Two kernels, chosen by the query rows per KV head:
//   * up to 64 (the MHA trees of 64 nodes): attn_split_mfma, a small
//     streaming kernel (K/V through registers into LDS, 16x16x32 MFMAs, the
//     tree rows as one extra split) of which two workgroups share a CU; it
//     hides the prefix stream's latency better at these few rows;
//   * more (256-row trees, GQA): attn_tile_mfma, below.
// attn_tile_mfma:
//   * every wave owns 32 query rows as one 32-column tile of
//     v_mfma_f32_32x32x16_bf16;
//   * the keys of a (sequence, KV head) are cut into splits; a split takes a
//     range of the paged prefix and a share of the tree keys, so no split is
//     tree-only; one workgroup (4 waves) per split and query tile;
//   * 32-key tiles of K and V reach LDS straight from memory
//     (global_load_lds_dwordx4, no staging registers), several tiles in
//     flight, each stage its own LDS object so that reading one stage never
//     waits for the fill of another; rows keep their 16-byte chunks XOR-ed by
//     2 (key mod 8), which spreads both the K operand reads and the transposed
//     V reads over the banks;
//   * S^T = K . Q^T puts each query in one lane column (a column's maximum is
//     one cross-lane swap away) and leaves the probabilities in the B-operand
//     layout of O^T = V^T . P^T; V^T comes from the row-major V tile through
//     gfx950's transposing LDS read (ds_read_b64_tr_b16), with the keys of a
//     16-key step permuted identically on both operands;
//   * eight waves per workgroup split the queries and share every K/V tile
//     (up to 256 rows), or split the keys into groups that merge their
//     states in LDS at the end (128 rows: two groups); the query tiles of one
//     split run on the same XCD (workgroup ids 8 apart), so all but the first
//     read the tiles from L2;
//   * the tree keys are masked by the ancestor table (v visible to u iff
//     anc[u][depth v] == v), no dense mask;
//   * splits write unnormalised partials; a combine kernel merges them with
//     their log-sum-exps and rounds the output to bf16.
#include "common.h"

namespace hydra {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

constexpr int kTK = 32;                     // keys per tile
constexpr int kD = 128;                     // head dim of the matrix-core path
constexpr int kTileElems = kTK * kD;        // one K or V tile: 8 KB
constexpr int kMaxWGPages = 2048;           // page ids a workgroup stages in LDS

// The running offset of a row moves only when a tile's maximum exceeds it by
// more than this (log2 units): probabilities stay below 2^8, and most tiles
// skip rescaling the accumulators.
constexpr float kRescaleSlack = 8.f;

struct AttnArgs {
  int B, N, Hq, Hkv, G, Dmax;
  float scale_log2;
  const bf16_t* q;
  const bf16_t* k_tree;
  const bf16_t* v_tree;
  const bf16_t* k_pages;
  const bf16_t* v_pages;
  int n_pages, page_shift, max_pages;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int32_t* anc;
  const int32_t* depth;
  int S;        // splits per (sequence, KV head)
  int QT;       // query tiles per (sequence, KV head)
  int NQ;       // query rows per (sequence, KV head) = N * G
  int NQpad;    // QT * rows per tile
  int nchunks;  // B * Hkv * S
  float* opart;
  float* mpart;
  float* lpart;
};

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// max / sum of the two lanes l and l ^ 32 (one column of a 32 x 32 tile): the
// gfx950 swap hands each lane its partner's value, and the pair {a[0], a[1]}
// holds the lane's own value and its partner's (in an order that depends on
// the half), so both halves get the same result
__device__ __forceinline__ float pair_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// 32-bit LDS address of a pointer into a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Transposing LDS read (8 bytes per lane) issued as an instruction the
// compiler does not track: it cannot tell these reads from the tiles still
// being filled by DMA and would wait for every fill before them. The caller
// waits for them with lds_wait, which threads the values through so nothing
// reads them earlier.
template <int OFF>
__device__ __forceinline__ u32x2_t tr_read(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// Workgroup barrier without the memory fence of __syncthreads (whose release
// half waits for every outstanding load, the tile fills included); the
// memory clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// f(integral_constant<int, I>) for I = I0 .. N - 1, unrolled
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int QC, int WQ, int WK, int NS>
__global__ __launch_bounds__(64 * WQ * WK, 1) void attn_tile_mfma(AttnArgs a) {
  static_assert(QC * WQ * WK == 8 && WQ >= 2 && NS >= 2 && NS <= 8 && 16 % WQ == 0, "layout");
  constexpr int NT = 64 * WQ * WK;  // threads
  constexpr int QW = 32 * QC;       // query rows of a wave
  constexpr int QR = QW * WQ;       // query rows of the workgroup
  constexpr int INS = 16 / WQ;      // 1 KB DMA instructions per wave per tile (16 per tile)
  __shared__ __align__(16) bf16_t st0[WK][2][kTileElems];
  __shared__ __align__(16) bf16_t st1[NS > 1 ? WK : 1][2][NS > 1 ? kTileElems : 8];
  __shared__ __align__(16) bf16_t st2[NS > 2 ? WK : 1][2][NS > 2 ? kTileElems : 8];
  __shared__ __align__(16) bf16_t st3[NS > 3 ? WK : 1][2][NS > 3 ? kTileElems : 8];
  __shared__ __align__(16) bf16_t st4[NS > 4 ? WK : 1][2][NS > 4 ? kTileElems : 8];
  __shared__ __align__(16) bf16_t st5[NS > 5 ? WK : 1][2][NS > 5 ? kTileElems : 8];
  __shared__ __align__(16) bf16_t st6[NS > 6 ? WK : 1][2][NS > 6 ? kTileElems : 8];
  __shared__ __align__(16) bf16_t st7[NS > 7 ? WK : 1][2][NS > 7 ? kTileElems : 8];
  __shared__ int s_pages[kMaxWGPages];
  __shared__ int s_dep[HYDRA_MAX_VERIFY];
  __shared__ int s_anc[QR][HYDRA_MAX_DEPTH + 1];
  // per stage and key of a tile: -1 masked, -2 prefix key, else tree key depth
  __shared__ __align__(16) int s_kd[WK][NS][kTK];

  // the wave index is uniform: readfirstlane keeps everything derived from it
  // (tile counts, pipeline branches) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave % WQ, wk = wave / WQ;
  const int hl = lane >> 5, l32 = lane & 31;

  // workgroup -> (query tile, split, sequence, KV head): id runs on XCD id % 8,
  // and the query tiles of one split take consecutive slots of one XCD
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int qt = slot % a.QT;
  const int chunk = (slot / a.QT) * 8 + xcd;
  if (chunk >= a.nchunks) return;  // whole workgroup: no barrier is pending
  const int split = chunk % a.S;
  const int b = (chunk / a.S) / a.Hkv, hkv = (chunk / a.S) % a.Hkv;
  const int G = a.G, N = a.N;
  const int page_size = 1 << a.page_shift;

  // this split's keys: prefix range [p0, p1) (whole tiles from p0) and the
  // tree tiles t0 + S j
  int L = a.prefix_len[b];
  const int cap = a.max_pages << a.page_shift;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int per = (L + a.S - 1) / a.S;
  const int lsp = (per + kTK - 1) / kTK * kTK;
  const int p0 = min(L, split * lsp), p1 = min(L, p0 + lsp);
  const int npt = (p1 - p0 + kTK - 1) / kTK;
  const int ntt = (N + kTK - 1) / kTK;
  const int t0 = a.S - 1 - split;
  const int ntr = t0 < ntt ? (ntt - 1 - t0) / a.S + 1 : 0;

  // tree depths (the DMA issue reads them) with the first page ids; the
  // ancestor rows and Q, needed only once tiles are computed, are loaded
  // after the first tiles' DMA is in flight
  if (ntr > 0)
    for (int e = tid; e < N; e += NT) s_dep[e] = a.depth[static_cast<size_t>(b) * N + e];
  const int q0 = qt * QR + wq * QW;
  bf16x8_t qreg[QC][8];
  // Q^T operands: column l32 of tile c is query row q0 + 32 c + l32, dims
  // 16 ks + 8 hl .. + 7
  auto load_q = [&]() __attribute__((always_inline)) {
    if (ntr > 0) {
      for (int e = tid; e < QR * (a.Dmax + 1); e += NT) {
        const int rr = e / (a.Dmax + 1), j = e % (a.Dmax + 1);
        const int qi = qt * QR + rr;
        s_anc[rr][j] = qi < a.NQ ? a.anc[(static_cast<size_t>(b) * N + qi / G) * (a.Dmax + 1) + j] : -1;
      }
    }
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const int qi = q0 + 32 * c + l32;
      const bool qv = qi < a.NQ;
      const int u = qv ? qi / G : 0, gq = qv ? qi % G : 0;
      const bf16_t* qp = a.q + ((static_cast<size_t>(b) * N + u) * a.Hq + hkv * G + gq) * kD + 8 * hl;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4_t v = qv ? *reinterpret_cast<const u32x4_t*>(qp + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u};
        qreg[c][ks] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  };

  float m_run[QC], l_run[QC];
  f32x16_t oacc[QC][4];
#pragma unroll
  for (int c = 0; c < QC; ++c) m_run[c] = -INFINITY, l_run[c] = 0.f;
#pragma unroll
  for (int c = 0; c < QC; ++c)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[c][dt][r] = 0.f;

  const size_t pstride = static_cast<size_t>(a.Hkv) << (a.page_shift + 7);  // elements per page
  const size_t head_off = static_cast<size_t>(hkv) << (a.page_shift + 7);
  const size_t tree_stride = static_cast<size_t>(a.Hkv) * kD;
  const size_t tree_base = (static_cast<size_t>(b) * N * a.Hkv + hkv) * kD;
  // K operand of this lane: key row l32, chunk 2 ks + hl at (2 ks + hl) ^ kx.
  // K rows keep chunk c of key r at c ^ 2 (r % 8) ^ ((r / 16) % 2): a 16-byte
  // read is served 16 lanes at a time (lanes 0-7 with 16-23, 8-15 with
  // 24-31, ...), which here are keys r and r + 16 of one chunk; the last
  // term puts those two in different bank groups (without it half of the
  // LDS cycles went to bank conflicts). V rows keep c ^ 2 (r % 8).
  const int krow = l32 * kD;
  const int kx = (2 * (l32 & 7)) ^ ((l32 >> 4) & 1);
  // V^T operands: lane 4 i + q of each 16-lane group points at key
  // 16 kc + 4 hl + 8 t + i, dims 32 dt + 16 (group % 2) + 4 q .. + 3; the
  // swizzle depends on the key mod 8 only, so kc and t are offsets
  const int grp = lane >> 4, li = (lane >> 2) & 3, lq = lane & 3;
  int voff[4];  // bytes from the tile's V base, per dt
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int row = 4 * hl + li;
    const int d0 = 32 * dt + 16 * (grp & 1) + 4 * lq;
    voff[dt] = 2 * (row * kD + (((d0 >> 3) ^ (2 * (row & 7))) << 3) + (d0 & 7));
  }

  auto stage_ptr = [&](auto ST) __attribute__((always_inline)) -> bf16_t* {
    constexpr int sti = decltype(ST)::value;
    if constexpr (sti == 0) return &st0[wk][0][0];
    else if constexpr (sti == 1) return &st1[wk][0][0];
    else if constexpr (sti == 2) return &st2[wk][0][0];
    else if constexpr (sti == 3) return &st3[wk][0][0];
    else if constexpr (sti == 4) return &st4[wk][0][0];
    else if constexpr (sti == 5) return &st5[wk][0][0];
    else if constexpr (sti == 6) return &st6[wk][0][0];
    else return &st7[wk][0][0];
  };

  // per-lane byte offsets of the DMA sources: row lane / 16 of an
  // instruction's four, chunk (lane % 16) ^ 2 (row % 8) with row % 8 =
  // 4 (ins % 2) + lane / 16
  const int lrow = lane >> 4;
  uint32_t lchunk[2], loff_pool[2], loff_tree[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int ch = (lane & 15) ^ (2 * (4 * par + lrow));
    lchunk[par] = ch * 16;
    loff_pool[par] = lrow * kD * 2 + ch * 16;
    loff_tree[par] = static_cast<uint32_t>(lrow * tree_stride * 2) + ch * 16;
  }

  // Windows of prefix tiles whose page ids fit in LDS (one window unless a
  // split is longer than kWinTiles tiles); the tree tiles run in the last.
  constexpr int kWinTiles = kMaxWGPages / 2 - 1;
  for (int w0 = 0;; w0 += kWinTiles) {
    const int wnp = max(0, min(npt - w0, kWinTiles));
    const bool last = w0 + kWinTiles >= npt;
    const int T = wnp + (last ? ntr : 0);
    const int wp0 = p0 + kTK * w0;                    // first key of the window
    const int wp1 = min(p1, wp0 + kTK * kWinTiles);   // end of its prefix keys
    const int pg0 = wp0 >> a.page_shift;
    const int npg = wp1 > wp0 ? ((wp1 - 1) >> a.page_shift) - pg0 + 1 : 0;
    if (w0 > 0) __syncthreads();  // the previous window's readers are done
    int bad = 0;
    for (int e = tid; e < npg; e += NT) {
      const int pg = a.block_table[static_cast<size_t>(b) * a.max_pages + pg0 + e];
      s_pages[e] = pg;
      bad |= pg < 0 || pg >= a.n_pages;
    }
    const bool pages_ok = __syncthreads_or(bad) == 0;

    // tiles of this key group: window tile wk + WK j, j < Tg (every group runs
    // Tmax iterations so that shared-tile barriers pair up)
    const int Tg = T > wk ? (T - 1 - wk) / WK + 1 : 0;
    const int Tmax = (T + WK - 1) / WK;

    // DMA of this wave's share of group tile j into stage ST: instruction ins
    // (0..15) fills rows 4 (ins % 8) .. + 3 of K (ins < 8) or V; lane i writes
    // position i % 16 of row i / 16 there, i.e. chunk (i % 16) ^ 2 (row % 8)
    // (K rows 16 .. 31: also ^ 1).
    // The four keys of an instruction are consecutive slots of one page (or
    // four consecutive tree rows), so the source is a wave-uniform base (page
    // and slot, computed on the scalar unit) plus a per-lane offset fixed for
    // the launch. The K instructions also record each key's mask code in s_kd.
    auto issue = [&](auto ST, int j) __attribute__((always_inline)) {
      if (j >= Tg) return;
      const int i = wk + WK * j;
      bf16_t* kd = stage_ptr(ST);
#pragma unroll
      for (int n = 0; n < INS; ++n) {
        const int ins = wq * INS + n;
        const int tensor = ins >> 3;
        const int par = ins & 1;
        // K rows 16 .. 31 of the tile (K instructions 4 .. 7) take the extra
        // chunk swizzle; bit 4 of a per-lane source offset is bit 0 of its chunk
        const uint32_t flip = tensor == 0 ? static_cast<uint32_t>((ins >> 2) & 1) << 4 : 0u;
        const char* src;
        int code;
        if (i < wnp) {
          const int tu = wp0 + kTK * i + 4 * (ins & 7);  // first key of the instruction
          int pg = tu < wp1 ? __builtin_amdgcn_readfirstlane(s_pages[(tu >> a.page_shift) - pg0]) : -1;
          const bool pvalid = pg >= 0 && pg < a.n_pages;
          code = pvalid && tu + lrow < wp1 ? -2 : -1;
          int slot0 = tu & (page_size - 1);
          if (!pvalid) {  // masked: read four mapped slots instead
            pg = __builtin_amdgcn_readfirstlane(s_pages[0]);
            pg = pg >= 0 && pg < a.n_pages ? pg : 0;
            slot0 = 0;
          }
          const bf16_t* base = (tensor ? a.v_pages : a.k_pages) + pg * pstride + head_off +
                               (static_cast<size_t>(slot0) << 7);
          src = reinterpret_cast<const char*>(base) + (loff_pool[par] ^ flip);
        } else {
          const int vu = kTK * (t0 + a.S * (i - wnp)) + 4 * (ins & 7);  // first tree row
          const int v = vu + lrow;
          const int dv = v < N ? s_dep[v] : -1;
          code = dv >= 0 && dv <= a.Dmax ? dv : -1;
          const bf16_t* tb = tensor ? a.v_tree : a.k_tree;
          if (vu + 3 < N) {
            src = reinterpret_cast<const char*>(tb + tree_base + vu * tree_stride) + (loff_tree[par] ^ flip);
          } else {  // the last rows: clamp each lane's row
            const int vc = v < N ? v : N - 1;
            src = reinterpret_cast<const char*>(tb + tree_base + vc * tree_stride) + (lchunk[par] ^ flip);
          }
        }
        if (tensor == 0 && (lane & 15) == 0) s_kd[wk][decltype(ST)::value][4 * (ins & 7) + lrow] = code;
        __builtin_amdgcn_global_load_lds((glb_void_t*)src,
                                         (lds_void_t*)(kd + tensor * kTileElems + 4 * (ins & 7) * kD), 16, 0, 0);
      }
    };

    // one tile from stage ST: S^T, online softmax, O^T += V^T P^T
    auto compute = [&](auto ST, int j) __attribute__((always_inline)) {
      const bf16_t* kt = stage_ptr(ST);
      const uint32_t vb = lds_addr(kt + kTileElems);
      const int i = wk + WK * j;
      f32x16_t sacc[QC];
#pragma unroll
      for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[c][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t ka =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(kt + krow + (((2 * ks + hl) ^ kx) << 3)));
#pragma unroll
        for (int c = 0; c < QC; ++c)
          sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c][ks], sacc[c], 0, 0, 0);
      }
      // V^T operands, in flight during the softmax: [kc][dt][t]
      u32x2_t vr[2][4][2];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        vr[0][dt][0] = tr_read<0>(vb + voff[dt]);
        vr[0][dt][1] = tr_read<8 * kD * 2>(vb + voff[dt]);
        vr[1][dt][0] = tr_read<16 * kD * 2>(vb + voff[dt]);
        vr[1][dt][1] = tr_read<24 * kD * 2>(vb + voff[dt]);
      }
      // scores of lane: key 8 (r / 4) + 4 hl + r % 4 of the tile, query column l32
      const bool tree_tile = i >= wnp;
      const bool masked = tree_tile || !pages_ok || wp0 + kTK * (i + 1) > wp1;
      if (masked) {
        // mask codes of this lane's keys 8 g + 4 hl + 0..3 (g = 0..3)
        const int* kcode = &s_kd[wk][decltype(ST)::value][4 * hl];
        const int vb0 = tree_tile ? kTK * (t0 + a.S * (i - wnp)) : 0;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int4 k4 = *reinterpret_cast<const int4*>(kcode + 8 * g4);
          const int kc4[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e, code = kc4[e];
            const int v = vb0 + 8 * g4 + 4 * hl + e;
#pragma unroll
            for (int c = 0; c < QC; ++c) {
              const bool vis = tree_tile ? code >= 0 && s_anc[wq * QW + 32 * c + l32][code < 0 ? 0 : code] == v
                                         : code != -1;
              sacc[c][r] = vis ? sacc[c][r] : -INFINITY;
            }
          }
        }
      }
      bf16x8_t pb[QC][2];
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        float mt = sacc[c][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[c][r]);
        mt = pair_max(mt) * a.scale_log2;
        const bool grow = mt > m_run[c] + kRescaleSlack;
        if (__any(grow)) {  // wave-uniform: rescale only when an offset moved
          const float m_new = grow ? fmaxf(m_run[c], mt) : m_run[c];
          const float alpha = m_new == m_run[c] ? 1.f : __builtin_amdgcn_exp2f(m_run[c] - m_new);
          l_run[c] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[c][dt] *= alpha;
          m_run[c] = m_new;
        }
        const float neg_m = m_run[c] == -INFINITY ? 0.f : -m_run[c];
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[c][r], a.scale_log2, neg_m));
          ps += pe;
          pb[c][r >> 3][r & 7] = static_cast<__bf16>(pe);
        }
        l_run[c] += ps;
      }
      // the transposed reads have landed: thread their values through the wait
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vr[0][0][0]), "+v"(vr[0][0][1]), "+v"(vr[0][1][0]), "+v"(vr[0][1][1]),
                     "+v"(vr[0][2][0]), "+v"(vr[0][2][1]), "+v"(vr[0][3][0]), "+v"(vr[0][3][1]),
                     "+v"(vr[1][0][0]), "+v"(vr[1][0][1]), "+v"(vr[1][1][0]), "+v"(vr[1][1][1]),
                     "+v"(vr[1][2][0]), "+v"(vr[1][2][1]), "+v"(vr[1][3][0]), "+v"(vr[1][3][1]));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4_t w = {vr[kc][dt][0].x, vr[kc][dt][0].y, vr[kc][dt][1].x, vr[kc][dt][1].y};
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
          for (int c = 0; c < QC; ++c)
            oacc[c][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c][kc], oacc[c][dt], 0, 0, 0);
        }
      }
    };

    // pipeline: NS - 1 tiles in flight ahead of the one being computed
    auto iter = [&](auto ST, int j) __attribute__((always_inline)) {
      constexpr int sti = decltype(ST)::value;
      if (j + NS - 2 < Tg) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * INS));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      // every wave's share of tile j landed; every wave finished tile j - 1
      if constexpr (WQ > 1) barrier_only();
      issue(std::integral_constant<int, (sti + NS - 1) % NS>{}, j + NS - 1);
      if (j < Tg) compute(ST, j);
    };
    auto prologue = [&](auto P) __attribute__((always_inline)) { issue(P, decltype(P)::value); };
    static_for<0, NS - 1>(prologue);
    if (w0 == 0) load_q();
    for (int j0 = 0; j0 < Tmax; j0 += NS) {
      auto step = [&](auto P) __attribute__((always_inline)) {
        if (j0 + decltype(P)::value < Tmax) iter(P, j0 + decltype(P)::value);
      };
      static_for<0, NS>(step);
    }
    if (last) break;
  }

  // column sums: each lane holds half of its column's keys
#pragma unroll
  for (int c = 0; c < QC; ++c) l_run[c] = pair_sum(l_run[c]);

  if constexpr (WK > 1) {
    // key groups 1.. hand their states to group 0 through LDS (the stages
    // are free once every wave is past its loop): O^T of a wave is QC * 16 KB
    // and a stage object holds 16 WK KB
    constexpr int kSlotFloats = QC * 4 * 16 * 64;
    constexpr int per_obj = WK / QC;
    static_assert(per_obj >= 1 && (WK - 1) * WQ <= NS * per_obj, "hand-over area");
    auto xo_of = [&](int s) -> float* {
      const int obj = s / per_obj;
      float* base = obj == 0 ? reinterpret_cast<float*>(&st0[0][0][0])
                  : obj == 1 ? reinterpret_cast<float*>(&st1[0][0][0])
                  : obj == 2 ? reinterpret_cast<float*>(&st2[0][0][0])
                             : reinterpret_cast<float*>(&st3[0][0][0]);
      return base + (s % per_obj) * kSlotFloats;
    };
    float* xm = reinterpret_cast<float*>(&s_pages[0]);  // [2][WK - 1][WQ][QC][64]: m, then l
    constexpr int kML = (WK - 1) * WQ * QC * 64;
    static_assert(2 * kML <= kMaxWGPages, "m and l hand-over");
    __syncthreads();
    if (wk > 0) {
      const int slotw = (wk - 1) * WQ + wq;
      float* xo = xo_of(slotw);
#pragma unroll
      for (int c = 0; c < QC; ++c) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) xo[(((c * 4 + dt) * 16 + r) << 6) + lane] = oacc[c][dt][r];
        xm[((slotw * QC + c) << 6) + lane] = m_run[c];
        xm[kML + ((slotw * QC + c) << 6) + lane] = l_run[c];
      }
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      float M = m_run[c];
      for (int o = 1; o < WK; ++o) M = fmaxf(M, xm[((((o - 1) * WQ + wq) * QC + c) << 6) + lane]);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float w0 = __builtin_amdgcn_exp2f(m_run[c] - Mu);
      l_run[c] *= w0;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[c][dt] *= w0;
      for (int o = 1; o < WK; ++o) {
        const int slotw = (o - 1) * WQ + wq;
        const float* xo = xo_of(slotw);
        const float wo = __builtin_amdgcn_exp2f(xm[((slotw * QC + c) << 6) + lane] - Mu);
        l_run[c] += wo * xm[kML + ((slotw * QC + c) << 6) + lane];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[c][dt][r] += wo * xo[(((c * 4 + dt) * 16 + r) << 6) + lane];
      }
      m_run[c] = M;
    }
  }

  // unnormalised partial of this split: rows (split, b, hkv, query)
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int qi = q0 + 32 * c + l32;
    if (qi < a.NQ) {
      const size_t row = (static_cast<size_t>(split * a.B + b) * a.Hkv + hkv) * a.NQpad + qi;
      float* op = a.opart + row * kD + 4 * hl;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<float4*>(op + 32 * dt + 8 * r4) =
              make_float4(oacc[c][dt][4 * r4], oacc[c][dt][4 * r4 + 1], oacc[c][dt][4 * r4 + 2],
                          oacc[c][dt][4 * r4 + 3]);
      if (hl == 0) {
        a.mpart[row] = m_run[c];
        a.lpart[row] = l_run[c];
      }
    }
  }
}

constexpr int kMaxSplitPages = 1024;  // page ids a split of the streaming kernel stages in LDS

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query column
// of a 16 x 16 S^T tile): the gfx950 row swaps hand every lane its partner's
// value in a VALU step
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

// Streaming kernel for up to 64 query rows per KV head (the 64-node MHA
// trees): NW waves of RT 16-row query tiles each (16 NW RT query rows); a
// thread loads KPT keys x 8 dims of K and V into registers, so a tile holds
// 4 NW KPT keys, and PD tiles are in flight; 16x16x32 MFMAs on S^T = K Q^T
// and O^T = V^T P^T with V transposed into LDS as it is stored; the tree rows
// are one extra split of their own, masked by the ancestor table. Small
// (about 40 KB of LDS) so that two workgroups share a CU and the tree split
// overlaps the prefix splits.
template <int NW, int RT, int PD, int KPT>
__global__ __launch_bounds__(NW * 64, 2) void attn_split_mfma(
    int B, int N, int Hq, int Hkv, float scale_log2, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k_tree, const bf16_t* __restrict__ v_tree,
    const bf16_t* __restrict__ k_pages, const bf16_t* __restrict__ v_pages, int n_pages,
    int page_shift, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ anc,
    const int32_t* __restrict__ depth, int Dmax, int nsplit, int NQ, int NQpad,
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

  // this split's share of the sequence's own prefix (the split count is
  // planned, the range length follows the sequence), in windows whose page
  // ids fit the LDS staging area
  int L = prefix_len[b];
  const int cap = max_pages << page_shift;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int lsp = nsplit > 0 ? ((L + nsplit - 1) / nsplit + TK - 1) / TK * TK : 0;
  const int s_begin = tree_part ? 0 : min(L, split * lsp);
  const int s_end = tree_part ? N : min(L, s_begin + lsp);
  constexpr int kWinKeys = (kMaxSplitPages - 1) * 16 / TK * TK;
  const int32_t* dep_b = depth + static_cast<size_t>(b) * N;
  if (tree_part) {
    for (int e = tid; e < QR * (Dmax + 1); e += NT) {
      const int rr = e / (Dmax + 1), j = e % (Dmax + 1);
      const int qr = qtile * QR + rr;
      s_anc[rr][j] = qr < NQ ? anc[(static_cast<size_t>(b) * N + qr / G) * (Dmax + 1) + j] : -1;
    }
  }

  float m_run[RT], l_run[RT];
  f32x4_t oacc[RT][DD];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) oacc[r][dd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int wb = s_begin;; wb += kWinKeys) {
  const int t_begin = wb;
  const int t_end = tree_part ? s_end : min(s_end, wb + kWinKeys);
  const int p0 = t_begin >> page_shift;
  if (wb > s_begin) __syncthreads();  // the previous window's tiles are consumed
  int pages_bad = 0;
  if (!tree_part) {
    const int np = t_end > t_begin ? ((t_end - 1) >> page_shift) - p0 + 1 : 0;
    for (int e = tid; e < np; e += NT) {
      const int pg = block_table[static_cast<size_t>(b) * max_pages + p0 + e];
      s_pages[e] = pg;
      pages_bad |= pg < 0 || pg >= n_pages;
    }
  }
  // every page of the window valid: whole tiles then need no mask (the
  // barrier also publishes the ancestor rows)
  const bool pages_ok = __syncthreads_or(pages_bad) == 0;

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

  using Whole = std::true_type;
  using Part = std::false_type;
  // whole prefix tiles over valid pages run unmasked in a loop of their own
  // (PD at a time, one per register slot), the rest masked; tile i lives in
  // slot i % PD and its slot's refill fetches tile i + PD
  const int ntiles = t_end > t_begin ? (t_end - t_begin + TK - 1) / TK : 0;
  const int nwhole = tree_part || !pages_ok ? 0 : (t_end - t_begin) / TK / PD * PD;
  auto prologue = [&](auto SLOT) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    if (sl < ntiles) {
      if (sl < nwhole) load_tile(SLOT, Whole{}, t_begin + sl * TK);
      else load_tile(SLOT, Part{}, t_begin + sl * TK);
    }
  };
  static_for<0, PD>(prologue);
  int it = 0;
  for (; it < nwhole; it += PD) {
    auto whole_step = [&](auto SLOT) __attribute__((always_inline)) {
      process(SLOT, Whole{}, t_begin + (it + decltype(SLOT)::value) * TK);
    };
    static_for<0, PD>(whole_step);
  }
  for (; it < ntiles; it += PD) {
    auto part_step = [&](auto SLOT) __attribute__((always_inline)) {
      if (it + decltype(SLOT)::value < ntiles) process(SLOT, Part{}, t_begin + (it + decltype(SLOT)::value) * TK);
    };
    static_for<0, PD>(part_step);
  }

  if (tree_part || t_end >= s_end) break;
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


struct TilePlan {
  int qc, wq, wk, ns;  // 32-row query tiles per wave, waves along queries, key groups, stages
  int S, QT, NQ, NQpad;
};

// Waves split the queries when a KV head has more than 64 query rows, else
// the keys; splits aim at about one workgroup per CU (each at least four
// tiles of the longest prefix, and short enough that its page ids fit the
// LDS staging area). Each sequence cuts its own prefix into S equal ranges,
// so the plan only sizes the work: any prefix_len up to the block table's
// capacity is covered whatever max_prefix_len says.
TilePlan plan_tiles(int B, int N, int Hq, int Hkv, int max_prefix_len) {
  TilePlan p;
  p.NQ = N * (Hq / Hkv);
  // eight waves of 32 query rows (two per SIMD)
  p.qc = 1;
  if (p.NQ <= 64) {
    p.wq = 2, p.wk = 4, p.ns = 2;
  } else if (p.NQ <= 128) {
    p.wq = 4, p.wk = 2, p.ns = 4;
  } else {
    p.wq = 8, p.wk = 1, p.ns = 6;
  }
  const int qr = 32 * p.qc * p.wq;
  p.QT = (p.NQ + qr - 1) / qr;
  p.NQpad = p.QT * qr;
  const long long units = static_cast<long long>(B) * Hkv * p.QT;
  const int Lr = max_prefix_len > 0 ? max_prefix_len : 0;
  long long S = (256 + units / 2) / units;
  const long long smax = (Lr + 4 * kTK - 1) / (4 * kTK);
  if (S > smax) S = smax;
  const long long smin = (Lr + (kMaxWGPages - 2) * 16 - 1) / ((kMaxWGPages - 2) * 16);
  if (S < smin) S = smin;
  if (S < 1) S = 1;
  p.S = static_cast<int>(S);
  return p;
}

// Streaming kernel plan (up to 64 query rows per KV head): about 512
// workgroups, each split at least four 64-key tiles (and at most 16) of the
// planned prefix, at least one split so that prefixes beyond the plan are
// still covered; the tree rows are the extra split.
struct SplitPlan {
  int nsplit, NQ, NQpad;
};
SplitPlan plan_splits(int B, int N, int Hq, int Hkv, int max_prefix_len) {
  constexpr int TK = 64;
  SplitPlan p;
  p.NQ = N * (Hq / Hkv);
  p.NQpad = 64;
  const int base = B * Hkv;
  const int Lr = max_prefix_len > 0 ? max_prefix_len : 0;
  int s = 512 / base - 1;  // the tree split takes one slot
  const int maxs = (Lr + 4 * TK - 1) / (4 * TK);
  if (s > maxs) s = maxs;
  const int mins = (Lr + 16 * TK - 1) / (16 * TK);
  if (s < mins) s = mins;
  if (s < 1) s = 1;
  int ls = (Lr + s - 1) / s;
  ls = (ls + TK - 1) / TK * TK;
  if (ls < TK) ls = TK;
  p.nsplit = Lr > 0 ? (Lr + ls - 1) / ls : 1;
  return p;
}

bool use_mfma(int dtype, int D) { return dtype == HYDRA_BF16 && D == 128; }
bool use_streaming(int N, int Hq, int Hkv) { return N * (Hq / Hkv) <= 64; }

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" size_t tree_attention_verify_workspace_size(int dtype, int B, int N, int Hq, int Hkv, int D,
                                                       int max_prefix_len) {
  if (!use_mfma(dtype, D) || B <= 0 || N <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv) return 0;
  size_t rows;
  if (use_streaming(N, Hq, Hkv)) {
    const SplitPlan p = plan_splits(B, N, Hq, Hkv, max_prefix_len);
    rows = static_cast<size_t>(p.nsplit + 1) * B * Hkv * p.NQpad;
  } else {
    const TilePlan p = plan_tiles(B, N, Hq, Hkv, max_prefix_len);
    rows = static_cast<size_t>(p.S) * B * Hkv * p.NQpad;
  }
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
  HY_CHECK(n_pages >= 1 && k_pages && v_pages, HYDRA_ERR_INVALID,
           "tree_attention: a page pool (n_pages >= 1, K and V) is needed");
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

  Arena arena(ws, ws_bytes);
  const float scale_log2 = scale * 1.4426950408889634f;
  const int page_shift = page_size == 16 ? 4 : (page_size == 32 ? 5 : 6);
  if (use_streaming(N, Hq, Hkv)) {
    const SplitPlan p = plan_splits(B, N, Hq, Hkv, max_prefix_len);
    const int nparts = p.nsplit + 1;
    const size_t rows = static_cast<size_t>(nparts) * B * Hkv * p.NQpad;
    float* opart = arena.take<float>(rows * D);
    float* mpart = arena.take<float>(rows);
    float* lpart = arena.take<float>(rows);
    attn_split_mfma<4, 1, 2, 4><<<dim3(nparts, 1, B * Hkv), 256, 0, stream>>>(
        B, N, Hq, Hkv, scale_log2, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_tree),
        static_cast<const bf16_t*>(v_tree), static_cast<const bf16_t*>(k_pages), static_cast<const bf16_t*>(v_pages),
        n_pages, page_shift, block_table, max_pages, prefix_len, anc, depth, Dmax, p.nsplit, p.NQ, p.NQpad, opart,
        mpart, lpart);
    HY_LAUNCH_CHECK("tree_attention(split)");
    const long long cthreads = static_cast<long long>(B) * Hkv * p.NQ * (D / 4);
    attn_combine<bf16_t><<<static_cast<int>((cthreads + 255) / 256), 256, 0, stream>>>(
        B, N, Hq, Hkv, D, nparts, p.NQ, p.NQpad, opart, mpart, lpart, static_cast<bf16_t*>(out), lse);
    HY_LAUNCH_CHECK("tree_attention(combine)");
    return HYDRA_OK;
  }
  const TilePlan p = plan_tiles(B, N, Hq, Hkv, max_prefix_len);
  const size_t rows = static_cast<size_t>(p.S) * B * Hkv * p.NQpad;
  AttnArgs a;
  a.B = B, a.N = N, a.Hq = Hq, a.Hkv = Hkv, a.G = Hq / Hkv, a.Dmax = Dmax;
  a.scale_log2 = scale_log2;
  a.q = static_cast<const bf16_t*>(q);
  a.k_tree = static_cast<const bf16_t*>(k_tree);
  a.v_tree = static_cast<const bf16_t*>(v_tree);
  a.k_pages = static_cast<const bf16_t*>(k_pages);
  a.v_pages = static_cast<const bf16_t*>(v_pages);
  a.n_pages = n_pages, a.max_pages = max_pages;
  a.page_shift = page_shift;
  a.block_table = block_table, a.prefix_len = prefix_len, a.anc = anc, a.depth = depth;
  a.S = p.S, a.QT = p.QT, a.NQ = p.NQ, a.NQpad = p.NQpad;
  a.nchunks = B * Hkv * p.S;
  a.opart = arena.take<float>(rows * D);
  a.mpart = arena.take<float>(rows);
  a.lpart = arena.take<float>(rows);
  const int grid = (a.nchunks + 7) / 8 * 8 * p.QT;
  const int nt = 64 * p.wq * p.wk;
  if (p.wq == 2) attn_tile_mfma<1, 2, 4, 2><<<grid, nt, 0, stream>>>(a);
  else if (p.wq == 4) attn_tile_mfma<1, 4, 2, 4><<<grid, nt, 0, stream>>>(a);
  else attn_tile_mfma<1, 8, 1, 6><<<grid, nt, 0, stream>>>(a);
  HY_LAUNCH_CHECK("tree_attention(tiles)");
  const long long cthreads = static_cast<long long>(B) * Hkv * p.NQ * (D / 4);
  attn_combine<bf16_t><<<static_cast<int>((cthreads + 255) / 256), 256, 0, stream>>>(
      B, N, Hq, Hkv, D, p.S, p.NQ, p.NQpad, a.opart, a.mpart, a.lpart, static_cast<bf16_t*>(out), lse);
  HY_LAUNCH_CHECK("tree_attention(combine)");
  return HYDRA_OK;
}
