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
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// 16-byte LDS read the compiler does not track (see tr_read), at a constant
// offset from addr; the caller waits for it with an s_waitcnt that threads
// the value through
template <int OFF>
__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// attn_tile_mfma: 8 waves, each 32 query rows of one (sequence, KV head);
// WQ waves along the queries, WK key groups. Per key group a ring of four
// stages (K and V of one 32-key tile, 16 KB) is filled by LDS DMA two tiles
// ahead; the stage index is static in the unrolled loop, so every LDS read
// names its stage by the instruction's offset field.
template <int WQ, int WK>
__global__ __launch_bounds__(512, 1) void attn_tile_mfma(AttnArgs a) {
  static_assert(WQ * WK == 8 && 16 % WQ == 0, "layout");
  constexpr int NS = 4;                           // stages
  constexpr int NT = 512;                         // threads
  constexpr int QR = 32 * WQ;                     // query rows of the workgroup
  constexpr int INS = 16 / WQ;                    // 1 KB DMA instructions per wave per tile (16 per tile)
  constexpr int kStageBytes = 2 * kTileElems * 2;  // a stage: K tile, then V tile
  constexpr int kWinTiles = 128;                  // tiles of a window: page ids in two registers per lane
  static_assert(NS * kStageBytes <= 65536, "stage offsets fit the LDS offset field");
  // stages of each key group: one object, read only through untracked reads
  // (a tracked read would make the compiler wait for every fill in flight)
  __shared__ __align__(16) bf16_t stg[WK][NS][2][kTileElems];
  __shared__ int s_anc[QR][HYDRA_MAX_DEPTH + 1];

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

  const int q0 = qt * QR + wq * 32;
  bf16x8_t qreg[8];
  // Q^T operand: column l32 is query row q0 + l32, dims 16 ks + 8 hl .. + 7;
  // the ancestor rows of the workgroup's queries go to LDS
  auto load_q = [&]() __attribute__((always_inline)) {
    if (ntr > 0) {
      for (int e = tid; e < QR * (a.Dmax + 1); e += NT) {
        const int rr = e / (a.Dmax + 1), j = e % (a.Dmax + 1);
        const int qi = qt * QR + rr;
        s_anc[rr][j] = qi < a.NQ ? a.anc[(static_cast<size_t>(b) * N + qi / G) * (a.Dmax + 1) + j] : -1;
      }
    }
    const int qi = q0 + l32;
    const bool qv = qi < a.NQ;
    const int u = qv ? qi / G : 0, gq = qv ? qi % G : 0;
    const bf16_t* qp = a.q + ((static_cast<size_t>(b) * N + u) * a.Hq + hkv * G + gq) * kD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4_t v = qv ? *reinterpret_cast<const u32x4_t*>(qp + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u};
      qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;

  // K operand of this lane: key row l32, chunk 2 ks + hl at (2 ks + hl) ^ kx.
  // K rows keep chunk c of key r at c ^ 2 (r % 8) ^ ((r / 16) % 2): a 16-byte
  // read is served 16 lanes at a time (lanes 0-7 with 16-23, 8-15 with
  // 24-31, ...), which here are keys r and r + 16 of one chunk; the last
  // term puts those two in different bank groups. V rows keep c ^ 2 (r % 8).
  const uint32_t stg0 = lds_addr(&stg[wk][0][0][0]);
  const int kx = (2 * (l32 & 7)) ^ ((l32 >> 4) & 1);
  uint32_t kaddr[8];  // stage 0 addresses; stage s is s * kStageBytes further
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kaddr[ks] = stg0 + 2 * (l32 * kD + (((2 * ks + hl) ^ kx) << 3));
  // V^T operands: lane 4 i + q of each 16-lane group points at key
  // 16 kc + 4 hl + 8 t + i, dims 32 dt + 16 (group % 2) + 4 q .. + 3; the
  // swizzle depends on the key mod 8 only, so kc and t are offsets
  const int grp = lane >> 4, li = (lane >> 2) & 3, lq = lane & 3;
  uint32_t vaddr[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int row = 4 * hl + li;
    const int d0 = 32 * dt + 16 * (grp & 1) + 4 * lq;
    vaddr[dt] = stg0 + 2 * kTileElems + 2 * (row * kD + (((d0 >> 3) ^ (2 * (row & 7))) << 3) + (d0 & 7));
  }

  // DMA: instruction ins (0..15) of a tile fills rows 4 (ins % 8) .. + 3 of K
  // (ins < 8) or V; lane i writes position i % 16 of row i / 16 there, i.e.
  // chunk (i % 16) ^ 2 (row % 8) (K rows 16 .. 31: also ^ 1, bit 4 of the
  // source offset). This wave issues ins = wq INS .. + INS - 1: one tensor,
  // rows rowbase .. + 4 INS - 1, which lie in one page (pages hold at least
  // 16 keys and tiles start at multiples of 32). The source is a uniform
  // base plus a per-lane 32-bit offset.
  const int lrow = lane >> 4;
  const int tensor = (wq * INS) >> 3;
  const int rowbase = 4 * ((wq * INS) & 7);
  const uint32_t flip = tensor == 0 ? static_cast<uint32_t>(((wq * INS) >> 2) & 1) << 4 : 0u;
  const size_t tree_stride_b = static_cast<size_t>(a.Hkv) * kD * 2;
  uint32_t dofs[INS], dofs_tree[INS];
#pragma unroll
  for (int n = 0; n < INS; ++n) {
    const uint32_t ch = static_cast<uint32_t>((lane & 15) ^ (2 * (4 * (n & 1) + lrow))) * 16;
    dofs[n] = ((lrow * kD * 2 + ch) ^ flip) + n * 4 * kD * 2;
    dofs_tree[n] = static_cast<uint32_t>((lrow + 4 * n) * tree_stride_b) + (ch ^ flip);
  }
  const size_t pstride_b = (static_cast<size_t>(a.Hkv) << (a.page_shift + 7)) * 2;  // bytes per page
  const char* kv_base = reinterpret_cast<const char*>((tensor ? a.v_pages : a.k_pages)) +
                        (static_cast<size_t>(hkv) << (a.page_shift + 7)) * 2;
  const char* tree_b = reinterpret_cast<const char*>(tensor ? a.v_tree : a.k_tree) +
                       ((static_cast<size_t>(b) * N * a.Hkv + hkv) * kD) * 2;

  // Windows of up to kWinTiles prefix tiles (one unless a split is longer);
  // the tree tiles run in the last.
  for (int w0 = 0;; w0 += kWinTiles) {
    const int wnp = max(0, min(npt - w0, kWinTiles));
    const bool last = w0 + kWinTiles >= npt;
    const int T = wnp + (last ? ntr : 0);
    const int wp0 = p0 + kTK * w0;                    // first key of the window
    const int wp1 = min(p1, wp0 + kTK * kWinTiles);   // end of its prefix keys
    if (w0 > 0) __syncthreads();  // the previous window's readers are done
    // page of this wave's rows in window tiles lane and lane + 64 (-1: none
    // or out of range; those keys are masked and read page 0 instead)
    int pgA = -1, pgB = -1, bad = 0;
    {
      const int32_t* bt = a.block_table + static_cast<size_t>(b) * a.max_pages;
      const int kA = wp0 + kTK * lane + rowbase, kB = kA + 64 * kTK;
      if (lane < wnp && kA < wp1) {
        pgA = bt[kA >> a.page_shift];
        bad |= pgA < 0 || pgA >= a.n_pages;
        pgA = pgA < 0 || pgA >= a.n_pages ? -1 : pgA;
      }
      if (lane + 64 < wnp && kB < wp1) {
        pgB = bt[kB >> a.page_shift];
        bad |= pgB < 0 || pgB >= a.n_pages;
        pgB = pgB < 0 || pgB >= a.n_pages ? -1 : pgB;
      }
    }
    const bool pages_ok = __syncthreads_or(bad) == 0;

    // tiles of this key group: window tile wk + WK j, j < Tg (every group runs
    // Tmax iterations so that the shared barriers pair up); the first Tfull
    // are whole prefix tiles
    const int Tg = T > wk ? (T - 1 - wk) / WK + 1 : 0;
    const int Tmax = (T + WK - 1) / WK;
    const int wfull = pages_ok ? (wp1 - wp0) / kTK : 0;
    const int Tfull = wfull > wk ? (wfull - 1 - wk) / WK + 1 : 0;

    // this wave's DMA share of group tile j into stage ST
    auto issue = [&](auto FAST, auto ST, int j) __attribute__((always_inline)) {
      if (!decltype(FAST)::value && j >= Tg) return;
      const int i = wk + WK * j;
      bf16_t* dst = &stg[wk][decltype(ST)::value][tensor][rowbase * kD];
      if (decltype(FAST)::value || i < wnp) {
        int pg = __builtin_amdgcn_readlane(i < 64 ? pgA : pgB, i & 63);
        if (!decltype(FAST)::value) pg = pg >= 0 ? pg : 0;
        const int slot0 = (wp0 + kTK * i + rowbase) & (page_size - 1);  // of the share's first row
        const char* src = kv_base + static_cast<size_t>(pg) * pstride_b + (static_cast<uint32_t>(slot0) << 8);
#pragma unroll
        for (int n = 0; n < INS; ++n)
          __builtin_amdgcn_global_load_lds((glb_void_t*)(src + dofs[n]), (lds_void_t*)(dst + 4 * n * kD), 16, 0, 0);
      } else {
        const int vu = kTK * (t0 + a.S * (i - wnp)) + rowbase;  // first tree row of the share
        if (vu + 4 * INS <= N) {
          const char* src = tree_b + static_cast<size_t>(vu) * tree_stride_b;
#pragma unroll
          for (int n = 0; n < INS; ++n)
            __builtin_amdgcn_global_load_lds((glb_void_t*)(src + dofs_tree[n]), (lds_void_t*)(dst + 4 * n * kD), 16,
                                             0, 0);
        } else {  // the last rows: clamp each lane's row
#pragma unroll
          for (int n = 0; n < INS; ++n) {
            const int v = vu + 4 * n + lrow;
            const int vc = v < N ? v : N - 1;
            const uint32_t ch = static_cast<uint32_t>((lane & 15) ^ (2 * (4 * (n & 1) + lrow))) * 16;
            __builtin_amdgcn_global_load_lds((glb_void_t*)(tree_b + static_cast<size_t>(vc) * tree_stride_b + (ch ^ flip)),
                                             (lds_void_t*)(dst + 4 * n * kD), 16, 0, 0);
          }
        }
      }
    };

    // scores of lane: key 8 (r / 4) + 4 hl + r % 4 of the tile, query column l32
    auto mask = [&](int j, f32x16_t& s) __attribute__((always_inline)) {
      const int i = wk + WK * j;
      if (i >= wnp) {
        // tree rows vb0 .. vb0 + 31: bit k of mk is set when row vb0 + k is
        // in the query's ancestor row (itself included)
        const int vb0 = kTK * (t0 + a.S * (i - wnp));
        const int* ar = &s_anc[wq * 32 + l32][0];
        uint32_t mk = 0;
#pragma unroll
        for (int d = 0; d <= HYDRA_MAX_DEPTH; ++d) {
          if (d <= a.Dmax) {
            const uint32_t o = static_cast<uint32_t>(ar[d] - vb0);
            mk |= o < 32u ? 1u << (o & 31u) : 0u;
          }
        }
        mk >>= 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = (mk >> (8 * (r >> 2) + (r & 3))) & 1u ? s[r] : -INFINITY;
      } else {
        // prefix keys: visible below wp1 and on a valid page
        const int ts = wp0 + kTK * i;
        bool pv0 = true, pv1 = true;  // pages of keys ts .. + 15 and ts + 16 .. + 31
        if (!pages_ok) {
          const int32_t* bt = a.block_table + static_cast<size_t>(b) * a.max_pages;
          const int pa = ts < wp1 ? bt[ts >> a.page_shift] : -1;
          const int pb2 = ts + 16 < wp1 ? bt[(ts + 16) >> a.page_shift] : -1;
          pv0 = pa >= 0 && pa < a.n_pages;
          pv1 = pb2 >= 0 && pb2 < a.n_pages;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool vis = ts + off < wp1 && (off < 16 ? pv0 : pv1);
          s[r] = vis ? s[r] : -INFINITY;
        }
      }
    };

    // One group tile j from stage ST: the next tile's K and this tile's V^T
    // are read from LDS; the softmax of tile j runs on the vector unit while
    // the matrix core computes S^T of tile j + 1 (into s_nxt), then
    // O^T += V^T P^T. A wave issues in order and each S^T step depends on the
    // previous one, so the exponentials are placed between the matrix
    // instructions by hand (sched_barrier keeps the compiler from regrouping
    // them):
    //   K reads; mask, maximum; E0..E2 | S step ks, two V reads, E(3 + ks) |
    //   O^T += V^T P^T for keys 0..15 with E11..E14 | E15, keys 16..31
    // where E r = exponential and bf16 packing of score r. The row sum adds
    // the packed probabilities (the values the product uses) by dot2.
    auto compute = [&](auto FAST, auto ST, int j, f32x16_t& s_cur, f32x16_t& s_nxt) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value, sn = (st + 1) % NS;
      u32x4_t kr[8];  // a stale stage after the last tile: the result is unused
      kr[0] = lds_read16<sn * kStageBytes>(kaddr[0]);
      kr[1] = lds_read16<sn * kStageBytes>(kaddr[1]);
      kr[2] = lds_read16<sn * kStageBytes>(kaddr[2]);
      kr[3] = lds_read16<sn * kStageBytes>(kaddr[3]);
      kr[4] = lds_read16<sn * kStageBytes>(kaddr[4]);
      kr[5] = lds_read16<sn * kStageBytes>(kaddr[5]);
      kr[6] = lds_read16<sn * kStageBytes>(kaddr[6]);
      kr[7] = lds_read16<sn * kStageBytes>(kaddr[7]);
      if (!decltype(FAST)::value) mask(j, s_cur);
      float mt = s_cur[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s_cur[r]);
      mt = pair_max(mt) * a.scale_log2;
      const bool grow = mt > m_run + kRescaleSlack;
      if (__any(grow)) {  // wave-uniform: rescale only when an offset moved
        const float m_new = grow ? fmaxf(m_run, mt) : m_run;
        const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float pe[16];
      bf16x8_t pb[2];
      auto E = [&](int r) __attribute__((always_inline)) {
        pe[r] = __builtin_amdgcn_exp2f(fmaf(s_cur[r], a.scale_log2, neg_m));
        if (r & 1) {
          pb[r >> 3][(r & 7) - 1] = static_cast<__bf16>(pe[r - 1]);
          pb[r >> 3][r & 7] = static_cast<__bf16>(pe[r]);
        }
      };
      E(0);
      E(1);
      E(2);
      __builtin_amdgcn_sched_barrier(0);
      // the K operands have landed
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(kr[0]), "+v"(kr[1]), "+v"(kr[2]), "+v"(kr[3]), "+v"(kr[4]), "+v"(kr[5]), "+v"(kr[6]),
                     "+v"(kr[7]));
      // V^T of tile j: [kc][dt][t], keys 0..15 first
      constexpr int vo = st * kStageBytes;
      u32x2_t vr[2][4][2];
      f32x16_t sn_acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sn_acc[r] = 0.f;
      static_for<0, 8>([&](auto KS) __attribute__((always_inline)) {
        constexpr int ks = decltype(KS)::value, kc = ks >> 2, dt = ks & 3;
        sn_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[ks]), qreg[ks], sn_acc, 0, 0,
                                                         0);
        vr[kc][dt][0] = tr_read<vo + (16 * kc) * kD * 2>(vaddr[dt]);
        vr[kc][dt][1] = tr_read<vo + (16 * kc + 8) * kD * 2>(vaddr[dt]);
        E(3 + ks);
        __builtin_amdgcn_sched_barrier(0);
      });
      s_nxt = sn_acc;
      // the reads of keys 0..15 have landed (8 more after them)
      asm volatile("s_waitcnt lgkmcnt(8)"
                   : "+v"(vr[0][0][0]), "+v"(vr[0][0][1]), "+v"(vr[0][1][0]), "+v"(vr[0][1][1]),
                     "+v"(vr[0][2][0]), "+v"(vr[0][2][1]), "+v"(vr[0][3][0]), "+v"(vr[0][3][1]));
      const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
      float ps = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x4_t w = {vr[0][dt][0].x, vr[0][dt][0].y, vr[0][dt][1].x, vr[0][dt][1].y};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb[0], oacc[dt], 0, 0, 0);
        E(11 + dt);
        const bf16x2_t pp = {pb[0][2 * dt], pb[0][2 * dt + 1]};
        ps = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ps, false);
        __builtin_amdgcn_sched_barrier(0);
      }
      E(15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // (built from the elements: a bit_cast of a lane of the packed vector
        // is folded to its first lane by this compiler)
        const bf16x2_t pp = {pb[1][2 * e], pb[1][2 * e + 1]};
        ps = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ps, false);
      }
      l_run += ps;
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vr[1][0][0]), "+v"(vr[1][0][1]), "+v"(vr[1][1][0]), "+v"(vr[1][1][1]),
                     "+v"(vr[1][2][0]), "+v"(vr[1][2][1]), "+v"(vr[1][3][0]), "+v"(vr[1][3][1]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x4_t w = {vr[1][dt][0].x, vr[1][dt][0].y, vr[1][dt][1].x, vr[1][dt][1].y};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb[1], oacc[dt], 0, 0, 0);
      }
    };

    // iteration j (stage j % NS): every wave's share of tile j + 1 has
    // landed and every wave is done with tile j - 1, whose stage takes tile
    // j + NS - 1. FAST: tiles j .. j + NS - 1 are whole prefix tiles, so
    // there is no mask, no tail test and the wait count is fixed.
    auto iter = [&](auto FAST, auto ST, int j, f32x16_t& s_cur, f32x16_t& s_nxt) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      if (decltype(FAST)::value) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 3) * INS));
      } else if (j + 1 < Tg) {
        if (j + NS - 2 < Tg) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 3) * INS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      barrier_only();
      issue(FAST, std::integral_constant<int, (st + NS - 1) % NS>{}, j + NS - 1);
      if (decltype(FAST)::value || j < Tg) compute(FAST, ST, j, s_cur, s_nxt);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using Fast = std::integral_constant<bool, true>;
    using Slow = std::integral_constant<bool, false>;
    issue(Slow{}, I0{}, 0);
    issue(Slow{}, I1{}, 1);
    issue(Slow{}, I2{}, 2);
    if (w0 == 0) {
      load_q();
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // Q, and the first tiles
    } else if (NS - 2 < Tg) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * INS));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();  // tile 0 of every group (and the ancestor rows) in LDS
    f32x16_t sa, sb;
    if (Tg > 0) {
      u32x4_t kr[8];
      kr[0] = lds_read16<0>(kaddr[0]);
      kr[1] = lds_read16<0>(kaddr[1]);
      kr[2] = lds_read16<0>(kaddr[2]);
      kr[3] = lds_read16<0>(kaddr[3]);
      kr[4] = lds_read16<0>(kaddr[4]);
      kr[5] = lds_read16<0>(kaddr[5]);
      kr[6] = lds_read16<0>(kaddr[6]);
      kr[7] = lds_read16<0>(kaddr[7]);
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(kr[0]), "+v"(kr[1]), "+v"(kr[2]), "+v"(kr[3]), "+v"(kr[4]), "+v"(kr[5]), "+v"(kr[6]),
                     "+v"(kr[7]));
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[ks]), qreg[ks], sa, 0, 0, 0);
    }
    // whole prefix tiles in groups of four, then the rest (tail, partial and
    // tree tiles) one checked iteration at a time
    const int jfast = max(0, Tfull - (NS - 1)) & ~3;
    int j = 0;
    for (; j < jfast; j += 4) {
      iter(Fast{}, I0{}, j, sa, sb);
      iter(Fast{}, I1{}, j + 1, sb, sa);
      iter(Fast{}, I2{}, j + 2, sa, sb);
      iter(Fast{}, I3{}, j + 3, sb, sa);
    }
    for (; j < Tmax; j += 4) {
      iter(Slow{}, I0{}, j, sa, sb);
      if (j + 1 < Tmax) iter(Slow{}, I1{}, j + 1, sb, sa);
      if (j + 2 < Tmax) iter(Slow{}, I2{}, j + 2, sa, sb);
      if (j + 3 < Tmax) iter(Slow{}, I3{}, j + 3, sb, sa);
    }
    if (last) break;
  }

  // column sums: each lane holds half of its column's keys
  l_run = pair_sum(l_run);

  if constexpr (WK > 1) {
    // key groups 1.. hand their states to group 0 through LDS (the stages
    // are free once every wave is past its loop): O^T of a wave is 16 KB
    constexpr int kSlotFloats = 4 * 16 * 64;
    constexpr int kML = (WK - 1) * WQ * 64;
    static_assert(((WK - 1) * WQ * kSlotFloats + 2 * kML) * 4 <= static_cast<int>(sizeof(stg)), "hand-over area");
    float* xo0 = reinterpret_cast<float*>(&stg[0][0][0][0]);
    float* xm = xo0 + (WK - 1) * WQ * kSlotFloats;  // [2][WK - 1][WQ][64]: m, then l
    __syncthreads();
    if (wk > 0) {
      const int slotw = (wk - 1) * WQ + wq;
      float* xo = xo0 + slotw * kSlotFloats;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[((dt * 16 + r) << 6) + lane] = oacc[dt][r];
      xm[(slotw << 6) + lane] = m_run;
      xm[kML + (slotw << 6) + lane] = l_run;
    }
    __syncthreads();
    if (wk > 0) return;
    float M = m_run;
    for (int o = 1; o < WK; ++o) M = fmaxf(M, xm[(((o - 1) * WQ + wq) << 6) + lane]);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float w0 = __builtin_amdgcn_exp2f(m_run - Mu);
    l_run *= w0;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] *= w0;
    for (int o = 1; o < WK; ++o) {
      const int slotw = (o - 1) * WQ + wq;
      const float* xo = xo0 + slotw * kSlotFloats;
      const float wo = __builtin_amdgcn_exp2f(xm[(slotw << 6) + lane] - Mu);
      l_run += wo * xm[kML + (slotw << 6) + lane];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] += wo * xo[((dt * 16 + r) << 6) + lane];
    }
    m_run = M;
  }

  // unnormalised partial of this split: rows (split, b, hkv, query)
  const int qi = q0 + l32;
  if (qi < a.NQ) {
    const size_t row = (static_cast<size_t>(split * a.B + b) * a.Hkv + hkv) * a.NQpad + qi;
    float* op = a.opart + row * kD + 4 * hl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(op + 32 * dt + 8 * r4) =
            make_float4(oacc[dt][4 * r4], oacc[dt][4 * r4 + 1], oacc[dt][4 * r4 + 2], oacc[dt][4 * r4 + 3]);
    if (hl == 0) {
      a.mpart[row] = m_run;
      a.lpart[row] = l_run;
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
  int wq, wk;  // waves along queries, key groups
  int S, QT, NQ, NQpad;
};

// Eight waves of 32 query rows: they split the queries when a KV head has
// more than 128 query rows, else form two key groups of four. Splits aim at
// about one workgroup per CU (each at least four tiles of the longest prefix,
// and, where that allows, at most one 128-tile window). Each sequence cuts its
// own prefix into S equal ranges, so the plan only sizes the work: any
// prefix_len up to the block table's capacity is covered whatever
// max_prefix_len says. (The tile kernel serves more than 64 query rows only.)
TilePlan plan_tiles(int B, int N, int Hq, int Hkv, int max_prefix_len) {
  TilePlan p;
  p.NQ = N * (Hq / Hkv);
  if (p.NQ <= 128) p.wq = 4, p.wk = 2;
  else p.wq = 8, p.wk = 1;
  const int qr = 32 * p.wq;
  p.QT = (p.NQ + qr - 1) / qr;
  p.NQpad = p.QT * qr;
  const long long units = static_cast<long long>(B) * Hkv * p.QT;
  const int Lr = max_prefix_len > 0 ? max_prefix_len : 0;
  long long S = (256 + units / 2) / units;
  const long long smax = (Lr + 4 * kTK - 1) / (4 * kTK);
  if (S > smax) S = smax;
  const long long smin = (Lr + 128 * kTK - 1) / (128 * kTK);
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
  if (p.wq == 4) attn_tile_mfma<4, 2><<<grid, nt, 0, stream>>>(a);
  else attn_tile_mfma<8, 1><<<grid, nt, 0, stream>>>(a);
  HY_LAUNCH_CHECK("tree_attention(tiles)");
  const long long cthreads = static_cast<long long>(B) * Hkv * p.NQ * (D / 4);
  attn_combine<bf16_t><<<static_cast<int>((cthreads + 255) / 256), 256, 0, stream>>>(
      B, N, Hq, Hkv, D, p.S, p.NQ, p.NQpad, a.opart, a.mpart, a.lpart, static_cast<bf16_t*>(out), lse);
  HY_LAUNCH_CHECK("tree_attention(combine)");
  return HYDRA_OK;
}
