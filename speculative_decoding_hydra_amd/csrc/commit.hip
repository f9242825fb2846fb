// Commit of the kept branch into the paged KV cache, after acceptance.
//
// "Hydra Guide: Sequentially-Dependent Speculative AI", section "Production
// Engineering and Training Best Practices" (items on tree KV-cache page sizing
// and branch management): the tree's K/V sit in statically reserved blocks
// and rejected nodes are rolled back without freeing memory. "Speculative
// Decoding", section "The acceptance criterion": the next round starts from
// the last accepted or resampled token and the rejected suffix leaves the
// caches. "Medusa Heads", section "Tree Attention und Akzeptanz": the longest
// accepted branch stays and its last hidden state feeds the heads next round.
//
// Here the verify pass keeps the tree rows' K/V in their own buffer, so
// rollback costs nothing: the commit copies the root and the m accepted rows
// to cache positions L .. L + m of every layer and never touches a rejected
// row. At most (Dmax + 1) rows per sequence and layer move, so the launch is
// latency-bound; one workgroup per (row, sequence, layer) copies that row's
// K and V with 16-byte loads and stores.
#include "common.h"

namespace hydra {
namespace {

constexpr int kCommitThreads = 256;

struct CommitArgs {
  int B, N, Hkv, D, Dmax, esz, n_pages, page_size, max_pages, d;
  const char* k_tree;
  const char* v_tree;
  char* k_pages;
  char* v_pages;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int32_t* n_accepted;
  const int32_t* path;
  const int32_t* out_tok;
  const char* hidden;
  int32_t* next_len;
  int32_t* next_root;
  char* next_h;
};

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitArgs a) {
  const int j = blockIdx.x, b = blockIdx.y, layer = blockIdx.z;
  const int* path = a.path + static_cast<size_t>(b) * (a.Dmax + 1);
  const int m = a.n_accepted[b];
  const int L = a.prefix_len[b];
  bool ok = m >= 0 && m <= a.Dmax;
  for (int i = 0; ok && i <= m; ++i) ok = path[i] >= 0 && path[i] < a.N;
  const bool seq_writer = j == 0 && layer == 0;
  if (!ok) {  // nothing to commit: the length stays and there is no next root
    if (seq_writer && threadIdx.x == 0) {
      a.next_len[b] = L;
      a.next_root[b] = -1;
    }
    return;
  }
  if (seq_writer) {
    if (threadIdx.x == 0) {
      a.next_len[b] = L + m + 1;
      a.next_root[b] = a.out_tok[static_cast<size_t>(b) * (a.Dmax + 1) + m];
    }
    if (a.hidden) {  // next h: the hidden state of the last accepted row
      const size_t hb = static_cast<size_t>(a.d) * a.esz;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.hidden + (static_cast<size_t>(b) * a.N + path[m]) * hb);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.next_h + static_cast<size_t>(b) * hb);
      for (size_t v = threadIdx.x; v < hb / 16; v += kCommitThreads) dst[v] = src[v];
    }
  }
  if (j > m) return;
  const long long pos = static_cast<long long>(L) + j;
  if (pos < 0) return;
  const long long pidx = pos / a.page_size;
  if (pidx >= a.max_pages) return;
  const int page = a.block_table[static_cast<size_t>(b) * a.max_pages + pidx];
  if (page < 0 || page >= a.n_pages) return;
  const int slot = static_cast<int>(pos % a.page_size);
  const size_t head_bytes = static_cast<size_t>(a.D) * a.esz;  // a multiple of 16
  const size_t row_bytes = head_bytes * a.Hkv;
  const int hv = static_cast<int>(head_bytes / 16);             // vectors per head
  const int nv = hv * a.Hkv;                                     // vectors per row
  const size_t src_off = ((static_cast<size_t>(layer) * a.B + b) * a.N + path[j]) * row_bytes;
  const size_t layer_off = static_cast<size_t>(layer) * a.n_pages * a.page_size * row_bytes;
  const size_t page_off = layer_off + (static_cast<size_t>(page) * a.Hkv * a.page_size + slot) * head_bytes;
  const size_t head_stride = static_cast<size_t>(a.page_size) * head_bytes;
  for (int v = threadIdx.x; v < nv; v += kCommitThreads) {
    const int hk = v / hv, w = v % hv;
    const size_t so = src_off + static_cast<size_t>(v) * 16;
    const size_t dof = page_off + hk * head_stride + static_cast<size_t>(w) * 16;
    const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(a.k_tree + so);
    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(a.v_tree + so);
    *reinterpret_cast<u32x4_t*>(a.k_pages + dof) = kv;
    *reinterpret_cast<u32x4_t*>(a.v_pages + dof) = vv;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace hydra

extern "C" int tree_commit(int dtype, int n_layers, int B, int N, int Hkv, int D, int Dmax, const void* k_tree,
                           const void* v_tree, void* k_pages, void* v_pages, int n_pages, int page_size,
                           const int32_t* block_table, int max_pages, const int32_t* prefix_len,
                           const int32_t* n_accepted, const int32_t* path, const int32_t* out_tok, int d,
                           const void* hidden, int32_t* next_prefix_len, int32_t* next_root_tok, void* next_h,
                           void* stream) {
  using namespace hydra;
  clear_error();
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "tree_commit: bad dtype %d", dtype);
  HY_CHECK(n_layers >= 1 && B >= 0 && N >= 1 && Hkv >= 1 && D >= 1 && n_pages >= 1 && page_size >= 1 &&
               max_pages >= 1,
           HYDRA_ERR_INVALID, "tree_commit: bad sizes layers=%d B=%d N=%d Hkv=%d D=%d pages=%d page_size=%d "
           "max_pages=%d", n_layers, B, N, Hkv, D, n_pages, page_size, max_pages);
  HY_CHECK(Dmax >= 0 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "tree_commit: Dmax=%d", Dmax);
  HY_CHECK(D % 8 == 0, HYDRA_ERR_UNSUPPORTED, "tree_commit: D %% 8 != 0 (D=%d)", D);
  if (B == 0) return HYDRA_OK;
  HY_CHECK(k_tree && v_tree && k_pages && v_pages && block_table && prefix_len && n_accepted && path && out_tok &&
               next_prefix_len && next_root_tok,
           HYDRA_ERR_INVALID, "tree_commit: null pointer");
  HY_CHECK(!hidden == !next_h, HYDRA_ERR_INVALID, "tree_commit: hidden and next_h go together");
  HY_CHECK(!hidden || (d >= 8 && d % 8 == 0), HYDRA_ERR_UNSUPPORTED, "tree_commit: d %% 8 != 0 (d=%d)", d);
  HY_CHECK(aligned16(k_tree) && aligned16(v_tree) && aligned16(k_pages) && aligned16(v_pages) &&
               aligned16(hidden) && aligned16(next_h),
           HYDRA_ERR_INVALID, "tree_commit: K/V and hidden-state buffers must be 16-byte aligned");
  HY_CHECK(static_cast<const void*>(next_prefix_len) != static_cast<const void*>(prefix_len), HYDRA_ERR_INVALID,
           "tree_commit: next_prefix_len must not alias prefix_len");
  HY_CHECK(B <= 65535 && n_layers <= 65535, HYDRA_ERR_UNSUPPORTED, "tree_commit: B=%d or layers=%d > 65535", B,
           n_layers);
  CommitArgs a{};
  a.B = B;
  a.N = N;
  a.Hkv = Hkv;
  a.D = D;
  a.Dmax = Dmax;
  a.esz = dtype == HYDRA_F32 ? 4 : 2;
  a.n_pages = n_pages;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.d = d;
  a.k_tree = static_cast<const char*>(k_tree);
  a.v_tree = static_cast<const char*>(v_tree);
  a.k_pages = static_cast<char*>(k_pages);
  a.v_pages = static_cast<char*>(v_pages);
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.n_accepted = n_accepted;
  a.path = path;
  a.out_tok = out_tok;
  a.hidden = static_cast<const char*>(hidden);
  a.next_len = next_prefix_len;
  a.next_root = next_root_tok;
  a.next_h = static_cast<char*>(next_h);
  commit_kernel<<<dim3(Dmax + 1, B, n_layers), kCommitThreads, 0, static_cast<hipStream_t>(stream)>>>(a);
  HY_LAUNCH_CHECK("tree_commit");
  return HYDRA_OK;
}
