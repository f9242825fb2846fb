// The draft heads' feed-forward layer for few rows:
//   a = W1 x + b1,  u = h + SiLU(a)  (or SiLU(a)),  stored as bf16.
// ("Medusa Heads", section "So sagen die Köpfe voraus": one SiLU layer with a
// residual connection; "Hydra Guide", section "1. Embedding Conditioning
// Mechanics": the Hydra layer reads [h || e(x_parent)].)
//
// W1 is [d, in] with d = 4096..8192, while the rows are few (one per expanded
// node, B * P <= 32). Tiling N in 64-row workgroups leaves too few
// workgroups, and split-K over the grid needs a second pass. Here a
// workgroup owns 16 rows of W1 and its NWV waves split K: each wave streams
// its K range of the 16 rows (the MFMA A operand) and reads the matching X
// slice straight from L2 (the B operand), with PF steps in flight. The waves'
// partial tiles meet in LDS and are summed in a fixed order, so the result is
// deterministic, then the epilogue runs before the workgroup ends.
//
// The Hydra input splits as W1 [h || e] = W1[:, :d] h + W1[:, d:] e. The h
// half does not depend on the tree, so the row merge of depth k - 1 runs it
// for head k in extra workgroups of its launch (epi 0) and depth k streams
// only the embedding half here (epi 2); Medusa heads read h alone and run all
// at once (several heads per launch, blockIdx.y = head).
#include "ffn.h"

namespace hydra {
namespace {

template <int MT, int PF, int NWV>
__global__ __launch_bounds__(NWV * 64) void mlp_fused_kernel(MlpArgs a) {
  mlp_tile<MT, PF, NWV>(a, blockIdx.x, blockIdx.y);
}

// waves per workgroup: 4, each streaming a quarter of K (measured on MI355X
// for one to 32 rows and K = 4096 .. 8192: 4 waves beat 8 by 10-20% and 16
// by 15-30%, as each wave keeps a longer stream of 16-byte loads in flight)
int mlp_waves(int) { return 4; }

template <int MT, int NWV>
void launch_mt(const MlpArgs& a, hipStream_t stream) {
  const int steps = a.K / NWV / 32;
  dim3 grid(a.d / 16, a.heads);
  if (steps % 8 == 0) {
    mlp_fused_kernel<MT, 8, NWV><<<grid, NWV * 64, 0, stream>>>(a);
  } else {
    mlp_fused_kernel<MT, 1, NWV><<<grid, NWV * 64, 0, stream>>>(a);
  }
}

template <int NWV>
void launch_nwv(const MlpArgs& a, hipStream_t stream) {
  if (a.M <= 16) launch_mt<1, NWV>(a, stream);
  else launch_mt<2, NWV>(a, stream);
}

}  // namespace

bool mlp_fused_supported(int dtype, int M, int K, int d) {
  // beyond 32 rows the per-wave row loads outweigh the weight stream
  return dtype == HYDRA_BF16 && M >= 1 && M <= 32 && K % (mlp_waves(K) * 32) == 0 && d % 16 == 0;
}

int launch_mlp_fused(const MlpArgs& a, hipStream_t stream) {
  if (a.heads < 1 || a.heads > HYDRA_MAX_DEPTH) {
    set_error("draft_heads: %d heads in one feed-forward launch", a.heads);
    return HYDRA_ERR_INVALID;
  }
  launch_nwv<4>(a, stream);
  HY_LAUNCH_CHECK("draft_heads: fused mlp");
  return HYDRA_OK;
}

}  // namespace hydra
