// Greedy acceptance walk of one sequence, shared by the stand-alone walk
// kernel and the row merge that finishes the target's arg maxes ("Hydra
// Guide: Sequentially-Dependent Speculative AI", section "Parallel
// Verification and Greedy Acceptance Algorithm"): from the root, follow the
// child whose token equals the target's arg max at the current node; the arg
// max at the last node reached is the bonus token.
#pragma once

#include "common.h"

namespace hydra {

// One wave (64 lanes) walks sequence b; lanes <= Dmax write path / out_tok.
__device__ __forceinline__ void greedy_walk_seq(int b, int N, int Dmax, const int32_t* amax, const int32_t* tok,
                                                const int32_t* parent, int32_t* n_accepted, int32_t* path,
                                                int32_t* out_tok) {
  const int lane = threadIdx.x & 63;
  const int32_t* tb = tok + static_cast<size_t>(b) * N;
  const int32_t* pb = parent + static_cast<size_t>(b) * N;
  int u = 0, m = 0;
  int my_path = lane == 0 ? 0 : -1, my_out = -1;  // lane j keeps entry j
  while (true) {
    const int y = amax[static_cast<size_t>(b) * N + u];
    int found = -1;
    for (int c0 = 0; c0 < N && found < 0; c0 += 64) {
      const int c = c0 + lane;
      const bool hit = c < N && pb[c] == u && tb[c] == y;
      const unsigned long long mask = __ballot(hit);
      if (mask) found = c0 + __ffsll(static_cast<long long>(mask)) - 1;
    }
    if (lane == m) my_out = y;
    if (found < 0 || m >= Dmax) break;
    ++m;
    u = found;
    if (lane == m) my_path = u;
  }
  if (lane <= Dmax) {
    path[static_cast<size_t>(b) * (Dmax + 1) + lane] = my_path;
    out_tok[static_cast<size_t>(b) * (Dmax + 1) + lane] = my_out;
  }
  if (lane == 0) n_accepted[b] = m;
}

}  // namespace hydra
