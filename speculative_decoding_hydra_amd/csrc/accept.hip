// Stage 4: target vocabulary projection and acceptance walk.
//
// Greedy: "Hydra Guide: Sequentially-Dependent Speculative AI", section
// "Parallel Verification and Greedy Acceptance Algorithm": follow the branch
// whose tokens equal the target's arg max, stop at the first mismatch and emit
// the target's token there as the bonus (m accepted drafts give m + 1 tokens).
//
// Rejection: "Speculative Decoding", sections "The acceptance criterion" and
// "The correctness guarantee": accept a drafted x with probability
// min(1, p(x)/q(x)), written division-free as u * q(x) < p(x); on rejection
// the target becomes norm(max(p - q, 0)). On a tree the children of the
// current node are tried in rank order against the current residual with q
// unchanged; a node without children, or with every child rejected, ends the
// walk with one inverse-CDF draw from the current target ("How much faster?":
// the bonus token is drawn from the target distribution when every draft is
// accepted). p and q are the post-temperature distributions ("Common
// misconceptions").
//
// Typical: "Medusa Heads", section "Tree Attention und Akzeptanz": a
// candidate is kept when its target probability exceeds a threshold tied to
// the entropy of the target's distribution, and the longest accepted branch
// is kept (not distribution-exact). Threshold form (a reading):
// tau = min(eps, delta * exp(-H(p))) at the parent, p = softmax(z / T); the
// kept branch ends at the deepest node whose whole path passes (smallest
// breadth-first index among equals) and one token is drawn from p there.
#include "walk.h"

#include <mutex>

namespace hydra {
namespace {

// One wave per sequence.
__global__ __launch_bounds__(64) void greedy_walk(int N, int Dmax, const int32_t* __restrict__ amax,
                                                  const int32_t* __restrict__ tok,
                                                  const int32_t* __restrict__ parent,
                                                  int32_t* __restrict__ n_accepted, int32_t* __restrict__ path,
                                                  int32_t* __restrict__ out_tok) {
  greedy_walk_seq(blockIdx.x, N, Dmax, amax, tok, parent, n_accepted, path, out_tok);
}

constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;

template <int NW = kWalkWaves>
__device__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < NW; ++w) t += red[w];
  return t;
}

template <int NW = kWalkWaves>
__device__ float block_max_f(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int w = 0; w < NW; ++w) t = fmaxf(t, red[w]);
  return t;
}

// Unnormalised current target r at x: from the logits (mode < 0) or from a
// residual buffer.
struct Target {
  const float* z;   // logits row (mode < 0)
  float invT, m;    // scaled max of the row
  const float* buf; // residual buffer (mode >= 0)
  double total;     // sum of the unnormalised values
  __device__ __forceinline__ float at(int x) const {
    return buf ? buf[x] : exp2f((z[x] * invT - m) * 1.4426950408889634f);
  }
};

// Inverse-CDF draw: the smallest x with cumsum_{y<=x} r(y) > u * total.
__device__ int block_sample(const Target& r, int V, float u, double* red, int* s_pick) {
  const int tid = threadIdx.x;
  const int C = (V + kWalkThreads - 1) / kWalkThreads;
  const int lo = tid * C, hi = min(V, lo + C);
  double part = 0.0;
  int lastpos = -1;
  for (int x = lo; x < hi; ++x) {
    const float v = r.at(x);
    part += v;
    if (v > 0.f) lastpos = x;
  }
  // exclusive scan of the chunk sums across the block
  const int lane = tid & 63, wave = tid >> 6;
  double incl = part;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == 63) red[wave] = incl;
  if (tid == 0) {
    s_pick[0] = -1;
    s_pick[1] = -1;
  }
  __syncthreads();
  double before = 0.0, total = 0.0;
  for (int w = 0; w < kWalkWaves; ++w) {
    if (w < wave) before += red[w];
    total += red[w];
  }
  const double excl = before + incl - part;
  const double thr = static_cast<double>(u) * total;
  if (lastpos >= 0) atomicMax(&s_pick[1], lastpos);
  if (excl <= thr && thr < excl + part) {
    double run = excl;
    for (int x = lo; x < hi; ++x) {
      run += r.at(x);
      if (run > thr) {
        s_pick[0] = x;
        break;
      }
    }
  }
  __syncthreads();
  const int pick = s_pick[0] >= 0 ? s_pick[0] : s_pick[1];
  __syncthreads();
  return pick;
}

__global__ __launch_bounds__(kWalkThreads) void reject_walk(
    int N, int V, int R, int Dmax, float invT, const float* __restrict__ Z, const float* __restrict__ HZ,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ parent, const int32_t* __restrict__ q_row,
    const float* __restrict__ u_acc, const float* __restrict__ u_res, float* __restrict__ rbuf,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ path, int32_t* __restrict__ out_tok) {
  __shared__ double red[kWalkWaves];
  __shared__ float redf[kWalkWaves];
  __shared__ int s_path[HYDRA_MAX_DEPTH + 1], s_out[HYDRA_MAX_DEPTH + 1];
  __shared__ int s_pick[2];
  __shared__ int s_kid[2];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid <= Dmax) {
    s_path[tid] = -1;
    s_out[tid] = -1;
  }
  if (tid == 0) s_path[0] = 0;
  const int32_t* tb = tok + static_cast<size_t>(b) * N;
  const int32_t* pb = parent + static_cast<size_t>(b) * N;
  float* buf[2] = {rbuf + static_cast<size_t>(b) * 2 * V, rbuf + (static_cast<size_t>(b) * 2 + 1) * V};
  int u = 0, m = 0;
  while (true) {
    // p at u
    const float* zu = Z + (static_cast<size_t>(b) * N + u) * V;
    float mx = -INFINITY;
    for (int x = tid; x < V; x += kWalkThreads) mx = fmaxf(mx, zu[x] * invT);
    Target r{zu, invT, block_max_f(mx, redf), nullptr, 0.0};
    double s = 0.0;
    for (int x = tid; x < V; x += kWalkThreads) s += r.at(x);
    r.total = block_sum_d(s, red);
    // children of u: contiguous, in rank order
    if (tid == 0) {
      s_kid[0] = N;
      s_kid[1] = 0;
    }
    __syncthreads();
    for (int c = tid; c < N; c += kWalkThreads)
      if (pb[c] == u) {
        atomicMin(&s_kid[0], c);
        atomicAdd(&s_kid[1], 1);
      }
    __syncthreads();
    const int c0 = s_kid[0], cnt = s_kid[1];
    __syncthreads();
    if (cnt == 0 || m >= Dmax) {
      const int x = block_sample(r, V, u_res[static_cast<size_t>(b) * N + u], red, s_pick);
      if (tid == 0) s_out[m] = x;
      break;
    }
    // q at u: the head row that drafted u's children
    const int qr = q_row[static_cast<size_t>(b) * N + u];
    const float* hz = HZ + (static_cast<size_t>(b) * R + (qr < 0 ? 0 : (qr >= R ? R - 1 : qr))) * V;
    float qm = -INFINITY;
    for (int x = tid; x < V; x += kWalkThreads) qm = fmaxf(qm, hz[x] * invT);
    qm = block_max_f(qm, redf);
    double qs = 0.0;
    for (int x = tid; x < V; x += kWalkThreads) qs += exp2f((hz[x] * invT - qm) * 1.4426950408889634f);
    const float qinv = static_cast<float>(1.0 / block_sum_d(qs, red));
    int nb = 0;
    bool moved = false;
    for (int j = 0; j < cnt; ++j) {
      const int c = c0 + j;
      const int x = tb[c];
      const float rx = static_cast<float>(r.at(x) / r.total);
      const float qx = exp2f((hz[x] * invT - qm) * 1.4426950408889634f) * qinv;
      if (u_acc[static_cast<size_t>(b) * N + c] * qx < rx) {
        ++m;
        if (tid == 0) {
          s_path[m] = c;
          s_out[m - 1] = x;
        }
        u = c;
        moved = true;
        break;
      }
      // residual: norm(max(r - q, 0)), kept unless it has no mass
      const float rinv = static_cast<float>(1.0 / r.total);
      float* dst = buf[nb];
      double ns = 0.0;
      for (int y = tid; y < V; y += kWalkThreads) {
        const float v = fmaxf(r.at(y) * rinv - exp2f((hz[y] * invT - qm) * 1.4426950408889634f) * qinv, 0.f);
        dst[y] = v;
        ns += v;
      }
      ns = block_sum_d(ns, red);
      if (ns > 0.0) {
        r.buf = dst;
        r.total = ns;
        nb ^= 1;
      }
      __syncthreads();
    }
    if (!moved) {
      const int x = block_sample(r, V, u_res[static_cast<size_t>(b) * N + u], red, s_pick);
      if (tid == 0) s_out[m] = x;
      break;
    }
  }
  __syncthreads();
  if (tid <= Dmax) {
    path[static_cast<size_t>(b) * (Dmax + 1) + tid] = s_path[tid];
    out_tok[static_cast<size_t>(b) * (Dmax + 1) + tid] = s_out[tid];
  }
  if (tid == 0) n_accepted[b] = m;
}

// Typical acceptance, part 1: one workgroup per tree row u with children.
// Over the row's scaled logits y = z / T it forms S = sum exp(y - M) and
// W = sum exp(y - M) (y - M) (float32 per thread, float64 across threads),
// so H(p) = log S - W / S; each child c of u passes iff
// log p(tok[c]) = y_x - M - log S exceeds log tau = min(log eps,
// log delta - H). Rows without children exit.
constexpr int kTypThreads = 1024;

__global__ __launch_bounds__(kTypThreads) void typical_rows(int N, int V, float invT, float log_eps,
                                                            float log_delta, const float* __restrict__ Z,
                                                            const int32_t* __restrict__ tok,
                                                            const int32_t* __restrict__ parent,
                                                            int32_t* __restrict__ pass) {
  __shared__ int s_kid[2];
  __shared__ float s_m[kTypThreads / 64];
  __shared__ double s_s[kTypThreads / 64], s_w[kTypThreads / 64];
  const int b = blockIdx.x / N, u = blockIdx.x % N, tid = threadIdx.x;
  const int32_t* pb = parent + static_cast<size_t>(b) * N;
  if (tid == 0) {
    s_kid[0] = N;
    s_kid[1] = 0;
    if (u == 0) pass[static_cast<size_t>(b) * N] = 1;  // the root
  }
  __syncthreads();
  for (int c = tid; c < N; c += kTypThreads)
    if (pb[c] == u) {
      atomicMin(&s_kid[0], c);
      atomicAdd(&s_kid[1], 1);
    }
  __syncthreads();
  const int c0 = s_kid[0], cnt = s_kid[1];
  if (cnt == 0) return;
  const float* zu = Z + (static_cast<size_t>(b) * N + u) * V;
  float mx = -INFINITY;
  for (int x = tid; x < V; x += kTypThreads) mx = fmaxf(mx, zu[x] * invT);
  mx = wave_max(mx);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) s_m[wave] = mx;
  __syncthreads();
  float M = s_m[0];
#pragma unroll
  for (int w = 1; w < kTypThreads / 64; ++w) M = fmaxf(M, s_m[w]);
  float Sf = 0.f, Wf = 0.f;
  for (int x = tid; x < V; x += kTypThreads) {
    const float t = zu[x] * invT - M;
    const float e = exp2f(t * 1.4426950408889634f);
    Sf += e;
    Wf += e * t;
  }
  double S = Sf, W = Wf;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S += __shfl_xor(S, off, 64);
    W += __shfl_xor(W, off, 64);
  }
  if (lane == 0) {
    s_s[wave] = S;
    s_w[wave] = W;
  }
  __syncthreads();
  S = 0.0;
  W = 0.0;
#pragma unroll
  for (int w = 0; w < kTypThreads / 64; ++w) {
    S += s_s[w];
    W += s_w[w];
  }
  const double logS = log(S);
  const double H = logS - W / S;
  const double log_tau = fmin(static_cast<double>(log_eps), static_cast<double>(log_delta) - H);
  for (int j = tid; j < cnt; j += kTypThreads) {
    const int c = c0 + j;
    const int x = tok[static_cast<size_t>(b) * N + c];
    const bool ok = x >= 0 && x < V &&
                    static_cast<double>(zu[x < 0 ? 0 : (x >= V ? V - 1 : x)] * invT - M) - logS > log_tau;
    pass[static_cast<size_t>(b) * N + c] = ok ? 1 : 0;
  }
}

// Typical acceptance, part 2: one workgroup per sequence finds the kept
// branch from the pass flags (parents precede children), then draws the last
// token from the target at its end by inverse CDF.
__global__ __launch_bounds__(kWalkThreads) void typical_walk(int N, int V, int Dmax, float invT,
                                                             const float* __restrict__ Z,
                                                             const int32_t* __restrict__ tok,
                                                             const int32_t* __restrict__ parent,
                                                             const int32_t* __restrict__ pass,
                                                             const float* __restrict__ u_res,
                                                             int32_t* __restrict__ n_accepted,
                                                             int32_t* __restrict__ path, int32_t* __restrict__ out_tok) {
  __shared__ double red[kWalkWaves];
  __shared__ float redf[kWalkWaves];
  __shared__ int s_pick[2];
  __shared__ int s_end, s_m;
  __shared__ int s_path[HYDRA_MAX_DEPTH + 1];
  __shared__ uint8_t s_ok[HYDRA_MAX_VERIFY];
  __shared__ uint8_t s_depth[HYDRA_MAX_VERIFY];
  __shared__ int s_par[HYDRA_MAX_VERIFY];
  __shared__ uint8_t s_pass[HYDRA_MAX_VERIFY];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* pb = parent + static_cast<size_t>(b) * N;
  for (int c = tid; c < N; c += kWalkThreads) {  // the tree into LDS, all loads at once
    s_par[c] = pb[c];
    s_pass[c] = pass[static_cast<size_t>(b) * N + c] != 0;
  }
  __syncthreads();
  if (tid == 0) {  // N <= 256 nodes in breadth-first order: a sequential pass over LDS
    int end = 0, dend = 0;
    s_ok[0] = 1;
    s_depth[0] = 0;
    for (int c = 1; c < N; ++c) {
      const int u = s_par[c];
      const bool valid = u >= 0 && u < c;
      const int dc = valid ? s_depth[u] + 1 : 0;
      s_depth[c] = static_cast<uint8_t>(dc > 255 ? 255 : dc);
      s_ok[c] = valid && s_ok[u] && dc <= Dmax && s_pass[c];
      if (s_ok[c] && dc > dend) {
        end = c;
        dend = dc;
      }
    }
    for (int j = 0; j <= Dmax; ++j) s_path[j] = -1;
    int v = end;
    for (int j = dend; j >= 0; --j) {
      s_path[j] = v;
      v = s_par[v] < 0 ? 0 : s_par[v];
    }
    s_end = end;
    s_m = dend;
  }
  __syncthreads();
  const int end = s_end, m = s_m;
  const float* ze = Z + (static_cast<size_t>(b) * N + end) * V;
  float mx = -INFINITY;
  for (int x = tid; x < V; x += kWalkThreads) mx = fmaxf(mx, ze[x] * invT);
  Target r{ze, invT, block_max_f(mx, redf), nullptr, 0.0};
  const int x = block_sample(r, V, u_res[static_cast<size_t>(b) * N + end], red, s_pick);
  if (tid <= Dmax) {
    const int pc = s_path[tid];
    path[static_cast<size_t>(b) * (Dmax + 1) + tid] = pc;
    int o = -1;
    if (tid < m) o = tok[static_cast<size_t>(b) * N + s_path[tid + 1]];
    else if (tid == m) o = x;
    out_tok[static_cast<size_t>(b) * (Dmax + 1) + tid] = o;
  }
  if (tid == 0) n_accepted[b] = m;
}

// ---------------------------------------------------------------------------
// Register-resident rows (V <= EPT * NT for a launch of NT threads). The walks
// above stream a logits row from memory on every pass (maximum, sum,
// residual, draw), one load per thread at a time, so each pass costs tens of
// memory round trips. Here a row is loaded once, with all of a thread's loads
// in flight together: element x = i * NT + tid sits in register i of thread
// tid, so every load is coalesced, and the passes run on registers. The steps
// are the walks' own; the float partial sums group the elements by thread of
// the launch (float per thread and wave, float64 across waves).

constexpr int kNodeThreads = 512;  // node kernels: two rows of up to 64 registers each without spilling
constexpr int kNodeWaves = kNodeThreads / 64;

constexpr float kLog2e = 1.4426950408889634f;

// float sum over the wave, the same value in every lane: rows of 16 by DPP,
// then the row pairs and halves by the gfx950 row swaps (VALU only; every
// partial is a commutative pair, so all lanes add in the same order)
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dppf<kDppXor1>(v);
  v += dppf<kDppXor2>(v);
  v += dppf<kDppHalfMirror>(v);
  v += dppf<kDppMirror>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// block sum: float within each wave (DPP), float64 across the NW waves
template <int NW>
__device__ __forceinline__ double block_sum_fd(float v, double* red) {
  v = wave_sum_dpp(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < NW; ++w) t += red[w];
  return t;
}


// row `row` of the [rows][V] float matrix z; buffer loads share one lane
// offset (register i adds i * 4 KB as a scalar offset), so all EPT loads are
// in flight at once without a 64-bit address per load
template <int EPT, int NT>
__device__ __forceinline__ void reg_load_scaled(float (&v)[EPT], const float* __restrict__ z, size_t row, int V,
                                                float invT) {
  const size_t r = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row));
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(z + r * V), 0, V * 4, 0x00020000);
  const int lane_off = static_cast<int>(threadIdx.x) * 4;
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, lane_off, i * NT * 4, 0));
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int x = i * NT + static_cast<int>(threadIdx.x);
    v[i] = x < V ? v[i] * invT : -INFINITY;  // past V the buffer returns 0
  }
}

// v <- exp(v - max v) (0 past V); returns the block sum in float64
template <int EPT, int NT>
__device__ __forceinline__ double reg_exp(float (&v)[EPT], double* red, float* redf) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPT; ++i) mx = fmaxf(mx, v[i]);
  const float M = block_max_f<NT / 64>(mx, redf);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    v[i] = v[i] == -INFINITY ? 0.f : exp2f((v[i] - M) * kLog2e);
    s += v[i];
  }
  return block_sum_fd<NT / 64>(s, red);
}

// a[x] and b[x] for one token x < V, broadcast to the whole block
template <int EPT, int NT>
__device__ __forceinline__ float2 reg_at2(const float (&a)[EPT], const float (&b)[EPT], int x, float2* s_bc) {
  __syncthreads();
  if (static_cast<int>(threadIdx.x) == x % NT) {
    float2 t = make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (i == x / NT) t = make_float2(a[i], b[i]);
    *s_bc = t;
  }
  __syncthreads();
  return *s_bc;
}

// Inverse-CDF draw over the unnormalised r held in registers: the smallest x
// with sum_{y <= x} r(y) > u * sum r. Tile i (register i of every thread,
// ids i * NT ...) is located from the tile sums (float per wave,
// float64 across waves), then one float64 block scan inside it finds x; if
// rounding between the two leaves no crossing there, the tile's last x with
// r > 0 is taken. s_pick holds 3 ints.
template <int EPT, int NT>
__device__ int reg_sample(const float (&r)[EPT], float u, double* s_tile, double* red, int* s_pick) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double s_thr, s_before;
  __shared__ double s_tsum[EPT];
  __shared__ int s_it;
  int lastpos = -1;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const float t = wave_sum_dpp(r[i]);  // locates the tile only; the scan inside it is float64
    if (lane == 0) s_tile[wave * EPT + i] = t;
    if (r[i] > 0.f) lastpos = i * NT + tid;
  }
  if (tid == 0) {
    s_pick[0] = -1;
    s_pick[1] = -1;
    s_pick[2] = -1;
  }
  __syncthreads();
  if (lastpos >= 0) atomicMax(&s_pick[1], lastpos);
  if (tid < EPT) {
    double t = 0.0;
    for (int w = 0; w < (NT / 64); ++w) t += s_tile[w * EPT + tid];
    s_tsum[tid] = t;
  }
  __syncthreads();
  if (tid == 0) {
    double total = 0.0;
    for (int i = 0; i < EPT; ++i) total += s_tsum[i];
    const double thr = static_cast<double>(u) * total;
    double before = 0.0;
    int it = -1;
    for (int i = 0; i < EPT; ++i) {
      if (before + s_tsum[i] > thr) {
        it = i;
        break;
      }
      before += s_tsum[i];
    }
    s_thr = thr;
    s_before = before;
    s_it = it;
  }
  __syncthreads();
  const int it = s_it;
  if (it >= 0) {
    float val = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (i == it) val = r[i];
    double inc = val;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(inc, off, 64);
      if (lane >= off) inc += o;
    }
    if (lane == 63) red[wave] = inc;
    __syncthreads();
    double woff = s_before;
    for (int w = 0; w < wave; ++w) woff += red[w];
    const double incl = woff + inc, excl = incl - val;
    const double thr = s_thr;
    if (val > 0.f && excl <= thr && thr < incl) s_pick[0] = it * NT + tid;
    if (val > 0.f) atomicMax(&s_pick[2], it * NT + tid);
  }
  __syncthreads();
  // no crossing: u * total beyond the last tile (the last x with r > 0), or
  // lost to rounding at the tile's end (its last x with r > 0)
  const int pick = s_pick[0] >= 0 ? s_pick[0] : (s_pick[2] >= 0 ? s_pick[2] : s_pick[1]);
  __syncthreads();
  return pick;
}

// ---------------------------------------------------------------------------
// Node-parallel acceptance. What the walk does at a node depends only on that
// node: its target row, the head row that drafted its children, the
// children's tokens and uniforms, its own residual uniform and its depth (the
// walk reaches node u having accepted depth(u) drafts). So one workgroup per
// tree row settles the node's outcome - the child it accepts, or else the
// token it draws - all rows at once on different CUs, and a small kernel per
// sequence then follows the accepted children from the root. The result is
// the walk's, decision for decision, and its latency no longer grows with the
// accepted length.

// the sequence's parents into LDS (N <= 256), all loads at once
__device__ __forceinline__ void load_parents(const int32_t* __restrict__ parent, int b, int N, int* s_par) {
  for (int c = threadIdx.x; c < N; c += blockDim.x) s_par[c] = parent[static_cast<size_t>(b) * N + c];
  __syncthreads();
}

// rejection mode: next[b, u] = the child accepted at u (children tried in rank
// order against the current residual, q unchanged), or -1 with draw[b, u] the
// inverse-CDF draw from the residual (from p when u has no children or sits
// at depth Dmax)
template <int EPT>
__global__ __launch_bounds__(kNodeThreads) void reject_node_reg(
    int N, int V, int R, int Dmax, float invT, const float* __restrict__ Z, const float* __restrict__ HZ,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ parent, const int32_t* __restrict__ q_row,
    const float* __restrict__ u_acc, const float* __restrict__ u_res, int32_t* __restrict__ next,
    int32_t* __restrict__ draw) {
  __shared__ double red[kNodeWaves];
  __shared__ float redf[kNodeWaves];
  __shared__ double s_tile[kNodeWaves * EPT];
  __shared__ int s_pick[3];
  __shared__ int s_kid[3];
  __shared__ float2 s_bc;
  __shared__ float3 s_next[2];
  __shared__ int s_par[HYDRA_MAX_VERIFY];
  const int b = blockIdx.x / N, u = blockIdx.x % N, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * N + u;
  load_parents(parent, b, N, s_par);
  if (tid == 0) {
    int d = 0, v = u;
    while (v > 0 && v < N && d <= N) {  // depth of u (a malformed chain stops within N steps)
      v = s_par[v];
      ++d;
    }
    if (v != 0) d = N + 1;  // not connected to the root: draw at u
    s_kid[0] = N;
    s_kid[1] = 0;
    s_kid[2] = d;
  }
  __syncthreads();
  for (int c = tid; c < N; c += kNodeThreads)
    if (s_par[c] == u) {
      atomicMin(&s_kid[0], c);
      atomicAdd(&s_kid[1], 1);
    }
  __syncthreads();
  const int c0 = s_kid[0], cnt = s_kid[1], depth = s_kid[2];
  const bool tries = cnt > 0 && depth < Dmax;
  // both rows in flight together: the target's, and the head row that
  // drafted u's children when there are children to try
  float r[EPT], q[EPT];
  reg_load_scaled<EPT, kNodeThreads>(r, Z, row, V, invT);
  if (tries) {
    const int qr = q_row[row];
    const size_t hrow = static_cast<size_t>(b) * R + (qr < 0 ? 0 : (qr >= R ? R - 1 : qr));
    reg_load_scaled<EPT, kNodeThreads>(q, HZ, hrow, V, invT);
  }
  double total = reg_exp<EPT, kNodeThreads>(r, red, redf);
  int taken = -1;
  if (tries) {
    const float qinv = static_cast<float>(1.0 / reg_exp<EPT, kNodeThreads>(q, red, redf));
#pragma unroll
    for (int i = 0; i < EPT; ++i) q[i] *= qinv;
    auto child_tok = [&](int c) {
      const int x = tok[static_cast<size_t>(b) * N + c];
      return x < 0 ? 0 : (x >= V ? V - 1 : x);
    };
    float2 rq = reg_at2<EPT, kNodeThreads>(r, q, child_tok(c0), &s_bc);
    for (int j = 0; j < cnt; ++j) {
      const int c = c0 + j;
      const float rx = static_cast<float>(rq.x / total);
      if (u_acc[static_cast<size_t>(b) * N + c] * rq.y < rx) {
        taken = c;
        break;
      }
      // residual norm(max(r - q, 0)), kept unless it has no mass; the
      // thread holding the next child's token posts that token's r before
      // and after the update and its q, so the sum's barriers also publish
      // the next lookup (two slots, alternating: a slot is rewritten only
      // after every thread has passed the barriers that follow its read)
      const float rinv = static_cast<float>(1.0 / total);
      float nsf = 0.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        float t = fmaxf(r[i] * rinv - q[i], 0.f);
        asm volatile("" : "+v"(t));  // recomputed below rather than kept: the rows fill the registers
        nsf += t;
      }
      const bool more = j + 1 < cnt;
      if (more) {
        const int xn = child_tok(c + 1);
        if (static_cast<int>(threadIdx.x) == xn % kNodeThreads) {
          float3 t = make_float3(0.f, 0.f, 0.f);
#pragma unroll
          for (int i = 0; i < EPT; ++i)
            if (i == xn / kNodeThreads) t = make_float3(r[i], fmaxf(r[i] * rinv - q[i], 0.f), q[i]);
          s_next[j & 1] = t;
        }
      }
      const double ns = block_sum_fd<kNodeWaves>(nsf, red);
      if (ns > 0.0) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) r[i] = fmaxf(r[i] * rinv - q[i], 0.f);
        total = ns;
      }
      if (more) {
        const float3 t = s_next[j & 1];
        rq = make_float2(ns > 0.0 ? t.y : t.x, t.z);
      }
    }
  }
  int x = -1;
  if (taken < 0) x = reg_sample<EPT, kNodeThreads>(r, u_res[row], s_tile, red, s_pick);
  if (tid == 0) {
    next[row] = taken;
    draw[row] = x;
  }
}

// typical mode: pass[b, c] for the children of u (see typical_rows) and
// draw[b, u], the inverse-CDF draw from p at u (used if the kept branch ends
// there)
template <int EPT>
__global__ __launch_bounds__(kNodeThreads) void typical_node_reg(int N, int V, float invT, float log_eps,
                                                                 float log_delta, const float* __restrict__ Z,
                                                                 const int32_t* __restrict__ tok,
                                                                 const int32_t* __restrict__ parent,
                                                                 const float* __restrict__ u_res,
                                                                 int32_t* __restrict__ pass,
                                                                 int32_t* __restrict__ draw) {
  __shared__ double red[kNodeWaves];
  __shared__ float redf[kNodeWaves];
  __shared__ double s_tile[kNodeWaves * EPT];
  __shared__ double s_w[kNodeWaves];
  __shared__ int s_pick[3];
  __shared__ int s_kid[2];
  const int b = blockIdx.x / N, u = blockIdx.x % N, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * N + u;
  if (tid == 0) {
    s_kid[0] = N;
    s_kid[1] = 0;
    if (u == 0) pass[static_cast<size_t>(b) * N] = 1;  // the root
  }
  __syncthreads();
  for (int c = tid; c < N; c += kNodeThreads)
    if (parent[static_cast<size_t>(b) * N + c] == u) {
      atomicMin(&s_kid[0], c);
      atomicAdd(&s_kid[1], 1);
    }
  float r[EPT];
  reg_load_scaled<EPT, kNodeThreads>(r, Z, row, V, invT);
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPT; ++i) mx = fmaxf(mx, r[i]);
  const float M = block_max_f<kNodeWaves>(mx, redf);
  float Sf = 0.f, Wf = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const float t = r[i] - M;
    const float e = r[i] == -INFINITY ? 0.f : exp2f(t * kLog2e);
    Sf += e;
    Wf += r[i] == -INFINITY ? 0.f : e * t;
    r[i] = e;
  }
  const double S = block_sum_d<kNodeWaves>(Sf, red);
  double Wd = Wf;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Wd += __shfl_xor(Wd, off, 64);
  if ((tid & 63) == 0) s_w[tid >> 6] = Wd;
  __syncthreads();
  double W = 0.0;
  for (int w = 0; w < kNodeWaves; ++w) W += s_w[w];
  const int c0 = s_kid[0], cnt = s_kid[1];
  if (cnt > 0) {
    const double logS = log(S);
    const double H = logS - W / S;
    const double log_tau = fmin(static_cast<double>(log_eps), static_cast<double>(log_delta) - H);
    const float* zu = Z + row * V;
    for (int j = tid; j < cnt; j += kNodeThreads) {
      const int c = c0 + j;
      const int x = tok[static_cast<size_t>(b) * N + c];
      const bool ok = x >= 0 && x < V &&
                      static_cast<double>(zu[x < 0 ? 0 : (x >= V ? V - 1 : x)] * invT - M) - logS > log_tau;
      pass[static_cast<size_t>(b) * N + c] = ok ? 1 : 0;
    }
  }
  const int x = reg_sample<EPT, kNodeThreads>(r, u_res[row], s_tile, red, s_pick);
  if (tid == 0) draw[row] = x;
}

// one wave per sequence: follow next[] from the root (rejection mode) and
// emit the accepted tokens plus the draw where the walk stops
__global__ __launch_bounds__(64) void reject_pick(int N, int Dmax, const int32_t* __restrict__ tok,
                                                  const int32_t* __restrict__ next, const int32_t* __restrict__ draw,
                                                  int32_t* __restrict__ n_accepted, int32_t* __restrict__ path,
                                                  int32_t* __restrict__ out_tok) {
  __shared__ int s_next[HYDRA_MAX_VERIFY], s_tok[HYDRA_MAX_VERIFY], s_draw[HYDRA_MAX_VERIFY];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int c = lane; c < N; c += 64) {
    s_next[c] = next[static_cast<size_t>(b) * N + c];
    s_tok[c] = tok[static_cast<size_t>(b) * N + c];
    s_draw[c] = draw[static_cast<size_t>(b) * N + c];
  }
  __syncthreads();
  if (lane == 0) {
    int u = 0, m = 0;
    int32_t* pb = path + static_cast<size_t>(b) * (Dmax + 1);
    int32_t* ob = out_tok + static_cast<size_t>(b) * (Dmax + 1);
    pb[0] = 0;
    while (m < Dmax && s_next[u] > u && s_next[u] < N) {  // children follow their parents
      const int c = s_next[u];
      ob[m] = s_tok[c];
      ++m;
      pb[m] = c;
      u = c;
    }
    ob[m] = s_draw[u];
    for (int j = m + 1; j <= Dmax; ++j) {
      pb[j] = -1;
      ob[j] = -1;
    }
    n_accepted[b] = m;
  }
}

// one workgroup per sequence: the kept branch of the typical mode from the
// pass flags, then the accepted tokens and the draw at its end
__global__ __launch_bounds__(256) void typical_pick(int N, int Dmax, const int32_t* __restrict__ tok,
                                                    const int32_t* __restrict__ parent,
                                                    const int32_t* __restrict__ pass,
                                                    const int32_t* __restrict__ draw,
                                                    int32_t* __restrict__ n_accepted, int32_t* __restrict__ path,
                                                    int32_t* __restrict__ out_tok) {
  __shared__ int s_par[HYDRA_MAX_VERIFY];
  __shared__ uint8_t s_pass[HYDRA_MAX_VERIFY];
  __shared__ uint32_t s_keys[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int c = tid; c < N; c += 256) {
    s_par[c] = parent[static_cast<size_t>(b) * N + c];
    s_pass[c] = pass[static_cast<size_t>(b) * N + c] != 0;
  }
  __syncthreads();
  // every node walks up to the root (at most Dmax steps): it is kept when each
  // node on the way passes; the kept branch is the largest (depth, -index)
  uint32_t key = 0;
  if (tid < N) {
    int v = tid, dc = 0;
    bool ok = true;
    while (v > 0 && ok) {
      const int pv = s_par[v];
      ok = pv >= 0 && pv < v && s_pass[v] && dc < Dmax;
      ++dc;
      v = pv;
    }
    if (ok && v == 0) key = (static_cast<uint32_t>(dc) << 16) | (0xFFFFu - static_cast<uint32_t>(tid));
  }
  key = wave_max_u32(key);
  if ((tid & 63) == 0) s_keys[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    const uint32_t best = max(max(s_keys[0], s_keys[1]), max(s_keys[2], s_keys[3]));
    const int end = static_cast<int>(0xFFFFu - (best & 0xFFFFu)), m = static_cast<int>(best >> 16);
    int32_t* pb = path + static_cast<size_t>(b) * (Dmax + 1);
    int32_t* ob = out_tok + static_cast<size_t>(b) * (Dmax + 1);
    for (int j = m + 1; j <= Dmax; ++j) {
      pb[j] = -1;
      ob[j] = -1;
    }
    ob[m] = draw[static_cast<size_t>(b) * N + end];
    int v = end;
    for (int j = m; j >= 1; --j) {
      pb[j] = v;
      ob[j - 1] = tok[static_cast<size_t>(b) * N + v];
      v = s_par[v];
    }
    pb[0] = 0;
    n_accepted[b] = m;
  }
}

// register tiles per thread for a vocabulary of V, or 0 past 32 (streamed walks)
// registers per row and thread of the node kernels, 0 when the row does not
// fit (then the streaming walks run)
int walk_ept(int V) {
  const int e = (V + kNodeThreads - 1) / kNodeThreads;
  for (int t = 1; t <= 64; t *= 2)
    if (e <= t) return t;
  return 0;
}

template <typename F>
void with_ept(int ept, F f) {
  switch (ept) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    case 16: f(std::integral_constant<int, 16>{}); break;
    case 32: f(std::integral_constant<int, 32>{}); break;
    default: f(std::integral_constant<int, 64>{}); break;
  }
}

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" size_t tree_accept_workspace_size(int mode, int B, int N, int V) {
  if (B <= 0 || N <= 0 || V <= 0) return 0;
  const size_t rows = static_cast<size_t>(B) * N;
  if (mode == 0)
    return align_up(rows * sizeof(int32_t), 256) + align_up(rows * projection_nwg(V) * sizeof(uint64_t), 256) +
           align_up(static_cast<size_t>(B) * sizeof(int), 256) + 256;
  // modes 1 and 2: two int32 per row (next child or pass flag, and the draw)
  const size_t per_row = 2 * align_up(rows * sizeof(int32_t), 256);
  if (mode == 2) return per_row + 256;
  return per_row + align_up(static_cast<size_t>(B) * 2 * V * sizeof(float), 256) + 256;
}

extern "C" int tree_accept(int dtype, int mode, int B, int N, int d, int V, int Dmax, const void* o,
                           const void* W_t, float temperature, float eps, float delta, const int32_t* tok,
                           const int32_t* parent,
                           const int32_t* q_row, const float* head_logits, int R, const float* u_acc,
                           const float* u_res, float* target_logits, int32_t* n_accepted, int32_t* path,
                           int32_t* out_tok, void* ws, size_t ws_bytes, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int vpack = dtype & HYDRA_VOCAB_PACKED;  // packed vocabulary weights (hydra_pack_weight)
  dtype &= ~HYDRA_VOCAB_PACKED;
  HY_CHECK(dtype == HYDRA_F32 || dtype == HYDRA_BF16, HYDRA_ERR_INVALID, "tree_accept: bad dtype %d", dtype);
  HY_CHECK(!vpack || dtype == HYDRA_BF16, HYDRA_ERR_UNSUPPORTED, "tree_accept: packed vocabulary weights are bf16");
  HY_CHECK(mode >= 0 && mode <= 2, HYDRA_ERR_INVALID, "tree_accept: mode %d not in {0, 1, 2}", mode);
  HY_CHECK(B > 0 && N > 0 && d > 0 && V > 0, HYDRA_ERR_INVALID, "tree_accept: bad sizes B=%d N=%d d=%d V=%d", B, N,
           d, V);
  HY_CHECK(N <= HYDRA_MAX_VERIFY, HYDRA_ERR_INVALID, "tree_accept: N=%d > %d", N, HYDRA_MAX_VERIFY);
  HY_CHECK(Dmax >= 1 && Dmax <= HYDRA_MAX_DEPTH, HYDRA_ERR_INVALID, "tree_accept: Dmax=%d", Dmax);
  HY_CHECK(o && W_t && tok && parent && target_logits && n_accepted && path && out_tok, HYDRA_ERR_INVALID,
           "tree_accept: null pointer");
  HY_CHECK(dtype == HYDRA_F32 || d % 256 == 0, HYDRA_ERR_UNSUPPORTED, "tree_accept: bf16 needs d %% 256 == 0 (d=%d)",
           d);
  if (mode == 1) {
    HY_CHECK(q_row && head_logits && u_acc && u_res && R > 0, HYDRA_ERR_INVALID,
             "tree_accept: rejection mode needs q_row, head_logits, R, u_acc and u_res");
    HY_CHECK(temperature > 0.f, HYDRA_ERR_INVALID, "tree_accept: temperature must be > 0");
  }
  if (mode == 2) {
    HY_CHECK(u_res, HYDRA_ERR_INVALID, "tree_accept: typical mode needs u_res");
    HY_CHECK(temperature > 0.f, HYDRA_ERR_INVALID, "tree_accept: temperature must be > 0");
    HY_CHECK(eps >= 0.f && delta >= 0.f, HYDRA_ERR_INVALID, "tree_accept: eps and delta must be >= 0");
  }
  const size_t need = tree_accept_workspace_size(mode, B, N, V);
  HY_CHECK(ws_bytes >= need && ws, HYDRA_ERR_WORKSPACE, "tree_accept: workspace %zu < %zu", ws_bytes, need);

  XSource xs{};
  xs.x = o;
  xs.ldx = d;
  xs.mode = 0;
  const int M = B * N;
  Arena arena(ws, ws_bytes);
  if (mode == 0) {
    // target logits with fused arg-max partials, merged per row, then the walk
    int32_t* amax = arena.take<int32_t>(static_cast<size_t>(M));
    const int nwg = projection_nwg(V);
    uint64_t* keys = arena.take<uint64_t>(static_cast<size_t>(M) * nwg);
    int* walk_count = arena.take<int>(static_cast<size_t>(B));
    // with up to 256 sequences the projection clears the walk counters and
    // the row merge's last workgroup per sequence walks; otherwise a walk kernel
    const bool fused_walk = B <= 256;
    TopkPartials tp{keys, nullptr, fused_walk ? walk_count : nullptr, fused_walk ? B : 0};
    int rc = launch_projection(dtype | vpack, M, d, V, xs, W_t, target_logits, RowMap{M, 0, 0}, V, 1, nullptr, tp, stream);
    if (rc != HYDRA_OK) return rc;
    MergeArgs ma{};
    ma.M = M;
    ma.nwg = nwg;
    ma.k = 1;
    ma.keys = keys;
    ma.ms = nullptr;  // the greedy walk needs the arg max only
    ma.Y = target_logits;
    ma.ldy = V;
    ma.V = V;
    ma.map = RowMap{M, 0, 0};
    ma.amax = amax;
    ma.P = 1;
    if (fused_walk) {
      ma.N = N;
      ma.walk_count = walk_count;
      ma.wtok = tok;
      ma.wparent = parent;
      ma.wDmax = Dmax;
      ma.n_accepted = n_accepted;
      ma.path = path;
      ma.out_tok = out_tok;
    }
    rc = launch_topk_merge(ma, stream);
    if (rc != HYDRA_OK) return rc;
    if (!fused_walk) {
      greedy_walk<<<B, 64, 0, stream>>>(N, Dmax, amax, tok, parent, n_accepted, path, out_tok);
      HY_LAUNCH_CHECK("tree_accept: greedy walk");
    }
  } else if (mode == 2) {
    int rc = launch_projection(dtype | vpack, M, d, V, xs, W_t, target_logits, RowMap{M, 0, 0}, V, 1, nullptr,
                               TopkPartials{nullptr, nullptr}, stream);
    if (rc != HYDRA_OK) return rc;
    int32_t* pass = arena.take<int32_t>(static_cast<size_t>(M));
    int32_t* drawn = arena.take<int32_t>(static_cast<size_t>(M));
    const float invT = 1.0f / temperature;
    if (const int ept = walk_ept(V)) {
      with_ept(ept, [&](auto e) {
        typical_node_reg<decltype(e)::value><<<M, kNodeThreads, 0, stream>>>(
            N, V, invT, logf(eps), logf(delta), target_logits, tok, parent, u_res, pass, drawn);
      });
      HY_LAUNCH_CHECK("tree_accept: typical nodes");
      typical_pick<<<B, 256, 0, stream>>>(N, Dmax, tok, parent, pass, drawn, n_accepted, path, out_tok);
      HY_LAUNCH_CHECK("tree_accept: typical pick");
    } else {
      typical_rows<<<M, kTypThreads, 0, stream>>>(N, V, invT, logf(eps), logf(delta), target_logits, tok, parent,
                                                  pass);
      HY_LAUNCH_CHECK("tree_accept: typical rows");
      typical_walk<<<B, kWalkThreads, 0, stream>>>(N, V, Dmax, invT, target_logits, tok, parent, pass, u_res,
                                                   n_accepted, path, out_tok);
      HY_LAUNCH_CHECK("tree_accept: typical walk");
    }
  } else {
    int rc = launch_projection(dtype | vpack, M, d, V, xs, W_t, target_logits, RowMap{M, 0, 0}, V, 1, nullptr,
                               TopkPartials{nullptr, nullptr}, stream);
    if (rc != HYDRA_OK) return rc;
    int32_t* nxt = arena.take<int32_t>(static_cast<size_t>(M));
    int32_t* drawn = arena.take<int32_t>(static_cast<size_t>(M));
    float* rbuf = arena.take<float>(static_cast<size_t>(B) * 2 * V);
    const float invT = 1.0f / temperature;
    if (const int ept = walk_ept(V)) {
      with_ept(ept, [&](auto e) {
        reject_node_reg<decltype(e)::value><<<M, kNodeThreads, 0, stream>>>(
            N, V, R, Dmax, invT, target_logits, head_logits, tok, parent, q_row, u_acc, u_res, nxt, drawn);
      });
      HY_LAUNCH_CHECK("tree_accept: rejection nodes");
      reject_pick<<<B, 64, 0, stream>>>(N, Dmax, tok, nxt, drawn, n_accepted, path, out_tok);
    } else {
      reject_walk<<<B, kWalkThreads, 0, stream>>>(N, V, R, Dmax, invT, target_logits, head_logits, tok, parent,
                                                  q_row, u_acc, u_res, rbuf, n_accepted, path, out_tok);
    }
    HY_LAUNCH_CHECK("tree_accept: rejection walk");
  }
  return HYDRA_OK;
}

// ------------------------------------------------------------------------
// Allocation-free variant: the scratch tree_accept takes from a caller
// workspace lives instead in this module's static device array, one copy per
// GPU. Its device address is taken once per device (hipGetSymbolAddress, with
// that device current) and kept; host code never passes the array's own name
// to a kernel. Every call on a GPU shares that GPU's array and leaves its
// contents behind; nothing in it has to start at zero (the walk counters are
// cleared by the projection launch of the same call), and calls that overlap
// on one GPU race.

namespace hydra {
namespace {

constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(32) << 20;  // 32 MiB
constexpr int kNoAllocMaxDevices = 64;

}  // namespace
}  // namespace hydra

static __device__ __align__(256) uint8_t scratch[hydra::kNoAllocScratchBytes];

namespace hydra {
namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call made with that device current.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  HY_CHECK(e == hipSuccess && dev >= 0 && dev < kNoAllocMaxDevices, HYDRA_ERR_HIP,
           "tree_accept_noalloc: no usable current device (%s, device %d)", hipGetErrorString(e), dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    HY_CHECK(e == hipSuccess && p, HYDRA_ERR_HIP, "tree_accept_noalloc: hipGetSymbolAddress failed on device %d (%s)",
             dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HYDRA_OK;
}

}  // namespace
}  // namespace hydra

extern "C" int tree_accept_noalloc(int dtype, int mode, int B, int N, int d, int V, int Dmax, const void* o,
                                   const void* W_t, float temperature, float eps, float delta, const int32_t* tok,
                                   const int32_t* parent, const int32_t* q_row, const float* head_logits, int R,
                                   const float* u_acc, const float* u_res, float* target_logits,
                                   int32_t* n_accepted, int32_t* path, int32_t* out_tok, void* stream) {
  clear_error();
  HY_CHECK(B > 0 && N > 0 && V > 0, HYDRA_ERR_INVALID, "tree_accept_noalloc: bad sizes B=%d N=%d V=%d", B, N, V);
  const size_t need = tree_accept_workspace_size(mode, B, N, V);
  HY_CHECK(need <= kNoAllocScratchBytes, HYDRA_ERR_WORKSPACE,
           "tree_accept_noalloc: this call needs %zu bytes of scratch, more than the %zu the library holds per "
           "device (use tree_accept with a workspace)",
           need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != HYDRA_OK) return rc;
  return tree_accept(dtype, mode, B, N, d, V, Dmax, o, W_t, temperature, eps, delta, tok, parent, q_row,
                     head_logits, R, u_acc, u_res, target_logits, n_accepted, path, out_tok, ws,
                     kNoAllocScratchBytes, stream);
}
