// Host side of libhydra: status strings, the thread-local error message and
// the tree-plan builders (no device work).
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "../../include/hydra.h"

namespace hydra {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

namespace {

typedef std::vector<int> Path;

// Breadth-first plan from a prefix-closed set of rank paths: ordered by depth,
// then by the path itself, which sorts siblings by rank under parents that
// are already in breadth-first order.
int emit_plan(std::vector<Path> paths, int max_nodes, int32_t* parent, int32_t* rank, int32_t* depth) {
  std::sort(paths.begin(), paths.end(), [](const Path& a, const Path& b) {
    if (a.size() != b.size()) return a.size() < b.size();
    return a < b;
  });
  const int n = static_cast<int>(paths.size()) + 1;
  if (n > max_nodes) {
    set_error("plan: %d nodes exceed capacity %d", n, max_nodes);
    return HYDRA_ERR_INVALID;
  }
  std::map<Path, int> index;
  index[Path()] = 0;
  parent[0] = -1;
  rank[0] = -1;
  depth[0] = 0;
  for (int i = 1; i < n; ++i) {
    const Path& p = paths[i - 1];
    Path up(p.begin(), p.end() - 1);
    auto it = index.find(up);
    if (it == index.end()) {
      set_error("plan: path set is not closed under parents");
      return HYDRA_ERR_INVALID;
    }
    index[p] = i;
    parent[i] = it->second;
    rank[i] = p.back();
    depth[i] = static_cast<int32_t>(p.size());
  }
  return n;
}

}  // namespace
}  // namespace hydra

using namespace hydra;

extern "C" const char* hydra_status_string(int code) {
  switch (code) {
    case HYDRA_OK: return "ok";
    case HYDRA_ERR_INVALID: return "invalid argument";
    case HYDRA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HYDRA_ERR_WORKSPACE: return "workspace too small";
    case HYDRA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" const char* hydra_last_error(void) { return g_last_error.c_str(); }

extern "C" int hydra_abi_version(void) { return 9; }

extern "C" int hydra_plan_cartesian(const int32_t* b, int K, int max_nodes, int32_t* parent, int32_t* rank,
                                    int32_t* depth) {
  clear_error();
  if (!b || !parent || !rank || !depth || K < 1 || K > HYDRA_MAX_DEPTH || max_nodes < 1) {
    set_error("plan_cartesian: bad arguments (K=%d, max_nodes=%d)", K, max_nodes);
    return HYDRA_ERR_INVALID;
  }
  long long total = 1, level = 1;
  for (int k = 0; k < K; ++k) {
    if (b[k] < 1 || b[k] > HYDRA_MAX_TOPK) {
      set_error("plan_cartesian: b[%d]=%d out of [1, %d]", k, b[k], HYDRA_MAX_TOPK);
      return HYDRA_ERR_INVALID;
    }
    level *= b[k];
    total += level;
    if (total > max_nodes) {
      set_error("plan_cartesian: %lld nodes exceed capacity %d", total, max_nodes);
      return HYDRA_ERR_INVALID;
    }
  }
  std::vector<Path> paths, frontier(1);
  for (int k = 0; k < K; ++k) {
    std::vector<Path> next;
    for (const Path& p : frontier)
      for (int r = 0; r < b[k]; ++r) {
        Path q = p;
        q.push_back(r);
        next.push_back(q);
      }
    paths.insert(paths.end(), next.begin(), next.end());
    frontier.swap(next);
  }
  return emit_plan(paths, max_nodes, parent, rank, depth);
}

extern "C" int hydra_plan_sparse(const int32_t* caps, int K, int n_nodes, int max_nodes, int32_t* parent,
                                 int32_t* rank, int32_t* depth) {
  clear_error();
  if (!caps || !parent || !rank || !depth || K < 1 || K > HYDRA_MAX_DEPTH || n_nodes < 1 || n_nodes > max_nodes) {
    set_error("plan_sparse: bad arguments (K=%d, n_nodes=%d, max_nodes=%d)", K, n_nodes, max_nodes);
    return HYDRA_ERR_INVALID;
  }
  long long count = 0, level = 1;
  for (int k = 0; k < K; ++k) {
    if (caps[k] < 1 || caps[k] > HYDRA_MAX_TOPK) {
      set_error("plan_sparse: caps[%d]=%d out of [1, %d]", k, caps[k], HYDRA_MAX_TOPK);
      return HYDRA_ERR_INVALID;
    }
    level *= caps[k];
    count += level;
    if (count > 4000000) {
      set_error("plan_sparse: too many candidate paths");
      return HYDRA_ERR_INVALID;
    }
  }
  if (count + 1 < n_nodes) {
    set_error("plan_sparse: only %lld candidates for %d nodes", count, n_nodes);
    return HYDRA_ERR_INVALID;
  }
  struct Cand {
    double score;
    Path path;
  };
  std::vector<Cand> cands;
  std::vector<Path> frontier(1);
  for (int k = 0; k < K; ++k) {
    std::vector<Path> next;
    for (const Path& p : frontier)
      for (int r = 0; r < caps[k]; ++r) {
        Path q = p;
        q.push_back(r);
        double s = static_cast<double>(1ll << q.size());
        for (int x : q) s *= x + 1;
        cands.push_back({s, q});
        next.push_back(q);
      }
    frontier.swap(next);
  }
  // rank prior 2^d * prod(r + 1), then depth, then the path
  std::sort(cands.begin(), cands.end(), [](const Cand& a, const Cand& b) {
    if (a.score != b.score) return a.score < b.score;
    if (a.path.size() != b.path.size()) return a.path.size() < b.path.size();
    return a.path < b.path;
  });
  std::vector<Path> keep;
  for (int i = 0; i < n_nodes - 1; ++i) keep.push_back(cands[i].path);
  return emit_plan(keep, max_nodes, parent, rank, depth);
}

extern "C" int hydra_plan_rows(int N, const int32_t* parent, const int32_t* rank, const int32_t* depth, int hydra_mode,
                               int32_t* node_row, int32_t* row_node, int32_t* row_first, int32_t* depth_first,
                               int32_t* k_per_depth) {
  clear_error();
  if (N < 2 || N > HYDRA_MAX_TREE || !parent || !rank || !depth || !node_row || !row_node || !row_first ||
      !depth_first || !k_per_depth) {
    set_error("plan_rows: bad arguments (N=%d)", N);
    return HYDRA_ERR_INVALID;
  }
  if (parent[0] != -1 || depth[0] != 0) {
    set_error("plan_rows: node 0 must be the root");
    return HYDRA_ERR_INVALID;
  }
  std::vector<int> nkids(N, 0);
  for (int i = 1; i < N; ++i) {
    const int p = parent[i];
    if (p < 0 || p >= i || depth[i] != depth[p] + 1 || depth[i] < depth[i - 1] || depth[i] > HYDRA_MAX_DEPTH) {
      set_error("plan_rows: node %d breaks breadth-first order", i);
      return HYDRA_ERR_INVALID;
    }
    if (rank[i] != nkids[p] || (nkids[p] > 0 && parent[i - 1] != p)) {
      set_error("plan_rows: children of node %d are not contiguous with ranks 0..n-1", p);
      return HYDRA_ERR_INVALID;
    }
    ++nkids[p];
    if (nkids[p] > HYDRA_MAX_TOPK) {
      set_error("plan_rows: node %d has more than %d children", p, HYDRA_MAX_TOPK);
      return HYDRA_ERR_INVALID;
    }
  }
  const int dmax = depth[N - 1];
  for (int k = 0; k <= dmax + 1; ++k) depth_first[k] = N;
  for (int i = N - 1; i >= 0; --i) depth_first[depth[i]] = i;
  depth_first[dmax + 1] = N;
  for (int k = 0; k < dmax; ++k) k_per_depth[k] = 0;
  for (int i = 0; i < N; ++i)
    if (nkids[i] > 0) k_per_depth[depth[i]] = std::max(k_per_depth[depth[i]], nkids[i]);
  int R = 0;
  row_first[0] = 0;
  for (int i = 0; i < N; ++i) node_row[i] = -1;
  if (hydra_mode) {
    for (int k = 0; k < dmax; ++k) {
      for (int i = depth_first[k]; i < depth_first[k + 1]; ++i)
        if (nkids[i] > 0) {
          node_row[i] = R;
          row_node[R] = i;
          ++R;
        }
      row_first[k + 1] = R;
    }
  } else {
    for (int k = 0; k < dmax; ++k) {
      for (int i = depth_first[k]; i < depth_first[k + 1]; ++i)
        if (nkids[i] > 0) node_row[i] = k;
      row_node[R] = -1;
      ++R;
      row_first[k + 1] = R;
    }
  }
  return R;
}
