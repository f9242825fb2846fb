"""Oracle: a plain, slow CPU implementation of one Hydra/Medusa round.

TEST INFRASTRUCTURE ONLY. This module exists to check the device path. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product never calls it, and it shares no code
with the product (no helpers, tables or constants); the two meet only through
the seeded arrays that ``hydra_inputs`` generates.

Sources (cited by page title and section):

* [HG] "Hydra Guide: Sequentially-Dependent Speculative AI" (AiFetchly blog).
* [SD] "Speculative Decoding" (thegustafson.com blog).
* [MH] "Medusa Heads" (Ultralytics glossary, German).

Arithmetic is float64 throughout. For bfloat16 workloads the inputs arrive
already rounded to bfloat16, and the oracle rounds to bfloat16 (round to
nearest even) at exactly the two points where the device path stores a
bfloat16 tensor: the head hidden state ``u`` and the attention output ``O``.
Logits, log-sum-exps and cumulative log-probabilities stay float64.

Readings of points the pages leave open:

* Hydra head form: one layer, ``u = h + SiLU(W1 [h || e(parent)] + b1)``; the
  residual on ``h`` is the Medusa block with its input widened.
* The root of the tree is the last known token that is not yet in the KV
  cache; it is row 0 of the verify pass and attends to the prefix and itself.
* Ties in top-k and argmax go to the lowest token id; top-k output is sorted by
  (logit descending, id ascending).
* Cumulative score of a node is the sum of log-softmax values on its path.
* Dense tree pruning keeps the root plus the best ``n_keep - 1`` nodes by
  (cumulative log-prob descending, depth ascending, full-tree index ascending)
  and renumbers the survivors in breadth-first order.
* Sparse template: rank paths with ranks below the per-depth fan-out caps,
  ordered by (2**depth * prod(rank + 1), depth, path) ascending; the first
  ``n_nodes - 1`` plus the root.
* Positions: tree row u of sequence b stands at L_b + depth(u); rotary
  embedding in the LLaMA half-split layout with base theta (10000).
* Full-path conditioning ([HG] "2. Generalizing to Arbitrary Tree Depths":
  head k reads h and the embeddings of every token before its position): the
  one-layer head with x = [h || e(t_0) || ... || e(t_{k-1})], t_j the token
  of the depth-j node on the path from the root to the expanded node (t_0 the
  root's, so head 1 reads [h || e(root)] as with parent-only conditioning);
  W1 of head k is [d, (k + 1) d].
* Hydra++ self-attention fusion ([HG] "3. Hydra++": one causal
  self-attention layer over the candidate token embeddings): one layer
  shared by all heads, single head, no biases, scale 1/sqrt(d). At an
  expanded node with path tokens t_0 .. t_{k-1}, x_j = e(t_j), the query is
  Wq x_{k-1}, keys Wk x_j, values Wv x_j (j <= k - 1: causal), and
  c = x_{k-1} + Wo sum_j softmax_j(q . K_j / sqrt(d)) V_j replaces e(parent)
  in the one-layer head. In bf16 the attention output and c are rounded
  (stored), q, K and V are not.
* Two-layer heads of the [HG] sketch: head 1 LayerNorm(SiLU(Wa h + ba)), later
  heads LayerNorm(Wb SiLU(Wa [h || e(parent)] + ba) + bb), LayerNorm eps 1e-5.
* Decoder layer of the verify pass: the LLaMA pre-norm layer (RMSNorm,
  rotated Q/K, tree attention, output projection, residual, RMSNorm, SwiGLU
  feed-forward, residual) over every tree row at once.
* Typical acceptance: at the parent u, with p = softmax(Z[u] / T), a child
  passes iff p(x) > min(eps, delta * exp(-H(p))); the kept branch is the
  deepest node whose whole path passes (smallest breadth-first index among
  equals), and one token is drawn from p at its end with that node's u_res.
* Commit after acceptance: the root and the accepted drafts take cache
  positions L .. L + m in path order; the bonus token is the next root and
  the hidden state of the last accepted row the next h.
* Stochastic acceptance on a tree (rule S1): siblings are tried in rank order;
  after each rejection the target becomes the normalised residual while the
  draft distribution stays the same.

Parity unpinned: the choice of nodes in the sparse template beyond its
invariants (a construction of this oracle's own), rule S1 on a tree whose
children are deterministic top-k tokens (the pages prove exactness only for a
drafted chain), and the threshold form of typical acceptance (the pages only
tie it to the entropy; its pins are its limits and closed forms).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "round_bf16", "silu", "logsumexp", "softmax", "topk_sorted", "topk_margin",
    "TreePlan", "plan_cartesian", "plan_sparse_template", "head_rows",
    "head_hidden", "head_logits", "draft_heads", "prune_tree", "ancestors",
    "tree_mask", "tree_attention", "target_logits", "argmax_lowest",
    "greedy_accept", "residual", "sample_inverse_cdf", "rejection_accept",
    "commit_path", "entropy", "typical_passes", "kept_branch", "typical_accept",
    "tree_positions", "rope", "rms_norm", "decoder_layer", "layer_norm", "sketch_hidden", "path_tokens", "path_attention",
]


# ---------------------------------------------------------------------------
# Scalar building blocks
# ---------------------------------------------------------------------------

def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (7 stored plus the implicit one) and the
    float32 exponent range. Written as: split x = m * 2**e with 0.5 <= |m| < 1,
    round m * 2**8 to the nearest integer (ties to even), scale back.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def silu(a):
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a))  [MH, "So sagen die Köpfe voraus"]."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def logsumexp(z):
    """log(sum(exp(z))) with the maximum factored out."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z)
    return float(m + np.log(np.sum(np.exp(z - m))))


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def topk_sorted(z, k):
    """Ids of the k largest entries, sorted by (value descending, id ascending).

    [HG, "Candidate Tree Construction"]: head k keeps its top-b_k tokens.
    np.lexsort sorts by its last key first: -z ascending, then id ascending.
    """
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.shape[0]), -z))
    return order[:k].astype(np.int64)


def topk_margin(z, k):
    """Smallest gap between consecutive sorted values among the first k+1.

    A top-k decision (which ids, in which order) can only change under a
    perturbation of z larger than half this gap.
    """
    s = np.sort(np.asarray(z, dtype=np.float64))[::-1][: k + 1]
    if s.shape[0] < 2:
        return math.inf
    return float(np.min(s[:-1] - s[1:]))


def argmax_lowest(z):
    """Arg max with ties going to the lowest id."""
    z = np.asarray(z, dtype=np.float64)
    return int(np.flatnonzero(z == np.max(z))[0])


# ---------------------------------------------------------------------------
# Tree plans (shape of the candidate tree, independent of token values)
# ---------------------------------------------------------------------------

@dataclass
class TreePlan:
    """A candidate tree in breadth-first order.

    Node 0 is the root. ``parent[i] < i``; the children of a node are
    contiguous and sorted by ``rank`` (which entry of the parent's top-k list
    the child takes).
    """
    parent: np.ndarray
    rank: np.ndarray
    depth: np.ndarray

    @property
    def n(self) -> int:
        return int(self.parent.shape[0])

    @property
    def dmax(self) -> int:
        return int(self.depth.max())

    def children(self, u):
        return [int(c) for c in np.flatnonzero(self.parent == u)]


def _plan_from_paths(paths):
    """Build a breadth-first plan from a prefix-closed set of rank paths."""
    paths = sorted(set(tuple(p) for p in paths), key=lambda p: (len(p), p))
    index = {(): 0}
    parent, rank, depth = [-1], [-1], [0]
    for p in paths:
        index[p] = len(parent)
        parent.append(index[p[:-1]])
        rank.append(p[-1])
        depth.append(len(p))
    return TreePlan(np.array(parent), np.array(rank), np.array(depth))


def plan_cartesian(b):
    """Cartesian tree from a branching vector b = [b_1 .. b_K].

    [HG, "Candidate Tree Construction"]: head 1 keeps its top-b_1 tokens and,
    for every node at depth k-1, head k keeps its top-b_k continuations, so the
    tree has sum_k prod_{j<=k} b_j candidate nodes (plus the root here).
    """
    paths = []
    frontier = [()]
    for bk in b:
        frontier = [p + (r,) for p in frontier for r in range(bk)]
        paths.extend(frontier)
    return _plan_from_paths(paths)


def plan_sparse_template(caps=(10, 4, 2, 1), n_nodes=64):
    """Static sparse tree of n_nodes rows (root included).

    [MH, "Tree Attention und Akzeptanz"] only says the 64-node sparse tree is
    made of the most accurate combinations. With no accuracy statistics, the
    rank paths are ordered by the prior 2**depth * prod(rank + 1) (then depth,
    then the path itself) and the first n_nodes - 1 are kept.
    """
    cands = []
    frontier = [()]
    for cap in caps:
        frontier = [p + (r,) for p in frontier for r in range(cap)]
        cands.extend(frontier)

    def key(p):
        s = 2 ** len(p)
        for r in p:
            s *= r + 1
        return (s, len(p), p)

    cands.sort(key=key)
    return _plan_from_paths(cands[: n_nodes - 1])


def head_rows(plan: TreePlan, hydra: bool):
    """Head rows of a round: which node each row conditions on, and per node
    the row whose top-k list gives that node's children.

    Hydra [HG, "Candidate Tree Construction"]: head k runs once for every node
    at depth k-1 that has children, on [h || e(token of that node)].
    Medusa [MH, "Tree Attention und Akzeptanz"]: head k reads only h, so one
    row per depth serves every parent at that depth.
    Returns (row_node, row_depth, node_row) where row_depth is the head index
    (1-based) and node_row[u] = -1 for a node without children.
    """
    n = plan.n
    has_child = np.zeros(n, dtype=bool)
    has_child[plan.parent[1:]] = True
    node_row = -np.ones(n, dtype=np.int64)
    row_node, row_depth = [], []
    if hydra:
        for u in range(n):
            if has_child[u]:
                node_row[u] = len(row_node)
                row_node.append(u)
                row_depth.append(int(plan.depth[u]) + 1)
    else:
        for k in range(plan.dmax):
            row_node.append(-1)
            row_depth.append(k + 1)
        for u in range(n):
            if has_child[u]:
                node_row[u] = int(plan.depth[u])
    return np.array(row_node), np.array(row_depth), node_row


# ---------------------------------------------------------------------------
# Stage 1: draft heads
# ---------------------------------------------------------------------------

def head_hidden(h, e, W1, b1, residual=True, bf16=False):
    """Hidden state of one head row.

    Medusa [MH, "So sagen die Köpfe voraus"]: one feed-forward layer with SiLU
    and a residual connection, u = h + SiLU(W1 h + b1). Hydra
    [HG, "1. Embedding Conditioning Mechanics"]: the layer reads
    [h || e(x_parent)] instead of h. W1 has shape [d, in] (in = d or 2 d).
    """
    h = np.asarray(h, dtype=np.float64)
    x = h if e is None else np.concatenate([h, np.asarray(e, dtype=np.float64)])
    a = np.asarray(W1, dtype=np.float64) @ x + np.asarray(b1, dtype=np.float64)
    u = h + silu(a) if residual else silu(a)
    return round_bf16(u) if bf16 else u


def layer_norm(x, g, b, eps=1e-5):
    """(x - mean) / sqrt(var + eps) * g + b over the last axis (biased var)."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, dtype=np.float64) + np.asarray(b, dtype=np.float64)


def sketch_hidden(h, e, head, bf16=False):
    """Hidden state of one row of the two-layer head of the [HG] sketch
    ("Python code block" of the implementation section: HydraHeadLayer and
    HydraDraftEngine). Head 1 reads h alone: LayerNorm(SiLU(Wa h + ba)).
    Later heads read [h || e(parent)]: LayerNorm(Wb SiLU(Wa [h || e] + ba) + bb),
    Wa [H, 2d] (H = 1024 in the sketch), Wb [d, H]; every Linear has a bias
    and the LayerNorm a gain and a bias. With bf16 the two stored tensors (the
    SiLU output and u) are rounded."""
    r = round_bf16 if bf16 else (lambda t: t)
    f = lambda t: np.asarray(t, dtype=np.float64)  # noqa: E731
    x = f(h) if e is None else np.concatenate([f(h), f(e)])
    a = r(silu(f(head["Wa"]) @ x + f(head["ba"])))
    if "Wb" in head:
        a = f(head["Wb"]) @ a + f(head["bb"])
    return r(layer_norm(a, head["ln_g"], head["ln_b"]))


def head_logits(u, W2):
    """Vocabulary projection of a head, z = W2 u (W2 has no bias)."""
    return np.asarray(W2, dtype=np.float64) @ np.asarray(u, dtype=np.float64)


def path_tokens(plan: TreePlan, tok_b, root_tok_b, node):
    """Tokens t_0 .. t_depth(node) on the path from the root to ``node``."""
    path = []
    while node != 0:
        path.append(int(tok_b[node]))
        node = int(plan.parent[node])
    path.append(int(root_tok_b))
    return path[::-1]


def path_attention(X, attn, bf16=False):
    """Hydra++ fusion of the path embeddings X [k, d] (root first): the
    causal self-attention output at the last position plus the residual,
    c = x_{k-1} + Wo softmax(q K^T / sqrt(d)) V with q = Wq x_{k-1}."""
    X = np.asarray(X, dtype=np.float64)
    f = lambda n: np.asarray(attn[n], dtype=np.float64)  # noqa: E731
    r = round_bf16 if bf16 else (lambda t: t)
    q = f("Wq") @ X[-1]
    K = X @ f("Wk").T
    Vv = X @ f("Wv").T
    s = K @ q / math.sqrt(X.shape[1])
    p = np.exp(s - np.max(s))
    a = r(p @ Vv / np.sum(p))
    return r(X[-1] + f("Wo") @ a)


def draft_heads(h, root_tok, E, heads, plan: TreePlan, hydra=True,
                residual=True, bf16=False, forced_tok=None, full_path=False, attn=None):
    """All draft heads of one round, filling the candidate tree.

    h [B, d], root_tok [B], E [V, d] (Hydra only), heads = list of (W1, b1, W2)
    with head k at index k-1, or of dicts for the sketch's two-layer heads
    (Wa, ba, [Wb, bb,] ln_g, ln_b, W2; see sketch_hidden). Node c at depth k
    takes entry rank[c] of the top-k list of the row that expanded its parent;
    its cumulative score adds that token's log-softmax to the parent's.

    ``full_path``: Hydra heads read the embeddings of the whole path from the
    root to the expanded node instead of its token alone (W1 of head k is
    [d, (k + 1) d]).

    ``attn``: Hydra++ fusion (dict of Wq, Wk, Wv, Wo, [d, d] each): the
    head reads [h || path_attention(embeddings of the path)] instead of
    [h || e(parent)].

    ``forced_tok`` [B, N] (stage-wise checking): when given, conditioning
    tokens and cumulative scores follow these tokens instead of the oracle's
    own decisions, while ``tok`` still reports the oracle's own choice.
    """
    B = h.shape[0]
    N = plan.n
    row_node, row_depth, node_row = head_rows(plan, hydra)
    R = len(row_node)
    d = h.shape[1]
    V = (heads[0]["W2"] if isinstance(heads[0], dict) else heads[0][2]).shape[0]
    tok = -np.ones((B, N), dtype=np.int64)
    logp = np.zeros((B, N), dtype=np.float64)
    u_all = np.zeros((B, R, d))
    z_all = np.zeros((B, R, V))
    lse_all = np.zeros((B, R))
    margin = np.full((B, R), math.inf)
    kmax = {}
    for c in range(1, N):
        r = node_row[plan.parent[c]]
        kmax[r] = max(kmax.get(r, 0), int(plan.rank[c]) + 1)
    for b in range(B):
        tok[b, 0] = root_tok[b]
        follow = tok if forced_tok is None else np.asarray(forced_tok)
        for k in range(1, plan.dmax + 1):
            sketch = isinstance(heads[k - 1], dict)
            if sketch:
                W2 = heads[k - 1]["W2"]
            else:
                W1, b1, W2 = heads[k - 1]
            for r in np.flatnonzero(row_depth == k):
                if hydra:
                    p = row_node[r]
                    if attn is not None:
                        toks = path_tokens(plan, follow[b], root_tok[b], p)
                        e = path_attention(np.stack([np.asarray(E[t], dtype=np.float64) for t in toks]), attn, bf16)
                    elif full_path:
                        toks = path_tokens(plan, follow[b], root_tok[b], p)
                        e = np.concatenate([np.asarray(E[t], dtype=np.float64) for t in toks])
                    else:
                        ptok = int(root_tok[b]) if p == 0 else int(follow[b, p])
                        e = np.asarray(E[ptok], dtype=np.float64)
                else:
                    e = None
                if sketch:
                    u = sketch_hidden(h[b], e if k > 1 else None, heads[k - 1], bf16)
                else:
                    u = head_hidden(h[b], e, W1, b1, residual, bf16)
                z = head_logits(u, W2)
                lse = logsumexp(z)
                u_all[b, r], z_all[b, r], lse_all[b, r] = u, z, lse
                ids = topk_sorted(z, kmax[r])
                margin[b, r] = topk_margin(z, kmax[r])
                for c in range(1, N):
                    if plan.depth[c] == k and node_row[plan.parent[c]] == r:
                        tok[b, c] = ids[plan.rank[c]]
                        t = int(follow[b, c]) if forced_tok is not None else int(tok[b, c])
                        logp[b, c] = logp[b, plan.parent[c]] + z[t] - lse
    return dict(tok=tok, logp=logp, u=u_all, z=z_all, lse=lse_all,
                margin=margin, row_node=row_node, row_depth=row_depth,
                node_row=node_row)


# ---------------------------------------------------------------------------
# Stage 2: tree build
# ---------------------------------------------------------------------------

def prune_tree(plan: TreePlan, logp, n_keep):
    """Keep the root and the best n_keep - 1 candidates, renumbered breadth-first.

    Candidates are ranked by (cumulative log-prob descending, depth ascending,
    full-tree index ascending); since log-probs are <= 0 a child never beats
    its parent, so the kept set is closed under taking parents. The survivors
    are renumbered depth by depth, ordered by (new index of the parent, rank).
    Returns (kept_plan, src) where src[new] = index in the full tree.
    """
    N = plan.n
    cand = sorted(range(1, N), key=lambda i: (-float(logp[i]), int(plan.depth[i]), i))
    kept = {0} | set(cand[: n_keep - 1])
    new_index = {0: 0}
    src = [0]
    for k in range(1, plan.dmax + 1):
        level = [i for i in kept if plan.depth[i] == k]
        level.sort(key=lambda i: (new_index[int(plan.parent[i])], int(plan.rank[i])))
        for i in level:
            new_index[i] = len(src)
            src.append(i)
    src = np.array(src)
    parent = np.array([-1] + [new_index[int(plan.parent[i])] for i in src[1:]])
    return TreePlan(parent, plan.rank[src].copy(), plan.depth[src].copy()), src


def ancestors(parent, dmax):
    """anc[u][j] = the node at depth j on the path root -> u (u itself at its
    own depth), -1 beyond depth(u)."""
    parent = np.asarray(parent)
    N = parent.shape[0]
    anc = -np.ones((N, dmax + 1), dtype=np.int64)
    for u in range(N):
        chain = [u]
        while parent[chain[-1]] >= 0:
            chain.append(int(parent[chain[-1]]))
        chain.reverse()
        anc[u, : len(chain)] = chain
    return anc


def tree_mask(parent):
    """Dense topology mask over the tree nodes [HG, "Tree Attention Matrix with
    Topology-Aware Causal Masking"]: M(u, v) = 0 if v is an ancestor of u or
    u == v, and -inf otherwise. parent[i] = -1 marks a node that hangs off the
    prefix directly."""
    parent = np.asarray(parent)
    N = parent.shape[0]
    M = np.full((N, N), -np.inf)
    for u in range(N):
        v = u
        while v >= 0:
            M[u, v] = 0.0
            v = int(parent[v])
    return M


# ---------------------------------------------------------------------------
# Positions of the tree rows and their rotary embedding
# ---------------------------------------------------------------------------

def tree_positions(prefix_len, depth):
    """Position of every tree row: L_b + depth [SD, "Beyond draft models:
    Medusa": the candidates of one head stand at the same future position;
    HG, "Parallel Verification and Greedy Acceptance Algorithm": accepting a
    depth-k node advances to position t + k]. Siblings share a position; the
    root (depth 0) is at L_b, the first position not in the cache.
    prefix_len [B], depth [B, N]."""
    L = np.asarray(prefix_len, dtype=np.int64)
    return L[:, None] + np.asarray(depth, dtype=np.int64)


def rope(x, pos, theta=10000.0):
    """Rotary position embedding of the rows of x [..., D] at positions pos
    (broadcast over the leading axes), in the half-split layout of the
    LLaMA family: dimension i pairs with i + D/2 and rotates by the angle
    pos * theta^(-2i/D). This is how position ids enter the pages' models
    (Vicuna, LLaMA-2); the pages only fix the positions themselves."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# Stage 3: tree-masked attention verify (one attention layer's share)
# ---------------------------------------------------------------------------

def tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, anc, bf16=False):
    """Attention of every tree node over the prefix plus its own ancestors.

    [HG, "Tree Attention Matrix with Topology-Aware Causal Masking"]: the tree
    is flattened after the prefix and node u sees the prompt history and the
    nodes v with M(u, v) = 0. [MH, "Tree Attention und Akzeptanz"] says the
    same. Scores are q.k / sqrt(D); softmax over the visible keys.

    q [B, N, Hq, D], k_tree/v_tree [B, N, Hkv, D], k_prefix/v_prefix: per
    sequence arrays [L_b, Hkv, D], anc [B, N, Dmax+1]. Query head hq reads key
    head hq // (Hq // Hkv). Returns (O [B, N, Hq, D], lse [B, N, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, N, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, N, Hq))
    for b in range(B):
        kp = np.asarray(k_prefix[b], dtype=np.float64)
        vp = np.asarray(v_prefix[b], dtype=np.float64)
        kt = np.asarray(k_tree[b], dtype=np.float64)
        vt = np.asarray(v_tree[b], dtype=np.float64)
        for hk in range(Hkv):
            for u in range(N):
                vis = [int(a) for a in anc[b][u] if a >= 0]
                keys = np.concatenate([kp[:, hk, :], kt[vis, hk, :]], axis=0)
                vals = np.concatenate([vp[:, hk, :], vt[vis, hk, :]], axis=0)
                for hq in range(hk * G, (hk + 1) * G):
                    s = keys @ q[b, u, hq] * scale
                    m = np.max(s)
                    w = np.exp(s - m)
                    out[b, u, hq] = (w @ vals) / np.sum(w)
                    lse[b, u, hq] = m + np.log(np.sum(w))
    if bf16:
        out = round_bf16(out)
    return out, lse


# ---------------------------------------------------------------------------
# One decoder layer of the target over the tree rows (verification pass)
# ---------------------------------------------------------------------------

def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)


def decoder_layer(x, w, k_prefix, v_prefix, anc, depth, prefix_len, Hq, Hkv, D, eps, theta=10000.0,
                  bf16=False):
    """The target's decoder layer over every tree row, all rows in one pass
    [SD, "Draft, then verify": the target scores all candidates in one
    forward pass; HG, "Tree Attention Matrix with Topology-Aware Causal
    Masking": each row sees the prefix and its ancestors].

    Reading (the pages name the models, Vicuna / LLaMA, not their layer):
    the LLaMA pre-norm layer,
      a = rms(x) g1;  q, k, v = a Wq^T, a Wk^T, a Wv^T;  q, k rotated at L + depth;
      o = tree attention;  x1 = x + o Wo^T;
      b = rms(x1) g2;  x2 = x1 + (silu(b Wg^T) * (b Wu^T)) Wd^T.
    x [B, N, d]; w: dict of g1, Wq [Hq D, d], Wk/Wv [Hkv D, d], Wo [d, Hq D],
    g2, Wg/Wu [F, d], Wd [d, F]; k_prefix/v_prefix: per sequence [L_b, Hkv, D]
    (already rotated keys). With bf16, the tensors the device stores in
    bfloat16 (a, q, k, v, o, x1, b, the gated product, x2) are rounded there.
    Returns (x2, k_rot, v) with k_rot, v [B, N, Hkv, D] (the rows a commit
    copies into this layer's cache).
    """
    r = round_bf16 if bf16 else (lambda t: t)
    f = lambda t: np.asarray(t, dtype=np.float64)  # noqa: E731
    x = f(x)
    B, N, d = x.shape
    a = r(rms_norm(x, w["g1"], eps))
    q = r(a @ f(w["Wq"]).T).reshape(B, N, Hq, D)
    k = r(a @ f(w["Wk"]).T).reshape(B, N, Hkv, D)
    v = r(a @ f(w["Wv"]).T).reshape(B, N, Hkv, D)
    pos = tree_positions(prefix_len, depth)[..., None]
    q, k = r(rope(q, pos, theta)), r(rope(k, pos, theta))
    o, _ = tree_attention(q, k, v, k_prefix, v_prefix, anc, bf16=bf16)
    x1 = r(x + o.reshape(B, N, Hq * D) @ f(w["Wo"]).T)
    b = r(rms_norm(x1, w["g2"], eps))
    g = r(silu(b @ f(w["Wg"]).T) * (b @ f(w["Wu"]).T))
    x2 = r(x1 + g @ f(w["Wd"]).T)
    return x2, k, v


def verify_layers(tok, E, layers, g_f, k_prefix, v_prefix, anc, depth, prefix_len, Hq, Hkv, D, eps,
                  theta=10000.0, bf16=False):
    """The target's whole forward pass over the tree rows [SD, "Draft, then
    verify": one forward pass of the target scores every candidate; HG,
    "Tree Attention Matrix with Topology-Aware Causal Masking": the tree mask
    applies in every layer's attention].

    Each row's input is the embedding of its own token (a token outside the
    table reads zeros); the decoder layers follow in order, each with its own
    weights and its own cached prefix; the final RMSNorm (gain g_f) gives the
    hidden state h that the target's vocabulary projection reads.
    tok [B, N]; E [V, d]; layers: list of decoder_layer weight dicts;
    k_prefix/v_prefix: per layer, per sequence [L_b, Hkv, D].
    Returns (h [B, N, d], k_rot [n, B, N, Hkv, D], v [n, B, N, Hkv, D]).
    """
    r = round_bf16 if bf16 else (lambda t: t)
    E = np.asarray(E, dtype=np.float64)
    tok = np.asarray(tok, dtype=np.int64)
    ok = (tok >= 0) & (tok < E.shape[0])
    x = np.where(ok[..., None], E[np.where(ok, tok, 0)], 0.0)
    ks, vs = [], []
    for w, kp, vp in zip(layers, k_prefix, v_prefix):
        x, k, v = decoder_layer(x, w, kp, vp, anc, depth, prefix_len, Hq, Hkv, D, eps, theta, bf16=bf16)
        ks.append(k)
        vs.append(v)
    return r(rms_norm(x, g_f, eps)), np.stack(ks), np.stack(vs)


# ---------------------------------------------------------------------------
# Stage 4: target projection and acceptance
# ---------------------------------------------------------------------------

def target_logits(O, W_t):
    """Target logits of every tree row: Z = W_t O, with O flattened over
    (query head, head dim) into the hidden size."""
    O = np.asarray(O, dtype=np.float64)
    B, N = O.shape[:2]
    flat = O.reshape(B * N, -1)
    return (flat @ np.asarray(W_t, dtype=np.float64).T).reshape(B, N, -1)


def greedy_accept(Z, tok, parent, dmax):
    """Greedy longest-accepted-branch walk [HG, "Parallel Verification and
    Greedy Acceptance Algorithm"].

    From the root: take the target's arg max at the current node; if a child
    carries that token, accept it and move there; otherwise stop. The target
    token at the stopping node is emitted as the bonus, so m accepted drafts
    give m + 1 tokens. Z [N, V], tok [N], parent [N] for one sequence.
    Returns (m, path, out) with path starting at the root.
    """
    u, path, out = 0, [0], []
    while True:
        y = argmax_lowest(Z[u])
        nxt = [c for c in range(len(parent)) if parent[c] == u and tok[c] == y]
        out.append(y)
        if not nxt:
            break
        u = nxt[0]
        path.append(u)
    m = len(path) - 1
    assert m <= dmax
    return m, path, out


def residual(r, q):
    """Residual target after a rejection [SD, "The acceptance criterion" and
    "The correctness guarantee"]: norm(max(r - q, 0)). Returns None when the
    residual has no mass."""
    res = np.maximum(np.asarray(r, dtype=np.float64) - np.asarray(q, dtype=np.float64), 0.0)
    s = np.sum(res)
    return None if s <= 0.0 else res / s


def sample_inverse_cdf(r, u):
    """Inverse-CDF draw: the smallest id x with sum_{y<=x} r(y) > u * sum(r),
    scanning ids in ascending order."""
    r = np.asarray(r, dtype=np.float64)
    c = np.cumsum(r)
    thr = u * c[-1]
    for x in range(r.shape[0]):
        if c[x] > thr:
            return x
    return int(np.flatnonzero(r > 0)[-1])


def rejection_accept(Z, head_z, q_row, tok, parent, u_acc, u_res, T, follow=None, trace=None):
    """Stochastic acceptance on a tree (rule S1), for one sequence.

    Chain rule [SD, "The acceptance criterion"]: accept a drafted token x with
    probability min(1, p(x)/q(x)); on rejection resample from
    norm(max(p - q, 0)) and discard the rest. With a uniform draw u the test
    "u < p/q" is written without a division as u * q(x) < p(x). Both p and q
    are the post-temperature distributions [SD, "Common misconceptions"].

    On a tree the children of the current node are tried in rank order; after
    each rejection the target becomes the residual and q stays the same. At a
    node without children, or after every child is rejected, one token is
    drawn from the current target with that node's residual uniform. If a
    residual has no mass, the draw uses the target before that rejection.

    Z [N, V] target logits, head_z [R, V] head logits, q_row [N] the head row
    whose distribution drafted each node's children, u_acc [N] (used when the
    node is tested as a child), u_res [N] (used when a draw happens at it).
    Returns (m, path, out).

    Checking aid: with ``follow = (path, out)`` from another implementation,
    the walk takes that implementation's decisions instead of its own and, if
    ``trace`` is a list, appends one record per decision: ("accept", own,
    taken, margin) with margin = |u q(x) - r(x)| / r(x), or ("sample", own,
    taken, margin) with margin = distance of u * sum(r) to the cumulative
    boundary between the two tokens, over sum(r).
    """
    u, path, out = 0, [0], []
    fpath = None if follow is None else [int(x) for x in follow[0]]
    fout = None if follow is None else [int(x) for x in follow[1]]

    def draw(r, uu):
        own = sample_inverse_cdf(r, uu)
        if fout is None:
            return own
        taken = fout[len(out)]
        if trace is not None:
            c = np.cumsum(r)
            thr = uu * c[-1]
            lo, hi = min(own, taken), max(own, taken)
            edge = c[lo:hi]  # boundaries separating the two tokens
            margin = float(np.min(np.abs(edge - thr)) / c[-1]) if hi > lo else np.inf
            trace.append(("sample", own, taken, margin))
        return taken

    while True:
        p = softmax(np.asarray(Z[u], dtype=np.float64) / T)
        kids = [c for c in range(len(parent)) if parent[c] == u]
        if not kids:
            out.append(draw(p, u_res[u]))
            break
        q = softmax(np.asarray(head_z[q_row[u]], dtype=np.float64) / T)
        r = p
        moved = False
        for c in kids:
            x = int(tok[c])
            own = bool(u_acc[c] * q[x] < r[x])
            take = own
            if fpath is not None:
                take = len(path) < len(fpath) and fpath[len(path)] == c
                if trace is not None:
                    margin = abs(u_acc[c] * q[x] - r[x]) / max(r[x], 1e-300)
                    trace.append(("accept", own, take, margin))
            if take:
                out.append(x)
                path.append(c)
                u = c
                moved = True
                break
            nr = residual(r, q)
            if nr is not None:
                r = nr
        if not moved:
            out.append(draw(r, u_res[u]))
            break
    return len(path) - 1, path, out


# ---------------------------------------------------------------------------
# Typical acceptance (not distribution-exact)
# ---------------------------------------------------------------------------

def entropy(p):
    """Shannon entropy in nats, -sum p log p over the tokens with p > 0."""
    p = np.asarray(p, dtype=np.float64)
    nz = p[p > 0]
    return float(-np.sum(nz * np.log(nz)))


def typical_passes(Z, tok, parent, T, eps, delta):
    """Per-node test of typical acceptance [MH, "Tree Attention und
    Akzeptanz"]: a candidate is kept when its probability under the target
    exceeds a threshold tied to the entropy of the target's distribution.

    Reading (the pages give no formula): at the parent u, p = softmax(Z[u] / T)
    and the threshold is tau = min(eps, delta * exp(-H(p))), so a flat
    distribution (high entropy) lowers the bar and a peaked one raises it up
    to eps. Node c passes iff p(tok[c]) > tau. The root passes by definition.
    Returns (passes [N] bool, margin [N]) with margin = |p(x) - tau| / tau,
    the relative distance of each decision from its boundary (inf at the root).
    """
    N = len(parent)
    passes = np.zeros(N, dtype=bool)
    margin = np.full(N, np.inf)
    passes[0] = True
    cache = {}
    for c in range(1, N):
        u = int(parent[c])
        if u not in cache:
            p = softmax(np.asarray(Z[u], dtype=np.float64) / T)
            cache[u] = (p, min(eps, delta * math.exp(-entropy(p))))
        p, tau = cache[u]
        px = p[int(tok[c])]
        passes[c] = px > tau
        margin[c] = abs(px - tau) / tau if tau > 0 else np.inf
    return passes, margin


def kept_branch(passes, parent):
    """End node of the kept branch: among the nodes whose whole root path
    passes, the deepest [MH, "Tree Attention und Akzeptanz": the longest
    accepted branch is kept]; equally deep ones go to the smallest
    breadth-first index (the tree's rank order). Parents precede children."""
    N = len(parent)
    ok = np.zeros(N, dtype=bool)
    depth = np.zeros(N, dtype=np.int64)
    ok[0] = True
    end = 0
    for c in range(1, N):
        u = int(parent[c])
        depth[c] = depth[u] + 1
        ok[c] = ok[u] and bool(passes[c])
        if ok[c] and depth[c] > depth[end]:
            end = c
    return end


def typical_accept(Z, tok, parent, u_res, T, eps, delta):
    """Typical acceptance on a tree, for one sequence: the kept branch of
    ``kept_branch`` over ``typical_passes``, then one token drawn from the
    target's distribution at the branch's end by inverse CDF with that
    node's u_res (as the rejection mode's final draw). Returns (m, path, out)
    like the other walks: m accepted drafts, then the drawn token."""
    passes, _ = typical_passes(Z, tok, parent, T, eps, delta)
    end = kept_branch(passes, parent)
    path = [end]
    while parent[path[-1]] >= 0:
        path.append(int(parent[path[-1]]))
    path.reverse()
    out = [int(tok[c]) for c in path[1:]]
    out.append(sample_inverse_cdf(softmax(np.asarray(Z[end], dtype=np.float64) / T), u_res[end]))
    return len(path) - 1, path, out


# ---------------------------------------------------------------------------
# After acceptance: commit of the kept branch into the paged KV cache
# ---------------------------------------------------------------------------

def commit_path(k_pages, v_pages, block_table, prefix_len, k_tree, v_tree,
                n_acc, path, out_tok, dmax, hidden=None):
    """Commit the accepted branch of every sequence to its KV cache.

    [HG, "Production Engineering and Training Best Practices", items "Tree
    KV-Cache Page Sizing" and "KV-Cache Tree Branch Management"]: the tree's
    K/V live in statically reserved blocks, and rejected nodes are rolled back
    without freeing anything. [SD, "The acceptance criterion"]: the next round
    continues from the last accepted or resampled token and the rejected
    suffix is dropped from the caches. [MH, "Tree Attention und Akzeptanz"]:
    the longest accepted branch is kept and its last hidden state feeds the
    heads next round.

    Reading: the root (row 0, the last known token, not yet cached) and the
    m accepted drafts path[1..m] go to cache positions L, ..., L + m in path
    order; nothing else is written, so a rejected node never reaches the
    cache. The emitted bonus (or resampled) token out_tok[m] is not cached:
    it is the next round's root, and the hidden state of the last accepted
    row path[m] is the next round's h. The next prefix length is L + m + 1.

    k_pages, v_pages [n_layers, n_pages, Hkv, page_size, D]; block_table
    [B, max_pages]; k_tree, v_tree [n_layers, B, N, Hkv, D]; n_acc [B];
    path, out_tok [B, dmax + 1]; hidden [B, N, d] or None.
    A position whose page index is past max_pages or whose page id is not in
    [0, n_pages) is skipped; a sequence with m outside [0, dmax] or a path
    row outside [0, N) commits nothing and gets next root -1.
    Returns (k_pages, v_pages, next_len [B], next_root [B], next_h [B, d]
    or None); the pools are new arrays.
    """
    kp = np.array(k_pages, dtype=np.float64, copy=True)
    vp = np.array(v_pages, dtype=np.float64, copy=True)
    kt = np.asarray(k_tree, dtype=np.float64)
    vt = np.asarray(v_tree, dtype=np.float64)
    n_pages, ps = kp.shape[1], kp.shape[3]
    B, N = kt.shape[1], kt.shape[2]
    max_pages = np.asarray(block_table).shape[1]
    next_len = np.array([int(x) for x in prefix_len], dtype=np.int64)
    next_root = -np.ones(B, dtype=np.int64)
    next_h = None
    if hidden is not None:
        hid = np.asarray(hidden, dtype=np.float64)
        next_h = np.zeros((B, hid.shape[2]))
    for b in range(B):
        L, m = int(prefix_len[b]), int(n_acc[b])
        rows = [int(path[b][j]) for j in range(m + 1)] if 0 <= m <= dmax else []
        if not rows or any(r < 0 or r >= N for r in rows):
            continue
        for j, r in enumerate(rows):
            pos = L + j
            if pos // ps >= max_pages:
                continue
            page = int(block_table[b][pos // ps])
            if not 0 <= page < n_pages:
                continue
            kp[:, page, :, pos % ps, :] = kt[:, b, r]
            vp[:, page, :, pos % ps, :] = vt[:, b, r]
        next_len[b] = L + m + 1
        next_root[b] = int(out_tok[b][m])
        if hidden is not None:
            next_h[b] = hid[b, rows[-1]]
    return kp, vp, next_len, next_root, next_h
