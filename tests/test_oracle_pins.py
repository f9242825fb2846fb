"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (fixtures under tests/golden/), library routines (torch, numpy,
scipy), closed forms, or brute force on small inputs. Chosen so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one.
"""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
from oracle import hydra_oracle as H


# --------------------------------------------------------------------- scalars

def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000)).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with both parities of the kept lsb
    bits = rng.integers(0, 2**31, 20000, dtype=np.uint64).astype(np.uint32)
    bits = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    ties = bits.view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) > 1e-30) & (np.abs(ties) < 1e30)]
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = H.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_silu_matches_torch():
    a = np.linspace(-40, 40, 10001)
    ref = torch.nn.functional.silu(torch.from_numpy(a)).numpy()
    assert np.allclose(H.silu(a), ref, rtol=1e-14, atol=1e-300)


def test_topk_sorted_matches_stable_argsort_and_ties():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.integers(0, 20, 300).astype(np.float64)  # many ties
        k = int(rng.integers(1, 30))
        ref = np.argsort(-z, kind="stable")[:k]
        assert np.array_equal(H.topk_sorted(z, k), ref)
    z = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert list(H.topk_sorted(z, 4)) == [1, 2, 4, 3]
    assert H.argmax_lowest(z) == 1


def test_logsumexp_matches_scipy():
    rng = np.random.default_rng(2)
    z = rng.standard_normal(5000) * 30
    assert math.isclose(H.logsumexp(z), float(scipy.special.logsumexp(z)), rel_tol=1e-13)


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(3)
    for _ in range(200):
        r = rng.random(37) * (rng.random(37) < 0.6)
        if r.sum() == 0:
            continue
        u = rng.random()
        ref = int(np.searchsorted(np.cumsum(r), u * r.sum(), side="right"))
        assert H.sample_inverse_cdf(r, u) == ref


def _margin_brute_force(z, k):
    """Smallest |a - b| over all pairs of the k + 1 largest values of z (the
    k + 1 largest taken by repeatedly removing a maximum)."""
    rest = [float(x) for x in z]
    top = []
    for _ in range(min(k + 1, len(rest))):
        i = max(range(len(rest)), key=lambda j: rest[j])
        top.append(rest.pop(i))
    if len(top) < 2:
        return math.inf
    return min(abs(a - b) for i, a in enumerate(top) for b in top[i + 1:])


def test_topk_margin_matches_brute_force_over_pairs():
    rng = np.random.default_rng(4)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        z = np.round(rng.standard_normal(n) * 3, int(rng.integers(0, 4)))  # rounding makes ties
        k = int(rng.integers(1, n + 2))
        assert H.topk_margin(z, k) == _margin_brute_force(z, k)
    # the k / k + 1 boundary counts: the first k values are far apart, the
    # (k + 1)-th sits just below the k-th; a margin over the first k alone
    # would call this decision safe
    z = np.array([9.0, 5.0, 1.0, 1.0 - 3e-5, -4.0])
    assert H.topk_margin(z, 3) == pytest.approx(3e-5)
    first_k_only = float(np.min(-np.diff(np.sort(z)[::-1][:3])))
    assert first_k_only == 4.0 and H.topk_margin(z, 3) < 1e-4


def test_topk_margin_bounds_the_perturbation_that_changes_top_k():
    """Below half the margin no perturbation changes the sorted top-k ids;
    just above it, moving the two closest of the k + 1 largest values
    towards each other does."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(3, 30))
        z = rng.standard_normal(n)
        k = int(rng.integers(1, n))
        m = H.topk_margin(z, k)
        base = H.topk_sorted(z, k)
        for _ in range(5):
            dz = rng.uniform(-1, 1, n) * 0.49 * m
            assert np.array_equal(H.topk_sorted(z + dz, k), base)
        order = np.argsort(-z, kind="stable")[: k + 1]
        gaps = z[order[:-1]] - z[order[1:]]
        j = int(np.argmin(gaps))
        hi, lo = order[j], order[j + 1]
        dz = np.zeros(n)
        dz[hi] -= 0.51 * m
        dz[lo] += 0.51 * m
        assert not np.array_equal(H.topk_sorted(z + dz, k), base)


# ------------------------------------------------------------------- heads

def test_medusa_zero_init_reproduces_lm_head(golden):
    spec = dict(ln.split(None, 1) for ln in golden("medusa_zero_init.txt"))
    d, V, K = int(spec["hidden"]), int(spec["vocab"]), int(spec["heads"])
    expected = [s == "True" for s in spec["expected"].split()]
    rng = np.random.default_rng(4)
    lm_head = rng.standard_normal((V, d)) * 0.02
    h = rng.standard_normal(d)
    # The page applies one projection routine to u and to h; the check is exact
    # because the zero-initialised layer leaves u bit-identical to h.
    base = H.head_logits(h, lm_head)
    got = []
    for _ in range(K):
        u = H.head_hidden(h, None, np.zeros((d, d)), np.zeros(d))
        assert np.array_equal(u, h)
        got.append(bool(np.array_equal(H.head_logits(u, lm_head), base)))
    assert got == expected
    # and the projection is the base model's head (torch's routine, to rounding)
    ref = (torch.from_numpy(lm_head) @ torch.from_numpy(h)).numpy()
    assert np.allclose(base, ref, rtol=0, atol=1e-12)
    # Hydra head under the same initialisation (wider input) reduces the same way
    e = rng.standard_normal(d)
    u = H.head_hidden(h, e, np.zeros((d, 2 * d)), np.zeros(d))
    assert np.array_equal(u, h) and np.array_equal(H.head_logits(u, lm_head), base)
    # the residual connection is what makes it exact: without it, logits vanish
    u0 = H.head_hidden(h, None, np.zeros((d, d)), np.zeros(d), residual=False)
    assert not np.array_equal(H.head_logits(u0, lm_head), base)


def test_head_matches_torch_modules():
    rng = np.random.default_rng(5)
    d, V = 48, 97
    for hydra in (False, True):
        ind = 2 * d if hydra else d
        lin1 = torch.nn.Linear(ind, d).double()
        lin2 = torch.nn.Linear(d, V, bias=False).double()
        h = rng.standard_normal(d)
        e = rng.standard_normal(d) if hydra else None
        x = torch.from_numpy(np.concatenate([h, e]) if hydra else h)
        ref = lin2(torch.from_numpy(h) + torch.nn.functional.silu(lin1(x))).detach().numpy()
        u = H.head_hidden(h, e, lin1.weight.detach().numpy(), lin1.bias.detach().numpy())
        got = H.head_logits(u, lin2.weight.detach().numpy())
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_head_bf16_rounds_hidden_state():
    rng = np.random.default_rng(6)
    d = 32
    W1, b1 = rng.standard_normal((d, d)), rng.standard_normal(d)
    h = rng.standard_normal(d)
    u = H.head_hidden(h, None, W1, b1, bf16=True)
    ref = torch.from_numpy(h + H.silu(W1 @ h + b1)).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(u, ref)


def _sketch_modules(d, V, n_heads, hidden, seed):
    """Heads built as torch modules after the two-layer sketch: head 1 is
    Linear(d, d), SiLU, LayerNorm(d), Linear(d, V); later heads fuse
    [h || e(parent)] with Linear(2d, hidden), SiLU, Linear(hidden, d),
    LayerNorm(d) and project with Linear(d, V). Returns the modules and the
    same weights as the oracle's dicts."""
    torch.manual_seed(seed)
    mods, dicts = [], []
    for k in range(1, n_heads + 1):
        if k == 1:
            lin_a, ln = torch.nn.Linear(d, d), torch.nn.LayerNorm(d)
            body = torch.nn.Sequential(lin_a, torch.nn.SiLU(), ln)
            w = {}
        else:
            lin_a, lin_b, ln = torch.nn.Linear(2 * d, hidden), torch.nn.Linear(hidden, d), torch.nn.LayerNorm(d)
            body = torch.nn.Sequential(lin_a, torch.nn.SiLU(), lin_b, ln)
            w = {"Wb": lin_b.weight, "bb": lin_b.bias}
        with torch.no_grad():  # the default LayerNorm is the identity affine map
            ln.weight.uniform_(0.5, 1.5)
            ln.bias.uniform_(-0.5, 0.5)
        head = torch.nn.Linear(d, V, bias=False)
        body, head = body.double(), head.double()
        mods.append((body, head))
        w.update(Wa=lin_a.weight, ba=lin_a.bias, ln_g=ln.weight, ln_b=ln.bias, W2=head.weight)
        dicts.append({n: t.detach().double().numpy().copy() for n, t in w.items()})
    return mods, dicts


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(11)
    x, g, b = rng.standard_normal((3, 40)) * 4 + 2, rng.standard_normal(40), rng.standard_normal(40)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    assert np.allclose(H.layer_norm(x, g, b), ref.numpy(), rtol=1e-12, atol=1e-12)
    # a constant row has no spread: only the bias survives
    assert np.allclose(H.layer_norm(np.full(8, 3.0), np.ones(8), np.arange(8.0)), np.arange(8.0))


def test_sketch_heads_match_torch_modules():
    rng = np.random.default_rng(12)
    d, V, hidden = 24, 61, 40
    mods, dicts = _sketch_modules(d, V, 3, hidden, seed=3)
    h, e = rng.standard_normal(d), rng.standard_normal(d)
    for k, ((body, head), w) in enumerate(zip(mods, dicts), start=1):
        x = torch.from_numpy(h if k == 1 else np.concatenate([h, e]))
        ref = head(body(x)).detach().numpy()
        got = H.head_logits(H.sketch_hidden(h, None if k == 1 else e, w), w["W2"])
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_sketch_tree_matches_brute_force_expansion():
    # Expand every candidate as the sketch describes, head by head: softmax of
    # the head's logits, its top-k tokens, cumulative probability as the
    # product along the branch. The oracle's tree must hold the same branches
    # with the same probabilities (exp of its cumulative log-softmax).
    rng = np.random.default_rng(13)
    d, V, hidden, branching = 16, 50, 32, [3, 2, 2]
    mods, dicts = _sketch_modules(d, V, 3, hidden, seed=4)
    E = rng.standard_normal((V, d))
    h = rng.standard_normal((1, d))
    ht = torch.from_numpy(h[0])
    want = {}
    frontier = [((), 1.0)]
    for k, ((body, head), kk) in enumerate(zip(mods, branching), start=1):
        nxt = []
        for path, prob in frontier:
            x = ht if k == 1 else torch.cat([ht, torch.from_numpy(E[path[-1]])])
            p = torch.softmax(head(body(x)), dim=-1).detach().numpy()
            for t in np.argsort(-p, kind="stable")[:kk]:
                nxt.append((path + (int(t),), prob * p[t]))
        want.update(nxt)
        frontier = nxt
    plan = H.plan_cartesian(branching)
    res = H.draft_heads(h, [0], E, dicts, plan, hydra=True)
    got = {}
    for c in range(1, plan.n):
        path, u = [], c
        while u:
            path.append(int(res["tok"][0, u]))
            u = plan.parent[u]
        got[tuple(reversed(path))] = math.exp(res["logp"][0, c])
    assert got.keys() == want.keys()
    for key in want:
        assert got[key] == pytest.approx(want[key], rel=1e-10)


def test_sketch_bf16_rounds_both_stored_tensors():
    rng = np.random.default_rng(14)
    d, hidden = 16, 24
    w = {"Wa": rng.standard_normal((hidden, 2 * d)), "ba": rng.standard_normal(hidden),
         "Wb": rng.standard_normal((d, hidden)), "bb": rng.standard_normal(d),
         "ln_g": rng.standard_normal(d), "ln_b": rng.standard_normal(d)}
    h, e = rng.standard_normal(d), rng.standard_normal(d)
    bf = lambda t: torch.from_numpy(t).float().to(torch.bfloat16).double().numpy()  # noqa: E731
    a = bf(H.silu(w["Wa"] @ np.concatenate([h, e]) + w["ba"]))
    ref = bf(H.layer_norm(w["Wb"] @ a + w["bb"], w["ln_g"], w["ln_b"]))
    assert np.array_equal(H.sketch_hidden(h, e, w, bf16=True), ref)
    assert not np.array_equal(H.sketch_hidden(h, e, w, bf16=False), ref)


def test_full_path_reduces_to_parent_only_when_earlier_blocks_vanish():
    # with W1_k = [W_h, 0, ..., 0, W_e] the full-path head reads only h and
    # the parent's embedding: the parent-only head with [W_h, W_e]
    rng = np.random.default_rng(21)
    d, V = 8, 40
    plan = H.plan_cartesian([3, 2, 2])
    E, h = rng.standard_normal((V, d)), rng.standard_normal((2, d))
    parent_only, full = [], []
    for k in range(1, 4):
        Wh, We = rng.standard_normal((d, d)) * 0.5, rng.standard_normal((d, d)) * 0.5
        b1, W2 = rng.standard_normal(d) * 0.1, rng.standard_normal((V, d))
        parent_only.append((np.hstack([Wh, We]), b1, W2))
        full.append((np.hstack([Wh] + [np.zeros((d, d))] * (k - 1) + [We]), b1, W2))
    a = H.draft_heads(h, [3, 7], E, parent_only, plan)
    b = H.draft_heads(h, [3, 7], E, full, plan, full_path=True)
    assert np.array_equal(a["tok"], b["tok"])
    assert np.allclose(a["logp"], b["logp"], rtol=0, atol=1e-12)


def test_full_path_block_j_reads_the_depth_j_token():
    # only block j of head 3's input weights is nonzero: every depth-3 row's
    # hidden state is h + SiLU(W E[t_j] + b1) for the depth-j token of its
    # own path, found here by walking parent links by hand
    rng = np.random.default_rng(22)
    d, V = 6, 30
    plan = H.plan_cartesian([2, 2, 2])
    E, h = rng.standard_normal((V, d)), rng.standard_normal((1, d))
    base = [(rng.standard_normal((d, (k + 1) * d)), rng.standard_normal(d), rng.standard_normal((V, d)))
            for k in range(1, 4)]
    row_node, row_depth, _ = H.head_rows(plan, True)
    for j in range(3):
        W = rng.standard_normal((d, d))
        W1 = np.zeros((d, 4 * d))
        W1[:, (j + 1) * d:(j + 2) * d] = W
        heads = base[:2] + [(W1, base[2][1], base[2][2])]
        res = H.draft_heads(h, [5], E, heads, plan, full_path=True)
        for r in np.flatnonzero(row_depth == 3):
            node, chain = int(row_node[r]), []
            while node:
                chain.append(int(res["tok"][0, node]))
                node = int(plan.parent[node])
            chain.append(5)
            t_j = chain[::-1][j]
            want = h[0] + torch.nn.functional.silu(torch.from_numpy(W @ E[t_j] + base[2][1])).numpy()
            assert np.allclose(res["u"][0, r], want, rtol=1e-12, atol=1e-12)


def _attn_weights(rng, d, scale=0.3):
    return {n: rng.standard_normal((d, d)) * scale for n in ("Wq", "Wk", "Wv", "Wo")}


def test_path_attention_matches_torch_causal_attention():
    # the fusion is one causal self-attention layer over the path embeddings,
    # read at the last position, plus the residual: torch's SDPA with a
    # causal mask over the whole sequence gives the same last row
    rng = np.random.default_rng(31)
    d = 16
    for k in (1, 2, 5):
        X = rng.standard_normal((k, d))
        w = _attn_weights(rng, d)
        t = lambda a: torch.from_numpy(a)[None, None]  # noqa: E731
        out = torch.nn.functional.scaled_dot_product_attention(t(X @ w["Wq"].T), t(X @ w["Wk"].T),
                                                               t(X @ w["Wv"].T), is_causal=True)[0, 0]
        want = X[-1] + w["Wo"] @ out[-1].numpy()
        assert np.allclose(H.path_attention(X, w), want, rtol=1e-12, atol=1e-12)


def test_path_attention_special_cases():
    rng = np.random.default_rng(32)
    d = 8
    X = rng.standard_normal((4, d))
    w = _attn_weights(rng, d)
    # one position: the softmax is 1 and c = x + Wo Wv x
    assert np.allclose(H.path_attention(X[:1], w), X[0] + w["Wo"] @ w["Wv"] @ X[0], atol=1e-12)
    # zero query: uniform weights, c = x_last + Wo mean(V)
    wz = dict(w, Wq=np.zeros((d, d)))
    assert np.allclose(H.path_attention(X, wz), X[-1] + w["Wo"] @ (w["Wv"] @ X.mean(axis=0)), atol=1e-12)


def test_hydra_pp_with_zero_output_projection_is_parent_only():
    # Wo = 0 leaves c = e(parent): the Hydra++ heads become the parent-only heads
    rng = np.random.default_rng(33)
    d, V = 8, 40
    plan = H.plan_cartesian([3, 2, 2])
    E, h = rng.standard_normal((V, d)), rng.standard_normal((2, d))
    heads = [(rng.standard_normal((d, 2 * d)) * 0.5, rng.standard_normal(d) * 0.1, rng.standard_normal((V, d)))
             for _ in range(3)]
    w = dict(_attn_weights(rng, d), Wo=np.zeros((d, d)))
    a = H.draft_heads(h, [3, 7], E, heads, plan)
    b = H.draft_heads(h, [3, 7], E, heads, plan, attn=w)
    assert np.array_equal(a["tok"], b["tok"])
    assert np.allclose(a["logp"], b["logp"], rtol=0, atol=1e-12)
    c = H.draft_heads(h, [3, 7], E, heads, plan, attn=_attn_weights(rng, d))
    assert not np.allclose(a["u"], c["u"])


# -------------------------------------------------------------------- trees

def test_cartesian_counts(golden):
    for ln in golden("tree_counts.txt"):
        b, total, per = [s.strip() for s in ln.split("|")]
        b = [int(x) for x in b.split(",")]
        plan = H.plan_cartesian(b)
        assert plan.n - 1 == int(total)
        counts = [int(np.sum(plan.depth == k)) for k in range(1, len(b) + 1)]
        assert counts == [int(x) for x in per.split()]
    rng = np.random.default_rng(7)
    for _ in range(20):
        b = list(rng.integers(1, 5, rng.integers(1, 5)))
        closed = sum(math.prod(b[: k + 1]) for k in range(len(b)))
        assert H.plan_cartesian(b).n - 1 == closed


def test_cartesian_2x3_six_candidates_share_prefixes():
    plan = H.plan_cartesian([2, 3])
    leaves = [u for u in range(plan.n) if not plan.children(u)]
    assert len(leaves) == 6
    d1 = plan.children(0)
    assert len(d1) == 2
    for a in d1:
        assert [int(plan.rank[c]) for c in plan.children(a)] == [0, 1, 2]
    paths = {tuple(int(x) for x in H.ancestors(plan.parent, 2)[u]) for u in leaves}
    assert len(paths) == 6 and {p[1] for p in paths} == set(d1)


def _tiny_heads(rng, d, V, K, hydra):
    ind = 2 * d if hydra else d
    return [(rng.standard_normal((d, ind)) * 0.02, rng.standard_normal(d) * 0.02,
             rng.standard_normal((V, d)) * 0.02) for _ in range(K)]


def test_medusa_same_tokens_under_every_parent():
    rng = np.random.default_rng(8)
    d, V = 64, 200
    plan = H.plan_cartesian([2, 3])
    h = rng.standard_normal((1, d))
    E = rng.standard_normal((V, d))
    res = H.draft_heads(h, [5], E, _tiny_heads(rng, d, V, 3, False), plan, hydra=False)
    sets = [tuple(res["tok"][0, plan.children(a)]) for a in plan.children(0)]
    assert sets[0] == sets[1]
    # Hydra conditions head 2 on the parent token: lists differ under each parent
    heads = [(W1 * 25.0, b1, W2) for W1, b1, W2 in _tiny_heads(rng, d, V, 3, True)]
    res = H.draft_heads(h, [5], E, heads, plan, hydra=True)
    sets = [tuple(res["tok"][0, plan.children(a)]) for a in plan.children(0)]
    assert sets[0] != sets[1]
    # depth-1 node tokens are head 1's top-2 and depth-2 its rows' top-3
    for a in plan.children(0):
        z = res["z"][0, res["node_row"][a]]
        assert list(res["tok"][0, plan.children(a)]) == list(np.argsort(-z, kind="stable")[:3])


def test_cumulative_logp_is_sum_of_log_softmax():
    rng = np.random.default_rng(9)
    d, V = 32, 50
    plan = H.plan_cartesian([3, 2, 2])
    h = rng.standard_normal((1, d))
    E = rng.standard_normal((V, d))
    res = H.draft_heads(h, [7], E, _tiny_heads(rng, d, V, 3, True), plan)
    for c in range(1, plan.n):
        chain = [int(a) for a in H.ancestors(plan.parent, 3)[c] if a >= 0]
        tot = 0.0
        for a, b in zip(chain[:-1], chain[1:]):
            z = torch.from_numpy(res["z"][0, res["node_row"][a]])
            tot += float(torch.log_softmax(z, 0)[res["tok"][0, b]])
        assert math.isclose(res["logp"][0, c], tot, rel_tol=1e-12, abs_tol=1e-12)


def test_sparse_template_invariants():
    plan = H.plan_sparse_template((10, 4, 2, 1), 64)
    assert plan.n == 64
    assert all(plan.parent[i] < i for i in range(1, 64))
    assert [int(np.sum(plan.depth == k)) for k in range(1, 5)] == [10, 27, 20, 6]
    fan = {}
    for u in range(64):
        kids = plan.children(u)
        if kids:
            assert kids == list(range(kids[0], kids[0] + len(kids)))
            assert [int(plan.rank[c]) for c in kids] == list(range(len(kids)))
            k = int(plan.depth[u]) + 1
            fan[k] = max(fan.get(k, 0), len(kids))
    assert fan == {1: 10, 2: 4, 3: 2, 4: 1}
    _, row_depth, _ = H.head_rows(plan, True)
    assert [int(np.sum(row_depth == k)) for k in range(1, 5)] == [1, 10, 13, 6]
    _, row_depth, _ = H.head_rows(plan, False)
    assert list(row_depth) == [1, 2, 3, 4]


def _brute_prune(plan, logp, n_keep):
    recs = np.array([(-logp[i], plan.depth[i], i) for i in range(1, plan.n)],
                    dtype=[("a", "f8"), ("b", "i8"), ("c", "i8")])
    order = np.argsort(recs, order=("a", "b", "c"))
    return {0} | {int(recs[j]["c"]) for j in order[: n_keep - 1]}


def test_prune_matches_brute_force():
    rng = np.random.default_rng(10)
    plan = H.plan_cartesian([4, 4, 4, 4])
    assert plan.n == 341
    for trial in range(20):
        step = np.log(rng.dirichlet(np.ones(4), size=plan.n))
        if trial % 4 == 0:
            step = np.round(step, 1)  # force ties
        logp = np.zeros(plan.n)
        for c in range(1, plan.n):
            logp[c] = logp[plan.parent[c]] + step[plan.parent[c], plan.rank[c]]
        kept, src = H.prune_tree(plan, logp, 256)
        assert set(int(s) for s in src) == _brute_prune(plan, logp, 256)
        assert kept.n == 256
        # breadth-first: parents first, depth non-decreasing, siblings by rank
        assert all(kept.parent[i] < i for i in range(1, 256))
        assert all(np.diff(kept.depth) >= 0)
        for i in range(1, 256):
            assert src[kept.parent[i]] == plan.parent[src[i]]
        for i in range(2, 256):
            if kept.parent[i] == kept.parent[i - 1]:
                assert kept.rank[i] > kept.rank[i - 1]
            elif kept.depth[i] == kept.depth[i - 1]:
                assert kept.parent[i] > kept.parent[i - 1]


def test_ancestors_follow_parent_chain():
    plan = H.plan_sparse_template((10, 4, 2, 1), 64)
    anc = H.ancestors(plan.parent, 4)
    for u in range(64):
        d = int(plan.depth[u])
        assert anc[u, d] == u and anc[u, 0] == 0
        assert all(anc[u, d + 1:] == -1)
        for j in range(1, d + 1):
            assert plan.parent[anc[u, j]] == anc[u, j - 1]


def test_tree_mask_matches_printed_table(golden):
    names, parents, rows = [], [], []
    for ln in golden("tree_mask_2x2.txt"):
        left, right = ln.split("|")
        nm, par = left.split()
        names.append(nm)
        parents.append(par)
        rows.append([0.0 if t == "0" else -np.inf for t in right.split()])
    parent = [-1 if p == "-" else names.index(p) for p in parents]
    M = H.tree_mask(parent)
    printed = np.array(rows)
    assert np.all(printed[:, 0] == 0.0)  # every node sees the prompt history
    assert np.array_equal(M, printed[:, 1:])


# ---------------------------------------------------------------- attention

def _causal_sdpa(q, k, v):
    """torch's attention with a causal mask; q [S, H, D], k/v [S, Hkv, D]."""
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True)
    return o.transpose(0, 1)


@pytest.mark.parametrize("L,tree", [(11, [2, 3]), (0, [2, 2, 2]), (5, [1, 1, 1, 1]), (7, [])])
def test_tree_attention_equals_causal_attention_per_branch(L, tree):
    rng = np.random.default_rng(11 + L)
    plan = H.plan_cartesian(tree) if tree else H.TreePlan(np.array([-1]), np.array([-1]), np.array([0]))
    N, Hq, Hkv, D, B = plan.n, 4, 2, 16, 2
    dmax = max(plan.dmax, 1)
    q = rng.standard_normal((B, N, Hq, D))
    kt, vt = rng.standard_normal((B, N, Hkv, D)), rng.standard_normal((B, N, Hkv, D))
    kp = [rng.standard_normal((L, Hkv, D)) for _ in range(B)]
    vp = [rng.standard_normal((L, Hkv, D)) for _ in range(B)]
    anc = np.stack([H.ancestors(plan.parent, dmax)] * B)
    out, lse = H.tree_attention(q, kt, vt, kp, vp, anc)
    for b in range(B):
        for leaf in [u for u in range(N) if not plan.children(u)]:
            branch = [int(a) for a in anc[b, leaf] if a >= 0]
            qs = torch.from_numpy(np.concatenate([np.zeros((L, Hq, D)), q[b, branch]]))
            ks = torch.from_numpy(np.concatenate([kp[b], kt[b, branch]]))
            vs = torch.from_numpy(np.concatenate([vp[b], vt[b, branch]]))
            ref = _causal_sdpa(qs, ks, vs).numpy()[L:]
            assert np.allclose(out[b, branch], ref, rtol=1e-10, atol=1e-12)
    if N == 1:  # single-query decode: softmax over the prefix plus the row itself
        s = np.concatenate([kp[0][:, 0], kt[0, [0], 0]]) @ q[0, 0, 0] / 4.0
        assert math.isclose(lse[0, 0, 0], float(scipy.special.logsumexp(s)), rel_tol=1e-12)


# --------------------------------------------------------------- acceptance

def test_target_logits_sum_over_query_heads():
    """Z[b, u] = sum over query heads hq of W_t[:, hq D:(hq + 1) D] O[b, u, hq]
    (the attention output is laid out head-major in the hidden vector), by
    explicit loops and by torch's F.linear on the flattened rows. A D-major
    flatten, or W_t used untransposed (a square W_t lets that run), fails."""
    rng = np.random.default_rng(21)
    for (B, N, Hq, D, V) in [(2, 5, 3, 4, 11), (1, 3, 2, 6, 12)]:  # the second has V = Hq D
        O_ = rng.standard_normal((B, N, Hq, D))
        Wt = rng.standard_normal((V, Hq * D))
        Z = H.target_logits(O_, Wt)
        ref = np.zeros((B, N, V))
        for b in range(B):
            for u in range(N):
                for hq in range(Hq):
                    for v in range(V):
                        ref[b, u, v] += sum(Wt[v, hq * D + j] * O_[b, u, hq, j] for j in range(D))
        assert Z.shape == (B, N, V)
        assert np.allclose(Z, ref, rtol=1e-12, atol=1e-12)
        lin = torch.nn.functional.linear(torch.from_numpy(O_.reshape(B, N, Hq * D)), torch.from_numpy(Wt)).numpy()
        assert np.allclose(Z, lin, rtol=1e-12, atol=1e-12)
        d_major = O_.transpose(0, 1, 3, 2).reshape(B, N, -1) @ Wt.T
        assert not np.allclose(d_major, ref, atol=1e-6)
        if V == Hq * D:
            untransposed = O_.reshape(B, N, -1) @ Wt
            assert not np.allclose(untransposed, ref, atol=1e-6)


def _planted_Z(rng, plan, tok, path, stop_tok, V):
    Z = rng.standard_normal((plan.n, V))
    for a, b in zip(path[:-1], path[1:]):
        Z[a, tok[b]] = 50.0
    Z[path[-1], stop_tok] = 50.0
    return Z


def test_greedy_planted_paths():
    rng = np.random.default_rng(12)
    V = 40
    plan = H.plan_sparse_template((4, 3, 2, 1), 30)
    anc = H.ancestors(plan.parent, plan.dmax)
    for trial in range(200):
        tok = np.zeros(plan.n, dtype=np.int64)
        for u in range(plan.n):
            kids = plan.children(u)
            tok[kids] = rng.choice(V, len(kids), replace=False)
        target = int(rng.integers(0, plan.n))
        path = [int(a) for a in anc[target] if a >= 0]
        kid_toks = {int(tok[c]) for c in plan.children(target)}
        stop = int(rng.choice([t for t in range(V) if t not in kid_toks]))
        Z = _planted_Z(rng, plan, tok, path, stop, V)
        m, got_path, out = H.greedy_accept(Z, tok, plan.parent, plan.dmax)
        assert m == len(path) - 1 and got_path == path
        assert out == [int(tok[c]) for c in path[1:]] + [stop]


def test_greedy_chain_is_longest_matching_prefix():
    rng = np.random.default_rng(13)
    V, k = 6, 5
    plan = H.plan_cartesian([1] * k)
    for _ in range(300):
        tok = rng.integers(0, V, k + 1)
        Z = rng.standard_normal((k + 1, V))
        m, _, out = H.greedy_accept(Z, tok, plan.parent, k)
        top = Z.argmax(axis=1)
        expect = 0
        while expect < k and tok[expect + 1] == top[expect]:
            expect += 1
        assert m == expect and out[-1] == top[expect] and len(out) == m + 1


def _chain_case(p_rows, q_rows, toks):
    """Chain tree: node i+1 carries toks[i]; Z[i] = log p_rows[i]; head row i =
    log q_rows[i]."""
    k = len(toks)
    parent = np.arange(-1, k)
    tok = np.array([0] + list(toks))
    with np.errstate(divide="ignore"):
        Z = np.log(np.asarray(p_rows, dtype=np.float64))
        hz = np.log(np.asarray(q_rows, dtype=np.float64))
    q_row = np.array(list(range(k)) + [-1])
    return parent, tok, Z, hz, q_row


def test_rejection_worked_example(golden):
    rows = [ln.split() for ln in golden("rejection_worked_example.txt")]
    total = int(rows[-1][1])
    drafted = rows[:-1]
    V = 10
    words = [r[0] for r in drafted]
    ids = {w: i for i, w in enumerate(words)}  # The=0 cat=1 sat=2 on=3 the=4
    ids["down"] = 7
    p_rows, q_rows = [], []
    for i, r in enumerate(drafted):
        p, q = np.full(V, 0.0), np.full(V, 0.0)
        if r[1] != "-":
            p[ids[r[0]]], q[ids[r[0]]] = float(r[1]), float(r[2])
        if r[0] == "on":  # the residual puts its mass where p exceeds q
            p[ids["down"]] += 0.5
            q[ids["down"]] += 0.05
        p += (1.0 - p.sum()) / V
        q += (1.0 - q.sum()) / V
        p_rows.append(p)
        q_rows.append(q)
    p_rows.append(np.full(V, 1.0 / V))  # after the last drafted token
    toks = [ids[w] for w in words]
    parent, tok, Z, hz, q_row = _chain_case(p_rows, q_rows, toks)
    n = len(tok)
    # the coin for "on" comes up reject: any u above p/q = 1/3 of that token
    pq = p_rows[3][ids["on"]] / q_rows[3][ids["on"]]
    u_acc = np.full(n, 0.99)
    u_acc[4] = 0.5
    assert u_acc[4] >= pq
    res = H.residual(p_rows[3], q_rows[3])
    u_res = np.zeros(n)
    u_res[3] = (np.cumsum(res)[ids["down"] - 1] + 0.5 * res[ids["down"]]) / res.sum()
    m, path, out = H.rejection_accept(Z, hz, q_row, tok, parent, u_acc, u_res, 1.0)
    verdict = [r[3] for r in drafted]
    assert m == verdict.count("accept") == 3
    assert len(out) == total
    assert out[:3] == toks[:3] and out[3] == ids["down"]
    assert p_rows[3][out[3]] > q_rows[3][out[3]]  # drawn from the residual support
    # a coin below p/q accepts "on" instead
    u_acc[4] = 0.3
    m2, _, out2 = H.rejection_accept(Z, hz, q_row, tok, parent, u_acc, u_res, 1.0)
    assert m2 >= 4 and out2[3] == ids["on"]


def _first_token_histogram(p, q, trials, rng):
    parent, tok, Z, hz, q_row = _chain_case([p, p], [q], [0])
    counts = np.zeros(len(p))
    cq = np.cumsum(q)
    for _ in range(trials):
        x = int(np.searchsorted(cq, rng.random() * cq[-1], side="right"))
        tok[1] = x
        u = rng.random(2)
        _, _, out = H.rejection_accept(Z, hz, q_row, tok, parent, u, rng.random(2), 1.0)
        counts[out[0]] += 1
    return counts


def test_rejection_identity_chi_square(monkeypatch):
    rng = np.random.default_rng(14)
    V = 8
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V) * 0.3)
    alpha = np.minimum(p, q).sum()
    assert 0.2 < alpha < 0.9
    trials = 20000
    counts = _first_token_histogram(p, q, trials, rng)
    assert scipy.stats.chisquare(counts, p * trials).pvalue > 1e-3
    # planted mistake: resample from the target itself instead of the residual
    monkeypatch.setattr(H, "residual", lambda r, qq: np.asarray(r, dtype=np.float64))
    naive = _first_token_histogram(p, q, trials, rng)
    assert scipy.stats.chisquare(naive, p * trials).pvalue < 1e-6
    mix = np.minimum(p, q) + (1 - alpha) * p  # the pages' closed form for this mistake
    assert scipy.stats.chisquare(naive, mix * trials).pvalue > 1e-3


def test_rejection_follow_own_decisions_is_identity():
    """The checking aid: following the walk's own decisions changes nothing
    and records no disagreement."""
    rng = np.random.default_rng(17)
    V = 12
    plan = H.plan_cartesian([3, 2, 2])
    _, _, node_row = H.head_rows(plan, True)
    for _ in range(100):
        tok = rng.integers(0, V, plan.n)
        Z = rng.standard_normal((plan.n, V)) * 2
        hz = rng.standard_normal((int(node_row.max()) + 1, V)) * 2
        ua, ur = rng.random(plan.n), rng.random(plan.n)
        m, path, out = H.rejection_accept(Z, hz, node_row, tok, plan.parent, ua, ur, 0.7)
        trace = []
        m2, path2, out2 = H.rejection_accept(Z, hz, node_row, tok, plan.parent, ua, ur, 0.7,
                                             follow=(path, out), trace=trace)
        assert (m, path, out) == (m2, path2, out2)
        assert trace and all(own == taken for _, own, taken, _ in trace)


def test_rejection_equal_distributions_never_resample():
    rng = np.random.default_rng(15)
    V = 6
    for _ in range(200):
        p = rng.dirichlet(np.ones(V))
        parent, tok, Z, hz, q_row = _chain_case([p, p], [p], [int(rng.integers(V))])
        m, _, _ = H.rejection_accept(Z, hz, q_row, tok, parent, rng.random(2), rng.random(2), 1.0)
        assert m == 1  # alpha = 1: p >= q everywhere, the draft is always accepted
        q = rng.dirichlet(np.ones(V))
        x = int(np.argmax(p - q))  # a token with p >= q
        parent, tok, Z, hz, q_row = _chain_case([p, p], [q], [x])
        m, _, _ = H.rejection_accept(Z, hz, q_row, tok, parent, rng.random(2), rng.random(2), 1.0)
        assert m == 1


def test_expected_yield_monte_carlo(golden):
    rng = np.random.default_rng(16)
    trials = 6000
    for ln in golden("yield_examples.txt"):
        alpha, k, printed = float(ln.split()[0]), int(ln.split()[1]), float(ln.split()[2])
        # closed form (1 - alpha^(k+1)) / (1 - alpha), reading of the garbled formula
        assert round((1 - alpha ** (k + 1)) / (1 - alpha), 1) == printed
        V = 4
        q = np.array([1.0, 1e-300, 1e-300, 1e-300])
        p = np.array([alpha] + [(1 - alpha) / 3] * 3)
        parent, tok, Z, hz, q_row = _chain_case([p] * (k + 1), [q] * k, [0] * k)
        n_out = []
        for _ in range(trials):
            _, _, out = H.rejection_accept(Z, hz, q_row, tok, parent, rng.random(k + 1),
                                           rng.random(k + 1), 1.0)
            n_out.append(len(out))
        mean, se = np.mean(n_out), np.std(n_out) / math.sqrt(trials)
        assert abs(mean - printed) < 0.05 + 4 * se, (alpha, k, mean)


def test_oracle_package_exports():
    for name in H.__all__:
        assert hasattr(oracle, name)


# -------------------------------------------------------------------- commit

def _paged_pool(rng, lens, reserve, n_layers, Hkv, D, ps):
    """Prefix K/V [n_layers][b] -> a scattered page pool with room for
    `reserve` more positions per sequence (test-side placement)."""
    per = [-(-(L + reserve) // ps) for L in lens]
    n_pages = sum(per) + 2  # two spare pages nobody maps
    order = rng.permutation(n_pages)
    bt = -np.ones((len(lens), max(per)), dtype=np.int64)
    kpool = rng.standard_normal((n_layers, n_pages, Hkv, ps, D))  # garbage outside the prefixes
    vpool = rng.standard_normal((n_layers, n_pages, Hkv, ps, D))
    kpre = [rng.standard_normal((n_layers, L, Hkv, D)) for L in lens]
    vpre = [rng.standard_normal((n_layers, L, Hkv, D)) for L in lens]
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(per[b]):
            bt[b, j] = order[nxt]
            nxt += 1
        for pos in range(L):
            kpool[:, bt[b, pos // ps], :, pos % ps] = kpre[b][:, pos]
            vpool[:, bt[b, pos // ps], :, pos % ps] = vpre[b][:, pos]
    return kpool, vpool, bt, kpre, vpre


def _gather(pool, bt, b, n, ps):
    """Positions 0..n-1 of sequence b read back through its block table."""
    return np.stack([pool[:, bt[b, p // ps], :, p % ps] for p in range(n)], axis=1)


@pytest.mark.parametrize("tree,ps", [([2, 3], 4), ([1, 1, 1, 1], 4), ([3, 2, 2], 16)])
def test_commit_turns_the_kept_branch_into_causal_attention(tree, ps):
    """After the commit, attention of the kept rows over the cache with a
    plain causal mask equals the tree-masked attention they had in the verify
    pass (the tree mask hides exactly the nodes off the branch)."""
    rng = np.random.default_rng(40 + ps + len(tree))
    plan = H.plan_cartesian(tree)
    N, Hq, Hkv, D, nl, dmax = plan.n, 4, 2, 8, 2, plan.dmax
    lens = [5, 7, 16]
    B = len(lens)
    kpool, vpool, bt, kpre, vpre = _paged_pool(rng, lens, dmax + 1, nl, Hkv, D, ps)
    q = rng.standard_normal((B, N, Hq, D))
    kt, vt = rng.standard_normal((nl, B, N, Hkv, D)), rng.standard_normal((nl, B, N, Hkv, D))
    anc = np.stack([H.ancestors(plan.parent, dmax)] * B)
    hidden = rng.standard_normal((B, N, 6))
    # kept branch of each sequence: root -> a random node (the root alone for b = 0)
    ends = [0] + [int(rng.integers(1, N)) for _ in range(B - 1)]
    path = -np.ones((B, dmax + 1), dtype=np.int64)
    out_tok = -np.ones((B, dmax + 1), dtype=np.int64)
    n_acc = np.zeros(B, dtype=np.int64)
    for b, e in enumerate(ends):
        br = [int(a) for a in anc[b, e] if a >= 0]
        n_acc[b] = len(br) - 1
        path[b, : len(br)] = br
        out_tok[b, : len(br)] = rng.integers(0, 100, len(br))
    kp2, vp2, nlen, nroot, nh = H.commit_path(kpool, vpool, bt, lens, kt, vt, n_acc, path, out_tok, dmax, hidden)
    for b in range(B):
        m, L = int(n_acc[b]), lens[b]
        assert nlen[b] == L + m + 1 and nroot[b] == out_tok[b, m]
        assert np.array_equal(nh[b], hidden[b, path[b, m]])
        br = [int(x) for x in path[b, : m + 1]]
        for layer in range(nl):
            o, _ = H.tree_attention(q[b:b + 1], kt[layer, b:b + 1], vt[layer, b:b + 1], [kpre[b][layer]],
                                    [vpre[b][layer]], anc[b:b + 1])
            ks = _gather(kp2, bt, b, L + m + 1, ps)[layer]
            vs = _gather(vp2, bt, b, L + m + 1, ps)[layer]
            qs = np.concatenate([np.zeros((L, Hq, D)), q[b, br]])
            ref = _causal_sdpa(torch.from_numpy(qs), torch.from_numpy(ks), torch.from_numpy(vs)).numpy()[L:]
            assert np.allclose(o[0, br], ref, rtol=1e-10, atol=1e-12)


def test_commit_writes_only_the_kept_positions():
    rng = np.random.default_rng(47)
    plan = H.plan_cartesian([2, 2])
    N, Hkv, D, nl, dmax, ps = plan.n, 2, 4, 1, plan.dmax, 4
    lens = [3, 8, 6, 2]
    B = len(lens)
    kpool, vpool, bt, _, _ = _paged_pool(rng, lens, dmax + 1, nl, Hkv, D, ps)
    kt, vt = rng.standard_normal((nl, B, N, Hkv, D)), rng.standard_normal((nl, B, N, Hkv, D))
    path = np.array([[0, 2, 6], [0, 1, -1], [0, 1, 3], [0, 2, 5]])
    out_tok = np.array([[7, 8, 9], [4, 5, -1], [1, 2, 3], [6, 6, 6]])
    n_acc = np.array([2, 1, 5, 2])   # sequence 2: count past dmax
    bt = bt.copy()
    bt[3, (lens[3] + 2) // ps] = -1  # sequence 3: the page of its position L + 2 is unmapped
    kp2, vp2, nlen, nroot, _ = H.commit_path(kpool, vpool, bt, lens, kt, vt, n_acc, path, out_tok, dmax)
    expect_k, expect_v = kpool.copy(), vpool.copy()
    for b in (0, 1, 3):
        for j in range(int(n_acc[b]) + 1):
            pos = lens[b] + j
            if bt[b, pos // ps] < 0:
                continue
            expect_k[:, bt[b, pos // ps], :, pos % ps] = kt[:, b, path[b, j]]
            expect_v[:, bt[b, pos // ps], :, pos % ps] = vt[:, b, path[b, j]]
    assert np.array_equal(kp2, expect_k) and np.array_equal(vp2, expect_v)
    assert not np.array_equal(kp2, kpool)
    assert list(nlen) == [lens[0] + 3, lens[1] + 2, lens[2], lens[3] + 3]
    assert list(nroot) == [9, 5, -1, 6]
    # pages no block table maps are untouched
    spare = sorted(set(range(kpool.shape[1])) - set(int(x) for x in bt.ravel()))
    assert len(spare) >= 2 and np.array_equal(kp2[:, spare], kpool[:, spare])


# -------------------------------------------------------- typical acceptance

def test_entropy_matches_scipy_and_closed_forms():
    rng = np.random.default_rng(50)
    for _ in range(20):
        p = rng.dirichlet(np.ones(int(rng.integers(2, 500))) * rng.uniform(0.05, 3))
        assert math.isclose(H.entropy(p), float(scipy.stats.entropy(p)), rel_tol=1e-12)
    assert math.isclose(H.entropy(np.full(1000, 1e-3)), math.log(1000), rel_tol=1e-12)
    assert H.entropy(np.eye(7)[3]) == 0.0


def test_typical_uniform_target_bar_scales_with_delta_over_V():
    """A flat target (entropy log V exactly) puts the bar at min(eps, delta / V):
    every candidate (probability 1 / V) passes iff delta < 1 (eps above 1 / V)."""
    plan = H.plan_cartesian([2, 2])
    V = 50
    Z = np.zeros((plan.n, V))
    tok = np.array([0] + list(range(1, plan.n)))
    for delta, want in ((0.5, True), (0.99, True), (1.01, False), (2.0, False)):
        passes, _ = H.typical_passes(Z, tok, plan.parent, 1.0, 0.3, delta)
        assert all(passes[1:] == want), delta
    passes, _ = H.typical_passes(Z, tok, plan.parent, 1.0, 0.5 / V, 0.5)  # eps below 1 / V binds
    assert all(passes[1:])


def test_typical_limits_nothing_everything_and_greedy():
    rng = np.random.default_rng(51)
    V = 60
    for tree in ([2, 3], [3, 2, 2], [1, 1, 1]):
        plan = H.plan_cartesian(tree)
        depth = plan.depth
        for _ in range(10):
            Z = rng.standard_normal((plan.n, V)) * 3
            tok = np.zeros(plan.n, dtype=np.int64)
            for u in range(plan.n):
                kids = plan.children(u)
                tok[kids] = rng.choice(V, len(kids), replace=False)
            u_res = rng.random(plan.n)
            # a bar of 1 passes nothing: the root's own draw
            m, path, out = H.typical_accept(Z, tok, plan.parent, u_res, 0.8, 1.0, 1e9)
            assert (m, path) == (0, [0])
            assert out == [H.sample_inverse_cdf(H.softmax(Z[0] / 0.8), u_res[0])]
            # a bar of 0 passes everything: the first deepest node
            m, path, _ = H.typical_accept(Z, tok, plan.parent, u_res, 0.8, 0.0, 0.5)
            end = int(np.flatnonzero(depth == depth.max())[0])
            assert m == depth.max() and path[-1] == end
            # temperature -> 0: the target becomes its arg max, which is greedy
            # acceptance, and the draw at the end is the arg max
            got = H.typical_accept(Z, tok, plan.parent, u_res, 1e-4, 0.3, 0.09)
            assert got == H.greedy_accept(Z, tok, plan.parent, plan.dmax)
            # scaling logits and temperature together changes nothing
            assert H.typical_accept(Z * 3, tok, plan.parent, u_res, 2.4, 0.3, 0.3) == \
                H.typical_accept(Z, tok, plan.parent, u_res, 0.8, 0.3, 0.3)


def test_typical_bar_is_monotone_in_eps_and_delta():
    rng = np.random.default_rng(52)
    plan = H.plan_cartesian([3, 3])
    V = 40
    for _ in range(20):
        Z = rng.standard_normal((plan.n, V)) * 2
        tok = rng.integers(0, V, plan.n)
        a, _ = H.typical_passes(Z, tok, plan.parent, 1.0, 0.2, 0.3)
        b, _ = H.typical_passes(Z, tok, plan.parent, 1.0, 0.1, 0.3)
        c, _ = H.typical_passes(Z, tok, plan.parent, 1.0, 0.2, 0.1)
        assert np.all(b >= a) and np.all(c >= a)  # a lower bar keeps a superset


def test_kept_branch_is_the_longest_fully_passing_path_by_brute_force():
    rng = np.random.default_rng(53)
    for tree in ([2, 3], [3, 2, 2], [2, 2, 2, 2]):
        plan = H.plan_cartesian(tree)
        anc = H.ancestors(plan.parent, plan.dmax)
        for _ in range(30):
            passes = rng.random(plan.n) < 0.6
            passes[0] = True
            best = (0, 0)
            for u in range(plan.n):
                chain = [int(a) for a in anc[u] if a >= 0]
                if all(passes[c] for c in chain):
                    best = max(best, (len(chain) - 1, -u))
            assert H.kept_branch(passes, plan.parent) == -best[1]


# ------------------------------------------------------- positions and RoPE

def test_rope_is_a_rotation_with_additive_angles():
    rng = np.random.default_rng(60)
    x = rng.standard_normal((7, 3, 64))
    pos = rng.integers(0, 20000, (7, 3))
    y = H.rope(x, pos)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    assert np.array_equal(H.rope(x, np.zeros((7, 3))), x)
    assert np.allclose(H.rope(H.rope(x, pos), pos + 5), H.rope(x, 2 * pos + 5), atol=1e-9)
    # the same rotation as multiplying (x_i + j x_{i+D/2}) by exp(j pos theta^(-2i/D))
    z = (x[..., :32] + 1j * x[..., 32:]) * np.exp(1j * pos[..., None] * 10000.0 ** (-np.arange(32) / 32))
    assert np.allclose(y, np.concatenate([z.real, z.imag], axis=-1), atol=1e-9)


def test_rope_scores_depend_on_position_differences_only():
    rng = np.random.default_rng(61)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n, s in ((3, 1, 100), (50, 70, 12345), (0, 0, 7)):
        a = H.rope(q, m) @ H.rope(k, n)
        b = H.rope(q, m + s) @ H.rope(k, n + s)
        assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


@pytest.mark.parametrize("tree", [[2, 3], [3, 2, 2]])
def test_tree_positions_make_each_branch_a_causal_sequence(tree):
    """With positions L + depth, tree attention over rotated Q/K equals causal
    attention over each root-to-leaf branch at consecutive positions L, L+1, ...
    (positions by breadth-first index would break this for every branch that
    is not the first)."""
    rng = np.random.default_rng(62 + len(tree))
    plan = H.plan_cartesian(tree)
    N, Hq, Hkv, D, L = plan.n, 4, 2, 16, 9
    anc = H.ancestors(plan.parent, plan.dmax)[None]
    q = rng.standard_normal((1, N, Hq, D))
    kt, vt = rng.standard_normal((1, N, Hkv, D)), rng.standard_normal((1, N, Hkv, D))
    kp, vp = rng.standard_normal((L, Hkv, D)), rng.standard_normal((L, Hkv, D))
    pos = H.tree_positions([L], plan.depth[None])
    assert pos[0, 0] == L and np.array_equal(pos[0], L + plan.depth)
    kp_rot = H.rope(kp, np.arange(L)[:, None])
    out, _ = H.tree_attention(H.rope(q, pos[..., None]), H.rope(kt, pos[..., None]), vt, [kp_rot], [vp], anc)
    for leaf in [u for u in range(N) if not plan.children(u)]:
        br = [int(a) for a in anc[0, leaf] if a >= 0]
        cpos = np.arange(L, L + len(br))[:, None]
        qs = np.concatenate([np.zeros((L, Hq, D)), H.rope(q[0, br], cpos)])
        ks = np.concatenate([kp_rot, H.rope(kt[0, br], cpos)])
        vs = np.concatenate([vp, vt[0, br]])
        ref = _causal_sdpa(torch.from_numpy(qs), torch.from_numpy(ks), torch.from_numpy(vs)).numpy()[L:]
        assert np.allclose(out[0, br], ref, rtol=1e-10, atol=1e-12)


# -------------------------------------------------------- decoder layer

def _llama_layer(d, F, Hq, Hkv, D, eps, theta, w):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding

    cfg = LlamaConfig(hidden_size=d, intermediate_size=F, num_attention_heads=Hq, num_key_value_heads=Hkv,
                      head_dim=D, rms_norm_eps=eps, rope_theta=theta, num_hidden_layers=1, vocab_size=16)
    cfg._attn_implementation = "eager"
    layer = LlamaDecoderLayer(cfg, layer_idx=0).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        layer.input_layernorm.weight.copy_(t(w["g1"]))
        layer.post_attention_layernorm.weight.copy_(t(w["g2"]))
        for name, key in (("q_proj", "Wq"), ("k_proj", "Wk"), ("v_proj", "Wv"), ("o_proj", "Wo")):
            getattr(layer.self_attn, name).weight.copy_(t(w[key]))
        for name, key in (("gate_proj", "Wg"), ("up_proj", "Wu"), ("down_proj", "Wd")):
            getattr(layer.mlp, name).weight.copy_(t(w[key]))
    return cfg, layer, LlamaRotaryEmbedding(cfg)


@pytest.mark.parametrize("tree,Hq,Hkv", [([2, 3], 4, 2), ([3, 2, 2], 4, 4)])
def test_decoder_layer_matches_transformers_llama_layer(tree, Hq, Hkv):
    """The oracle's decoder layer against transformers' LlamaDecoderLayer in
    float64, run per sequence with the prefix in its cache, position ids
    L + depth and an additive mask that opens the prefix and each row's
    ancestors (its rotary tables and its RMSNorm are float32: positions stay
    small and the tolerance is 1e-5)."""
    from transformers import DynamicCache

    rng = np.random.default_rng(70 + len(tree) + Hkv)
    plan = H.plan_cartesian(tree)
    N, D, F, eps, theta = plan.n, 8, 48, 1e-6, 10000.0
    d = Hq * D
    lens = [5, 11]
    B = len(lens)
    w = dict(g1=1 + 0.1 * rng.standard_normal(d), g2=1 + 0.1 * rng.standard_normal(d),
             Wq=0.2 * rng.standard_normal((Hq * D, d)), Wk=0.2 * rng.standard_normal((Hkv * D, d)),
             Wv=0.2 * rng.standard_normal((Hkv * D, d)), Wo=0.2 * rng.standard_normal((d, Hq * D)),
             Wg=0.2 * rng.standard_normal((F, d)), Wu=0.2 * rng.standard_normal((F, d)),
             Wd=0.2 * rng.standard_normal((d, F)))
    x = rng.standard_normal((B, N, d))
    kp = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vp = [rng.standard_normal((L, Hkv, D)) for L in lens]
    anc = np.stack([H.ancestors(plan.parent, plan.dmax)] * B)
    depth = np.stack([plan.depth] * B)
    got, k_rot, v = H.decoder_layer(x, w, kp, vp, anc, depth, lens, Hq, Hkv, D, eps, theta)
    cfg, layer, rot = _llama_layer(d, F, Hq, Hkv, D, eps, theta, w)
    vis = H.tree_mask(plan.parent)  # 0 / -inf over the tree rows
    for b, L in enumerate(lens):
        cache = DynamicCache()
        cache.update(torch.from_numpy(kp[b]).transpose(0, 1)[None], torch.from_numpy(vp[b]).transpose(0, 1)[None], 0)
        mask = np.concatenate([np.zeros((N, L)), np.where(np.isfinite(vis), 0.0, np.finfo(np.float64).min)], axis=1)
        hs = torch.from_numpy(x[b])[None]
        pos_ids = torch.from_numpy(L + plan.depth)[None]
        with torch.no_grad():
            out = layer(hs, attention_mask=torch.from_numpy(mask)[None, None], position_ids=pos_ids,
                        past_key_values=cache, use_cache=True, position_embeddings=rot(hs, pos_ids))
        out = out[0] if isinstance(out, tuple) else out
        assert np.allclose(got[b], out[0].numpy(), rtol=1e-5, atol=1e-5)
        # the cache now holds the layer's rotated tree keys and values after the prefix
        ck, cv = cache.layers[0].keys[0].transpose(0, 1).numpy(), cache.layers[0].values[0].transpose(0, 1).numpy()
        assert np.allclose(ck[L:], k_rot[b], rtol=1e-5, atol=1e-5) and np.allclose(cv[L:], v[b], rtol=1e-5, atol=1e-5)


# -------------------------------------------------------- the target's forward pass

def _layer_dict(rng, d, F, Hq, Hkv, D):
    return dict(g1=1 + 0.1 * rng.standard_normal(d), g2=1 + 0.1 * rng.standard_normal(d),
                Wq=0.2 * rng.standard_normal((Hq * D, d)), Wk=0.2 * rng.standard_normal((Hkv * D, d)),
                Wv=0.2 * rng.standard_normal((Hkv * D, d)), Wo=0.2 * rng.standard_normal((d, Hq * D)),
                Wg=0.2 * rng.standard_normal((F, d)), Wu=0.2 * rng.standard_normal((F, d)),
                Wd=0.2 * rng.standard_normal((d, F)))


def test_verify_layers_matches_transformers_llama_model_on_a_chain():
    """On a chain-shaped tree with nothing cached, tree attention is causal
    attention at positions 0..N-1, so the oracle's forward pass (embeddings,
    layers, final norm) must equal transformers' LlamaModel on the same ids in
    float64, hidden states and every layer's cached keys and values alike."""
    from transformers import LlamaConfig, LlamaModel

    rng = np.random.default_rng(81)
    n_layers, Hq, Hkv, D, F, V, eps, theta = 3, 4, 2, 8, 40, 50, 1e-6, 10000.0
    d = Hq * D
    plan = H.plan_cartesian([1, 1, 1, 1, 1])  # root and five drafts in a line
    assert list(plan.parent) == [-1, 0, 1, 2, 3, 4]
    B, N = 2, plan.n
    tok = rng.integers(0, V, (B, N))
    E = rng.standard_normal((V, d))
    layers = [_layer_dict(rng, d, F, Hq, Hkv, D) for _ in range(n_layers)]
    g_f = 1 + 0.1 * rng.standard_normal(d)
    empty = [np.zeros((0, Hkv, D))] * B
    anc = np.stack([H.ancestors(plan.parent, plan.dmax)] * B)
    depth = np.stack([plan.depth] * B)
    h, k, v = H.verify_layers(tok, E, layers, g_f, [empty] * n_layers, [empty] * n_layers, anc, depth, [0] * B,
                              Hq, Hkv, D, eps, theta)
    cfg = LlamaConfig(hidden_size=d, intermediate_size=F, num_attention_heads=Hq, num_key_value_heads=Hkv,
                      head_dim=D, rms_norm_eps=eps, rope_theta=theta, num_hidden_layers=n_layers, vocab_size=V)
    cfg._attn_implementation = "eager"
    model = LlamaModel(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        model.embed_tokens.weight.copy_(t(E))
        model.norm.weight.copy_(t(g_f))
        for layer, w in zip(model.layers, layers):
            layer.input_layernorm.weight.copy_(t(w["g1"]))
            layer.post_attention_layernorm.weight.copy_(t(w["g2"]))
            for name, key in (("q_proj", "Wq"), ("k_proj", "Wk"), ("v_proj", "Wv"), ("o_proj", "Wo")):
                getattr(layer.self_attn, name).weight.copy_(t(w[key]))
            for name, key in (("gate_proj", "Wg"), ("up_proj", "Wu"), ("down_proj", "Wd")):
                getattr(layer.mlp, name).weight.copy_(t(w[key]))
        out = model(input_ids=torch.from_numpy(tok), use_cache=True)
    assert np.allclose(h, out.last_hidden_state.numpy(), rtol=1e-5, atol=1e-5)
    for l in range(n_layers):
        ck = out.past_key_values.layers[l].keys.transpose(1, 2).numpy()
        cv = out.past_key_values.layers[l].values.transpose(1, 2).numpy()
        assert np.allclose(k[l], ck, rtol=1e-5, atol=1e-5) and np.allclose(v[l], cv, rtol=1e-5, atol=1e-5)


def test_verify_layers_on_a_tree_with_cached_prefixes_matches_transformers_modules():
    """A branching tree over per-layer cached prefixes of different lengths:
    the forward pass equals transformers' own pieces chained by hand (the
    embedding lookup, LlamaDecoderLayer per layer with that layer's prefix
    in its cache, position ids L + depth and the tree mask, LlamaRMSNorm); a
    token outside the table gives its row a zero input."""
    from transformers import DynamicCache
    from transformers.models.llama.modeling_llama import LlamaRMSNorm

    rng = np.random.default_rng(82)
    n_layers, Hq, Hkv, D, F, V, eps, theta = 2, 4, 2, 8, 40, 30, 1e-6, 10000.0
    d = Hq * D
    plan = H.plan_cartesian([2, 3])
    N, lens = plan.n, [4, 9]
    B = len(lens)
    tok = rng.integers(0, V, (B, N))
    tok[1, 2] = V + 5  # outside the table
    E = rng.standard_normal((V, d))
    layers = [_layer_dict(rng, d, F, Hq, Hkv, D) for _ in range(n_layers)]
    g_f = 1 + 0.1 * rng.standard_normal(d)
    kp = [[rng.standard_normal((L, Hkv, D)) for L in lens] for _ in range(n_layers)]
    vp = [[rng.standard_normal((L, Hkv, D)) for L in lens] for _ in range(n_layers)]
    anc = np.stack([H.ancestors(plan.parent, plan.dmax)] * B)
    depth = np.stack([plan.depth] * B)
    h, k, v = H.verify_layers(tok, E, layers, g_f, kp, vp, anc, depth, lens, Hq, Hkv, D, eps, theta)
    mods = [_llama_layer(d, F, Hq, Hkv, D, eps, theta, w) for w in layers]
    norm = LlamaRMSNorm(d, eps=eps).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(g_f))
    vis = H.tree_mask(plan.parent)
    Et = torch.from_numpy(np.concatenate([E, np.zeros((1, d))]))  # the zero row stands in for the bad token
    for b, L in enumerate(lens):
        ids = torch.from_numpy(np.where(tok[b] < V, tok[b], V))
        hs = torch.nn.functional.embedding(ids, Et)[None]
        mask = np.concatenate([np.zeros((N, L)), np.where(np.isfinite(vis), 0.0, np.finfo(np.float64).min)], axis=1)
        pos_ids = torch.from_numpy(L + plan.depth)[None]
        for l, (cfg, layer, rot) in enumerate(mods):
            cache = DynamicCache()
            cache.update(torch.from_numpy(kp[l][b]).transpose(0, 1)[None],
                         torch.from_numpy(vp[l][b]).transpose(0, 1)[None], 0)
            with torch.no_grad():
                hs = layer(hs, attention_mask=torch.from_numpy(mask)[None, None], position_ids=pos_ids,
                           past_key_values=cache, use_cache=True, position_embeddings=rot(hs, pos_ids))
            hs = hs[0] if isinstance(hs, tuple) else hs
            ck = cache.layers[0].keys[0].transpose(0, 1).numpy()
            assert np.allclose(ck[L:], k[l, b], rtol=1e-5, atol=1e-5)
        with torch.no_grad():
            ref = norm(hs)[0].numpy()
        assert np.allclose(h[b], ref, rtol=1e-5, atol=1e-5)
