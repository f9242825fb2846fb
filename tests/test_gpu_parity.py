"""Device path against the CPU oracle, through the C ABI (needs an MI355X).

Float tolerances (max-abs): 1e-4 in float32 mode, 2e-2 for bfloat16 inputs
with float32 accumulation. Integer results (tokens, tree indices, accepted
lengths) are bit-exact, with the 1e-4 margin rule of tests/helpers.py for
top-k decisions.
"""
import math

import numpy as np
import pytest
import torch

import hydra_inputs as HI
from oracle import hydra_oracle as O
from tests import helpers as T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import speculative_decoding_hydra_amd._lib as L

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()  # fails loudly if libhydra.so is missing
    torch.cuda.set_device(0)


def _bf16(x):
    return x.to(torch.bfloat16)


# ------------------------------------------------------------ projections

@pytest.mark.parametrize("M,K,N", [(1, 256, 1000), (5, 512, 640), (16, 4096, 4096), (17, 256, 2000),
                                   (33, 1024, 777), (64, 4096, 32000), (100, 512, 1000), (256, 256, 512),
                                   (300, 256, 130), (13, 8192, 4096), (0, 256, 64), (1024, 1024, 3000),
                                   (420, 2048, 1111), (65, 1024, 3001), (200, 2048, 4100), (64, 11008, 4096),
                                   (13, 11008, 1000), (18, 768, 640), (64, 4096, 22016)])
def test_projection_bf16(M, K, N):
    from speculative_decoding_hydra_amd import hydra_vocab_projection

    print(f"projection bf16 M={M} K={K} N={N}", flush=True)
    g = torch.Generator().manual_seed(M * 7 + K + N)
    X = _bf16(torch.randn(M, K, generator=g))
    W = _bf16(torch.randn(N, K, generator=g) * 0.02)
    Y = torch.full((M, N), float("nan"), device="cuda")
    hydra_vocab_projection(X.cuda(), W.cuda(), Y)
    torch.cuda.synchronize()
    if M == 0:
        return
    ref = HI.as_f64(X) @ HI.as_f64(W).T
    err = float(np.max(np.abs(Y.cpu().double().numpy() - ref)))
    assert err <= 1e-3, err  # bf16 inputs are exact in fp32; only the summation order differs


@pytest.mark.parametrize("M,K,N,k", [(1, 256, 1000, 10), (13, 4096, 32000, 10), (64, 4096, 32000, 1),
                                     (17, 512, 1000, 0), (33, 256, 777, 3), (100, 512, 1000, 5),
                                     (300, 256, 130, 0), (1024, 1024, 3000, 1), (5, 256, 70, 4)])
def test_projection_packed_weights_match_row_major(M, K, N, k):
    """The packed weight layout is a layout of the same values and the
    kernels keep their K order, so the logits (streaming kernel up to 64
    rows, tiled kernel from 65) and the fused top-k partials are bit-identical
    to those of the row-major weights; the packed copy itself holds every
    value of W at the offset the layout defines, and zeros past row N."""
    from speculative_decoding_hydra_amd import (hydra_pack_weight, hydra_vocab_projection,
                                                hydra_vocab_projection_workspace_size, hydra_vocab_topk)

    print(f"packed weights M={M} K={K} N={N} k={k}", flush=True)
    g = torch.Generator().manual_seed(M + 3 * K + N + k)
    X = _bf16(torch.randn(M, K, generator=g)).cuda()
    W = _bf16(torch.randn(N, K, generator=g) * 0.05).cuda()
    Wp = hydra_pack_weight(W)
    torch.cuda.synchronize()
    # the layout, spelled out: tile t, chunk c, step s, group g, row r
    T = (N + 15) // 16
    ref_pack = torch.zeros(T * 16, K, dtype=torch.bfloat16)
    ref_pack[:N] = W.cpu()
    ref_pack = ref_pack.view(T, 16, K // 256, 8, 4, 8).permute(2, 0, 3, 4, 1, 5).reshape(-1)
    assert torch.equal(Wp.data.cpu(), ref_pack)
    outs = []
    for Wm in (W, Wp):
        Y = torch.empty(M, N, device="cuda")
        ws = torch.empty(max(1, hydra_vocab_projection_workspace_size(M, N, k)), dtype=torch.uint8, device="cuda")
        hydra_vocab_projection(X, Wm, Y, k, ws if k else None)
        res = [Y]
        if k:
            lse = torch.empty(M, device="cuda")
            ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
            vals = torch.empty(M, k, device="cuda")
            hydra_vocab_topk(M, N, k, Y, ws, lse, ids, vals)
            res += [lse, ids, vals]
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in res])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    ref = HI.as_f64(X) @ HI.as_f64(W).T
    assert float(np.max(np.abs(outs[1][0].double().numpy() - ref))) <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,K,N,k", [(1, 256, 1000, 10), (13, 4096, 32000, 10), (64, 512, 32000, 1),
                                     (20, 256, 100, 16), (300, 256, 1000, 3), (5, 256, 70, 4)])
def test_vocab_topk(dtype, M, K, N, k):
    """Fused top-k / log-sum-exp of the projection: bit-exact against the CPU
    on the device logits, and against the oracle's own float64 logits under
    the 1e-4 margin rule."""
    from speculative_decoding_hydra_amd import (hydra_vocab_projection, hydra_vocab_projection_workspace_size,
                                                hydra_vocab_topk)

    print(f"vocab top-k {dtype} M={M} K={K} N={N} k={k}", flush=True)
    g = torch.Generator().manual_seed(M + K + N + k)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    X = torch.randn(M, K, generator=g).to(dt)
    W = (torch.randn(N, K, generator=g) * 0.05).to(dt)
    if N <= 100:  # force exact ties: duplicate rows of W
        W[N // 2:] = W[: N - N // 2]
    Y = torch.empty(M, N, device="cuda")
    ws = torch.empty(hydra_vocab_projection_workspace_size(M, N, k), dtype=torch.uint8, device="cuda")
    lse = torch.empty(M, device="cuda")
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    vals = torch.empty(M, k, device="cuda")
    hydra_vocab_projection(X.cuda(), W.cuda(), Y, k, ws)
    hydra_vocab_topk(M, N, k, Y, ws, lse, ids, vals)
    torch.cuda.synchronize()
    Yd = Y.cpu().double().numpy()
    ref = HI.as_f64(X) @ HI.as_f64(W).T
    for m in range(M):
        assert np.array_equal(ids[m].cpu().numpy(), O.topk_sorted(Yd[m], k)), f"row {m}"
        assert np.array_equal(vals[m].cpu().double().numpy(), Yd[m][O.topk_sorted(Yd[m], k)])
        T.check_topk(ref[m], Yd[m], k, ids[m].cpu().numpy(), f"row {m}")
        assert abs(float(lse[m]) - O.logsumexp(Yd[m])) <= 1e-4 * max(1.0, abs(O.logsumexp(Yd[m])))


@pytest.mark.gpu
@pytest.mark.parametrize("groups,k", [(8, 10), (1, 16), (3, 5)])
def test_vocab_topk_mass_ties(groups, k):
    """Every column repeats one of `groups` distinct weight rows, so each row of
    logits holds only `groups` values, each tied across hundreds of ids: the
    top k must be the lowest ids carrying the largest value, in id order."""
    from speculative_decoding_hydra_amd import (hydra_vocab_projection, hydra_vocab_projection_workspace_size,
                                                hydra_vocab_topk)

    M, K, N = 6, 256, 1000
    print(f"vocab top-k mass ties groups={groups} k={k}", flush=True)
    g = torch.Generator().manual_seed(groups * 100 + k)
    X = torch.randn(M, K, generator=g).to(torch.bfloat16)
    base = (torch.randn(groups, K, generator=g) * 0.05).to(torch.bfloat16)
    W = base[torch.arange(N) % groups].contiguous()
    Y = torch.empty(M, N, device="cuda")
    ws = torch.empty(hydra_vocab_projection_workspace_size(M, N, k), dtype=torch.uint8, device="cuda")
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    hydra_vocab_projection(X.cuda(), W.cuda(), Y, k, ws)
    hydra_vocab_topk(M, N, k, Y, ws, None, ids, None)
    torch.cuda.synchronize()
    Yd = Y.cpu().double().numpy()
    for m in range(M):
        assert np.array_equal(ids[m].cpu().numpy(), O.topk_sorted(Yd[m], k)), f"row {m}"
        first = int(np.argmax(Yd[m][:groups]))
        top_vals = Yd[m][:groups]
        if np.sum(top_vals == top_vals[first]) == 1:  # one group holds the maximum
            assert np.array_equal(ids[m].cpu().numpy(), first + groups * np.arange(k)), f"row {m}"


@pytest.mark.parametrize("M,K,N", [(1, 256, 1000), (9, 256, 1000), (7, 100, 33)])
def test_projection_f32(M, K, N):
    from speculative_decoding_hydra_amd import hydra_vocab_projection

    g = torch.Generator().manual_seed(M + K + N)
    X = torch.randn(M, K, generator=g)
    W = torch.randn(N, K, generator=g) * 0.02
    Y = torch.empty(M, N, device="cuda")
    hydra_vocab_projection(X.cuda(), W.cuda(), Y)
    torch.cuda.synchronize()
    ref = X.double().numpy() @ W.double().numpy().T
    assert float(np.max(np.abs(Y.cpu().double().numpy() - ref))) <= 1e-5


# -------------------------------------------------------------- attention

def _attn_case(B, N, Hq, Hkv, D, lens, dtype, seed, tree=None, scattered=True, page=16):
    g = torch.Generator().manual_seed(seed)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    if tree is None:
        # random breadth-first tree: parent[i] uniform over earlier nodes, depth <= 8
        parent = [-1]
        depth = [0]
        for i in range(1, N):
            while True:
                p = int(torch.randint(0, i, (1,), generator=g))
                if depth[p] < 8:
                    break
            parent.append(p)
            depth.append(depth[p] + 1)
        order = sorted(range(N), key=lambda i: (depth[i], i))
        new = {o: k for k, o in enumerate(order)}
        parent = [-1 if parent[o] < 0 else new[parent[o]] for o in order]
        parent = np.array(parent)
    else:
        parent = tree
    dm = 1
    anc = O.ancestors(parent, 8)
    dep = np.array([int(np.sum(a >= 0)) - 1 for a in anc])
    dm = max(1, int(dep.max()))
    anc = anc[:, : dm + 1]
    q = torch.randn(B, N, Hq, D, generator=g).to(dt)
    kt = torch.randn(B, N, Hkv, D, generator=g).to(dt)
    vt = torch.randn(B, N, Hkv, D, generator=g).to(dt)
    kp = [torch.randn(L, Hkv, D, generator=g).to(dt) for L in lens]
    vp = [torch.randn(L, Hkv, D, generator=g).to(dt) for L in lens]
    per = [max(1, math.ceil(L / page)) for L in lens]
    n_pages = sum(per)
    order = torch.randperm(n_pages, generator=g) if scattered else torch.arange(n_pages)
    kpool = torch.zeros(n_pages, Hkv, page, D, dtype=dt)
    vpool = torch.zeros(n_pages, Hkv, page, D, dtype=dt)
    bt = torch.full((B, max(per)), -1, dtype=torch.int32)
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(per[b]):
            pid = int(order[nxt])
            nxt += 1
            bt[b, j] = pid
            lo, hi = j * page, min(L, (j + 1) * page)
            if hi > lo:
                kpool[pid, :, : hi - lo] = kp[b][lo:hi].transpose(0, 1)
                vpool[pid, :, : hi - lo] = vp[b][lo:hi].transpose(0, 1)
    ancB = np.stack([anc] * B).astype(np.int32)
    depB = np.stack([dep] * B).astype(np.int32)
    return dict(q=q, kt=kt, vt=vt, kp=kp, vp=vp, kpool=kpool, vpool=vpool, bt=bt,
                lens=torch.tensor(lens, dtype=torch.int32), anc=ancB, dep=depB, dt=dt)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,N,Hq,Hkv,D,lens", [
    (1, 9, 8, 8, 32, [128]),
    (1, 64, 4, 4, 128, [2048 + 5]),
    (2, 64, 8, 1, 128, [300, 17]),
    (3, 100, 16, 2, 128, [0, 1, 777]),
    (1, 1, 4, 4, 128, [64]),
    (2, 256, 2, 2, 128, [1000, 64]),
    (1, 37, 4, 2, 64, [129]),
])
def test_tree_attention(dtype, B, N, Hq, Hkv, D, lens):
    from speculative_decoding_hydra_amd import tree_attention_verify, tree_attention_verify_workspace_size

    print(f"attention {dtype} B={B} N={N} Hq={Hq} Hkv={Hkv} D={D} L={lens}", flush=True)
    c = _attn_case(B, N, Hq, Hkv, D, lens, dtype, seed=N * 31 + Hq + sum(lens))
    dev = lambda t: t.cuda().contiguous()  # noqa: E731
    out = torch.full((B, N, Hq, D), float("nan"), dtype=c["dt"], device="cuda")
    lse = torch.empty(B, N, Hq, device="cuda")
    code = 0 if dtype == "fp32" else 1
    ws = torch.empty(max(1, tree_attention_verify_workspace_size(code, B, N, Hq, Hkv, D, max(lens))),
                     dtype=torch.uint8, device="cuda")
    tree_attention_verify(dev(c["q"]), dev(c["kt"]), dev(c["vt"]), dev(c["kpool"]), dev(c["vpool"]), dev(c["bt"]),
                          dev(c["lens"]), max(lens), dev(torch.from_numpy(c["anc"])), dev(torch.from_numpy(c["dep"])),
                          out, lse, ws)
    torch.cuda.synchronize()
    f = HI.as_f64
    ref, ref_lse = O.tree_attention(f(c["q"]), f(c["kt"]), f(c["vt"]), [f(x) for x in c["kp"]],
                                    [f(x) for x in c["vp"]], c["anc"], bf16=dtype == "bf16")
    t = 1e-4 if dtype == "fp32" else 2e-2
    e = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    el = float(np.max(np.abs(lse.cpu().double().numpy() - ref_lse)))
    print(f"  max-abs out {e:.3g} lse {el:.3g}", flush=True)
    assert e <= t and el <= t


# ------------------------------------------------------------ whole rounds

_cache = {}


def _round(name, pack_vocab=None, **over):
    key = (name, pack_vocab, tuple(sorted(over.items())))
    if key not in _cache:
        w = HI.workload(name, **over)
        print(f"round {name} {over} pack_vocab={pack_vocab}: generating", flush=True)
        inp = HI.generate(w)
        rnd, dev = T.round_inputs(inp, pack_vocab=pack_vocab)
        print(f"round {name}: running on the device", flush=True)
        T.run_round(rnd, dev)
        torch.cuda.synchronize()
        _cache.clear()
        _cache[key] = (inp, rnd, dev)
    return _cache[key]


@pytest.mark.parametrize("name", ["tiny", "tiny_medusa", "tiny_sketch", "tiny_path", "tiny_attn"])
def test_tiny_round_stagewise(name):
    inp, rnd, dev = _round(name)
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


@pytest.mark.parametrize("name", ["tiny", "tiny_medusa", "tiny_sketch", "tiny_path", "tiny_attn"])
def test_tiny_round_end_to_end(name):
    """Float32 workload: the oracle's own round from the inputs alone."""
    inp, rnd, _ = _round(name)
    w = inp["workload"]
    plan, _ = T.oracle_plan(w.tree)
    f = HI.as_f64
    if w.head == "sketch":
        heads = [{n: f(t) for n, t in hd.items()} for hd in inp["heads"]]
    else:
        heads = [(f(a), f(b), f(c)) for a, b, c in zip(inp["W1"], inp["b1"], inp["W2"])]
    res = O.draft_heads(f(inp["h"]), inp["root_tok"].numpy(), f(inp["E"]), heads, plan, hydra=w.hydra,
                        full_path=w.cond == "path", attn=T.oracle_attn(inp) if w.cond == "attn" else None)
    for r in range(res["z"].shape[1]):
        assert res["margin"][0, r] > T.MARGIN, "near tie: seed would need the margin rule"
    assert np.array_equal(res["tok"], rnd.cand_tok.cpu().numpy())
    anc = O.ancestors(plan.parent, plan.dmax)[None]
    pos = O.tree_positions(inp["prefix_len"].numpy(), plan.depth[None])[..., None]
    out, _ = O.tree_attention(O.rope(f(inp["q_tree"]), pos), O.rope(f(inp["k_tree"]), pos), f(inp["v_tree"]),
                              [f(x) for x in inp["k_prefix"]], [f(x) for x in inp["v_prefix"]], anc)
    Z = O.target_logits(out, f(inp["W_t"]))[0]
    m, path, toks = O.greedy_accept(Z, res["tok"][0], plan.parent, plan.dmax)
    assert int(rnd.n_accepted[0]) == m
    assert [int(x) for x in rnd.out_tok[0] if x >= 0] == toks
    assert [int(x) for x in rnd.path[0] if x >= 0] == path


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("hydra", [False, True])
def test_zero_init_heads_reproduce_lm_head_exactly(dtype, hydra):
    """Zero-initialised heads whose vocabulary projection is a copy of the
    base head give that head's logits bit for bit (same projection kernel)."""
    from speculative_decoding_hydra_amd import hydra_vocab_projection

    over = dict(zero_init=True)
    if dtype == "bf16":
        over.update(dtype="bf16", d=256)
    inp, rnd, dev = _round("tiny" if hydra else "tiny_medusa", **over)
    base = torch.empty(1, inp["workload"].V, device="cuda")
    hydra_vocab_projection(dev["h"], rnd.w["W_t"], base)
    torch.cuda.synchronize()
    got = rnd.head_logits[0]
    assert torch.equal(rnd.head_hidden[0], dev["h"].expand_as(rnd.head_hidden[0]))
    assert all(torch.equal(got[r], base[0]) for r in range(got.shape[0]))


@pytest.mark.parametrize("B,dtype", [(4, "fp32"), (4, "bf16"), (20, "bf16"), (300, "fp32")])
def test_greedy_planted_paths(B, dtype):
    """Target logits forced along a chosen branch give that accepted length.
    Up to 256 sequences the walk runs inside the arg-max merge (its counters
    cleared by the streaming projection, by the tiled one at 20 x 21 = 420
    rows, or by the float32 partials pass); 300 sequences take the separate
    walk kernel."""
    from speculative_decoding_hydra_amd import tree_accept, tree_accept_workspace_size

    print(f"greedy planted B={B} {dtype}", flush=True)
    g = np.random.default_rng(B)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    V, d = 1000, 256
    plan = O.plan_cartesian([2, 3, 2])
    N = plan.n
    anc = O.ancestors(plan.parent, plan.dmax)
    W = g.standard_normal((V, d)) * 0.02
    for trial in range(6 if B < 100 else 2):
        tok = np.zeros((B, N), dtype=np.int32)
        o = g.standard_normal((B, N, d)) * 0.1
        want = []
        for b in range(B):
            for u in range(N):
                kids = plan.children(u)
                tok[b, kids] = g.choice(V, len(kids), replace=False)
            target = int(g.integers(0, N)) if trial else 0
            path = [int(a) for a in anc[target] if a >= 0]
            kid = set(int(tok[b, c]) for c in plan.children(target))
            stop = int(g.choice([t for t in range(V) if t not in kid]))
            for a, nx in zip(path[:-1], path[1:]):
                o[b, a] = W[tok[b, nx]] * 40.0
            o[b, path[-1]] = W[stop] * 40.0
            want.append((len(path) - 1, path, [int(tok[b, c]) for c in path[1:]] + [stop]))
        ot = torch.tensor(o, dtype=torch.float32).to(dt).cuda()
        Wt = torch.tensor(W, dtype=torch.float32).to(dt).cuda()
        tk = torch.tensor(tok).cuda()
        par = torch.tensor(np.stack([plan.parent] * B).astype(np.int32)).cuda()
        Z = torch.empty(B, N, V, device="cuda")
        n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
        path_t = torch.empty(B, plan.dmax + 1, dtype=torch.int32, device="cuda")
        out_t = torch.empty_like(path_t)
        ws = torch.empty(tree_accept_workspace_size(0, B, N, V), dtype=torch.uint8, device="cuda")
        tree_accept(ot, Wt, tk, par, Z, n_acc, path_t, out_t, ws)
        torch.cuda.synchronize()
        for b in range(B):
            m, path, toks = want[b]
            ref = O.greedy_accept(Z[b].cpu().double().numpy(), tok[b], plan.parent, plan.dmax)
            assert ref == (m, path, toks), "planted branch not the oracle's"
            assert int(n_acc[b]) == m
            assert [int(x) for x in path_t[b] if x >= 0] == path
            assert [int(x) for x in out_t[b] if x >= 0] == toks


@pytest.mark.parametrize("pack_vocab", [None, False])
def test_7b_sparse64_round(pack_vocab):
    """The headline round; by default its bf16 vocabulary weights are packed,
    and once more with them row-major."""
    inp, rnd, dev = _round("7b_sparse64", pack_vocab=pack_vocab)
    assert rnd.pack_vocab == (pack_vocab is None)
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


def test_7b_dense256_round():
    inp, rnd, dev = _round("7b_dense256")
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


def test_tiny_stochastic_round():
    """Rejection acceptance at temperature 0.7 on the tiny workload."""
    inp, rnd, dev = _round("tiny", mode="stochastic", T=0.7)
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_tiny_stochastic_planted_acceptance(seed):
    """Planted attention outputs make the target favour the drafted tokens
    along one branch, so the rejection walk sees accepts as well as
    rejections, residual updates and the final draw; every decision is
    checked against the oracle following the device's path."""
    inp, rnd, dev = _round("tiny", mode="stochastic", T=0.7, seed=seed)
    g = np.random.default_rng(seed)
    plan, _ = T.oracle_plan(inp["workload"].tree)
    Wt = inp["W_t"]
    tok = rnd.tok.cpu().numpy()
    o = rnd.attn_out.clone()
    for b in range(o.shape[0]):
        u = 0
        while plan.children(u):
            c = int(g.choice(plan.children(u)))
            o[b, u] = (Wt[int(tok[b, c])] * 40.0).view(o.shape[2], o.shape[3]).to(o.device)
            u = c
    rnd.attn_out.copy_(o)
    rnd.accept(dev["u_acc"], dev["u_res"])
    torch.cuda.synchronize()
    rep = T.check_accept(inp, rnd)
    print(rep, "accepted", rnd.n_accepted.tolist(), flush=True)


@pytest.mark.parametrize("B,dtype", [(3, "bf16"), (2, "fp32")])
def test_rejection_planted_large_vocabulary(B, dtype):
    """Rule S1 over a 32000-token vocabulary (the register-resident node
    kernel holds 32 logits per thread). Planted attention outputs make the
    target put almost all its mass on one drafted token per node of a chosen
    branch, two to four deep; at one node the favoured child is the second
    in rank order, so the first is rejected, the residual norm(max(p - q, 0))
    is formed and the second is accepted from it. The device must take the
    planted branch, and every decision is checked against the oracle
    following the device's path."""
    from speculative_decoding_hydra_amd import tree_accept, tree_accept_workspace_size

    print(f"rejection planted V=32000 B={B} {dtype}", flush=True)
    g = np.random.default_rng(40 + B)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    V, d, Tm = 32000, 256, 0.7
    plan = O.plan_sparse_template((4, 3, 2, 1), 30)
    N = plan.n
    _, _, node_row = O.head_rows(plan, True)
    R = int(node_row.max()) + 1
    W = HI.as_f64(_bf16(torch.tensor(g.standard_normal((V, d)) * 0.02, dtype=torch.float32)))
    tok = np.zeros((B, N), dtype=np.int32)
    o = g.standard_normal((B, N, d)) * 0.01
    hz = (g.standard_normal((B, R, V)) * 2.0).astype(np.float32)
    u_acc = g.random((B, N)).astype(np.float32)
    u_res = g.random((B, N)).astype(np.float32)
    want = []
    for b in range(B):
        for u in range(N):
            kids = plan.children(u)
            tok[b, kids] = g.choice(V, len(kids), replace=False)
        depth_t = int(g.integers(2, plan.dmax + 1))
        r1_step = int(g.integers(0, 2))  # the step that takes a rank-1 child (nodes above depth 2 all have two or more)
        path = [0]
        for step in range(depth_t):
            kids = plan.children(path[-1])
            if not kids:
                break
            pick = [c for c in kids if plan.rank[c] == 1] if step == r1_step else kids
            pick = pick or kids
            if step + 1 < depth_t:
                pick = [c for c in pick if plan.children(c)] or pick
            path.append(int(g.choice(pick)))
        for a, nx in zip(path[:-1], path[1:]):
            o[b, a] = W[tok[b, nx]] * 400.0
        want.append(path)
    assert any(plan.rank[nx] == 1 for p in want for nx in p[1:]), "no rejected first sibling planted"
    ot = torch.tensor(o, dtype=torch.float32).to(dt).cuda()
    Wt = torch.tensor(W, dtype=torch.float32).to(dt).cuda()
    tk = torch.tensor(tok).cuda()
    par = torch.tensor(np.stack([plan.parent] * B).astype(np.int32)).cuda()
    qrow = torch.tensor(np.stack([node_row] * B).astype(np.int32)).cuda()
    Z = torch.empty(B, N, V, device="cuda")
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    path_t = torch.empty(B, plan.dmax + 1, dtype=torch.int32, device="cuda")
    out_t = torch.empty_like(path_t)
    ws = torch.empty(tree_accept_workspace_size(1, B, N, V), dtype=torch.uint8, device="cuda")
    tree_accept(ot, Wt, tk, par, Z, n_acc, path_t, out_t, ws, mode=1, temperature=Tm, q_row=qrow,
                head_logits=torch.tensor(hz).cuda(), u_acc=torch.tensor(u_acc).cuda(),
                u_res=torch.tensor(u_res).cuda())
    torch.cuda.synchronize()
    Zd = Z.cpu().double().numpy()
    Zo = O.target_logits(HI.as_f64(ot.cpu()), W)
    assert float(np.max(np.abs(Zo - Zd))) <= (1e-4 if dtype == "fp32" else 2e-2)
    depths, rejections = [], 0
    for b in range(B):
        got_p = [int(x) for x in path_t[b] if x >= 0]
        got_o = [int(x) for x in out_t[b] if x >= 0]
        assert int(n_acc[b]) == len(got_p) - 1
        assert got_p[: len(want[b])] == want[b], f"seq {b}: device path {got_p}, planted {want[b]}"
        trace = []
        m, p, ot_ = O.rejection_accept(Zd[b], hz[b].astype(np.float64), node_row, tok[b], plan.parent, u_acc[b],
                                       u_res[b], Tm, follow=(got_p, got_o), trace=trace)
        assert p == got_p and ot_ == got_o
        for kind, own, taken, margin in trace:
            if own != taken:
                bound = T.ACCEPT_EPS if kind == "accept" else T.SAMPLE_EPS
                assert margin < bound, f"seq {b}: {kind} decision {taken} vs oracle {own} (margin {margin:.3g})"
        rejections += sum(1 for e in trace if e[0] == "accept" and not e[2])
        depths.append(len(got_p) - 1)
    assert min(depths) >= 2 and rejections > 0, (depths, rejections)


def test_7b_batched16_round():
    """16 ragged sequences over scattered 16-token pages; sampled sequences
    checked stage by stage."""
    inp, rnd, dev = _round("7b_batched16")
    lens = inp["prefix_len"].tolist()
    seqs = sorted({0, int(np.argmin(lens)), int(np.argmax(lens)), 15})
    print("prefix lengths", lens, "checked", seqs, flush=True)
    rep = T.oracle_round_checks(inp, rnd, seqs=seqs)
    rep.update(T.check_commit(inp, rnd, dev, seqs=seqs))
    print(rep, flush=True)


def test_70b_gqa_stochastic_round():
    """70B-shaped GQA layer (64 query heads on 8 KV heads), prefix 16384,
    rejection acceptance at temperature 0.7; sequences 0 and 3 checked."""
    inp, rnd, dev = _round("70b_gqa")
    rep = T.oracle_round_checks(inp, rnd, seqs=[0, 3])
    rep.update(T.check_commit(inp, rnd, dev, seqs=[0, 3]))
    print(rep, flush=True)


@pytest.mark.parametrize("fold", [True, False])
@pytest.mark.parametrize("B,d,b1,hydra", [(4, 8192, 10, True), (3, 4096, 10, True), (3, 8192, 13, True),
                                           (2, 256, 16, True), (1, 8192, 16, True), (8, 4096, 10, True),
                                           (2, 4096, 13, True), (3, 4096, 4, False), (1, 8192, 16, False)])
def test_draft_first_layer_split_and_fused(B, d, b1, hydra, fold):
    """Head hidden states for row counts on both sides of the few-row kernel
    (B * b1 <= 32: head 2's h half runs inside the depth-1 row merge and its
    embedding half at depth 2; Medusa: every head in one launch) and the
    split-K projection path (more rows), d up to 8192; Hydra with and
    without the folded embedding tables (used when d % 1024 == 0)."""
    if fold and not hydra:
        pytest.skip("Medusa heads read no embedding")
    w = HI.workload("70b_gqa", B=B, d=d, V=1000, n_heads=2, tree=("cartesian", (b1, 1)), Hq=8, Hkv=8, D=32,
                    L=(64,), mode="greedy", T=1.0, hydra=hydra)
    print(f"first layer B={B} d={d} rows/depth2={B * b1} hydra={hydra} fold={fold}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp, fold_embedding=fold)
    rnd.draft(dev["h"], dev["root_tok"])  # the draft stage alone (the layer sizes differ from d)
    torch.cuda.synchronize()
    rep = T.check_draft(inp, rnd)
    print(rep, flush=True)


@pytest.mark.parametrize("residual", [True, False])
@pytest.mark.parametrize("fold", [True, False])
@pytest.mark.parametrize("tree", [("sparse", (10, 4, 2, 1), 64), ("cartesian", (3, 2, 2, 2))])
def test_draft_four_heads_folded_and_streamed(tree, fold, residual):
    """Four Hydra heads at d = 4096 (the folded path's next-depth rows are
    written by each row merge, and the h half of head k + 2 streams inside
    the merge of depth k), both against the oracle stage by stage, with and
    without the residual connection."""
    w = HI.workload("7b_sparse64", B=2, V=3000, tree=tree, L=(64,))
    print(f"four heads tree={tree} fold={fold} residual={residual}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp, fold_embedding=fold, residual=residual)
    assert (rnd.emb_proj is not None) == fold
    rnd.draft(dev["h"], dev["root_tok"])  # the draft stage alone (the layer sizes differ from d)
    torch.cuda.synchronize()
    rep = T.check_draft(inp, rnd)
    print(rep, flush=True)


@pytest.mark.parametrize("d", [4096, 8192])
def test_folded_heads_packed_h_halves_match_row_major(d):
    """The folded round streams only the h halves of W1; read from their
    packed copies (HYDRA_W1H_PACKED) they give bit-identical heads to the
    row-major W1 (same products in the same order)."""
    w = HI.workload("7b_sparse64", B=2, d=d, V=3000, L=(64,))
    print(f"folded heads, packed h halves, d={d}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp, fold_embedding=True)
    assert rnd.W1h is not None
    outs = []
    for packed in (True, False):
        saved = rnd.W1h
        rnd.W1h = saved if packed else None
        rnd.draft(dev["h"], dev["root_tok"])
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (rnd.cand_tok, rnd.cand_logp, rnd.head_logits, rnd.head_lse)])
        rnd.W1h = saved
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,d,hid,V,tree", [
    (1, 4096, 1024, 32000, ("sparse", (10, 4, 2, 1), 64)),   # the 7B sketch shape
    (3, 256, 512, 1000, ("cartesian", (4, 3, 2))),
    (2, 8192, 1024, 2000, ("cartesian", (10, 2))),           # 70B width, 20 rows at depth 2
    (20, 512, 768, 1000, ("sparse", (10, 4, 2, 1), 64)),     # 200 rows at depth 2: tiled second layer
    (1, 256, 256, 777, ("cartesian", (16, 1, 1))),           # ragged vocabulary, 16-wide first depth
])
def test_sketch_heads_stagewise(B, d, hid, V, tree):
    """Two-layer LayerNorm heads in bf16 against the oracle stage by stage:
    u within one bf16 step, logits, log-sum-exp and top-k under the margin
    rule, at row counts on both sides of the tiled-product threshold."""
    w = HI.workload("7b_sketch", B=B, d=d, V=V, head_hidden=hid, tree=tree, n_heads=len(tree[1]), Hq=8, Hkv=8,
                    D=32, L=(64,))
    print(f"sketch heads B={B} d={d} H={hid} V={V} tree={tree}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp)
    assert rnd.sketch and rnd.emb_proj is None
    rnd.draft(dev["h"], dev["root_tok"])  # the draft stage alone (the layer sizes differ from d)
    torch.cuda.synchronize()
    rep = T.check_draft(inp, rnd)
    print(rep, flush=True)


@pytest.mark.parametrize("B,d,V,tree", [
    (3, 256, 1000, ("cartesian", (4, 3, 2))),
    (2, 8192, 2000, ("cartesian", (10, 2))),            # 70B width: head 2 reads 3 x 8192 inputs
    (20, 512, 1000, ("sparse", (10, 4, 2, 1), 64)),     # 200 rows at depth 2: tiled product
    (1, 256, 777, ("cartesian", (2, 2, 2, 2, 2, 1))),   # six heads, ragged vocabulary
])
def test_full_path_heads_stagewise(B, d, V, tree):
    """Full-path conditioning in bf16 against the oracle stage by stage: each
    depth-k row gathers h and the embeddings of its k path tokens."""
    w = HI.workload("7b_path", B=B, d=d, V=V, tree=tree, n_heads=len(tree[1]), Hq=8, Hkv=8, D=32, L=(64,))
    print(f"full-path heads B={B} d={d} V={V} tree={tree}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp)
    assert rnd.full_path and rnd.emb_proj is None
    rnd.draft(dev["h"], dev["root_tok"])  # the draft stage alone (the layer sizes differ from d)
    torch.cuda.synchronize()
    rep = T.check_draft(inp, rnd)
    print(rep, flush=True)


@pytest.mark.parametrize("B,d,V,tree", [
    (3, 256, 1000, ("cartesian", (4, 3, 2))),
    (2, 8192, 2000, ("cartesian", (10, 2))),            # 70B width: 8 columns per thread in the path attention
    (20, 512, 1000, ("sparse", (10, 4, 2, 1), 64)),     # 200 rows at depth 2: tiled products
    (1, 256, 777, ("cartesian", (2, 2, 2, 2, 2, 2, 1, 1))),  # eight heads: the deepest path, ragged vocabulary
])
def test_hydra_pp_heads_stagewise(B, d, V, tree):
    """Hydra++ self-attention fusion in bf16 against the oracle stage by
    stage: each row attends over its own path's embeddings, keys and values
    of the ancestors coming from the rows of earlier depths."""
    w = HI.workload("7b_attn", B=B, d=d, V=V, tree=tree, n_heads=len(tree[1]), Hq=8, Hkv=8, D=32, L=(64,))
    print(f"Hydra++ heads B={B} d={d} V={V} tree={tree}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp)
    assert rnd.attn is not None and rnd.emb_proj is None
    rnd.draft(dev["h"], dev["root_tok"])  # the draft stage alone (the layer sizes differ from d)
    torch.cuda.synchronize()
    rep = T.check_draft(inp, rnd)
    print(rep, flush=True)


def test_hydra_pp_7b_round():
    """Whole round with Hydra++ heads at the 7B shape, every stage plus the
    commit."""
    inp, rnd, dev = _round("7b_attn")
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


def test_full_path_7b_round():
    """Whole round with full-path heads at the 7B shape, every stage plus the
    commit."""
    inp, rnd, dev = _round("7b_path")
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


def test_sketch_7b_round():
    """Whole round with the sketch heads at the 7B shape: stage-wise checks
    on every stage plus the commit."""
    inp, rnd, dev = _round("7b_sketch")
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


@pytest.mark.parametrize("V,d", [(1000, 256), (300, 1024), (2049, 4096)])
def test_fold_embedding_table(V, d):
    """hydra_fold_embedding against the float64 product of the same bf16
    inputs: out[t] = W1[:, d:] E[t]."""
    from speculative_decoding_hydra_amd import hydra_fold_embedding

    print(f"fold embedding V={V} d={d}", flush=True)
    g = torch.Generator().manual_seed(V + d)
    E = torch.randn(V, d, generator=g).to(torch.bfloat16)
    W1 = (torch.randn(d, 2 * d, generator=g) * 0.02).to(torch.bfloat16)
    out = torch.full((V, d), float("nan"), device="cuda")
    hydra_fold_embedding(E.cuda(), W1.cuda(), out)
    torch.cuda.synchronize()
    ref = HI.as_f64(E) @ HI.as_f64(W1)[:, d:].T
    err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
    assert err <= 1e-3, err  # bf16 inputs are exact in fp32; only the summation order differs


# ------------------------------------------------------- commit of the branch

def _commit_case(seed, B, N, Hkv, D, layers, page, dmax, dt):
    """Synthetic commit inputs: ragged prefixes over scattered pages with room
    for one commit, random root-to-node branches, and the edge cases (nothing
    accepted, the whole depth accepted, a count past Dmax, a branch row out of
    range, an unmapped page, a prefix ending on a page boundary)."""
    g = np.random.default_rng(seed)
    parent = np.array([-1] + [int(g.integers(0, i)) for i in range(1, N)])
    anc = O.ancestors(parent, N)
    depth = np.array([int(np.sum(a >= 0)) - 1 for a in anc])
    lens = [int(x) for x in g.integers(0, 3 * page, B)]
    lens[0], lens[-1] = page - 1, page  # the branch crosses a page boundary / starts on a new page
    per = [-(-(L + dmax + 1) // page) for L in lens]
    n_pages = sum(per) + 3
    order = g.permutation(n_pages)
    bt = -np.ones((B, max(per)), dtype=np.int32)
    nxt = 0
    for b in range(B):
        bt[b, : per[b]] = order[nxt: nxt + per[b]]
        nxt += per[b]
    kpool = g.standard_normal((layers, n_pages, Hkv, page, D))
    vpool = g.standard_normal((layers, n_pages, Hkv, page, D))
    kt = g.standard_normal((layers, B, N, Hkv, D))
    vt = g.standard_normal((layers, B, N, Hkv, D))
    hidden = g.standard_normal((B, N, 64))
    path = -np.ones((B, dmax + 1), dtype=np.int32)
    out_tok = -np.ones((B, dmax + 1), dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    deep = [u for u in range(N) if depth[u] <= dmax]
    for b in range(B):
        end = 0 if b == 1 else int(g.choice(deep))
        if b == 2:
            end = max(deep, key=lambda u: depth[u])
        br = [int(a) for a in anc[end] if a >= 0]
        n_acc[b] = len(br) - 1
        path[b, : len(br)] = br
        out_tok[b, : len(br)] = g.integers(0, 32000, len(br))
    if B > 4:
        n_acc[3] = dmax + 1          # count out of range: nothing committed
        path[4, min(1, n_acc[4])] = N  # a branch row out of range
        bt[5, (lens[5] + 1) // page] = -1 if n_acc[5] >= 1 else bt[5, (lens[5] + 1) // page]
    cast = lambda a: torch.from_numpy(a).to(torch.float32).to(dt)  # noqa: E731
    return dict(kpool=cast(kpool), vpool=cast(vpool), kt=cast(kt), vt=cast(vt), hidden=cast(hidden), bt=bt,
                lens=np.array(lens, dtype=np.int32), n_acc=n_acc, path=path, out_tok=out_tok)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,N,Hkv,D,layers,page,dmax", [
    (8, 9, 8, 32, 1, 16, 2), (6, 64, 32, 128, 2, 16, 4), (7, 40, 8, 128, 3, 4, 5),
    (9, 30, 2, 64, 1, 64, 8), (1, 1, 4, 32, 1, 16, 0), (300, 12, 1, 8, 1, 5, 3)])
def test_tree_commit(dtype, B, N, Hkv, D, layers, page, dmax):
    """Every byte of the page pools, the next lengths, roots and hidden states
    equal the oracle's commit on the same inputs."""
    from speculative_decoding_hydra_amd import tree_commit

    print(f"commit {dtype} B={B} N={N} Hkv={Hkv} D={D} layers={layers} page={page} Dmax={dmax}", flush=True)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    c = _commit_case(B * 13 + N + page, B, N, Hkv, D, layers, page, dmax, dt)
    dev = lambda a: (torch.from_numpy(a) if isinstance(a, np.ndarray) else a).cuda().contiguous()  # noqa: E731
    kp, vp = dev(c["kpool"]), dev(c["vpool"])
    nlen = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nroot = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nh = torch.full((B, 64), 5.0, dtype=dt, device="cuda")
    tree_commit(dev(c["kt"]), dev(c["vt"]), kp, vp, dev(c["bt"]), dev(c["lens"]), dev(c["n_acc"]), dev(c["path"]),
                dev(c["out_tok"]), nlen, nroot, hidden=dev(c["hidden"]), next_h=nh)
    torch.cuda.synchronize()
    f = HI.as_f64
    rk, rv, rlen, rroot, rh = O.commit_path(f(c["kpool"]), f(c["vpool"]), c["bt"], c["lens"], f(c["kt"]),
                                             f(c["vt"]), c["n_acc"], c["path"], c["out_tok"], dmax, f(c["hidden"]))
    assert np.array_equal(kp.cpu().double().numpy(), rk) and np.array_equal(vp.cpu().double().numpy(), rv)
    assert np.array_equal(nlen.cpu().numpy(), rlen) and np.array_equal(nroot.cpu().numpy(), rroot)
    got_h = nh.cpu().double().numpy()
    for b in range(B):
        if rroot[b] >= 0:
            assert np.array_equal(got_h[b], rh[b]), f"seq {b}: next h"
        else:
            assert np.all(got_h[b] == 5.0), f"seq {b}: next h written without a commit"
    if B > 4:
        assert rroot[3] == -1 and rroot[4] == -1  # the invalid sequences committed nothing


def _oracle_round(w, inp, plan, h, root, q, kt, vt, kpre, vpre, dev_logits, L):
    """The oracle's own greedy round (float32 workloads, B = 1). Its top-k
    decisions are the device's whenever every margin exceeds twice the
    largest difference between the two sides' head logits, so that is
    asserted instead of a fixed margin."""
    f = HI.as_f64
    heads = [(f(a), f(b), f(c)) for a, b, c in zip(inp["W1"], inp["b1"], inp["W2"])]
    res = O.draft_heads(h, root, f(inp["E"]), heads, plan, hydra=w.hydra)
    err = float(np.max(np.abs(res["z"] - dev_logits.cpu().double().numpy())))
    assert err <= 1e-4, f"head logits max-abs {err:.3g}"
    assert np.all(res["margin"] > 2 * err), f"top-k margin {res['margin'].min():.3g} within 2 x {err:.3g}"
    anc = O.ancestors(plan.parent, plan.dmax)[None]
    pos = O.tree_positions([L], plan.depth[None])[..., None]  # rows rotated at L + depth
    q, kt = O.rope(q, pos), O.rope(kt, pos)
    out, _ = O.tree_attention(q, kt, vt, kpre, vpre, anc)
    Z = O.target_logits(out, f(inp["W_t"]))[0]
    m, path, toks = O.greedy_accept(Z, res["tok"][0], plan.parent, plan.dmax)
    return res, out, m, path, toks, kt


@pytest.mark.parametrize("name", ["tiny", "tiny_medusa"])
def test_two_rounds_through_the_commit(name):
    """Round 2 starts from what round 1's commit hands over: the bonus token
    as root, the last accepted row's hidden state as h, the longer prefix and
    the cache with the committed rows. Float32, against the oracle's own two
    rounds from the inputs alone."""
    from speculative_decoding_hydra_amd import HydraRound

    w = HI.workload(name)
    plan, _ = T.oracle_plan(w.tree)
    inp = HI.generate(w, reserve=2 * (plan.dmax + 1))
    fresh = HI.generate(HI.workload(name, seed=w.seed + 100))  # round 2's tree Q/K/V
    rnd, dev = T.round_inputs(inp)
    T.run_round(rnd, dev)
    shape = dict(rnd.shape, max_prefix_len=int(inp["prefix_len"].max()) + plan.dmax + 1)
    rnd2 = HydraRound(rnd.w, w.tree, shape, hydra=w.hydra, keep_hidden=True)
    q2, kt2, vt2 = (fresh[k].cuda().contiguous() for k in ("q_tree", "k_tree", "v_tree"))
    rnd2.run(rnd.next_h, rnd.next_root_tok, q2, kt2, vt2, dev["k_pages"], dev["v_pages"], dev["block_table"],
             rnd.next_prefix_len)
    torch.cuda.synchronize()

    f = HI.as_f64
    L = int(inp["prefix_len"][0])
    res, out, m, path, toks, kt_rot = _oracle_round(w, inp, plan, f(inp["h"]), inp["root_tok"].numpy(),
                                                    f(inp["q_tree"]), f(inp["k_tree"]), f(inp["v_tree"]),
                                                    [f(inp["k_prefix"][0])], [f(inp["v_prefix"][0])],
                                                    rnd.head_logits, L)
    assert [int(x) for x in rnd.path[0] if x >= 0] == path and int(rnd.n_accepted[0]) == m
    bt = inp["block_table"].numpy()
    pad = lambda a: np.concatenate([a, -np.ones(plan.dmax + 1 - len(a), dtype=np.int64)])[None]  # noqa: E731
    kp, vp, nlen, nroot, nh = O.commit_path(f(inp["k_pages"])[None], f(inp["v_pages"])[None], bt, [L],
                                            kt_rot[None], f(inp["v_tree"])[None], [m], pad(path),
                                            pad(toks), plan.dmax, out.reshape(1, plan.n, -1))
    assert int(rnd.next_prefix_len[0]) == nlen[0] == L + m + 1 and int(rnd.next_root_tok[0]) == nroot[0]
    assert np.max(np.abs(rnd.next_h.cpu().double().numpy() - nh)) <= 1e-4
    ps = int(inp["page_size"])
    gather = lambda pool: np.stack([pool[0, bt[0, p // ps], :, p % ps] for p in range(nlen[0])])  # noqa: E731
    res2, out2, m2, path2, toks2, _ = _oracle_round(w, inp, plan, nh, nroot, f(fresh["q_tree"]),
                                                    f(fresh["k_tree"]), f(fresh["v_tree"]), [gather(kp)],
                                                    [gather(vp)], rnd2.head_logits, int(nlen[0]))
    assert np.array_equal(res2["tok"], rnd2.cand_tok.cpu().numpy())
    assert np.max(np.abs(out2 - rnd2.attn_out.cpu().double().numpy())) <= 1e-4
    assert int(rnd2.n_accepted[0]) == m2
    assert [int(x) for x in rnd2.path[0] if x >= 0] == path2
    assert [int(x) for x in rnd2.out_tok[0] if x >= 0] == toks2
    assert int(rnd2.next_prefix_len[0]) == L + m + 1 + m2 + 1


# ------------------------------------------------------ typical acceptance

def test_tiny_typical_round():
    """Typical acceptance at temperature 0.7 on the tiny workload, then the
    commit of its branch."""
    inp, rnd, dev = _round("tiny", mode="typical", T=0.7)
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


def test_7b_sparse64_typical_round():
    """Typical acceptance on the 7B-shaped round: nearly flat random targets
    put the bar low, so branches several levels deep are accepted."""
    inp, rnd, dev = _round("7b_sparse64", mode="typical", T=1.0)
    rep = T.oracle_round_checks(inp, rnd)
    rep.update(T.check_commit(inp, rnd, dev))
    print(rep, flush=True)


@pytest.mark.parametrize("B,dtype", [(4, "fp32"), (6, "bf16"), (300, "fp32")])
def test_typical_planted_branches(B, dtype):
    """Targets planted on two branches of different depth, with two siblings
    passing at once: the kept branch is the deeper one even where it starts
    at the lower-ranked sibling, and the stage-wise oracle agrees."""
    from speculative_decoding_hydra_amd import tree_accept, tree_accept_workspace_size

    print(f"typical planted B={B} {dtype}", flush=True)
    g = np.random.default_rng(B + 7)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    V, d, Tmp = 1000, 256, 1.0
    w = HI.workload("tiny", mode="typical", T=Tmp)
    plan = O.plan_cartesian([2, 3, 2])
    N = plan.n
    anc = O.ancestors(plan.parent, plan.dmax)
    depth = plan.depth
    W = g.standard_normal((V, d)) * 0.02
    tok = np.zeros((B, N), dtype=np.int32)
    o = g.standard_normal((B, N, d)) * 0.01
    want = []
    for b in range(B):
        for u in range(N):
            kids = plan.children(u)
            tok[b, kids] = g.choice(V, len(kids), replace=False)
        deep = [u for u in range(N) if depth[u] == plan.dmax]
        shallow = [u for u in range(N) if depth[u] == plan.dmax - 1 and plan.children(u)]
        t_deep = int(g.choice(deep))
        t_sh = int(g.choice([u for u in shallow if anc[u][1] != anc[t_deep][1]]))
        plant = {}
        for t in (t_deep, t_sh):
            path = [int(a) for a in anc[t] if a >= 0]
            for a, nx in zip(path[:-1], path[1:]):
                plant.setdefault(a, set()).add(int(tok[b, nx]))
        for a in range(N):
            kids = set(int(tok[b, c]) for c in plan.children(a))
            if a not in plant and kids:  # a peaked target on a token no child carries: every child fails
                plant[a] = {int(g.choice([t for t in range(V) if t not in kids]))}
        for a, xs in plant.items():  # the smallest o giving each planted token a logit of 12
            Wp = W[sorted(xs)]
            o[b, a] = Wp.T @ np.linalg.solve(Wp @ Wp.T, np.full(len(xs), 12.0))
        want.append(t_deep)
    ot = torch.tensor(o, dtype=torch.float32).to(dt).cuda()
    Wt = torch.tensor(W, dtype=torch.float32).to(dt).cuda()
    tk = torch.tensor(tok).cuda()
    par = torch.tensor(np.stack([plan.parent] * B).astype(np.int32)).cuda()
    u_res = torch.rand(B, N, generator=torch.Generator().manual_seed(B)).cuda()
    Z = torch.empty(B, N, V, device="cuda")
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    path_t = torch.empty(B, plan.dmax + 1, dtype=torch.int32, device="cuda")
    out_t = torch.empty_like(path_t)
    ws = torch.empty(tree_accept_workspace_size(2, B, N, V), dtype=torch.uint8, device="cuda")
    tree_accept(ot, Wt, tk, par, Z, n_acc, path_t, out_t, ws, mode=2, temperature=Tmp, u_res=u_res,
                eps=w.eps, delta=w.delta)
    torch.cuda.synchronize()
    Zc, ur = Z.cpu().double().numpy(), u_res.cpu().double().numpy()
    for b in range(B):
        got_p = [int(x) for x in path_t[b] if x >= 0]
        got_o = [int(x) for x in out_t[b] if x >= 0]
        assert int(n_acc[b]) == len(got_p) - 1
        assert got_p[-1] == want[b], f"seq {b}: kept branch ends at {got_p[-1]}, planted {want[b]}"
        T.check_typical(Zc[b], tok[b], plan.parent, ur[b], w, got_p, got_o, f"seq {b}")


# ---------------------------------------------------------- positions / RoPE

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,N,H,D,lens,inplace", [(1, 9, 8, 32, [128], False), (3, 64, 32, 128, [0, 2049, 16384], False),
                                                  (2, 37, 8, 64, [5, 700], True), (1, 1, 1, 2, [3], True)])
def test_tree_rope(dtype, B, N, H, D, lens, inplace):
    """Rotated rows against the oracle at positions prefix_len + depth:
    float32 within 1e-6, bfloat16 within one rounding step of the oracle's
    value rounded to bfloat16."""
    from speculative_decoding_hydra_amd import tree_rope

    print(f"rope {dtype} B={B} N={N} H={H} D={D} L={lens} inplace={inplace}", flush=True)
    g = torch.Generator().manual_seed(B * 100 + N + D)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    x = torch.randn(B, N, H, D, generator=g).to(dt)
    depth = torch.randint(0, 9, (B, N), generator=g, dtype=torch.int32)
    L = torch.tensor(lens, dtype=torch.int32)
    xd = x.cuda()
    out = xd if inplace else torch.full_like(xd, float("nan"))
    tree_rope(xd, depth.cuda(), L.cuda(), out=out)
    torch.cuda.synchronize()
    ref = O.rope(HI.as_f64(x), O.tree_positions(L.numpy(), depth.numpy())[..., None])
    got = out.cpu().double().numpy()
    if dtype == "fp32":
        assert np.max(np.abs(got - ref)) <= 1e-6
    else:
        step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
        assert np.all(np.abs(got - ref) <= step), float(np.max(np.abs(got - ref) / step))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,N,Hq,Hkv,D,lens", [(1, 64, 32, 32, 128, [2048]), (3, 21, 64, 8, 128, [0, 17, 16384]),
                                               (2, 5, 4, 2, 32, [3, 100])])
def test_tree_rope_qk_equals_two_rotations(dtype, B, N, Hq, Hkv, D, lens):
    """The one-launch Q/K rotation gives tree_rope's values bit for bit
    (tree_rope itself is checked against the oracle above), also in place."""
    from speculative_decoding_hydra_amd import tree_rope, tree_rope_qk

    print(f"rope qk {dtype} B={B} N={N} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    g = torch.Generator().manual_seed(B * 7 + N + Hq)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q = torch.randn(B, N, Hq, D, generator=g).to(dt).cuda()
    k = torch.randn(B, N, Hkv, D, generator=g).to(dt).cuda()
    depth = torch.randint(0, 9, (B, N), generator=g, dtype=torch.int32).cuda()
    L = torch.tensor(lens, dtype=torch.int32).cuda()
    qr, kr = torch.full_like(q, float("nan")), torch.full_like(k, float("nan"))
    tree_rope(q, depth, L, out=qr)
    tree_rope(k, depth, L, out=kr)
    qo, ko = torch.full_like(q, float("nan")), torch.full_like(k, float("nan"))
    tree_rope_qk(q, k, depth, L, q_out=qo, k_out=ko)
    torch.cuda.synchronize()
    assert torch.equal(qo, qr) and torch.equal(ko, kr)
    tree_rope_qk(q, k, depth, L)  # in place
    torch.cuda.synchronize()
    assert torch.equal(q, qr) and torch.equal(k, kr)


@pytest.mark.parametrize("over", [dict(), dict(head="sketch", head_hidden=256), dict(cond="path"), dict(cond="attn"),
                                  dict(mode="stochastic", T=0.7), dict(mode="typical")],
                         ids=["folded", "sketch", "path", "attn", "stochastic", "typical"])
def test_round_graph_replays_match_eager(over):
    """The whole round captured in a HIP graph (as bench.py times it) and
    replayed three times, with eager work and synchronisations between the
    replays: every replay reproduces the eager round bit for bit (the kernels
    are deterministic and nothing in the round is a memset or an allocation),
    and the commit writes the same cache contents again."""
    w = HI.workload("7b_sparse64", B=2, d=512, V=3000, Hq=4, Hkv=4, D=128, L=(256,), **over)
    print(f"graph replay {over}", flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp)
    outs = lambda: [t.clone() for t in (rnd.cand_tok, rnd.cand_logp, rnd.head_logits, rnd.head_lse, rnd.tok,  # noqa: E731
                                        rnd.anc, rnd.attn_out, rnd.target_logits, rnd.n_accepted, rnd.path,
                                        rnd.out_tok, rnd.next_prefix_len, rnd.next_root_tok, rnd.next_h)]
    T.run_round(rnd, dev)
    torch.cuda.synchronize()
    ref, kp, vp = outs(), dev["k_pages"].clone(), dev["v_pages"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        T.run_round(rnd, dev)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        T.run_round(rnd, dev)
    for rep in range(3):
        for t in (rnd.cand_tok, rnd.cand_logp, rnd.head_logits, rnd.target_logits, rnd.n_accepted, rnd.out_tok):
            t.fill_(-7)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs())):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager round"
        assert torch.equal(dev["k_pages"], kp) and torch.equal(dev["v_pages"], vp)


# ------------------------------------------------ the target's decoder layer

def _layer_weights(g, d, Hq, Hkv, D, F, dt):
    n = lambda *s: (torch.randn(*s, generator=g) * 0.02).to(dt)  # noqa: E731
    return dict(ln1=(1 + 0.1 * torch.randn(d, generator=g)).to(dt), Wqkv=n((Hq + 2 * Hkv) * D, d), Wo=n(d, Hq * D),
                ln2=(1 + 0.1 * torch.randn(d, generator=g)).to(dt), Wgu=n(2 * F, d), Wd=n(d, F))


def _oracle_weights(w, Hq, Hkv, D, F):
    f = HI.as_f64
    wqkv, wgu = f(w["Wqkv"]), f(w["Wgu"])
    return dict(g1=f(w["ln1"]), g2=f(w["ln2"]), Wq=wqkv[: Hq * D], Wk=wqkv[Hq * D:(Hq + Hkv) * D],
                Wv=wqkv[(Hq + Hkv) * D:], Wo=f(w["Wo"]), Wg=wgu[:F], Wu=wgu[F:], Wd=f(w["Wd"]))


def _close(got, ref, dtype, what, stream=False):
    """float32: 1e-4. bfloat16: 2e-2 plus two rounding steps of the value's
    scale; for the residual stream (stream=True) the scale is at least the
    row's RMS, since x_out is the rounded sum of two rounded operands of that
    size and keeps their rounding errors where they cancel to a small value."""
    if dtype == "fp32":
        e = float(np.max(np.abs(got - ref)))
        assert e <= 1e-4, f"{what}: max-abs {e:.3g}"
        return
    scale = np.abs(ref)
    if stream:
        scale = np.maximum(scale, np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)))
    step = np.ldexp(1.0, np.frexp(np.maximum(scale, 1e-30))[1] - 8)
    bad = np.abs(got - ref) > 2e-2 + 2 * step
    assert not bad.any(), f"{what}: {int(bad.sum())} values off, worst {float(np.max(np.abs(got - ref))):.3g}"


@pytest.mark.parametrize("dtype,B,tree,d,Hq,Hkv,D,F,lens,layers", [
    ("fp32", 2, ("cartesian", [2, 3]), 256, 8, 2, 32, 512, [5, 40], 2),
    ("bf16", 2, ("cartesian", [2, 3]), 256, 8, 2, 32, 512, [5, 40], 2),
    ("bf16", 3, ("cartesian", [3, 2, 2]), 512, 4, 4, 128, 1024, [0, 17, 300], 1),
    ("bf16", 1, ("sparse", (10, 4, 2, 1), 64), 4096, 32, 32, 128, 11008, [2048], 1),
    # head dim 128 at up to 16 and up to 32 rows (one- and two-tile row
    # shapes of the streaming products; GQA in the first)
    ("bf16", 1, ("cartesian", [2, 2]), 512, 4, 2, 128, 1024, [33], 2),
    ("bf16", 2, ("cartesian", [3, 4]), 512, 8, 8, 128, 1024, [64, 1000], 1),
    # 96 and 192 heads' rows in the Q/K/V product (unsplit streaming launch)
    # at 7 and 32 rows (GQA), and head dim 64 with K = 256
    ("bf16", 1, ("cartesian", [2, 2]), 512, 32, 16, 128, 1024, [33], 1),
    ("bf16", 2, ("cartesian", [3, 4]), 512, 32, 16, 128, 1024, [64, 1000], 2),
    ("bf16", 1, ("cartesian", [2, 3]), 256, 64, 64, 64, 512, [40], 1),
    # 73 rows at the 7B width: tiled split products with eight partials, so
    # the norms and the residual sum eight; and the 70B width at 7 rows
    ("bf16", 1, ("cartesian", [8, 8]), 4096, 32, 32, 128, 11008, [64], 1),
    ("bf16", 1, ("cartesian", [2, 2]), 8192, 8, 8, 128, 512, [40], 1),
])
def test_tree_decoder_layer(dtype, B, tree, d, Hq, Hkv, D, F, lens, layers):
    """Decoder layers over the tree rows (each with its own weights and paged
    prefix, the second reading the first's output) against the oracle's;
    also the rotated keys and values each layer hands to the commit."""
    from speculative_decoding_hydra_amd import tree_decoder_layer, tree_decoder_layer_workspace_size

    print(f"decoder layer {dtype} B={B} tree={tree} d={d} Hq={Hq} Hkv={Hkv} D={D} F={F} L={lens} x{layers}",
          flush=True)
    plan = T.oracle_plan(tree)[0]
    N = plan.n
    g = torch.Generator().manual_seed(d + N + B)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    anc = np.stack([O.ancestors(plan.parent, plan.dmax)] * B).astype(np.int32)
    depth = np.stack([plan.depth] * B).astype(np.int32)
    x = torch.randn(B, N, d, generator=g).to(dt)
    dev = lambda t: (torch.from_numpy(t) if isinstance(t, np.ndarray) else t).cuda().contiguous()  # noqa: E731
    xs_dev, xs_ref = dev(x), HI.as_f64(x)
    for layer in range(layers):
        w = _layer_weights(g, d, Hq, Hkv, D, F, dt)
        c = _attn_case(B, N, Hq, Hkv, D, lens, dtype, seed=100 * layer + d, tree=plan.parent)
        out = torch.empty(B, N, d, dtype=dt, device="cuda")
        kt = torch.empty(B, N, Hkv, D, dtype=dt, device="cuda")
        vt = torch.empty_like(kt)
        code = 0 if dtype == "fp32" else 1
        ws = torch.empty(tree_decoder_layer_workspace_size(code, B, N, d, Hq, Hkv, D, F, max(lens)),
                         dtype=torch.uint8, device="cuda")
        tree_decoder_layer(xs_dev, {k: dev(v) for k, v in w.items()}, Hq, Hkv, dev(c["kpool"]), dev(c["vpool"]),
                           dev(c["bt"]), dev(c["lens"]), max(lens), dev(anc), dev(depth), out, kt, vt, ws)
        torch.cuda.synchronize()
        ref, rk, rv = O.decoder_layer(xs_ref, _oracle_weights(w, Hq, Hkv, D, F), [HI.as_f64(t) for t in c["kp"]],
                                      [HI.as_f64(t) for t in c["vp"]], anc, depth, lens, Hq, Hkv, D, 1e-6,
                                      bf16=dtype == "bf16")
        _close(kt.cpu().double().numpy(), rk, dtype, f"layer {layer} keys")
        _close(vt.cpu().double().numpy(), rv, dtype, f"layer {layer} values")
        _close(out.cpu().double().numpy(), ref, dtype, f"layer {layer} output", stream=True)
        xs_dev, xs_ref = out, ref  # each side's next layer reads its own output


@pytest.mark.parametrize("B,tree,d,Hq,Hkv,D,F,lens", [
    (3, ("cartesian", [3, 2, 2]), 512, 4, 4, 128, 1024, [0, 17, 300]),
    (1, ("sparse", (10, 4, 2, 1), 64), 4096, 32, 32, 128, 11008, [2048]),
    (2, ("cartesian", [10, 4, 2]), 256, 8, 2, 32, 512, [5, 40]),  # 2 x 131 rows: the tiled split products
])
def test_tree_decoder_layer_packed_weights_match_row_major(B, tree, d, Hq, Hkv, D, F, lens):
    """The layer with its four weight matrices packed (HYDRA_LAYER_PACKED)
    gives bit for bit the outputs of the row-major weights: same values,
    same kernels, same K order."""
    from speculative_decoding_hydra_amd import (hydra_pack_weight, tree_decoder_layer,
                                                tree_decoder_layer_workspace_size)

    print(f"decoder layer packed B={B} tree={tree} d={d} F={F}", flush=True)
    plan = T.oracle_plan(tree)[0]
    N = plan.n
    g = torch.Generator().manual_seed(d + N + B + 1)
    dt = torch.bfloat16
    anc = torch.from_numpy(np.stack([O.ancestors(plan.parent, plan.dmax)] * B).astype(np.int32)).cuda()
    depth = torch.from_numpy(np.stack([plan.depth] * B).astype(np.int32)).cuda()
    x = torch.randn(B, N, d, generator=g).to(dt).cuda()
    w = {k: v.cuda() for k, v in _layer_weights(g, d, Hq, Hkv, D, F, dt).items()}
    wp = dict(w, **{k: hydra_pack_weight(w[k]) for k in ("Wqkv", "Wo", "Wgu", "Wd")})
    c = _attn_case(B, N, Hq, Hkv, D, lens, "bf16", seed=d + 7, tree=plan.parent)
    dev = lambda t: (torch.from_numpy(t) if isinstance(t, np.ndarray) else t).cuda().contiguous()  # noqa: E731
    ws = torch.empty(tree_decoder_layer_workspace_size(1, B, N, d, Hq, Hkv, D, F, max(lens)), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for weights in (w, wp):
        out = torch.empty(B, N, d, dtype=dt, device="cuda")
        kt = torch.empty(B, N, Hkv, D, dtype=dt, device="cuda")
        vt = torch.empty_like(kt)
        tree_decoder_layer(x, weights, Hq, Hkv, dev(c["kpool"]), dev(c["vpool"]), dev(c["bt"]), dev(c["lens"]),
                           max(lens), anc, depth, out, kt, vt, ws)
        torch.cuda.synchronize()
        outs.append((out.cpu(), kt.cpu(), vt.cpu()))
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("name,over", [("tiny_layers", {}), ("tiny_layers", {"dtype": "bf16"}),
                                       ("tiny_layers", {"mode": "stochastic", "T": 0.8, "layers": 2}),
                                       ("7b_layers", {"layers": 2})])
def test_round_through_the_target_layers(name, over):
    """A whole round whose verification runs the target's decoder layers over
    the tree tokens (tree_verify_layers): the device's final hidden states and
    every layer's rotated K/V against the oracle's chain of layers on the
    device's tree, acceptance on those hidden states, and the commit of every
    layer's K/V of the kept branch (bit-exact)."""
    w = HI.workload(name, **over)
    print(f"round through the target's layers {w.name} {w.dtype} layers={w.layers} B={w.B} mode={w.mode}",
          flush=True)
    inp = HI.generate(w)
    rnd, dev = T.round_inputs(inp, device="cuda")
    T.run_round(rnd, dev)
    torch.cuda.synchronize()
    seqs = [0] if w.d >= 4096 else None
    rep = T.oracle_round_checks(inp, rnd, seqs=seqs, rows=[0, 1] if seqs else None)
    rep.update(T.check_commit(inp, rnd, dev, seqs=seqs))
    print("  ", {k: v for k, v in rep.items() if not isinstance(v, list)}, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tree_attention_prefix_beyond_the_plan(dtype):
    """max_prefix_len only sizes the split plan: prefixes longer than it (a
    round object reused after its commit grew the cache) are attended in
    full, on both paths."""
    from speculative_decoding_hydra_amd import tree_attention_verify, tree_attention_verify_workspace_size

    B, N, Hq, Hkv, D, lens = 2, 64, 8, 2, (128 if dtype == "bf16" else 64), [2100, 700]
    print(f"attention beyond the plan {dtype} lens={lens} planned 600", flush=True)
    c = _attn_case(B, N, Hq, Hkv, D, lens, dtype, seed=99)
    dev = lambda t: t.cuda().contiguous()  # noqa: E731
    out = torch.full((B, N, Hq, D), float("nan"), dtype=c["dt"], device="cuda")
    lse = torch.empty(B, N, Hq, device="cuda")
    code = 0 if dtype == "fp32" else 1
    ws = torch.empty(max(1, tree_attention_verify_workspace_size(code, B, N, Hq, Hkv, D, 600)), dtype=torch.uint8,
                     device="cuda")
    tree_attention_verify(dev(c["q"]), dev(c["kt"]), dev(c["vt"]), dev(c["kpool"]), dev(c["vpool"]), dev(c["bt"]),
                          dev(c["lens"]), 600, dev(torch.from_numpy(c["anc"])), dev(torch.from_numpy(c["dep"])),
                          out, lse, ws)
    torch.cuda.synchronize()
    f = HI.as_f64
    ref, ref_lse = O.tree_attention(f(c["q"]), f(c["kt"]), f(c["vt"]), [f(x) for x in c["kp"]],
                                    [f(x) for x in c["vp"]], c["anc"], bf16=dtype == "bf16")
    t = 1e-4 if dtype == "fp32" else 2e-2
    assert float(np.max(np.abs(out.cpu().double().numpy() - ref))) <= t
    assert float(np.max(np.abs(lse.cpu().double().numpy() - ref_lse))) <= t
