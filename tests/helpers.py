"""Shared pieces of the GPU parity tests and the smoke check.

Parity is stage-wise: each oracle stage is fed the device's upstream outputs
(parent tokens, hidden states, tree, attention output), so that one
near-tie at depth 1 cannot cascade, and the float and integer results of
every stage are compared with the oracle on the same inputs:

* head hidden state u: oracle from the device's parent tokens; in bf16 mode
  at most one bf16 rounding step (or 1e-3 where h + SiLU(a) cancels to near
  zero) apart per element, differing on at most 1% of them;
* head logits z and log-sum-exp: oracle projection of the device's u;
* top-k tokens: bit-exact, except where the oracle's margin between
  consecutive sorted logits is below 1e-4, where the decision is recomputed
  on the CPU from the device's logits;
* tree: oracle prune / ancestors from the device's cumulative scores;
* attention output: oracle from the device's ancestor table;
* target logits: oracle projection of the device's attention output;
* target arg max of every row: the device's equals the oracle's, except
  where the oracle's top-1 margin is below 1e-4 (recomputed from the device
  logits);
* acceptance: oracle walk on the device's logits (greedy: and on the
  oracle's own logits, unless a visited row was recomputed).

Tolerances (max-abs): 1e-4 in float32 mode and 2e-2 for bfloat16 inputs
with float32 accumulation.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import hydra_inputs as HI
from oracle import hydra_oracle as O

MARGIN = 1e-4
# Rejection walk: a device decision may differ from the float64 oracle only
# when the oracle's own decision is that close to its boundary (relative):
# the accept test u q(x) < r(x), or the cumulative mass at the drawn token.
# float32 probabilities carry ~1e-7 relative error each, so these bounds leave
# two orders of magnitude of room.
ACCEPT_EPS = 1e-5
SAMPLE_EPS = 1e-5


def tol(w):
    return 1e-4 if w.dtype == "fp32" else 2e-2


def oracle_plan(tree):
    kind = tree[0]
    if kind == "cartesian":
        return O.plan_cartesian(tree[1]), None
    if kind == "sparse":
        return O.plan_sparse_template(tree[1], tree[2]), None
    return O.plan_cartesian(tree[1]), tree[2]


def round_inputs(inp, device="cuda", keep_hidden=True, fold_embedding=None, residual=True, pack_vocab=None):
    from speculative_decoding_hydra_amd import round_from_inputs

    return round_from_inputs(inp, device=device, keep_hidden=keep_hidden, fold_embedding=fold_embedding,
                             residual=residual, pack_vocab=pack_vocab)


def run_round(rnd, dev, stream=None):
    from speculative_decoding_hydra_amd import run_round as _run

    _run(rnd, dev, stream)


def np_(t):
    return t.detach().cpu().to(torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def check_topk(z_oracle, z_dev, k, got_ids, where):
    """Top-k decision of one row: bit-exact unless the oracle margin < 1e-4."""
    mine = O.topk_sorted(z_oracle, k)
    if np.array_equal(mine, got_ids):
        return False
    margin = O.topk_margin(z_oracle, k)
    assert margin < MARGIN, f"{where}: top-{k} {list(got_ids)} != oracle {list(mine)} (margin {margin:.3g})"
    recomputed = O.topk_sorted(z_dev, k)
    assert np.array_equal(recomputed, got_ids), f"{where}: top-{k} differs from the CPU on the device logits"
    return True


def sketch_u_slack(x, head):
    """Extra per-element slack on a bf16 two-layer head's u beyond its own
    rounding. The SiLU output a is rounded to bf16 before the LayerNorm (head
    1) or the second product: where the float32 sum (device) and the float64
    sum (oracle) of Wa x straddle a rounding midpoint, a_i differs by one bf16
    step, and u_j moves by rstd * |g_j| times that step (head 1) or times
    sum_i |Wb_ji| step_i over those i (later heads). The float32 error of a
    K-term sum is taken as 4 sqrt(K) 2^-24 sum |terms| (a random-walk bound)."""
    Wa, ba = head["Wa"], head["ba"]
    pre = Wa @ x + ba
    a = O.silu(pre)
    err = 4.0 * math.sqrt(x.size) * 2.0 ** -24 * (np.abs(Wa) @ np.abs(x) + np.abs(ba)) * 1.1  # |SiLU'| < 1.1
    ar = O.round_bf16(a)
    step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(a), 1e-30))[1] - 8)
    near = np.abs(np.abs(a - ar) - step / 2) <= err
    shift = np.where(near, step, 0.0)
    v = ar
    if "Wb" in head:
        shift = np.abs(head["Wb"]) @ shift
        v = head["Wb"] @ ar + head["bb"]
    rstd = 1.0 / math.sqrt(np.var(v) + 1e-5)
    return rstd * np.abs(head["ln_g"]) * shift


def _bf16_step(v):
    return np.ldexp(1.0, np.frexp(np.maximum(np.abs(v), 1e-30))[1] - 8)


def attn_u_slack(X, attn, W1):
    """Extra slack on a bf16 Hydra++ head's u. The attention output a and
    c = x + Wo a are rounded before use, so a one-step flip of a_l (where
    device and oracle fall on two sides of a rounding midpoint) moves c_i by
    Wo_il step_l, and a flip of c_i moves W1's sum by W1_ji step_i. A value
    perturbed with standard deviation sigma, at a uniform place in its
    rounding cell, flips with probability about 0.8 sigma / step; flips are
    independent with random signs, so each stage's perturbation has variance
    sum (weight * step)^2 * P(flip), and the slack is four standard
    deviations of W1's sum (times 1.1 >= |SiLU'|). The float32 error of a
    K-term sum has standard deviation about 2^-24 sqrt(K / 2) sqrt(sum terms^2)."""
    X = np.asarray(X)
    d = X.shape[1]
    u32 = 2.0 ** -24 * math.sqrt(d / 2)
    q, K, Vv = attn["Wq"] @ X[-1], X @ attn["Wk"].T, X @ attn["Wv"].T
    sc = K @ q / math.sqrt(d)
    p = np.exp(sc - sc.max())
    p /= p.sum()
    a = p @ Vv
    sd_a = u32 * np.sqrt((attn["Wv"] ** 2) @ (X ** 2).max(axis=0))
    step_a = _bf16_step(a)
    pf_a = np.minimum(1.0, 0.8 * sd_a / step_a)
    ar = O.round_bf16(a)
    c = X[-1] + attn["Wo"] @ ar
    var_c = (attn["Wo"] ** 2) @ (step_a ** 2 * pf_a) + (u32 ** 2) * ((attn["Wo"] ** 2) @ (ar ** 2))
    step_c = _bf16_step(c)
    pf_c = np.minimum(1.0, 0.8 * np.sqrt(var_c) / step_c)
    return 1.1 * 4.0 * np.sqrt((W1[:, d:] ** 2) @ (step_c ** 2 * pf_c))


def oracle_attn(inp):
    """The Hydra++ fusion weights of an input dict, as the oracle takes them."""
    Wqkv = HI.as_f64(inp["attn"]["Wqkv"])
    d = Wqkv.shape[1]
    return {"Wq": Wqkv[:d], "Wk": Wqkv[d:2 * d], "Wv": Wqkv[2 * d:], "Wo": HI.as_f64(inp["attn"]["Wo"])}


def check_draft(inp, rnd, seqs=None, rows=None):
    """Stage 1, stage-wise. Returns max errors."""
    w = inp["workload"]
    t = tol(w)
    bf16 = w.dtype == "bf16"
    plan, _ = oracle_plan(w.tree)
    dp = rnd.dplan
    assert np.array_equal(plan.parent, dp.plan.parent) and np.array_equal(plan.rank, dp.plan.rank)
    row_node, row_depth, node_row = O.head_rows(plan, w.hydra)
    assert np.array_equal(node_row, dp.rows.node_row)
    if w.hydra:
        assert np.array_equal(row_node, dp.rows.row_node)
    kmax = {}
    for c in range(1, plan.n):
        r = node_row[plan.parent[c]]
        kmax[r] = max(kmax.get(r, 0), int(plan.rank[c]) + 1)
    logits = np_(rnd.head_logits)
    lse = np_(rnd.head_lse)
    hidden = np_(rnd.head_hidden)
    ctok = np_(rnd.cand_tok)
    clogp = np_(rnd.cand_logp)
    h = HI.as_f64(inp["h"])
    seqs = range(w.B) if seqs is None else seqs
    rows = range(len(row_node)) if rows is None else rows
    err = dict(u=0.0, z=0.0, lse=0.0, logp=0.0, flips=0)
    sketch = getattr(w, "head", "mlp") == "sketch"
    attn_w = oracle_attn(inp) if getattr(w, "cond", "parent") == "attn" else None
    W1c, W2c = {}, {}
    for r in rows:
        k = int(row_depth[r])
        if k not in W1c:
            if sketch:
                W1c[k] = {n: HI.as_f64(t) for n, t in inp["heads"][k - 1].items()}
                W2c[k] = W1c[k]["W2"]
            else:
                W1c[k] = HI.as_f64(inp["W1"][k - 1])
                W2c[k] = HI.as_f64(inp["W2"][k - 1])
        W1, W2 = W1c[k], W2c[k]
        b1 = None if sketch else HI.as_f64(inp["b1"][k - 1])
        for b in seqs:
            e = None
            if w.hydra:
                p = int(row_node[r])
                if getattr(w, "cond", "parent") == "attn":
                    toks = O.path_tokens(plan, ctok[b], int(inp["root_tok"][b]), p)
                    e = O.path_attention(np.stack([HI.as_f64(inp["E"][t]) for t in toks]), attn_w, bf16)
                elif getattr(w, "cond", "parent") == "path":
                    toks = O.path_tokens(plan, ctok[b], int(inp["root_tok"][b]), p)
                    e = np.concatenate([HI.as_f64(inp["E"][t]) for t in toks])
                else:
                    ptok = int(inp["root_tok"][b]) if p == 0 else int(ctok[b, p])
                    e = HI.as_f64(inp["E"][ptok])
            if sketch:
                u = O.sketch_hidden(h[b], e if k > 1 else None, W1, bf16)
            else:
                u = O.head_hidden(h[b], e, W1, b1, rnd.residual, bf16)
            if bf16:
                # u is stored in bf16: a float32-vs-float64 difference in a can
                # flip one rounding, so compare in units of the bf16 step
                # (plus an absolute 1e-3 where h + SiLU(a) cancels to near zero)
                ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(u), 1e-30))[1] - 8)
                diff = np.abs(u - hidden[b, r])
                lim = np.maximum(ulp, 1e-3)
                if sketch:
                    x = h[b] if k == 1 else np.concatenate([h[b], e])
                    lim = lim + sketch_u_slack(x, W1)
                elif attn_w is not None:
                    extra = attn_u_slack(np.stack([HI.as_f64(inp["E"][t]) for t in toks]), attn_w, W1)
                    lim = lim + extra
                    # expected flips of u under the same model (sigma = extra / 4.4)
                    err["u_flips_model"] = err.get("u_flips_model", 0.0) + float(
                        np.sum(np.minimum(1.0, 0.8 * (extra / 4.4) / ulp)))
                bad = diff > lim
                j = int(np.argmax(diff / lim))
                assert not bad.any(), (f"seq {b} row {r}: u[{j}] = {hidden[b, r][j]!r} vs oracle {u[j]!r} "
                                       f"(bf16 step {ulp[j]:.3g})")
                err["u_flips"] = err.get("u_flips", 0) + int(np.sum(diff > 0))
                err["u_elems"] = err.get("u_elems", 0) + u.size
            else:
                err["u"] = max(err["u"], float(np.max(np.abs(u - hidden[b, r]))))
            z = O.head_logits(hidden[b, r], W2)
            err["z"] = max(err["z"], float(np.max(np.abs(z - logits[b, r]))))
            err["lse"] = max(err["lse"], abs(O.logsumexp(z) - lse[b, r]))
            kids = [c for c in range(1, plan.n) if node_row[plan.parent[c]] == r]
            # every parent served by the row takes a prefix of the row's list
            lists = [[int(ctok[b, c]) for c in sorted(plan.children(p), key=lambda c: plan.rank[c])]
                     for p in range(plan.n) if node_row[p] == r]
            ids = np.array(max(lists, key=len))
            assert len(ids) == kmax[r]
            for lst in lists:
                assert lst == list(ids[: len(lst)]), f"seq {b} row {r}: parents disagree"
            err["flips"] += check_topk(z, logits[b, r], kmax[r], ids, f"seq {b} row {r}")
            # device decision equals the CPU's on the device logits, always
            assert np.array_equal(O.topk_sorted(logits[b, r], kmax[r]), ids), f"seq {b} row {r}: top-k"
            for c in kids:
                ref = clogp[b, plan.parent[c]] + logits[b, r, ctok[b, c]] - O.logsumexp(logits[b, r])
                err["logp"] = max(err["logp"], abs(ref - clogp[b, c]))
    assert err["u"] <= t, f"head hidden max-abs {err['u']:.3g} > {t}"
    if bf16:
        # two-layer heads round twice: a flip in the SiLU output moves Wb a by
        # ~1e-4 relative, enough to move about 1 in 40 of that row's u across
        # a bf16 rounding boundary (one step, which the check above bounds)
        # (Hydra++ fusion rounds a and c first: the same effect through W1)
        # Hydra++: at d = 8192 the flips of c flip several percent of u; allow
        # twice the model's expectation on top of the one-layer 1%
        model = min(2 * err.get("u_flips_model", 0.0), 0.15 * err["u_elems"])
        allowed = 0.05 * err["u_elems"] if sketch else 0.01 * err["u_elems"] + model
        assert err["u_flips"] <= allowed, f"{err['u_flips']} rounding flips in u (allowed {allowed:.0f})"
    assert err["z"] <= t, f"head logits max-abs {err['z']:.3g} > {t}"
    assert err["lse"] <= t and err["logp"] <= t, (err["lse"], err["logp"])
    for b in seqs:
        assert ctok[b, 0] == int(inp["root_tok"][b]) and clogp[b, 0] == 0.0
    return err


def check_build(inp, rnd, seqs=None):
    w = inp["workload"]
    plan, n_keep = oracle_plan(w.tree)
    ctok, clogp = np_(rnd.cand_tok), np_(rnd.cand_logp)
    tok, par, dep = np_(rnd.tok), np_(rnd.parent), np_(rnd.depth)
    anc, qrow, src = np_(rnd.anc), np_(rnd.q_row), np_(rnd.src)
    _, _, node_row = O.head_rows(plan, w.hydra)
    seqs = range(w.B) if seqs is None else seqs
    for b in seqs:
        if n_keep is None:
            kept, s = plan, np.arange(plan.n)
        else:
            kept, s = O.prune_tree(plan, clogp[b], n_keep)
        assert np.array_equal(src[b], s), f"seq {b}: kept set / order"
        assert np.array_equal(par[b], kept.parent) and np.array_equal(dep[b], kept.depth)
        assert np.array_equal(tok[b], ctok[b][s])
        assert np.array_equal(anc[b], O.ancestors(kept.parent, plan.dmax))
        assert np.array_equal(qrow[b], node_row[s])


def close_stream(got, ref, dtype, what, layers=1):
    """float32: 1e-4 per layer. bfloat16: per layer 2e-2 plus two rounding
    steps of the value's scale, the scale at least the row's RMS: every
    layer rounds its stored tensors once more and hands what it inherited on
    through the residual sum, so the bound grows with the number of layers
    the value went through."""
    if dtype == "fp32":
        e = float(np.max(np.abs(got - ref)))
        assert e <= 1e-4 * layers, f"{what}: max-abs {e:.3g}"
        return e
    scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)))
    step = np.ldexp(1.0, np.frexp(np.maximum(scale, 1e-30))[1] - 8)
    bad = np.abs(got - ref) > layers * (2e-2 + 2 * step)
    assert not bad.any(), f"{what}: {int(bad.sum())} values off, worst {float(np.max(np.abs(got - ref))):.3g}"
    return float(np.max(np.abs(got - ref)))


def target_layers_f64(inp):
    """The oracle's per-layer weight dicts from the layer-stacked inputs."""
    w, t, f = inp["workload"], inp["target"], HI.as_f64
    qd, kd, F = w.Hq * w.D, w.Hkv * w.D, w.ffn
    out = []
    for layer in range(w.layers):
        wqkv, wgu = f(t["Wqkv"][layer]), f(t["Wgu"][layer])
        out.append(dict(g1=f(t["ln1"][layer]), g2=f(t["ln2"][layer]), Wq=wqkv[:qd], Wk=wqkv[qd:qd + kd],
                        Wv=wqkv[qd + kd:], Wo=f(t["Wo"][layer]), Wg=wgu[:F], Wu=wgu[F:], Wd=f(t["Wd"][layer])))
    return out


def check_verify(inp, rnd, seqs=None):
    """The target's forward pass over the device's tree (its tokens, ancestor
    table and depths) against the oracle's: embeddings, the chain of decoder
    layers over each layer's prefix, final norm; every layer's rotated K/V."""
    w = inp["workload"]
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    f = HI.as_f64
    kp = [[f(inp["k_prefix_layers"][layer][b]) for b in seqs] for layer in range(w.layers)]
    vp = [[f(inp["v_prefix_layers"][layer][b]) for b in seqs] for layer in range(w.layers)]
    h, k, v = O.verify_layers(np_(rnd.tok)[seqs], f(inp["E"]), target_layers_f64(inp), f(inp["ln_f"]), kp, vp,
                              np_(rnd.anc)[seqs], np_(rnd.depth)[seqs], inp["prefix_len"].numpy()[seqs], w.Hq, w.Hkv,
                              w.D, 1e-6, theta=rnd.rope_theta or 10000.0, bf16=w.dtype == "bf16")
    rep = {}
    for layer in range(w.layers):
        rep[f"k{layer}"] = close_stream(np_(rnd.k_layers[layer])[seqs], k[layer], w.dtype, f"layer {layer} keys",
                                        layer + 1)
        rep[f"v{layer}"] = close_stream(np_(rnd.v_layers[layer])[seqs], v[layer], w.dtype, f"layer {layer} values",
                                        layer + 1)
    rep["h"] = close_stream(np_(rnd.hidden)[seqs], h, w.dtype, "final hidden states", w.layers)
    return rep


def check_attention(inp, rnd, seqs=None):
    if rnd.target is not None:
        return check_verify(inp, rnd, seqs)
    w = inp["workload"]
    t = tol(w)
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    anc = np_(rnd.anc)[seqs]
    sub = lambda x: HI.as_f64(x[seqs])  # noqa: E731
    kp = [HI.as_f64(inp["k_prefix"][b]) for b in seqs]
    vp = [HI.as_f64(inp["v_prefix"][b]) for b in seqs]
    q, k = sub(inp["q_tree"]), sub(inp["k_tree"])
    if rnd.rope_theta:  # rows rotated at prefix_len + depth (the device's tree)
        pos = O.tree_positions(inp["prefix_len"].numpy()[seqs], np_(rnd.depth)[seqs])[..., None]
        q, k = O.rope(q, pos, rnd.rope_theta), O.rope(k, pos, rnd.rope_theta)
        t_rot = 1e-6 if w.dtype == "fp32" else 2e-2
        for name, mine, dev_rot in (("q", q, rnd.q_rot), ("k", k, rnd.k_rot)):
            e = float(np.max(np.abs(mine - np_(dev_rot)[seqs])))
            assert e <= t_rot, f"rotated {name} max-abs {e:.3g}"
    out, lse = O.tree_attention(q, k, sub(inp["v_tree"]), kp, vp, anc, bf16=w.dtype == "bf16")
    got = np_(rnd.attn_out)[seqs]
    e_o = float(np.max(np.abs(out - got)))
    e_l = float(np.max(np.abs(lse - np_(rnd.attn_lse)[seqs])))
    assert e_o <= t, f"attention output max-abs {e_o:.3g} > {t}"
    assert e_l <= t, f"attention lse max-abs {e_l:.3g} > {t}"
    return dict(o=e_o, lse=e_l)


def check_accept(inp, rnd, seqs=None):
    w = inp["workload"]
    t = tol(w)
    seqs = range(w.B) if seqs is None else seqs
    O_dev = np_(rnd.rows())
    Z_dev = np_(rnd.target_logits)
    Wt = HI.as_f64(inp["W_t"])
    tok, par, qrow = np_(rnd.tok), np_(rnd.parent), np_(rnd.q_row)
    n_acc, path, out = np_(rnd.n_accepted), np_(rnd.path), np_(rnd.out_tok)
    Dm = rnd.dplan.dmax
    e_z = 0.0
    amb = 0
    recomputed = 0
    for b in seqs:
        Z = O.target_logits(O_dev[b: b + 1], Wt)[0]
        e_z = max(e_z, float(np.max(np.abs(Z - Z_dev[b]))))
        # every row's arg max: the device's (over its own logits, as its walk
        # takes it) equals the oracle's unless the oracle's top-1 margin is
        # below 1e-4, where the decision is recomputed from the device logits
        for u in range(Z.shape[0]):
            mine, dev_y = O.argmax_lowest(Z[u]), O.argmax_lowest(Z_dev[b, u])
            if mine != dev_y:
                margin = O.topk_margin(Z[u], 1)
                assert margin < MARGIN, (f"seq {b} row {u}: device arg max {dev_y} != oracle {mine} "
                                         f"(margin {margin:.3g})")
                recomputed += 1
        got_p = [int(x) for x in path[b] if x >= 0]
        got_o = [int(x) for x in out[b] if x >= 0]
        assert n_acc[b] == len(got_p) - 1 and len(got_o) == len(got_p)
        if w.mode == "greedy":
            m, p, o = O.greedy_accept(Z_dev[b], tok[b], par[b], Dm)
            assert n_acc[b] == m and got_p == p and got_o == o, f"seq {b}: greedy walk {got_p}/{got_o} vs {p}/{o}"
            # and on the oracle's own logits, the same walk unless a row it
            # visits was recomputed above
            m2, p2, o2 = O.greedy_accept(Z, tok[b], par[b], Dm)
            if (p2, o2) != (p, o):
                near = [u for u in set(p) | set(p2) if O.topk_margin(Z[u], 1) < MARGIN]
                assert near, f"seq {b}: walk on the oracle's logits {p2}/{o2} vs device {p}/{o}"
        elif w.mode == "typical":
            amb += check_typical(Z_dev[b], tok[b], par[b], np_(inp["u_res"])[b], w, got_p, got_o, f"seq {b}")
        else:
            # the oracle follows the device's decisions and reports its own;
            # they may differ only within float32 rounding of the boundary
            hz = np_(rnd.head_logits)[b]
            trace = []
            m, p, o = O.rejection_accept(Z_dev[b], hz, qrow[b], tok[b], par[b], np_(inp["u_acc"])[b],
                                         np_(inp["u_res"])[b], w.T, follow=(got_p, got_o), trace=trace)
            assert p == got_p and o == got_o
            for kind, own, taken, margin in trace:
                if own != taken:
                    amb += 1
                    bound = ACCEPT_EPS if kind == "accept" else SAMPLE_EPS
                    assert margin < bound, f"seq {b}: {kind} decision {taken} vs oracle {own} (margin {margin:.3g})"
    assert e_z <= t, f"target logits max-abs {e_z:.3g} > {t}"
    return dict(z=e_z, ambiguous=amb, argmax_recomputed=recomputed)


def check_typical(Z, tok, parent, u_res, w, got_p, got_o, where):
    """Typical acceptance of one sequence on the device's target logits. A
    pass decision within ACCEPT_EPS (relative) of its bar may go either way:
    the device's branch must be the kept branch of one such choice, and its
    last token the oracle's draw at that branch's end (or within SAMPLE_EPS
    of a cumulative boundary). Returns the number of ambiguous decisions."""
    import itertools

    passes, margin = O.typical_passes(Z, tok, parent, w.T, w.eps, w.delta)
    amb = [int(c) for c in np.flatnonzero(margin < ACCEPT_EPS)]
    ends = set()
    for choice in itertools.product([False, True], repeat=len(amb)):
        f = passes.copy()
        f[amb] = choice
        ends.add(O.kept_branch(f, parent))
    end = got_p[-1]
    assert end in ends, f"{where}: typical branch ends at {end}, oracle {sorted(ends)} (ambiguous {amb})"
    chain = [end]
    while parent[chain[-1]] >= 0:
        chain.append(int(parent[chain[-1]]))
    assert got_p == chain[::-1], f"{where}: path {got_p} is not the root path of {end}"
    assert got_o[:-1] == [int(tok[c]) for c in got_p[1:]], f"{where}: accepted tokens"
    r = O.softmax(np.asarray(Z[end], dtype=np.float64) / w.T)
    x = O.sample_inverse_cdf(r, u_res[end])
    if got_o[-1] != x:
        assert ambiguous_sample(r, u_res[end], SAMPLE_EPS), f"{where}: drawn {got_o[-1]} vs oracle {x}"
        return len(amb) + 1
    return len(amb)


def oracle_round_checks(inp, rnd, seqs=None, rows=None):
    rep = {}
    for k, v in check_draft(inp, rnd, seqs, rows).items():
        rep["draft_" + k] = v
    check_build(inp, rnd, seqs)
    for k, v in check_attention(inp, rnd, seqs).items():
        rep["attn_" + k] = v
    for k, v in check_accept(inp, rnd, seqs).items():
        rep["accept_" + k] = v
    return rep


def ambiguous_sample(r, u, eps=1e-6):
    """True if u * sum(r) lies within eps * sum(r) of a cumulative boundary."""
    c = np.cumsum(np.asarray(r, dtype=np.float64))
    thr = u * c[-1]
    return float(np.min(np.abs(c - thr))) < eps * c[-1] or math.isclose(thr, 0.0)


def check_commit(inp, rnd, dev, seqs=None):
    """Commit after the round, stage-wise: the oracle commits the device's
    accepted branches (sub-pools of the sampled sequences, bit-exact); on the
    whole pool, nothing but the committed positions differs from the input."""
    w = inp["workload"]
    seqs = range(w.B) if seqs is None else seqs
    n_acc, path, out = np_(rnd.n_accepted), np_(rnd.path), np_(rnd.out_tok)
    Dm = rnd.dplan.dmax
    lens = inp["prefix_len"].numpy()
    bt = inp["block_table"].numpy()
    ps = int(inp["page_size"])
    nlen, nroot, nh = np_(rnd.next_prefix_len), np_(rnd.next_root_tok), rnd.next_h
    hid = rnd.rows()
    layered = rnd.target is not None  # pools and tree K/V stacked over the target's layers
    for b in seqs:
        pages = [int(p) for p in bt[b] if p >= 0]
        sub_bt = np.arange(len(pages))[None]
        if layered:
            sub = lambda pool: HI.as_f64(pool[:, pages])  # noqa: E731
            ksrc, vsrc = np_(rnd.k_layers[:, b:b + 1]), np_(rnd.v_layers[:, b:b + 1])
        else:
            sub = lambda pool: HI.as_f64(pool[pages])[None]  # noqa: E731
            ksrc = np_((rnd.k_rot if rnd.rope_theta else inp["k_tree"])[b:b + 1])[None]  # the keys committed
            vsrc = HI.as_f64(inp["v_tree"][b:b + 1])[None]
        rk, rv, rl, rr, _ = O.commit_path(sub(inp["k_pages"]), sub(inp["v_pages"]), sub_bt, lens[b:b + 1], ksrc,
                                          vsrc, n_acc[b:b + 1], path[b:b + 1], out[b:b + 1], Dm)
        got_k = np_(dev["k_pages"][:, pages]) if layered else np_(dev["k_pages"][pages])[None]
        got_v = np_(dev["v_pages"][:, pages]) if layered else np_(dev["v_pages"][pages])[None]
        assert np.array_equal(got_k, rk), f"seq {b}: committed K pages"
        assert np.array_equal(got_v, rv), f"seq {b}: committed V pages"
        assert nlen[b] == rl[0] and nroot[b] == rr[0], f"seq {b}: next length / root"
        assert torch.equal(nh[b], hid[b, int(path[b, n_acc[b]])]), f"seq {b}: next h"
    # whole pool: differences only at committed positions
    for name in ("k_pages", "v_pages"):
        ne = dev[name] != inp[name].to(dev[name].device)        # [(layers,) pages, Hkv, slot, D]
        if layered:
            ne = ne.any(dim=0)
        diff = ne.permute(0, 2, 1, 3).flatten(2).any(dim=2)      # [pages, slot]
        diff = diff.cpu().numpy().copy()
        for b in range(w.B):
            for j in range(int(n_acc[b]) + 1):
                pos = int(lens[b]) + j
                diff[bt[b, pos // ps], pos % ps] = False
        assert not diff.any(), f"{name}: {int(diff.sum())} positions changed outside the committed branches"
    return dict(accepted=[int(x) for x in n_acc])
