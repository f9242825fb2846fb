"""Throughput of one Hydra draft-and-verify round on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--acceptance MODE] [--no-graph]
                [--no-cpu] [--no-fold] [--no-configs]

A step is one whole round (draft heads -> tree build -> rotary embedding of
the tree Q/K rows at positions prefix + depth -> tree-attention verify ->
accept -> commit of the kept branch into the KV cache) over the workload's
synthetic batch, with every input resident in
HBM before timing starts. The default workload is the Vicuna-7B-shaped layer
with the 64-node sparse tree and a 2048-token prefix (batch 1). The value is
verified tree rows per second, B * N / t_round. Hydra heads use their folded
embedding tables (built once before timing; --no-fold streams W1[:, d:]
every round instead).

The JSON line also carries
  roofline      the dominant kernel (the head/target vocabulary projection
                that streams a [V, d] bf16 matrix): algorithmic bytes per
                launch / average launch duration from HIP events on its stream,
                against the 8 TB/s HBM peak;
  decoder_layer one target decoder layer over every tree row at the workload's
                shape (tree_decoder_layer; bytes, time, HBM fraction);
  commit_32_layers  the commit kernel moving each sequence's deepest kept
                branch across 32 layers of caches (bytes, time, HBM fraction);
  mfma          the tiled projection at an MFMA-bound shape (1024 rows x
                32000 x 4096, arg-max epilogue): flops / launch time against
                the 2.5 PFLOP/s dense bf16 peak, with the rocprofv3 MFMA
                counters committed for it (null when gemm.hip changed since);
  configs       the same round on the other workloads (7B dense 256-row
                tree at prefix 8192, the 64-node tree at prefix 8192, 16
                ragged sequences, the 70B GQA layer with rejection
                acceptance, the 7B round verified through all 32 of the
                target's decoder layers) and the headline round with W1's
                embedding half streamed, and with its vocabulary weights
                row-major rather than packed: ms, verified rows/s and round
                HBM fraction each
                (their inputs are drawn on the device; --no-configs skips);
  cpu_baseline  the CPU oracle timed on this host on one full round of the
                same workload (rank 0, one GPU only).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree-tokens/sec per round + % HBM roofline (64-node tree, 7B-shape)"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "vocab_projection_7b_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "tiled_projection_1024_mfma.json")
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
CAL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="7b_sparse64")
    ap.add_argument("--no-graph", action="store_true", help="eager launches everywhere (for counter runs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--acceptance", choices=["greedy", "stochastic", "typical"], default=None,
                    help="override the workload's acceptance mode")
    ap.add_argument("--no-fold", action="store_true",
                    help="stream W1[:, d:] every round instead of the folded embedding tables")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' rounds")
    ap.add_argument("--mfma-only", action="store_true",
                    help="only the tiled projection at 1024 rows (for counter runs); prints its object")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash():
    import hashlib

    h = hashlib.sha256()
    with open(os.path.join(ROOT, "speculative_decoding_hydra_amd", "csrc", "proj.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def file_hash(name):
    import hashlib

    with open(os.path.join(ROOT, "speculative_decoding_hydra_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_mfma():
    """MFMA counters of the tiled projection at 1024 rows from a committed
    rocprofv3 run, or None when missing or the kernel changed since."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t.get("counters") if t.get("gemm_hip_sha256_16") == file_hash("gemm.hip") else None


def _loop_us(call, n, reps, use_graph):
    """Average microseconds of call(i), i = 0 .. reps - 1 (n distinct
    operands cycled), launched back to back from one graph (or eagerly)."""
    import torch

    for i in range(n):
        call(i)
    torch.cuda.synchronize()
    g = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                call(i % n)
        g.replay()
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    if g is not None:
        g.replay()
    else:
        for i in range(reps):
            call(i % n)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3


def mfma_measure(W2s, M=1024, reps=10, use_graph=True):
    """The tiled projection at an MFMA-bound row count (M rows of one
    sequence batch x every tree row: 1024 x 32000 x 4096, the 16-sequence
    target projection), with the arg-max epilogue of the target projection,
    cycling the heads' W2 copies so the last-level cache cannot serve
    repeats: flops / average launch time against the dense bf16 peak. For
    context, the vendor GEMM (hipBLASLt through torch.mm: bf16 output, no
    epilogue) on as many row-major copies in the same loop form."""
    import torch

    from speculative_decoding_hydra_amd import hydra_vocab_projection, hydra_vocab_projection_workspace_size

    N, K = W2s[0].shape
    X = torch.randn(M, K, device="cuda").to(W2s[0].dtype)
    Y = torch.empty(M, N, device="cuda")
    ws = torch.empty(hydra_vocab_projection_workspace_size(M, N, 1), dtype=torch.uint8, device="cuda")
    us = _loop_us(lambda i: hydra_vocab_projection(X, W2s[i], Y, 1, ws), len(W2s), reps, use_graph)
    flops = 2.0 * M * N * K
    tf = flops / (us * 1e-6) / 1e12
    from speculative_decoding_hydra_amd import PackedWeight

    Wr = [(torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(len(W2s))]
    Yb = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    us_bl = _loop_us(lambda i: torch.mm(X, Wr[i].t(), out=Yb), len(Wr), reps, use_graph)
    del Wr, Yb
    return {"kernel": "proj_gemm_kernel (tiled vocabulary projection, arg-max epilogue)", "rows": M, "cols": N,
            "depth": K, "weight_layout": "packed" if isinstance(W2s[0], PackedWeight) else "row-major",
            "flops": flops, "avg_launch_us": us, "achieved_TFLOPs": tf, "peak_TFLOPs": MFMA_PEAK_TFLOPS,
            "frac": tf / MFMA_PEAK_TFLOPS,
            "hipblaslt_same_loop": {"avg_launch_us": us_bl, "frac": flops / (us_bl * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS},
            "counters": measured_mfma()}


def measured_traffic():
    """Per-launch HBM bytes of the projection kernel from committed counter
    runs, or None when they are missing or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t.get("bytes_per_launch") if t.get("proj_hip_sha256_16") == source_hash() else None


def round_bytes(w, rnd, prefix_len):
    """Algorithmic HBM bytes of one round: every weight matrix the round
    needs streamed once, the paged prefix K/V read once, the tree Q/K/V/O,
    the logits written, (folded Hydra heads) one float32 table row per head
    row instead of W1's embedding half (two-layer heads: their Wa and Wb),
    and the commit's K/V rows (read and written) plus the next hidden
    state."""
    d, V, B, esz = w.d, w.V, w.B, 2 if w.dtype == "bf16" else 4
    R, N, heads = rnd.dplan.R, rnd.n_keep, rnd.dplan.dmax
    rows_per_head = [int(rnd.dplan.rows.row_first[k + 1] - rnd.dplan.rows.row_first[k]) for k in range(heads)]
    draft = heads * V * d * esz  # W2
    if getattr(rnd, "sketch", False):
        hid = w.head_hidden
        draft += d * d * esz + (heads - 1) * 3 * d * hid * esz  # head 1's Wa; later heads' Wa and Wb
    elif w.hydra and w.cond == "attn":
        draft += heads * 2 * d * d * esz + 4 * heads * d * d * esz  # W1, and Wqkv + Wo once per depth
    elif w.hydra and w.cond == "path":
        draft += sum((k + 1) * d * d for k in range(1, heads + 1)) * esz  # W1 over [h, path embeddings]
    elif w.hydra:
        draft += heads * d * d * esz  # W1 h halves
        if rnd.emb_proj is None:
            draft += heads * d * d * esz  # W1 embedding halves, streamed
        else:
            draft += B * sum(rows_per_head) * d * 4  # one table row per head row
    else:
        draft += heads * d * d * esz
    draft += B * R * V * 4  # head logits
    prefix = int(prefix_len.sum())
    attn = prefix * w.Hkv * w.D * esz * 2 + B * N * (2 * w.Hq + 2 * w.Hkv) * w.D * esz
    target = V * d * esz + B * N * d * esz + B * N * V * 4
    kept = int(rnd.n_accepted.clamp(min=0).sum()) + B  # root + accepted rows
    commit = kept * w.Hkv * w.D * esz * 2 * 2 + B * d * esz * 2
    if w.layers:
        # the target's layers: each streams its weights and reads its prefix
        # K/V once; the rows' activations in and out; embedding rows read and
        # final hidden states written; the commit moves every layer's K/V
        weights = ((w.Hq + 2 * w.Hkv) * w.D * d + d * w.Hq * w.D + 3 * w.ffn * d + 2 * d) * esz
        acts = B * N * (2 * d + 2 * w.Hkv * w.D) * esz
        attn = w.layers * (weights + prefix * w.Hkv * w.D * esz * 2 + acts) + 2 * B * N * d * esz
        commit = w.layers * kept * w.Hkv * w.D * esz * 2 * 2 + B * d * esz * 2
    return draft + attn + target + commit


def commit_measure(w, rnd, dev, stream, layers=32, reps=20, use_graph=True):
    """The commit kernel at model depth: the round's own commit moves one
    layer (and, with random weights, only the root), so this times the
    commit of each sequence's deepest kept branch across a `layers`-deep
    stack of caches (synthetic tree K/V, the round's block table)."""
    import torch

    from speculative_decoding_hydra_amd import tree_commit

    B, K = rnd.attn_out.shape[:2]
    dt = rnd.dtype
    n_pages, _, ps, _ = dev["k_pages"].shape[-4:]  # one layer's pool (target layers stack them)
    kt = torch.randn(layers, B, K, w.Hkv, w.D, device="cuda").to(dt)
    vt = torch.randn(layers, B, K, w.Hkv, w.D, device="cuda").to(dt)
    kp = torch.zeros(layers, n_pages, w.Hkv, ps, w.D, dtype=dt, device="cuda")
    vp = torch.zeros_like(kp)
    deepest = rnd.depth.argmax(dim=1)
    n_acc = rnd.depth.gather(1, deepest[:, None])[:, 0].contiguous()
    path = rnd.anc[torch.arange(B, device="cuda"), deepest].contiguous()
    out_tok = torch.zeros_like(path)
    nlen = torch.empty(B, dtype=torch.int32, device="cuda")
    nroot = torch.empty_like(nlen)
    hidden = rnd.attn_out.view(B, K, -1)
    nh = torch.empty(B, hidden.shape[2], dtype=dt, device="cuda")
    launch = lambda: tree_commit(kt, vt, kp, vp, dev["block_table"], dev["prefix_len"], n_acc, path,  # noqa: E731
                                 out_tok, nlen, nroot, hidden=hidden, next_h=nh)
    launch()
    torch.cuda.synchronize()
    g = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                launch()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    if g is not None:
        g.replay()
    else:
        for _ in range(reps):
            launch()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    rows = int(n_acc.sum()) + B
    esz = kt.element_size()
    nbytes = layers * rows * w.Hkv * w.D * esz * 2 * 2 + B * hidden.shape[2] * esz * 2
    return {"layers": layers, "rows_per_layer": rows, "bytes": nbytes, "avg_launch_us": us,
            "achieved_GBps": nbytes / (us * 1e-6) / 1e9, "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


FFN_DIM = {4096: 11008, 8192: 28672}  # the LLaMA-family feed-forward widths of the two model shapes


def layer_measure(w, rnd, dev, stream, reps=10, use_graph=True):
    """One target decoder layer over every tree row of the round
    (tree_decoder_layer) at the workload's shape, cycling two weight sets so
    the last-level cache cannot serve repeats; random weights, the round's
    paged prefix, tree and positions."""
    import torch

    from speculative_decoding_hydra_amd import tree_decoder_layer, tree_decoder_layer_workspace_size

    B, K = rnd.attn_out.shape[:2]
    d, Hq, Hkv, D = w.d, w.Hq, w.Hkv, w.D
    F = FFN_DIM.get(d, 4 * d)
    dt = rnd.dtype
    g = torch.Generator(device="cuda").manual_seed(7)
    n = lambda *s: (torch.randn(*s, device="cuda", generator=g) * 0.02).to(dt)  # noqa: E731
    ones = torch.ones(d, device="cuda", dtype=dt)
    sets = [dict(ln1=ones, Wqkv=n((Hq + 2 * Hkv) * D, d), Wo=n(d, Hq * D), ln2=ones, Wgu=n(2 * F, d), Wd=n(d, F))
            for _ in range(2)]
    if rnd.pack_vocab:  # the layout the rounds keep their weights in
        from speculative_decoding_hydra_amd import hydra_pack_weight

        sets = [dict(s, **{k: hydra_pack_weight(s[k]) for k in ("Wqkv", "Wo", "Wgu", "Wd")}) for s in sets]
    x = torch.randn(B, K, d, device="cuda", generator=g).to(dt)
    out = torch.empty_like(x)
    kt = torch.empty(B, K, Hkv, D, device="cuda", dtype=dt)
    vt = torch.empty_like(kt)
    mpl = int(rnd.shape["max_prefix_len"])
    code = 0 if dt == torch.float32 else 1
    ws = torch.empty(tree_decoder_layer_workspace_size(code, B, K, d, Hq, Hkv, D, F, mpl), dtype=torch.uint8,
                     device="cuda")
    kp, vp = dev["k_pages"], dev["v_pages"]
    if kp.dim() == 5:  # one pool per target layer: the first layer's
        kp, vp = kp[0], vp[0]
    launch = lambda i: tree_decoder_layer(x, sets[i % 2], Hq, Hkv, kp, vp,  # noqa: E731
                                          dev["block_table"], dev["prefix_len"], mpl, rnd.anc, rnd.depth, out, kt,
                                          vt, ws)
    launch(0)
    launch(1)
    torch.cuda.synchronize()
    gr = None
    if use_graph:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(reps):
                launch(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    if gr is not None:
        gr.replay()
    else:
        for i in range(reps):
            launch(i)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    esz = x.element_size()
    weights = ((Hq + 2 * Hkv) * D * d + d * Hq * D + 3 * F * d) * esz
    prefix = int(dev["prefix_len"].sum()) * Hkv * D * esz * 2
    acts = B * K * (2 * d + 2 * Hkv * D) * esz
    nbytes = weights + prefix + acts
    return {"d": d, "ffn": F, "rows": B * K, "weight_layout": "packed" if rnd.pack_vocab else "row-major",
            "bytes": nbytes, "weight_bytes": weights, "avg_launch_us": us,
            "achieved_GBps": nbytes / (us * 1e-6) / 1e9, "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def time_round(rnd, dev, steps, warmup, use_graph=True):
    """Mean ms per round over `steps` graph-replayed rounds (after `warmup`),
    the graph (or None) and the per-round event distribution."""
    import torch

    from speculative_decoding_hydra_amd import run_round

    stream = torch.cuda.current_stream()
    for _ in range(max(1, warmup)):
        run_round(rnd, dev)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                run_round(rnd, dev)
            stream.wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                run_round(rnd, dev)
            torch.cuda.synchronize()
            for _ in range(max(1, warmup)):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001
            log(f"[bench] graph capture unavailable ({e}); timing eager launches")
            graph = None
    step = graph.replay if graph is not None else (lambda: run_round(rnd, dev))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    rev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    rev[0].record(stream)
    for i in range(steps):
        step()
        rev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(rev[i].elapsed_time(rev[i + 1]) for i in range(steps))
    pick = lambda q: per[min(len(per) - 1, int(q * len(per)))]  # noqa: E731
    return ms, graph, {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9)}


# the other workloads of the same round, each on its own synthetic inputs
# (drawn on the device); the first uses the headline's inputs with the
# embedding half of W1 streamed every round instead of the folded tables
CONFIGS = ["7b_sparse64:streamed", "7b_sparse64:row-major", "7b_dense256", "7b_sparse64_L8192", "7b_batched16",
           "70b_gqa", "7b_layers"]


def configs_measure(head_inp, steps, warmup, use_graph=True):
    import torch

    import hydra_inputs as HI
    from speculative_decoding_hydra_amd import round_from_inputs

    out = {}
    for spec in CONFIGS:
        name, _, variant = spec.partition(":")
        t0 = time.perf_counter()
        w = HI.workload(name)
        inp = head_inp if variant in ("streamed", "row-major") else HI.generate(w, device="cuda")
        rnd, dev = round_from_inputs(inp, device="cuda:0", keep_hidden=False,
                                     fold_embedding=False if variant == "streamed" else None,
                                     pack_vocab=False if variant == "row-major" else None)
        ms, graph, dist = time_round(rnd, dev, steps, warmup, use_graph)
        rows = w.B * rnd.n_keep
        rb = round_bytes(w, rnd, inp["prefix_len"].cpu())
        out[spec] = {"ms_per_round": ms, "round_ms": dist, "tokens_per_s": rows / (ms * 1e-3), "tree_rows": rows,
                     "round_bytes": rb, "round_hbm_frac": rb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "acceptance": w.mode, "embedding_half": ("folded table" if rnd.emb_proj is not None
                                                              else "streamed") if w.hydra else None,
                     "vocab_weights": "packed" if rnd.pack_vocab else "row-major",
                     "launch": "hip-graph" if graph is not None else "eager",
                     "target_layers": w.layers or None}
        log(f"[bench] {spec}: {ms:.4f} ms/round ({time.perf_counter() - t0:.1f} s)")
        del graph, rnd, dev
        if inp is not head_inp:
            del inp
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, n_rows):
    """The oracle, as it stands, on one full round of the same workload."""
    import numpy as np

    import hydra_inputs as HI
    from oracle import hydra_oracle as O

    w = inp["workload"]
    f = HI.as_f64
    if w.head == "sketch":
        heads = [{n: f(t) for n, t in hd.items()} for hd in inp["heads"]]
    else:
        heads = [(f(a), f(b), f(c)) for a, b, c in zip(inp["W1"], inp["b1"], inp["W2"])]
    attn = None
    if w.cond == "attn":
        Wqkv = f(inp["attn"]["Wqkv"])
        attn = {"Wq": Wqkv[:w.d], "Wk": Wqkv[w.d:2 * w.d], "Wv": Wqkv[2 * w.d:], "Wo": f(inp["attn"]["Wo"])}
    E, Wt, h = f(inp["E"]), f(inp["W_t"]), f(inp["h"])
    kp = [f(x) for x in inp["k_prefix"]]
    vp = [f(x) for x in inp["v_prefix"]]
    q, kt, vt = f(inp["q_tree"]), f(inp["k_tree"]), f(inp["v_tree"])
    kpool, vpool = f(inp["k_pages"])[None], f(inp["v_pages"])[None]
    bt, lens = inp["block_table"].numpy(), inp["prefix_len"].numpy()
    kind = w.tree[0]
    plan = O.plan_sparse_template(w.tree[1], w.tree[2]) if kind == "sparse" else O.plan_cartesian(w.tree[1])
    node_row = O.head_rows(plan, w.hydra)[2]
    u_acc = inp["u_acc"].numpy() if "u_acc" in inp else None
    u_res = inp["u_res"].numpy() if "u_res" in inp else None
    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    reps, total = 0, 0.0
    while reps < 5 and total < 10.0:  # a bounded sample: whole rounds, about 10 s
        t0 = time.perf_counter()
        res = O.draft_heads(h, inp["root_tok"].numpy(), E, heads, plan, hydra=w.hydra, bf16=w.dtype == "bf16",
                            full_path=w.cond == "path", attn=attn)
        if kind == "dense":
            trees = [O.prune_tree(plan, res["logp"][b], w.tree[2]) for b in range(w.B)]
        else:
            trees = [(plan, np.arange(plan.n)) for _ in range(w.B)]
        anc = np.stack([O.ancestors(t.parent, plan.dmax) for t, _ in trees])
        pos = O.tree_positions(lens, np.stack([t.depth for t, _ in trees]))[..., None]
        q_rot, kt_rot = O.rope(q, pos), O.rope(kt, pos)
        out, _ = O.tree_attention(q_rot, kt_rot, vt, kp, vp, anc, bf16=w.dtype == "bf16")
        Z = O.target_logits(out, Wt)
        n_acc = np.zeros(w.B, dtype=np.int64)
        path = -np.ones((w.B, plan.dmax + 1), dtype=np.int64)
        toks = -np.ones((w.B, plan.dmax + 1), dtype=np.int64)
        for b, (t, s) in enumerate(trees):
            tb = res["tok"][b][s]
            if w.mode == "greedy":
                m, pth, tk = O.greedy_accept(Z[b], tb, t.parent, plan.dmax)
            elif w.mode == "typical":
                m, pth, tk = O.typical_accept(Z[b], tb, t.parent, u_res[b], w.T, w.eps, w.delta)
            else:
                m, pth, tk = O.rejection_accept(Z[b], res["z"][b], node_row[s], tb, t.parent, u_acc[b], u_res[b],
                                                w.T)
            n_acc[b], path[b, : m + 1], toks[b, : m + 1] = m, pth, tk
        O.commit_path(kpool, vpool, bt, lens, kt_rot[None], vt[None], n_acc, path, toks, plan.dmax,
                      out.reshape(w.B, out.shape[1], -1))
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    return {"value": n_rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full round(s) of {w.name} (B={w.B}, N={n_rows // w.B}) in float64 NumPy, "
                      f"{dt:.2f} s per round; inputs converted to float64 before timing"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each sequence "
              "batch shards across GPUs with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import hydra_inputs as HI
    from speculative_decoding_hydra_amd import (hydra_vocab_projection, hydra_vocab_projection_workspace_size,
                                                 round_from_inputs)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.mfma_only:
        g = torch.Generator(device="cuda").manual_seed(1)
        from speculative_decoding_hydra_amd import hydra_pack_weight

        W2s = [hydra_pack_weight((torch.randn(32000, 4096, device="cuda", generator=g) * 0.02).to(torch.bfloat16))
               for _ in range(4)]  # packed, as the rounds hold their vocabulary weights
        print(json.dumps(mfma_measure(W2s, use_graph=not args.no_graph)), flush=True)
        return
    w = HI.workload(args.workload)
    if args.acceptance and args.acceptance != w.mode:
        w = HI.workload(args.workload, mode=args.acceptance, T=w.T if w.mode != "greedy" else 1.0)
    log(f"[bench] generating {w.name}")
    inp = HI.generate(w)
    rnd, dev = round_from_inputs(inp, device="cuda:0", keep_hidden=False,
                                 fold_embedding=False if args.no_fold else None)
    N = rnd.n_keep
    rows = w.B * N
    stream = torch.cuda.current_stream()
    ms, graph, round_ms = time_round(rnd, dev, args.steps, args.warmup, use_graph=not args.no_graph)
    log(f"[bench] {w.name}: {ms:.4f} ms/round ({'graph' if graph else 'eager'})")

    # per-stage times (eager, events on the launch stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    stage_ms = [0.0] * 5
    reps = 10
    for _ in range(reps):
        ev[0].record(stream)
        rnd.draft(dev["h"], dev["root_tok"])
        ev[1].record(stream)
        rnd.build()
        ev[2].record(stream)
        if rnd.target is not None:  # the target's layers over the tree tokens
            rnd.verify(dev["k_pages"], dev["v_pages"], dev["block_table"], dev["prefix_len"])
        else:
            rnd.attend(dev["q"], dev["k_tree"], dev["v_tree"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                       dev["prefix_len"])
        ev[3].record(stream)
        rnd.accept(dev.get("u_acc"), dev.get("u_res"))
        ev[4].record(stream)
        rnd.commit(dev.get("k_tree"), dev.get("v_tree"), dev["k_pages"], dev["v_pages"], dev["block_table"],
                   dev["prefix_len"])
        ev[5].record(stream)
        torch.cuda.synchronize()
        for i in range(5):
            stage_ms[i] += ev[i].elapsed_time(ev[i + 1]) / reps

    # dominant kernel: the [V, d] vocabulary projection of a head (largest row count of the round)
    # (same kernel instance as the round's head launches: fused top-k epilogue)
    M = int(max(rnd.dplan.rows.row_first[1:] - rnd.dplan.rows.row_first[:-1])) * w.B
    kk = int(max(rnd.dplan.rows.k_per_depth))
    X = torch.randn(M, w.d, device="cuda").to(rnd.dtype)
    Y = torch.empty(M, w.V, device="cuda")
    kws = torch.empty(hydra_vocab_projection_workspace_size(M, w.V, kk), dtype=torch.uint8, device="cuda")
    W2s = [hd["W2"] for hd in rnd.heads] if rnd.sketch else rnd.W2  # as the round holds them (packed or not)
    W2 = W2s[0]
    proj = lambda Wm: hydra_vocab_projection(X, Wm, Y, kk, kws)  # noqa: E731
    for _ in range(3):
        proj(W2)
    torch.cuda.synchronize()
    kgraph = None
    try:  # back-to-back launches from a graph, so the events see no launch gaps
        if args.no_graph:
            raise RuntimeError("--no-graph")
        s2 = torch.cuda.Stream()
        s2.wait_stream(stream)
        with torch.cuda.stream(s2):
            proj(W2)
        stream.wait_stream(s2)
        torch.cuda.synchronize()
        kgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(kgraph):
            for i in range(args.kernel_reps):
                proj(W2s[i % len(W2s)])
        kgraph.replay()
        torch.cuda.synchronize()
    except Exception as e:  # noqa: BLE001
        log(f"[bench] kernel graph unavailable ({e}); eager launches")
        kgraph = None
    ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ka.record(stream)
    if kgraph is not None:
        kgraph.replay()
    else:
        for i in range(args.kernel_reps):
            proj(W2s[i % len(W2s)])
    kb.record(stream)
    torch.cuda.synchronize()
    k_ms = ka.elapsed_time(kb) / args.kernel_reps

    # a plain elementwise pass of known size (reads and writes 256 MiB), so that
    # HBM counters taken over this command can be scaled to bytes
    cal = torch.ones(CAL_BYTES // 4, device="cuda")
    torch.neg(cal, out=torch.empty_like(cal))
    torch.cuda.synchronize()
    del cal
    esz = X.element_size()
    alg_bytes = w.V * w.d * esz + M * w.d * esz + M * w.V * 4
    achieved = alg_bytes / (k_ms * 1e-3) / 1e9

    mfma = mfma_measure(W2s, use_graph=not args.no_graph) if w.d == 4096 and rnd.dtype == torch.bfloat16 else None
    commit = commit_measure(w, rnd, dev, stream, use_graph=not args.no_graph)
    layer = layer_measure(w, rnd, dev, stream, use_graph=not args.no_graph)
    rbytes = round_bytes(w, rnd, inp["prefix_len"])
    configs = None
    if not args.no_configs and args.workload == "7b_sparse64" and not args.no_fold:
        configs = configs_measure(inp, args.steps, args.warmup, use_graph=not args.no_graph)
    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on one round")
        cpu = cpu_baseline(inp, rows)

    res = {
        "metric": METRIC,
        "value": rows / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; no checkpoint)",
        "config": {"workload": w.name, "batch": w.B, "tree_rows": N, "hidden": w.d, "vocab": w.V,
                   "heads": w.n_heads, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "prefix": list(w.L), "tree": str(w.tree[0]), "acceptance": w.mode,
                   "launch": "hip-graph" if graph is not None else "eager",
                   "embedding_half": ("folded table" if rnd.emb_proj is not None else "streamed")
                   if w.hydra else None,
                   "vocab_weights": "packed" if rnd.pack_vocab else "row-major"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": ("proj_bf16_kernel (streaming vocabulary projection, fused top-k epilogue)"
                                if M < 65 else "proj_gemm_kernel (tiled vocabulary projection, fused top-k epilogue)"),
                     "bytes_per_launch": alg_bytes, "rows": M, "topk": kk, "avg_launch_ms": k_ms,
                     "weight_layout": "packed" if rnd.pack_vocab else "row-major"},
        "mfma": mfma,
        "round_ms": round_ms,
        "round_bytes": rbytes,
        "round_hbm_frac": rbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stages_ms": {"draft": stage_ms[0], "build": stage_ms[1],
                      ("target_layers" if rnd.target is not None else "attention"): stage_ms[2],
                      "accept": stage_ms[3], "commit": stage_ms[4]},
        "commit_32_layers": commit,
        "decoder_layer": layer,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
