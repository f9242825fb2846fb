"""tree_accept_noalloc (library-held scratch) against tree_accept (caller
workspace), through the C ABI: the same outputs bit for bit, on two calls in
a row, the second with a smaller input, in each acceptance mode."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import hydra_oracle as O

pytestmark = pytest.mark.gpu


def _case(g, B, N_plan, V, d, dt, mode):
    plan = O.plan_sparse_template(*N_plan) if isinstance(N_plan, tuple) else O.plan_cartesian(N_plan)
    N = plan.n
    _, _, node_row = O.head_rows(plan, True)
    R = int(node_row.max()) + 1
    tok = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for u in range(N):
            kids = plan.children(u)
            tok[b, kids] = g.choice(V, len(kids), replace=False)
    o = torch.tensor(g.standard_normal((B, N, d)), dtype=torch.float32)
    W = torch.tensor(g.standard_normal((V, d)) * 0.02, dtype=torch.float32)
    # plant a few accepts so the walks go below the root
    for b in range(B):
        u = 0
        while plan.children(u) and g.random() < 0.8:
            c = int(g.choice(plan.children(u)))
            o[b, u] = W[int(tok[b, c])] * 300.0
            u = c
    dev = lambda t: t.cuda().contiguous()  # noqa: E731
    args = dict(
        o=dev(o.to(dt)), W_t=dev(W.to(dt)), tok=dev(torch.tensor(tok)),
        parent=dev(torch.tensor(np.stack([plan.parent] * B).astype(np.int32))),
        mode=mode, temperature=0.7,
        q_row=dev(torch.tensor(np.stack([node_row] * B).astype(np.int32))),
        head_logits=dev(torch.tensor(g.standard_normal((B, R, V)) * 2.0, dtype=torch.float32)),
        u_acc=dev(torch.tensor(g.random((B, N)), dtype=torch.float32)),
        u_res=dev(torch.tensor(g.random((B, N)), dtype=torch.float32)),
        eps=0.1, delta=0.3)
    if mode == 0:
        for k in ("q_row", "head_logits", "u_acc", "u_res"):
            args[k] = None
    return args, B, N, V, plan.dmax


def _outputs(B, N, V, Dmax):
    return dict(target_logits=torch.full((B, N, V), float("nan"), device="cuda"),
                n_accepted=torch.full((B,), -7, dtype=torch.int32, device="cuda"),
                path=torch.full((B, Dmax + 1), -7, dtype=torch.int32, device="cuda"),
                out_tok=torch.full((B, Dmax + 1), -7, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_entry_on_two_calls(mode, dtype):
    from speculative_decoding_hydra_amd import tree_accept, tree_accept_noalloc, tree_accept_workspace_size

    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = np.random.default_rng(100 + 7 * mode + (dtype == "bf16"))
    shapes = [(5, ((10, 4, 2, 1), 64), 32000, 512), (2, [2, 3], 1000, 256)]  # second call: smaller
    for call, (B, tree, V, d) in enumerate(shapes):
        print(f"noalloc mode {mode} {dtype} call {call}: B={B} V={V} d={d}", flush=True)
        args, B, N, V, Dmax = _case(g, B, tree, V, d, dt, mode)
        ref = _outputs(B, N, V, Dmax)
        ws = torch.empty(tree_accept_workspace_size(mode, B, N, V), dtype=torch.uint8, device="cuda")
        targs = {k: v for k, v in args.items() if k not in ("eps", "delta") or mode == 2}
        tree_accept(ws=ws, **targs, **ref)
        got = _outputs(B, N, V, Dmax)
        tree_accept_noalloc(**targs, **got)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], got[k]), f"mode {mode} call {call}: {k} differs"
        if mode != 0:
            assert int(got["n_accepted"].max()) >= 1  # the planted accepts were taken


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call needing more than the 32 MiB the library holds is refused
    before anything is touched (null pointers are never read)."""
    from speculative_decoding_hydra_amd._lib import lib

    L = lib()
    # greedy: B * N rows x 500 blocks of 8 bytes = 307 MB of partials
    rc = L.tree_accept_noalloc(1, 0, 300, 256, 4096, 32000, 4, None, None, C.c_float(1.0), C.c_float(0.0),
                               C.c_float(0.0), None, None, None, None, 0, None, None, None, None, None, None, None)
    assert rc == -3, rc
    assert b"32 MiB" in L.hydra_last_error() or b"33554432" in L.hydra_last_error()
