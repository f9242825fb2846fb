"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and its host-side tree-plan builders agree with the
oracle's independent ones."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import hydra_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hydra.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    from speculative_decoding_hydra_amd._lib import LIB_PATH, lib as load

    if not os.path.exists(LIB_PATH):
        from speculative_decoding_hydra_amd.build import build

        build()
    return load()


def test_header_declares_the_four_stages():
    names = set(header_functions())
    for fn in ("hydra_draft_heads", "tree_build", "tree_attention_verify", "tree_accept", "tree_commit"):
        assert fn in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    from speculative_decoding_hydra_amd._lib import SIGNATURES

    names = header_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"
        assert name in SIGNATURES, f"{name} has no binding signature"
    assert set(SIGNATURES) == set(names)
    raw = C.CDLL(os.path.join(ROOT, "speculative_decoding_hydra_amd", "libhydra.so"))
    for name in names:
        getattr(raw, name)


def test_status_strings(lib):
    assert lib.hydra_status_string(0) == b"ok"
    assert lib.hydra_status_string(-3) == b"workspace too small"
    assert lib.hydra_abi_version() == 9


@pytest.mark.parametrize("b", [[2, 3], [3, 2, 2], [4, 4, 4, 4], [1, 1, 1, 1, 1], [5, 2], [2, 1, 3]])
def test_cartesian_plan_matches_oracle(lib, b):
    import speculative_decoding_hydra_amd as S

    got = S.hydra_plan_cartesian(b)
    ref = O.plan_cartesian(b)
    assert np.array_equal(got.parent, ref.parent)
    assert np.array_equal(got.rank, ref.rank)
    assert np.array_equal(got.depth, ref.depth)


@pytest.mark.parametrize("caps,n", [((10, 4, 2, 1), 64), ((4, 3, 2, 1), 30), ((6, 6, 6), 100), ((3,), 4)])
def test_sparse_plan_matches_oracle(lib, caps, n):
    import speculative_decoding_hydra_amd as S

    got = S.hydra_plan_sparse(caps, n)
    ref = O.plan_sparse_template(caps, n)
    assert np.array_equal(got.parent, ref.parent)
    assert np.array_equal(got.rank, ref.rank)
    assert np.array_equal(got.depth, ref.depth)


@pytest.mark.parametrize("hydra", [True, False])
@pytest.mark.parametrize("tree", [("c", [2, 3]), ("s", ((10, 4, 2, 1), 64)), ("c", [4, 4, 4, 4])])
def test_plan_rows_match_oracle(lib, hydra, tree):
    import speculative_decoding_hydra_amd as S

    if tree[0] == "c":
        plan = S.hydra_plan_cartesian(tree[1])
    else:
        plan = S.hydra_plan_sparse(*tree[1])
    rows = S.hydra_plan_rows(plan, hydra)
    op = O.TreePlan(plan.parent.astype(np.int64), plan.rank.astype(np.int64), plan.depth.astype(np.int64))
    row_node, row_depth, node_row = O.head_rows(op, hydra)
    assert rows.R == len(row_node)
    assert np.array_equal(rows.node_row, node_row)
    if hydra:
        assert np.array_equal(rows.row_node, row_node)
    for k in range(1, plan.dmax + 1):
        assert list(range(rows.row_first[k - 1], rows.row_first[k])) == list(np.flatnonzero(row_depth == k))
        nodes = np.flatnonzero(plan.depth == k)
        assert rows.depth_first[k] == nodes[0] and rows.depth_first[k + 1] == nodes[-1] + 1
        fan = max(len(op.children(u)) for u in np.flatnonzero(plan.depth == k - 1))
        assert rows.k_per_depth[k - 1] == fan


def test_plan_rows_rejects_bad_trees(lib):
    import speculative_decoding_hydra_amd as S

    good = S.hydra_plan_cartesian([2, 2])
    for mutate in ("parent", "rank", "depth"):
        bad = S.TreePlan(good.parent.copy(), good.rank.copy(), good.depth.copy())
        if mutate == "parent":
            bad.parent[3] = 5  # parent after child
        elif mutate == "rank":
            bad.rank[4] = 0    # siblings 0, 0
        else:
            bad.depth[2] = 2
        with pytest.raises(S.HydraError):
            S.hydra_plan_rows(bad, True)


def test_plan_builders_reject_bad_arguments(lib):
    import speculative_decoding_hydra_amd as S

    with pytest.raises(S.HydraError):
        S.hydra_plan_cartesian([0, 2])
    with pytest.raises(S.HydraError):
        S.hydra_plan_cartesian([17])
    with pytest.raises(S.HydraError):
        S.hydra_plan_sparse((2, 2), 100)  # only 6 candidates


def test_workspace_queries(lib):
    import speculative_decoding_hydra_amd as S

    assert S.tree_attention_verify_workspace_size(1, 1, 64, 32, 32, 128, 2048) > 0
    assert S.tree_attention_verify_workspace_size(0, 1, 9, 8, 8, 32, 128) == 0  # float32 path needs none
    assert S.tree_accept_workspace_size(0, 1, 64, 32000) >= 64 * 4
    assert S.tree_accept_workspace_size(1, 4, 64, 32000) >= 4 * 2 * 32000 * 4
    plan = S.hydra_plan_sparse((10, 4, 2, 1), 64)

    class P:
        rows = S.hydra_plan_rows(plan, True)
        dmax = 4

    assert S.hydra_draft_heads_workspace_size(1, 1, 4096, 32000, True, P) >= 13 * 4096 * (4 + 2)


def test_binding_fails_loudly_without_the_library(monkeypatch):
    import speculative_decoding_hydra_amd._lib as L

    monkeypatch.setattr(L, "LIB_PATH", "/nonexistent/libhydra.so")
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        L.lib()


def test_tree_commit_rejects_bad_arguments_before_any_launch(lib):
    """Argument checks of tree_commit run on the host; fake (aligned,
    non-null) device addresses are never dereferenced on these paths."""
    p = [4096 * (i + 1) for i in range(16)]
    I32 = C.POINTER(C.c_int32)

    def call(dtype=1, layers=1, B=2, N=9, Hkv=8, D=32, Dmax=2, prefix=None, nxt=None, hidden=None, next_h=None,
             k_tree=None, d=0):
        ip = lambda a: C.cast(C.c_void_p(a), I32)  # noqa: E731
        return lib.tree_commit(dtype, layers, B, N, Hkv, D, Dmax, k_tree or p[0], p[1], p[2], p[3], 10, 16,
                               ip(p[4]), 4, ip(prefix or p[5]), ip(p[6]), ip(p[7]), ip(p[8]), d, hidden,
                               ip(nxt or p[9]), ip(p[10]), next_h, None)

    assert call(B=0) == 0                           # nothing to do
    assert call(dtype=7) == -1
    assert call(layers=0) == -1
    assert call(Dmax=9) == -1
    assert call(D=12) == -2                         # 16-byte vectors need D % 8 == 0
    assert call(prefix=p[9], nxt=p[9]) == -1        # next length aliases the input length
    assert b"alias" in lib.hydra_last_error()
    assert call(hidden=p[11]) == -1                 # hidden without next_h
    assert call(hidden=p[11], next_h=p[12], d=12) == -2
    assert call(k_tree=p[0] + 8) == -1              # misaligned K
    assert b"aligned" in lib.hydra_last_error()


def test_draft_heads_sketch_rejects_bad_arguments_before_any_launch(lib):
    """Argument checks of hydra_draft_heads_sketch run on the host; the fake
    device addresses are never dereferenced on these paths."""
    import speculative_decoding_hydra_amd as S

    plan = S.hydra_plan_cartesian([2, 3])
    rows = S.hydra_plan_rows(plan, True)
    I32 = C.POINTER(C.c_int32)
    host = lambda a: (C.c_int32 * len(a))(*[int(x) for x in a])  # noqa: E731
    rf, df, kp = host(rows.row_first), host(rows.depth_first), host(rows.k_per_depth)
    p = [4096 * (i + 1) for i in range(32)]
    arr = C.c_void_p * 2

    def call(dtype=1, d=256, hid=1024, eps=1e-5, n_heads=2, Wb=None, ws_bytes=1 << 30):
        Wb = arr(None, p[20]) if Wb is None else Wb
        heads = [arr(p[10 + 2 * i], p[11 + 2 * i]) for i in range(5)]
        ip = lambda a: C.cast(C.c_void_p(a), I32)  # noqa: E731
        return lib.hydra_draft_heads_sketch(
            dtype, 1, d, 1000, hid, p[0], ip(p[1]), p[2], n_heads, heads[0], heads[1], Wb, heads[2], heads[3],
            heads[4], arr(p[21], p[22]), eps, plan.n, 2, p[3], p[4], p[5], len(rows.row_node), p[6],
            C.cast(rf, I32), C.cast(df, I32), C.cast(kp, I32), p[7], p[8], None, p[9], p[23], p[24], ws_bytes, None)

    assert call(dtype=7) == -1
    assert call(d=300) == -2                        # bf16 needs d % 256 == 0
    assert call(hid=1000) == -2                     # ... and H % 256 == 0
    assert call(dtype=0, hid=9000) == -2            # rows held in LDS: H <= 8192
    assert call(eps=0.0) == -1
    assert call(n_heads=1) == -1                    # two depths, one head
    assert call(Wb=arr(p[20], None)) == -1          # head 2 has no second layer
    assert b"head 2" in lib.hydra_last_error()
    assert call(ws_bytes=16) == -3
    assert S.hydra_draft_heads_sketch_workspace_size(1, 1, 256, 1000, 1024, _Plan(rows)) >= 6 * 1024 * 4


class _Plan:
    def __init__(self, rows):
        self.rows, self.dmax = rows, 2


def test_draft_heads_attn_and_modes_reject_bad_arguments_before_any_launch(lib):
    """Host-side checks of hydra_draft_heads_attn and of hydra_draft_heads'
    hydra mode (2 = full path); fake device addresses are never touched."""
    import speculative_decoding_hydra_amd as S

    plan = S.hydra_plan_cartesian([2, 3])
    rows = S.hydra_plan_rows(plan, True)
    I32 = C.POINTER(C.c_int32)
    host = lambda a: (C.c_int32 * len(a))(*[int(x) for x in a])  # noqa: E731
    rf, df, kp = host(rows.row_first), host(rows.depth_first), host(rows.k_per_depth)
    p = [4096 * (i + 1) for i in range(40)]
    arr = C.c_void_p * 2
    ip = lambda a: C.cast(C.c_void_p(a), I32)  # noqa: E731
    plan_args = (plan.n, 2, p[3], p[4], p[5], len(rows.row_node), p[6], C.cast(rf, I32), C.cast(df, I32),
                 C.cast(kp, I32))

    def attn(dtype=1, d=256, Wo=None, ws_bytes=1 << 30):
        return lib.hydra_draft_heads_attn(dtype, 1, d, 1000, 1, p[0], ip(p[1]), p[2], p[30], Wo or p[31], 2,
                                          arr(p[10], p[11]), arr(p[12], p[13]), arr(p[14], p[15]), *plan_args,
                                          p[7], p[8], None, p[9], p[23], p[24], ws_bytes, None)

    assert attn(dtype=5) == -1
    assert attn(d=300) == -2                        # bf16 needs d % 256 == 0
    assert attn(dtype=0, d=9000) == -2              # d <= 8192
    assert attn(ws_bytes=16) == -3
    assert S.hydra_draft_heads_attn_workspace_size(1, 1, 256, 1000, _Plan2(rows, plan.n)) >= 2 * 6 * 256 * 4

    def heads(mode, d=256):
        return lib.hydra_draft_heads(1, 1, d, 1000, mode, 1, p[0], ip(p[1]), p[2], None, 2, arr(p[10], p[11]),
                                     arr(p[12], p[13]), arr(p[14], p[15]), *plan_args, p[7], p[8], None, p[9],
                                     p[23], p[24], 1 << 30, None)

    assert heads(3) == -1                           # modes are 0, 1, 2
    assert b"hydra mode" in lib.hydra_last_error()
    assert heads(2, d=300) == -2                    # full path in bf16 needs d % 256 == 0


class _Plan2:
    def __init__(self, rows, n):
        self.rows, self.dmax, self.N = rows, 2, n


def test_tree_rope_qk_rejects_bad_arguments_before_any_launch(lib):
    I32 = C.POINTER(C.c_int32)
    ip = lambda a: C.cast(C.c_void_p(a), I32)  # noqa: E731
    p = [4096 * (i + 1) for i in range(8)]

    def call(dtype=1, B=1, D=128, theta=10000.0, k=None):
        return lib.tree_rope_qk(dtype, B, 4, 8, 2, D, p[0], p[1], p[2] if k is None else k, p[3], ip(p[4]),
                                ip(p[5]), theta, None)

    assert call(B=0) == 0
    assert call(dtype=3) == -1
    assert call(D=7) == -1
    assert call(theta=1.0) == -1
    assert call(k=0) == -1                          # null K


def test_tree_accept_binding_rejects_mismatched_target_weights():
    """The target projection reads W_t rows as wide as the attention output:
    the binding refuses a W_t of another width before touching any pointer."""
    import torch

    import speculative_decoding_hydra_amd as S

    o = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError, match="W_t"):
        S.tree_accept(o, torch.zeros(10, 16), None, None, torch.zeros(1, 4, 10), None, torch.zeros(1, 3), None, None)
    with pytest.raises(ValueError, match="target_logits"):
        S.tree_accept(o, torch.zeros(10, 8), None, None, torch.zeros(1, 4, 9), None, torch.zeros(1, 3), None, None)


def _refuses(fn, good, bad):
    """fn(**good) gets past every shape check (it stops at the first CPU
    tensor, which is not a device pointer); each entry of bad, swapped in
    alone, is refused by name before any pointer is taken."""
    for name, t in bad.items():
        args = dict(good)
        key = name.split("[")[0]
        if "[" in name:  # one entry of a per-head list
            j = int(name.split("[")[1].rstrip("]"))
            args[key] = list(args[key])
            args[key][j] = t
        else:
            args[key] = t
        with pytest.raises(ValueError, match=re.escape(name) + " has shape"):
            fn(**args)
    with pytest.raises(ValueError, match="GPU tensor"):
        fn(**good)


def test_bindings_refuse_every_mismatched_shape():
    """The C entry points see pointers only: every tensor argument of every
    stage binding is checked against the shape the kernels index it with."""
    import torch

    import speculative_decoding_hydra_amd as S
    from speculative_decoding_hydra_amd import hydra as Hy

    f = lambda *s: torch.zeros(*s)  # noqa: E731
    i = lambda *s: torch.zeros(*s, dtype=torch.int32)  # noqa: E731
    B, d, V, heads = 2, 16, 40, 2
    dplan = Hy.DevicePlan(Hy.hydra_plan_cartesian([2, 3]), True, "cpu")
    N, R, Dm = dplan.N, dplan.R, dplan.dmax
    draft = dict(h=f(B, d), root_tok=i(B), emb=f(V, d), W1=[f(d, 2 * d)] * heads, b1=[f(d)] * heads,
                 W2=[f(V, d)] * heads, dplan=dplan, head_logits=f(B, R, V), head_lse=f(B, R), cand_tok=i(B, N),
                 cand_logp=f(B, N), ws=None, head_hidden=f(B, R, d))
    _refuses(S.hydra_draft_heads, draft,
             {"root_tok": i(B + 1), "emb": f(V, d + 1), "head_logits": f(B, R + 1, V), "head_lse": f(B, R, 2),
              "cand_tok": i(B, N - 1), "cand_logp": f(B + 1, N), "head_hidden": f(B, R, d - 1),
              "W1[1]": f(d, d), "b1[0]": f(d + 1), "W2[1]": f(V - 1, d)})
    sketch = {k: v for k, v in draft.items() if k not in ("W1", "b1", "W2")}
    hid = 8
    sketch["heads"] = [dict(Wa=f(d, d), ba=f(d), ln_g=f(d), ln_b=f(d), W2=f(V, d)),
                       dict(Wa=f(hid, 2 * d), ba=f(hid), Wb=f(d, hid), bb=f(d), ln_g=f(d), ln_b=f(d), W2=f(V, d))]
    for k, name, bad in [(1, "Wb", f(d, hid + 1)), (0, "Wa", f(d, 2 * d)), (1, "ln_g", f(d - 1))]:
        hs = [dict(x) for x in sketch["heads"]]
        hs[k][name] = bad
        with pytest.raises(ValueError, match=re.escape(f"heads[{k}].{name} has shape")):
            S.hydra_draft_heads_sketch(**{**sketch, "heads": hs})
    attn = dict(draft, Wqkv=f(3 * d, d), Wo=f(d, d))
    attn.pop("emb")
    attn = {"h": attn.pop("h"), "root_tok": attn.pop("root_tok"), "emb": f(V, d), **attn}
    _refuses(S.hydra_draft_heads_attn, attn, {"Wqkv": f(2 * d, d), "Wo": f(d, 2 * d), "cand_tok": i(B, N + 1)})

    K = N
    build = dict(dplan=dplan, cand_tok=i(B, N), cand_logp=f(B, N), n_keep=K, tok=i(B, K), parent=i(B, K),
                 depth=i(B, K), anc=i(B, K, Dm + 1), q_row=i(B, K), src=i(B, K))
    _refuses(S.tree_build, build, {"cand_logp": f(B, N + 1), "anc": i(B, K, Dm), "src": i(B, K - 1),
                                   "q_row": i(B + 1, K)})

    Hq, Hkv, D, P, ps, mp = 4, 2, 32, 6, 16, 3
    att = dict(q=f(B, N, Hq, D), k_tree=f(B, N, Hkv, D), v_tree=f(B, N, Hkv, D), k_pages=f(P, Hkv, ps, D),
               v_pages=f(P, Hkv, ps, D), block_table=i(B, mp), prefix_len=i(B), max_prefix_len=40,
               anc=i(B, N, Dm + 1), depth=i(B, N), out=f(B, N, Hq, D), lse=f(B, N, Hq))
    _refuses(S.tree_attention_verify, att,
             {"k_tree": f(B, N + 1, Hkv, D), "v_tree": f(B, N - 1, Hkv, D), "v_pages": f(P + 1, Hkv, ps, D),
              "prefix_len": i(B + 1), "depth": i(B, N + 1), "out": f(B, N, Hkv, D), "lse": f(B, N, Hq, 1)})

    acc = dict(o=f(B, N, d), W_t=f(V, d), tok=i(B, N), parent=i(B, N), target_logits=f(B, N, V), n_accepted=i(B),
               path=i(B, Dm + 1), out_tok=i(B, Dm + 1), ws=None, mode=1, q_row=i(B, N), head_logits=f(B, R, V),
               u_acc=f(B, N), u_res=f(B, N))
    _refuses(S.tree_accept, acc,
             {"tok": i(B, N + 1), "parent": i(B - 1, N), "q_row": i(B, N - 1), "head_logits": f(B, R, V + 1),
              "u_acc": f(B, 1), "u_res": f(1, N), "n_accepted": i(B + 1), "out_tok": i(B, Dm)})

    proj = dict(X=f(5, d), W=f(V, d), Y=f(5, V))
    _refuses(S.hydra_vocab_projection, proj, {"W": f(V, d + 1), "Y": f(5, V + 1)})


def test_packed_weight_size_and_the_mixing_rule(lib):
    """The packed copy of W [N, K] holds ceil(N / 16) tiles of 16 rows (K a
    multiple of 256, else 0); a call's vocabulary weights are all packed or
    all row-major."""
    import torch

    from speculative_decoding_hydra_amd import PackedWeight, hydra_packed_weight_size
    from speculative_decoding_hydra_amd.hydra import HYDRA_VOCAB_PACKED, _vocab_flag

    assert hydra_packed_weight_size(32000, 4096) == 32000 * 4096 * 2
    assert hydra_packed_weight_size(1000, 256) == 1008 * 256 * 2
    assert hydra_packed_weight_size(17, 512) == 32 * 512 * 2
    for N, K in ((100, 300), (0, 256), (16, 0), (-1, 256)):
        assert hydra_packed_weight_size(N, K) == 0
    pw = PackedWeight(torch.zeros(8), 16, 256)
    assert tuple(pw.shape) == (16, 256) and pw.dim() == 2
    row = torch.zeros(16, 256, dtype=torch.bfloat16)
    assert _vocab_flag("t", [pw, pw]) == HYDRA_VOCAB_PACKED
    assert _vocab_flag("t", [row, row]) == 0
    with pytest.raises(ValueError):
        _vocab_flag("t", [pw, row])


def test_dtype_flags_match_the_header():
    """The binding's dtype flags carry the values include/hydra.h defines
    (the library parses them from the same integer)."""
    import re

    from speculative_decoding_hydra_amd import hydra as H

    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hydra.h")).read()
    for name in ("HYDRA_VOCAB_PACKED", "HYDRA_W1H_PACKED"):
        m = re.search(rf"#define {name} (0x[0-9a-fA-F]+)", hdr)
        assert m, name
        assert getattr(H, name) == int(m.group(1), 16), name
    assert len({H.HYDRA_VOCAB_PACKED, H.HYDRA_W1H_PACKED, 0x200}) == 3  # distinct bits (0x200: layer weights)
