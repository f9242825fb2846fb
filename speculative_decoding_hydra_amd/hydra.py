"""Python binding of libhydra, one function per C entry point (same names).

Argument marshalling only: tensors are checked for device, dtype and layout,
turned into pointers and sizes, and passed to the library, which does all of
the work in its HIP kernels on the given stream. PyTorch provides device
memory and streams.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from ._lib import lib

HYDRA_F32, HYDRA_BF16 = 0, 1
HYDRA_VOCAB_PACKED = 0x100  # dtype flag: the call's vocabulary weights are packed (hydra_pack_weight)
HYDRA_W1H_PACKED = 0x400  # dtype flag: W1 holds the packed h halves of a folded call (hydra_pack_weight)
HYDRA_LAYER_PACKED = 0x200  # dtype flag: the decoder layers' weights are packed
MAX_DEPTH, MAX_TOPK, MAX_TREE, MAX_VERIFY = 8, 16, 1024, 256


class HydraError(RuntimeError):
    def __init__(self, fn, code):
        L = lib()
        msg = L.hydra_last_error().decode()
        super().__init__(f"{fn}: {L.hydra_status_string(code).decode()} ({code}): {msg}")
        self.code = code


def _check(fn, rc):
    if rc != 0:
        raise HydraError(fn, rc)
    return rc


def _dtype_code(t):
    if t.dtype == torch.float32:
        return HYDRA_F32
    if t.dtype == torch.bfloat16:
        return HYDRA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


class PackedWeight:
    """A bfloat16 weight W [N, K] (or a layer stack [n, N, K], each layer
    packed on its own) in the packed layout that hydra_pack_weight writes
    (see include/hydra.h). Accepted wherever a call takes vocabulary
    projection weights (the heads' W2, W_t, the W of hydra_vocab_projection)
    or decoder layer weights (Wqkv, Wo, Wgu, Wd); the binding then sets
    HYDRA_VOCAB_PACKED or HYDRA_LAYER_PACKED in the call's dtype."""

    dtype = torch.bfloat16

    def __init__(self, data, N, K, layers=None):
        self.data, self.N, self.K = data, int(N), int(K)
        self.layers = None if layers is None else int(layers)

    @property
    def shape(self):
        if self.layers is None:
            return torch.Size((self.N, self.K))
        return torch.Size((self.layers, self.N, self.K))

    def dim(self):
        return 2 if self.layers is None else 3


def hydra_packed_weight_size(N, K):
    return int(lib().hydra_packed_weight_size(int(N), int(K)))


def hydra_pack_weight(W, stream=None):
    """The packed copy of a bfloat16 W [N, K] (K % 256 == 0) as a
    PackedWeight; a layer stack [n, N, K] (N % 16 == 0, so that each layer's
    packed matrix keeps the row-major stride) is packed layer by layer."""
    if W.dim() not in (2, 3):
        raise ValueError(f"hydra_pack_weight: W must be [N, K] or [layers, N, K], got {tuple(W.shape)}")
    N, K = W.shape[-2:]
    size = hydra_packed_weight_size(N, K)
    if size == 0:
        raise ValueError(f"hydra_pack_weight: needs K % 256 == 0 and positive sizes (N={N}, K={K})")
    if W.dim() == 3 and N % 16 != 0:
        raise ValueError(f"hydra_pack_weight: a layer stack needs N % 16 == 0 (N={N})")
    n = W.shape[0] if W.dim() == 3 else 1
    out = torch.empty(n * size // 2, dtype=torch.bfloat16, device=W.device)
    Wc = W.reshape(n, N, K)
    for layer in range(n):
        _check("hydra_pack_weight", lib().hydra_pack_weight(N, K, _dev(Wc[layer], "W", torch.bfloat16),
                                                           out.data_ptr() + layer * size, _stream(stream)))
    return PackedWeight(out, N, K, layers=n if W.dim() == 3 else None)


def _vocab_flag(fn, weights, flag=HYDRA_VOCAB_PACKED):
    """flag when every given weight is packed, 0 when none is; a mix is
    refused."""
    packed = [isinstance(w, PackedWeight) for w in weights]
    if any(packed) and not all(packed):
        raise ValueError(f"{fn}: either every vocabulary or layer weight is packed or none is")
    return flag if packed and all(packed) else 0


def _dev(t, name, dtype=None):
    """Device pointer of a contiguous GPU tensor or of a packed weight's data
    (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, PackedWeight):
        if dtype is not None and dtype != torch.bfloat16:
            raise TypeError(f"{name}: packed weights are bfloat16, the call works in {dtype}")
        t = t.data
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shapes(fn, **want):
    """Raise ValueError unless every given tensor (None skipped) has its
    expected shape: the C entry points see pointers only, so this is where a
    mismatched tensor is refused before any kernel could read past it."""
    for name, (t, shape) in want.items():
        if t is None:
            continue
        if not isinstance(t, (torch.Tensor, PackedWeight)):
            raise TypeError(f"{fn}: {name}: expected a tensor")
        if tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")


def _host_i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ws(ws):
    if ws is None:
        return None, 0
    return _dev(ws, "ws"), ws.numel() * ws.element_size()


# --------------------------------------------------------------- tree plans

@dataclass
class TreePlan:
    """Breadth-first candidate tree shape (host int32 arrays)."""
    parent: np.ndarray
    rank: np.ndarray
    depth: np.ndarray

    @property
    def n(self):
        return int(self.parent.shape[0])

    @property
    def dmax(self):
        return int(self.depth.max())


@dataclass
class PlanRows:
    node_row: np.ndarray
    row_node: np.ndarray
    row_first: np.ndarray
    depth_first: np.ndarray
    k_per_depth: np.ndarray
    R: int


def _plan_out(n):
    return [np.zeros(n, dtype=np.int32) for _ in range(3)]


def hydra_plan_cartesian(b):
    b, bp = _host_i32(b)
    par, rk, dp = _plan_out(MAX_TREE)
    P = C.POINTER(C.c_int32)
    n = lib().hydra_plan_cartesian(bp, len(b), MAX_TREE, par.ctypes.data_as(P), rk.ctypes.data_as(P),
                                   dp.ctypes.data_as(P))
    if n < 0:
        raise HydraError("hydra_plan_cartesian", n)
    return TreePlan(par[:n].copy(), rk[:n].copy(), dp[:n].copy())


def hydra_plan_sparse(caps, n_nodes):
    caps, cp = _host_i32(caps)
    par, rk, dp = _plan_out(MAX_TREE)
    P = C.POINTER(C.c_int32)
    n = lib().hydra_plan_sparse(cp, len(caps), int(n_nodes), MAX_TREE, par.ctypes.data_as(P),
                                rk.ctypes.data_as(P), dp.ctypes.data_as(P))
    if n < 0:
        raise HydraError("hydra_plan_sparse", n)
    return TreePlan(par[:n].copy(), rk[:n].copy(), dp[:n].copy())


def hydra_plan_rows(plan: TreePlan, hydra: bool):
    P = C.POINTER(C.c_int32)
    N = plan.n
    par, _ = _host_i32(plan.parent)
    rk, _ = _host_i32(plan.rank)
    dp, _ = _host_i32(plan.depth)
    node_row = np.zeros(N, dtype=np.int32)
    row_node = np.zeros(N, dtype=np.int32)
    row_first = np.zeros(MAX_DEPTH + 2, dtype=np.int32)
    depth_first = np.zeros(MAX_DEPTH + 2, dtype=np.int32)
    k_per_depth = np.zeros(MAX_DEPTH + 2, dtype=np.int32)
    R = lib().hydra_plan_rows(N, par.ctypes.data_as(P), rk.ctypes.data_as(P), dp.ctypes.data_as(P),
                              int(bool(hydra)), node_row.ctypes.data_as(P), row_node.ctypes.data_as(P),
                              row_first.ctypes.data_as(P), depth_first.ctypes.data_as(P),
                              k_per_depth.ctypes.data_as(P))
    if R < 0:
        raise HydraError("hydra_plan_rows", R)
    dmax = plan.dmax
    return PlanRows(node_row, row_node[:R].copy(), row_first[: dmax + 1].copy(),
                    depth_first[: dmax + 2].copy(), k_per_depth[:dmax].copy(), int(R))


class DevicePlan:
    """A tree plan and its head rows, with device copies of the arrays the
    kernels read."""

    def __init__(self, plan: TreePlan, hydra: bool, device="cuda"):
        self.plan = plan
        self.hydra = bool(hydra)
        self.rows = hydra_plan_rows(plan, hydra)
        self.N, self.dmax, self.R = plan.n, plan.dmax, self.rows.R

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

        self.parent = up(plan.parent)
        self.rank = up(plan.rank)
        self.depth = up(plan.depth)
        self.node_row = up(self.rows.node_row)
        self.row_node = up(self.rows.row_node)


# ------------------------------------------------------------------ stages

def _draft_shapes(fn, h, root_tok, emb, W2, dplan, head_logits, head_lse, cand_tok, cand_logp, head_hidden):
    """Shapes shared by the three draft-stage bindings."""
    if h.dim() != 2:
        raise ValueError(f"{fn}: h must be [B, d], got {tuple(h.shape)}")
    B, d = h.shape
    V = W2[0].shape[0]
    if len(W2) < dplan.dmax:
        raise ValueError(f"{fn}: the tree is {dplan.dmax} deep but there are {len(W2)} heads")
    _shapes(fn, root_tok=(root_tok, (B,)), emb=(emb, (V, d)), head_logits=(head_logits, (B, dplan.R, V)),
            head_lse=(head_lse, (B, dplan.R)), cand_tok=(cand_tok, (B, dplan.N)), cand_logp=(cand_logp, (B, dplan.N)),
            head_hidden=(head_hidden, (B, dplan.R, d)))
    for k, w in enumerate(W2):
        _shapes(fn, **{f"W2[{k}]": (w, (V, d))})


def hydra_draft_heads_workspace_size(dtype_code, B, d, V, hydra, dplan: DevicePlan):
    rf, rfp = _host_i32(dplan.rows.row_first)
    return int(lib().hydra_draft_heads_workspace_size(dtype_code, B, d, V, int(hydra), dplan.dmax, rfp))


def hydra_draft_heads(h, root_tok, emb, W1, b1, W2, dplan: DevicePlan, head_logits, head_lse,
                      cand_tok, cand_logp, ws, head_hidden=None, residual=True, emb_proj=None, full_path=False,
                      stream=None):
    """Stage 1 (see include/hydra.h). h [B, d]; W1/b1/W2: lists, head k at k-1;
    emb_proj: optional list of folded embedding tables (hydra_fold_embedding);
    full_path: Hydra heads read every path token's embedding (W1_k [d, (k+1) d])."""
    if full_path and not dplan.hydra:
        raise ValueError("full-path conditioning needs a Hydra plan")
    dt = _dtype_code(h)
    B, d = h.shape
    V = W2[0].shape[0]
    n_heads = len(W2)
    if not (len(W1) == len(b1) == n_heads):
        raise ValueError("W1, b1 and W2 need one entry per head")
    _draft_shapes("hydra_draft_heads", h, root_tok, emb if dplan.hydra else None, W2, dplan, head_logits, head_lse,
                  cand_tok, cand_logp, head_hidden)
    # with folded tables W1 may be the packed h halves W1_k[:, :d] (all or none)
    w1h = emb_proj is not None and any(isinstance(w, PackedWeight) for w in W1)
    if w1h and not all(isinstance(w, PackedWeight) for w in W1):
        raise ValueError("hydra_draft_heads: packed h halves of W1 come for every head or none")
    for k in range(n_heads):
        in_k = d if w1h else ((k + 2) * d if full_path else (2 * d if dplan.hydra else d))
        _shapes("hydra_draft_heads", **{f"W1[{k}]": (W1[k], (d, in_k)), f"b1[{k}]": (b1[k], (d,))})
    arr = C.c_void_p * n_heads
    w1 = arr(*[_dev(w, "W1", h.dtype) for w in W1])
    bb = arr(*[_dev(w, "b1", h.dtype) for w in b1])
    w2 = arr(*[_dev(w, "W2", h.dtype) for w in W2])
    dt |= _vocab_flag("draft heads", W2)
    if w1h:
        dt |= HYDRA_W1H_PACKED
    rows = dplan.rows
    rf, rfp = _host_i32(rows.row_first)
    df, dfp = _host_i32(rows.depth_first)
    kp, kpp = _host_i32(rows.k_per_depth)
    ep = None
    if emb_proj is not None:
        if full_path:
            raise ValueError("full-path heads take no folded tables")
        if len(emb_proj) != n_heads:
            raise ValueError("emb_proj needs one table per head")
        for k, t in enumerate(emb_proj):
            _shapes("hydra_draft_heads", **{f"emb_proj[{k}]": (t, (V, d))})
        ep = arr(*[_dev(t, "emb_proj", torch.float32) for t in emb_proj])
    wsp, wsb = _ws(ws)
    rc = lib().hydra_draft_heads(
        dt, B, d, V, 2 if full_path else int(dplan.hydra), int(bool(residual)), _dev(h, "h"), _dev(root_tok, "root_tok", torch.int32),
        _dev(emb, "emb", h.dtype) if dplan.hydra else None, ep, n_heads, w1, bb, w2, dplan.N, dplan.dmax,
        _dev(dplan.parent, "parent"), _dev(dplan.rank, "rank"), _dev(dplan.node_row, "node_row"), dplan.R,
        _dev(dplan.row_node, "row_node"), rfp, dfp, kpp, _dev(head_logits, "head_logits", torch.float32),
        _dev(head_lse, "head_lse", torch.float32), _dev(head_hidden, "head_hidden", h.dtype),
        _dev(cand_tok, "cand_tok", torch.int32), _dev(cand_logp, "cand_logp", torch.float32), wsp, wsb,
        _stream(stream))
    return _check("hydra_draft_heads", rc)


def hydra_draft_heads_sketch_workspace_size(dtype_code, B, d, V, hidden_dim, dplan: DevicePlan):
    rf, rfp = _host_i32(dplan.rows.row_first)
    return int(lib().hydra_draft_heads_sketch_workspace_size(dtype_code, B, d, V, hidden_dim, dplan.dmax, rfp))


def hydra_draft_heads_sketch(h, root_tok, emb, heads, dplan: DevicePlan, head_logits, head_lse, cand_tok,
                             cand_logp, ws, head_hidden=None, ln_eps=1e-5, stream=None):
    """Stage 1 with two-layer LayerNorm heads (see include/hydra.h). heads: one
    dict per head (head k at k-1) with Wa, ba, ln_g, ln_b, W2 and, for k > 1,
    Wb, bb."""
    if not dplan.hydra:
        raise ValueError("two-layer heads read [h || e(parent)]: the plan must be a Hydra plan")
    dt = _dtype_code(h)
    B, d = h.shape
    n_heads = len(heads)
    V = heads[0]["W2"].shape[0]
    hidden_dim = heads[1]["Wa"].shape[0] if n_heads > 1 else d
    _draft_shapes("hydra_draft_heads_sketch", h, root_tok, emb, [w["W2"] for w in heads], dplan, head_logits,
                  head_lse, cand_tok, cand_logp, head_hidden)
    for k, w in enumerate(heads):
        want = {"Wa": (d, d) if k == 0 else (hidden_dim, 2 * d), "ba": (d,) if k == 0 else (hidden_dim,),
                "ln_g": (d,), "ln_b": (d,)}
        if k > 0:
            want.update(Wb=(d, hidden_dim), bb=(d,))
        _shapes("hydra_draft_heads_sketch", **{f"heads[{k}].{n}": (w[n], sh) for n, sh in want.items()})
    arr = C.c_void_p * n_heads

    def col(name, first=True):
        return arr(*[_dev(w[name], name, h.dtype) if (first or k > 0) else None for k, w in enumerate(heads)])

    dt |= _vocab_flag("hydra_draft_heads_sketch", [w["W2"] for w in heads])

    rows = dplan.rows
    rf, rfp = _host_i32(rows.row_first)
    df, dfp = _host_i32(rows.depth_first)
    kp, kpp = _host_i32(rows.k_per_depth)
    wsp, wsb = _ws(ws)
    rc = lib().hydra_draft_heads_sketch(
        dt, B, d, V, hidden_dim, _dev(h, "h"), _dev(root_tok, "root_tok", torch.int32), _dev(emb, "emb", h.dtype),
        n_heads, col("Wa"), col("ba"), col("Wb", False), col("bb", False), col("ln_g"), col("ln_b"), col("W2"),
        float(ln_eps), dplan.N, dplan.dmax, _dev(dplan.parent, "parent"), _dev(dplan.rank, "rank"),
        _dev(dplan.node_row, "node_row"), dplan.R, _dev(dplan.row_node, "row_node"), rfp, dfp, kpp,
        _dev(head_logits, "head_logits", torch.float32), _dev(head_lse, "head_lse", torch.float32),
        _dev(head_hidden, "head_hidden", h.dtype), _dev(cand_tok, "cand_tok", torch.int32),
        _dev(cand_logp, "cand_logp", torch.float32), wsp, wsb, _stream(stream))
    return _check("hydra_draft_heads_sketch", rc)


def hydra_draft_heads_attn_workspace_size(dtype_code, B, d, V, dplan: DevicePlan):
    rf, rfp = _host_i32(dplan.rows.row_first)
    return int(lib().hydra_draft_heads_attn_workspace_size(dtype_code, B, d, V, dplan.N, dplan.dmax, rfp))


def hydra_draft_heads_attn(h, root_tok, emb, Wqkv, Wo, W1, b1, W2, dplan: DevicePlan, head_logits, head_lse,
                           cand_tok, cand_logp, ws, head_hidden=None, residual=True, stream=None):
    """Stage 1 with Hydra++ self-attention fusion (see include/hydra.h).
    Wqkv [3d, d] (Wq, Wk, Wv rows), Wo [d, d]; W1/b1/W2 as hydra_draft_heads."""
    if not dplan.hydra:
        raise ValueError("self-attention fusion reads the candidate embeddings: the plan must be a Hydra plan")
    dt = _dtype_code(h)
    B, d = h.shape
    V = W2[0].shape[0]
    n_heads = len(W2)
    if not (len(W1) == len(b1) == n_heads):
        raise ValueError("W1, b1 and W2 need one entry per head")
    _draft_shapes("hydra_draft_heads_attn", h, root_tok, emb, W2, dplan, head_logits, head_lse, cand_tok, cand_logp,
                  head_hidden)
    _shapes("hydra_draft_heads_attn", Wqkv=(Wqkv, (3 * d, d)), Wo=(Wo, (d, d)))
    for k in range(n_heads):
        _shapes("hydra_draft_heads_attn", **{f"W1[{k}]": (W1[k], (d, 2 * d)), f"b1[{k}]": (b1[k], (d,))})
    arr = C.c_void_p * n_heads
    w1 = arr(*[_dev(w, "W1", h.dtype) for w in W1])
    bb = arr(*[_dev(w, "b1", h.dtype) for w in b1])
    w2 = arr(*[_dev(w, "W2", h.dtype) for w in W2])
    dt |= _vocab_flag("draft heads", W2)
    rows = dplan.rows
    rf, rfp = _host_i32(rows.row_first)
    df, dfp = _host_i32(rows.depth_first)
    kp, kpp = _host_i32(rows.k_per_depth)
    wsp, wsb = _ws(ws)
    rc = lib().hydra_draft_heads_attn(
        dt, B, d, V, int(bool(residual)), _dev(h, "h"), _dev(root_tok, "root_tok", torch.int32),
        _dev(emb, "emb", h.dtype), _dev(Wqkv, "Wqkv", h.dtype), _dev(Wo, "Wo", h.dtype), n_heads, w1, bb, w2,
        dplan.N, dplan.dmax, _dev(dplan.parent, "parent"), _dev(dplan.rank, "rank"), _dev(dplan.node_row, "node_row"),
        dplan.R, _dev(dplan.row_node, "row_node"), rfp, dfp, kpp, _dev(head_logits, "head_logits", torch.float32),
        _dev(head_lse, "head_lse", torch.float32), _dev(head_hidden, "head_hidden", h.dtype),
        _dev(cand_tok, "cand_tok", torch.int32), _dev(cand_logp, "cand_logp", torch.float32), wsp, wsb,
        _stream(stream))
    return _check("hydra_draft_heads_attn", rc)


def hydra_fold_embedding(emb, W1, out, stream=None):
    """out[t, n] = sum_j W1[n, d + j] * emb[t, j] (see include/hydra.h):
    emb [V, d] and W1 [d, 2d] bf16, out [V, d] float32."""
    V, d = emb.shape
    if tuple(W1.shape) != (d, 2 * d) or tuple(out.shape) != (V, d):
        raise ValueError(f"fold_embedding: W1 {tuple(W1.shape)} / out {tuple(out.shape)} do not match emb {(V, d)}")
    rc = lib().hydra_fold_embedding(_dtype_code(emb), V, d, _dev(emb, "emb"), _dev(W1, "W1", emb.dtype),
                                    _dev(out, "out", torch.float32), _stream(stream))
    return _check("hydra_fold_embedding", rc)


def hydra_vocab_projection_workspace_size(M, N, k):
    return int(lib().hydra_vocab_projection_workspace_size(M, N, k))


def hydra_vocab_projection(X, W, Y, k=0, ws=None, stream=None):
    """Y[M, N] = X[M, K] . W[N, K]^T in float32; with k > 0 also the fused
    top-k partials in ws (finish with hydra_vocab_topk)."""
    M, K = X.shape
    N = W.shape[0]
    _shapes("hydra_vocab_projection", W=(W, (N, K)), Y=(Y, (M, N)))
    wsp, wsb = _ws(ws)
    rc = lib().hydra_vocab_projection(_dtype_code(X) | _vocab_flag("hydra_vocab_projection", [W]), M, K, N, int(k),
                                      _dev(X, "X"), _dev(W, "W", X.dtype),
                                      _dev(Y, "Y", torch.float32), wsp, wsb, _stream(stream))
    return _check("hydra_vocab_projection", rc)


def hydra_vocab_topk(M, N, k, Y, ws, lse=None, ids=None, vals=None, stream=None):
    """Per-row log-sum-exp and sorted top-k from a k > 0 projection's logits Y
    and workspace."""
    _shapes("hydra_vocab_topk", Y=(Y, (M, N)), lse=(lse, (M,)), ids=(ids, (M, k)), vals=(vals, (M, k)))
    wsp, wsb = _ws(ws)
    rc = lib().hydra_vocab_topk(int(M), int(N), int(k), _dev(Y, "Y", torch.float32), wsp, wsb,
                                _dev(lse, "lse", torch.float32),
                                _dev(ids, "ids", torch.int32), _dev(vals, "vals", torch.float32), _stream(stream))
    return _check("hydra_vocab_topk", rc)


def tree_build_workspace_size(B, N, n_keep):
    return int(lib().tree_build_workspace_size(B, N, n_keep))


def tree_build(dplan: DevicePlan, cand_tok, cand_logp, n_keep, tok, parent, depth, anc, q_row, src,
               ws=None, stream=None):
    """Stage 2 (see include/hydra.h)."""
    B = cand_tok.shape[0]
    K = int(n_keep)
    _shapes("tree_build", cand_tok=(cand_tok, (B, dplan.N)), cand_logp=(cand_logp, (B, dplan.N)), tok=(tok, (B, K)),
            parent=(parent, (B, K)), depth=(depth, (B, K)), anc=(anc, (B, K, dplan.dmax + 1)), q_row=(q_row, (B, K)),
            src=(src, (B, K)))
    wsp, wsb = _ws(ws)
    rc = lib().tree_build(B, dplan.N, dplan.dmax, _dev(dplan.parent, "parent"), _dev(dplan.rank, "rank"),
                          _dev(dplan.depth, "depth"), _dev(dplan.node_row, "node_row"),
                          _dev(cand_tok, "cand_tok", torch.int32), _dev(cand_logp, "cand_logp", torch.float32),
                          int(n_keep), _dev(tok, "tok", torch.int32), _dev(parent, "parent", torch.int32),
                          _dev(depth, "depth", torch.int32), _dev(anc, "anc", torch.int32),
                          _dev(q_row, "q_row", torch.int32), _dev(src, "src", torch.int32), wsp, wsb,
                          _stream(stream))
    return _check("tree_build", rc)


def tree_rope(x, depth, prefix_len, out=None, theta=10000.0, stream=None):
    """Rotary embedding of the tree rows x [B, N, H, D] at positions
    prefix_len + depth (see include/hydra.h); out defaults to x (in place)."""
    B, N, H, D = x.shape
    if out is None:
        out = x
    if tuple(out.shape) != tuple(x.shape) or tuple(depth.shape) != (B, N) or tuple(prefix_len.shape) != (B,):
        raise ValueError(f"tree_rope: shapes x {tuple(x.shape)}, out {tuple(out.shape)}, depth "
                         f"{tuple(depth.shape)}, prefix_len {tuple(prefix_len.shape)}")
    rc = lib().tree_rope(_dtype_code(x), B, N, H, D, _dev(x, "x"), _dev(out, "out", x.dtype),
                         _dev(depth, "depth", torch.int32), _dev(prefix_len, "prefix_len", torch.int32), float(theta),
                         _stream(stream))
    return _check("tree_rope", rc)


def tree_rope_qk(q, k, depth, prefix_len, q_out=None, k_out=None, theta=10000.0, stream=None):
    """tree_rope of the tree Q [B, N, Hq, D] and K [B, N, Hkv, D] rows in one
    launch (see include/hydra.h); the outputs default to the inputs."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    q_out = q if q_out is None else q_out
    k_out = k if k_out is None else k_out
    if (tuple(k.shape) != (B, N, Hkv, D) or tuple(q_out.shape) != tuple(q.shape)
            or tuple(k_out.shape) != tuple(k.shape) or tuple(depth.shape) != (B, N) or tuple(prefix_len.shape) != (B,)):
        raise ValueError(f"tree_rope_qk: shapes q {tuple(q.shape)}, k {tuple(k.shape)}, depth {tuple(depth.shape)}")
    rc = lib().tree_rope_qk(_dtype_code(q), B, N, Hq, Hkv, D, _dev(q, "q"), _dev(q_out, "q_out", q.dtype),
                            _dev(k, "k", q.dtype), _dev(k_out, "k_out", q.dtype), _dev(depth, "depth", torch.int32),
                            _dev(prefix_len, "prefix_len", torch.int32), float(theta), _stream(stream))
    return _check("tree_rope_qk", rc)


def tree_attention_verify_workspace_size(dtype_code, B, N, Hq, Hkv, D, max_prefix_len):
    return int(lib().tree_attention_verify_workspace_size(dtype_code, B, N, Hq, Hkv, D, max_prefix_len))


def tree_attention_verify(q, k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, max_prefix_len,
                          anc, depth, out, lse=None, ws=None, scale=None, stream=None):
    """Stage 3 (see include/hydra.h). q [B, N, Hq, D]; pages [n_pages, Hkv, page, D]."""
    B, N, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    if k_pages.dim() != 4 or anc.dim() != 3 or block_table.dim() != 2:
        raise ValueError("tree_attention_verify: pages [n_pages, Hkv, page, D], anc [B, N, Dmax + 1] and "
                         "block_table [B, max_pages] expected")
    n_pages, _, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    Dmax = anc.shape[2] - 1
    _shapes("tree_attention_verify", k_tree=(k_tree, (B, N, Hkv, D)), v_tree=(v_tree, (B, N, Hkv, D)),
            k_pages=(k_pages, (n_pages, Hkv, page_size, D)), v_pages=(v_pages, (n_pages, Hkv, page_size, D)),
            block_table=(block_table, (B, max_pages)), prefix_len=(prefix_len, (B,)), anc=(anc, (B, N, Dmax + 1)),
            depth=(depth, (B, N)), out=(out, (B, N, Hq, D)), lse=(lse, (B, N, Hq)))
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    wsp, wsb = _ws(ws)
    rc = lib().tree_attention_verify(
        _dtype_code(q), B, N, Hq, Hkv, D, float(scale), _dev(q, "q"), _dev(k_tree, "k_tree", q.dtype),
        _dev(v_tree, "v_tree", q.dtype), _dev(k_pages, "k_pages", q.dtype), _dev(v_pages, "v_pages", q.dtype),
        n_pages, page_size, _dev(block_table, "block_table", torch.int32), max_pages,
        _dev(prefix_len, "prefix_len", torch.int32), int(max_prefix_len), _dev(anc, "anc", torch.int32),
        _dev(depth, "depth", torch.int32), Dmax, _dev(out, "out", q.dtype), _dev(lse, "lse", torch.float32),
        wsp, wsb, _stream(stream))
    return _check("tree_attention_verify", rc)


def tree_decoder_layer_workspace_size(dtype_code, B, N, d, Hq, Hkv, D, F, max_prefix_len):
    return int(lib().tree_decoder_layer_workspace_size(dtype_code, B, N, d, Hq, Hkv, D, F, max_prefix_len))


def tree_decoder_layer(x, w, Hq, Hkv, k_pages, v_pages, block_table, prefix_len, max_prefix_len, anc, depth,
                       x_out, k_tree, v_tree, ws, eps=1e-6, theta=10000.0, stream=None):
    """The target's decoder layer over the tree rows (see include/hydra.h).
    x [B, N, d]; w: dict of ln1 [d], Wqkv [(Hq + 2 Hkv) D, d], Wo [d, Hq D],
    ln2 [d], Wgu [2F, d], Wd [d, F]; pages [n_pages, Hkv, page, D]."""
    B, N, d = x.shape
    D = k_tree.shape[3]
    F = w["Wd"].shape[1]
    n_pages, _, page_size, _ = k_pages.shape
    shapes = {"Wqkv": ((Hq + 2 * Hkv) * D, d), "Wo": (d, Hq * D), "ln1": (d,), "ln2": (d,), "Wgu": (2 * F, d),
              "Wd": (d, F)}
    for name, shape in shapes.items():
        if tuple(w[name].shape) != shape:
            raise ValueError(f"tree_decoder_layer: {name} has shape {tuple(w[name].shape)}, expected {shape}")
    for name, t, shape in (("x_out", x_out, (B, N, d)), ("k_tree", k_tree, (B, N, Hkv, D)),
                           ("v_tree", v_tree, (B, N, Hkv, D)), ("anc", anc, (B, N, anc.shape[2])),
                           ("depth", depth, (B, N)), ("prefix_len", prefix_len, (B,))):
        if tuple(t.shape) != shape:
            raise ValueError(f"tree_decoder_layer: {name} has shape {tuple(t.shape)}, expected {shape}")
    dt = x.dtype
    wsp, wsb = _ws(ws)
    rc = lib().tree_decoder_layer(
        _dtype_code(x) | _vocab_flag("tree_decoder_layer", [w[n] for n in ("Wqkv", "Wo", "Wgu", "Wd")],
                                     HYDRA_LAYER_PACKED), B, N, d, Hq, Hkv, D, F, _dev(x, "x"), _dev(w["ln1"], "ln1", dt), _dev(w["Wqkv"], "Wqkv", dt),
        _dev(w["Wo"], "Wo", dt), _dev(w["ln2"], "ln2", dt), _dev(w["Wgu"], "Wgu", dt), _dev(w["Wd"], "Wd", dt),
        float(eps), float(theta), _dev(k_pages, "k_pages", dt), _dev(v_pages, "v_pages", dt), n_pages, page_size,
        _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(prefix_len, "prefix_len", torch.int32), int(max_prefix_len), _dev(anc, "anc", torch.int32),
        _dev(depth, "depth", torch.int32), anc.shape[2] - 1, _dev(x_out, "x_out", dt), _dev(k_tree, "k_tree", dt),
        _dev(v_tree, "v_tree", dt), wsp, wsb, _stream(stream))
    return _check("tree_decoder_layer", rc)


def tree_verify_layers_workspace_size(dtype_code, B, N, d, Hq, Hkv, D, F, max_prefix_len):
    return int(lib().tree_verify_layers_workspace_size(dtype_code, B, N, d, Hq, Hkv, D, F, max_prefix_len))


def tree_verify_layers(tok, emb, w, ln_f, Hq, Hkv, k_pages, v_pages, block_table, prefix_len, max_prefix_len, anc,
                       depth, h_out, k_tree, v_tree, ws, eps=1e-6, theta=10000.0, stream=None):
    """The target's forward pass over the tree rows (see include/hydra.h):
    embeddings of tok, every decoder layer, final norm. w: dict of
    layer-stacked ln1 [n, d], Wqkv [n, (Hq + 2 Hkv) D, d], Wo [n, d, Hq D],
    ln2 [n, d], Wgu [n, 2F, d], Wd [n, d, F]; pages [n, n_pages, Hkv, page, D];
    k_tree, v_tree [n, B, N, Hkv, D]; h_out [B, N, d]."""
    B, N = tok.shape
    V, d = emb.shape
    n = w["Wqkv"].shape[0]
    D = k_tree.shape[4]
    F = w["Wd"].shape[2]
    n_pages, page_size = k_pages.shape[1], k_pages.shape[3]
    dt = emb.dtype
    _shapes("tree_verify_layers", ln1=(w["ln1"], (n, d)), Wqkv=(w["Wqkv"], (n, (Hq + 2 * Hkv) * D, d)),
            Wo=(w["Wo"], (n, d, Hq * D)), ln2=(w["ln2"], (n, d)), Wgu=(w["Wgu"], (n, 2 * F, d)),
            Wd=(w["Wd"], (n, d, F)), ln_f=(ln_f, (d,)), k_pages=(k_pages, (n, n_pages, Hkv, page_size, D)),
            v_pages=(v_pages, (n, n_pages, Hkv, page_size, D)), h_out=(h_out, (B, N, d)),
            k_tree=(k_tree, (n, B, N, Hkv, D)), v_tree=(v_tree, (n, B, N, Hkv, D)),
            anc=(anc, (B, N, anc.shape[2])), depth=(depth, (B, N)), prefix_len=(prefix_len, (B,)),
            block_table=(block_table, (B, block_table.shape[1])))
    wsp, wsb = _ws(ws)
    rc = lib().tree_verify_layers(
        _dtype_code(emb) | _vocab_flag("tree_verify_layers", [w[n] for n in ("Wqkv", "Wo", "Wgu", "Wd")],
                                       HYDRA_LAYER_PACKED), n, B, N, d, Hq, Hkv, D, F, V, _dev(tok, "tok", torch.int32), _dev(emb, "emb"),
        _dev(w["ln1"], "ln1", dt), _dev(w["Wqkv"], "Wqkv", dt), _dev(w["Wo"], "Wo", dt), _dev(w["ln2"], "ln2", dt),
        _dev(w["Wgu"], "Wgu", dt), _dev(w["Wd"], "Wd", dt), _dev(ln_f, "ln_f", dt), float(eps), float(theta),
        _dev(k_pages, "k_pages", dt), _dev(v_pages, "v_pages", dt), n_pages, page_size,
        _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(prefix_len, "prefix_len", torch.int32), int(max_prefix_len), _dev(anc, "anc", torch.int32),
        _dev(depth, "depth", torch.int32), anc.shape[2] - 1, _dev(h_out, "h_out", dt), _dev(k_tree, "k_tree", dt),
        _dev(v_tree, "v_tree", dt), wsp, wsb, _stream(stream))
    return _check("tree_verify_layers", rc)


def tree_accept_workspace_size(mode, B, N, V):
    return int(lib().tree_accept_workspace_size(mode, B, N, V))


def tree_accept(o, W_t, tok, parent, target_logits, n_accepted, path, out_tok, ws, mode=0, temperature=1.0,
                q_row=None, head_logits=None, u_acc=None, u_res=None, eps=None, delta=None, stream=None):
    """Stage 4 (see include/hydra.h). o [B, N, d]; mode 0 greedy, 1 rejection,
    2 typical (needs eps and delta)."""
    if mode == 2 and (eps is None or delta is None):
        raise ValueError("tree_accept: typical acceptance needs eps and delta")
    B, N, d = o.shape
    V = W_t.shape[0]
    if W_t.dim() != 2 or W_t.shape[1] != d:
        raise ValueError(f"tree_accept: W_t {tuple(W_t.shape)} does not take rows of width {d} (o {tuple(o.shape)})")
    if tuple(target_logits.shape) != (B, N, V):
        raise ValueError(f"tree_accept: target_logits {tuple(target_logits.shape)}, expected {(B, N, V)}")
    Dmax = path.shape[1] - 1
    R = head_logits.shape[1] if head_logits is not None else 0
    _shapes("tree_accept", tok=(tok, (B, N)), parent=(parent, (B, N)), q_row=(q_row, (B, N)),
            head_logits=(head_logits, (B, R, V)), u_acc=(u_acc, (B, N)), u_res=(u_res, (B, N)),
            n_accepted=(n_accepted, (B,)), path=(path, (B, Dmax + 1)), out_tok=(out_tok, (B, Dmax + 1)))
    wsp, wsb = _ws(ws)
    rc = lib().tree_accept(
        _dtype_code(o) | _vocab_flag("tree_accept", [W_t]), int(mode), B, N, d, V, Dmax, _dev(o, "o"),
        _dev(W_t, "W_t", o.dtype), float(temperature),
        float(eps or 0.0), float(delta or 0.0), _dev(tok, "tok", torch.int32), _dev(parent, "parent", torch.int32), _dev(q_row, "q_row", torch.int32),
        _dev(head_logits, "head_logits", torch.float32), R, _dev(u_acc, "u_acc", torch.float32),
        _dev(u_res, "u_res", torch.float32), _dev(target_logits, "target_logits", torch.float32),
        _dev(n_accepted, "n_accepted", torch.int32), _dev(path, "path", torch.int32),
        _dev(out_tok, "out_tok", torch.int32), wsp, wsb, _stream(stream))
    return _check("tree_accept", rc)


def tree_accept_noalloc(o, W_t, tok, parent, target_logits, n_accepted, path, out_tok, mode=0, temperature=1.0,
                        q_row=None, head_logits=None, u_acc=None, u_res=None, eps=None, delta=None, stream=None):
    """tree_accept with the library's per-GPU scratch instead of a workspace
    (see include/hydra.h): for callers that cannot allocate."""
    if mode == 2 and (eps is None or delta is None):
        raise ValueError("tree_accept_noalloc: typical acceptance needs eps and delta")
    B, N, d = o.shape
    V = W_t.shape[0]
    if W_t.dim() != 2 or W_t.shape[1] != d:
        raise ValueError(f"tree_accept_noalloc: W_t {tuple(W_t.shape)} does not take rows of width {d}")
    Dmax = path.shape[1] - 1
    R = head_logits.shape[1] if head_logits is not None else 0
    _shapes("tree_accept_noalloc", target_logits=(target_logits, (B, N, V)), tok=(tok, (B, N)),
            parent=(parent, (B, N)), q_row=(q_row, (B, N)), head_logits=(head_logits, (B, R, V)),
            u_acc=(u_acc, (B, N)), u_res=(u_res, (B, N)), n_accepted=(n_accepted, (B,)), path=(path, (B, Dmax + 1)),
            out_tok=(out_tok, (B, Dmax + 1)))
    rc = lib().tree_accept_noalloc(
        _dtype_code(o) | _vocab_flag("tree_accept", [W_t]), int(mode), B, N, d, V, Dmax, _dev(o, "o"),
        _dev(W_t, "W_t", o.dtype), float(temperature),
        float(eps or 0.0), float(delta or 0.0), _dev(tok, "tok", torch.int32), _dev(parent, "parent", torch.int32),
        _dev(q_row, "q_row", torch.int32), _dev(head_logits, "head_logits", torch.float32), R,
        _dev(u_acc, "u_acc", torch.float32), _dev(u_res, "u_res", torch.float32),
        _dev(target_logits, "target_logits", torch.float32), _dev(n_accepted, "n_accepted", torch.int32),
        _dev(path, "path", torch.int32), _dev(out_tok, "out_tok", torch.int32), _stream(stream))
    return _check("tree_accept_noalloc", rc)


def tree_commit(k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, n_accepted, path, out_tok,
                next_prefix_len, next_root_tok, hidden=None, next_h=None, stream=None):
    """Kept branch into the paged KV cache (see include/hydra.h).

    k_tree/v_tree [B, N, Hkv, D] or [n_layers, B, N, Hkv, D]; k_pages/v_pages
    [n_pages, Hkv, page, D] or [n_layers, n_pages, Hkv, page, D] (in/out);
    hidden [B, N, d] and next_h [B, d] optional."""
    if k_tree.dim() == 4:
        k_tree, v_tree = k_tree.unsqueeze(0), v_tree.unsqueeze(0)
    if k_pages.dim() == 4:
        k_pages, v_pages = k_pages.unsqueeze(0), v_pages.unsqueeze(0)
    n_layers, B, N, Hkv, D = k_tree.shape
    if k_pages.shape[0] != n_layers or tuple(k_pages.shape[2:]) != (Hkv, k_pages.shape[3], D):
        raise ValueError(f"tree_commit: pages {tuple(k_pages.shape)} do not match tree K/V {tuple(k_tree.shape)}")
    n_pages, page_size = k_pages.shape[1], k_pages.shape[3]
    max_pages = block_table.shape[1]
    Dmax = path.shape[1] - 1
    d = hidden.shape[2] if hidden is not None else 0
    want = {"v_tree": (v_tree, tuple(k_tree.shape)), "v_pages": (v_pages, tuple(k_pages.shape)),
            "block_table": (block_table, (B, max_pages)), "prefix_len": (prefix_len, (B,)),
            "n_accepted": (n_accepted, (B,)), "path": (path, (B, Dmax + 1)), "out_tok": (out_tok, (B, Dmax + 1)),
            "next_prefix_len": (next_prefix_len, (B,)), "next_root_tok": (next_root_tok, (B,))}
    if hidden is not None:
        want["hidden"] = (hidden, (B, N, d))
        if next_h is not None:
            want["next_h"] = (next_h, (B, d))
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape:
            raise ValueError(f"tree_commit: {name} has shape {tuple(t.shape)}, expected {shape}")
    dt = k_tree.dtype
    rc = lib().tree_commit(
        _dtype_code(k_tree), n_layers, B, N, Hkv, D, Dmax, _dev(k_tree, "k_tree"), _dev(v_tree, "v_tree", dt),
        _dev(k_pages, "k_pages", dt), _dev(v_pages, "v_pages", dt), n_pages, page_size,
        _dev(block_table, "block_table", torch.int32), max_pages, _dev(prefix_len, "prefix_len", torch.int32),
        _dev(n_accepted, "n_accepted", torch.int32), _dev(path, "path", torch.int32),
        _dev(out_tok, "out_tok", torch.int32), d, _dev(hidden, "hidden", dt),
        _dev(next_prefix_len, "next_prefix_len", torch.int32), _dev(next_root_tok, "next_root_tok", torch.int32),
        _dev(next_h, "next_h", dt), _stream(stream))
    return _check("tree_commit", rc)
