"""One draft-and-verify round: buffers plus the library calls in order (the
four stages, then the commit of the kept branch into the KV cache).

Allocation and sequencing only; every step of the round runs in libhydra's
kernels. Buffers are allocated once per shape so a round can be replayed (or
captured in a HIP graph) without allocating.
"""
from __future__ import annotations

import torch

from . import hydra as H


def make_plan(tree):
    """Tree plan from a spec: ("cartesian", b), ("sparse", caps, n_nodes) or
    ("dense", b, n_keep). Returns (plan, n_keep)."""
    kind = tree[0]
    if kind == "cartesian":
        p = H.hydra_plan_cartesian(tree[1])
        return p, p.n
    if kind == "sparse":
        p = H.hydra_plan_sparse(tree[1], tree[2])
        return p, p.n
    if kind == "dense":
        return H.hydra_plan_cartesian(tree[1]), int(tree[2])
    raise ValueError(f"unknown tree kind {kind!r}")


class HydraRound:
    """Buffers and calls for one round of B sequences.

    weights: dict with emb [V, d] (Hydra), W1/b1/W2 lists, W_t [V, d]; or,
    for the two-layer LayerNorm heads (hydra_draft_heads_sketch), ``heads``:
    one dict per head (Wa, ba, [Wb, bb,] ln_g, ln_b, W2) instead of W1/b1/W2;
    with ``attn`` (dict of Wqkv [3d, d] and Wo [d, d]) the Hydra heads read
    Hydra++ self-attention fusion of the path embeddings
    (hydra_draft_heads_attn).
    shape: dict with B, d, V, Hq, Hkv, D, max_prefix_len.
    fold_embedding: build the folded embedding tables of the Hydra heads
    (hydra_fold_embedding, V * d * 4 bytes per head) once here and let the
    draft stage look the embedding half up; None folds for bf16 Hydra heads.
    full_path: Hydra heads read the embeddings of the whole path from the
    root (W1 of head k is [d, (k + 1) d]); never folded.
    pack_vocab: keep the vocabulary projection weights (the heads' W2 and
    W_t) and the target layers' weights in the packed layout
    (hydra_pack_weight, one copy each made here); None packs them for bf16
    with d % 256 == 0.
    rope_theta: rotate the tree Q/K rows at positions prefix_len + depth
    (tree_rope) before attention; None gives the rows to attention as they are.
    With ``target`` in weights (layer-stacked ln1, Wqkv, Wo, ln2, Wgu, Wd, the
    final norm gain ln_f and the embedding table emb) the verification runs
    the target's decoder layers over the tree tokens (tree_verify_layers)
    instead of one attention layer over given Q/K/V; the pools are then
    layer-stacked and the commit writes every layer's K/V.
    """

    def __init__(self, weights, tree, shape, hydra=True, mode=0, temperature=1.0, residual=True,
                 keep_hidden=False, device="cuda", fold_embedding=None, eps=None, delta=None, rope_theta=10000.0,
                 full_path=False, pack_vocab=None):
        self.w = weights
        plan, n_keep = make_plan(tree)
        self.dplan = H.DevicePlan(plan, hydra, device)
        self.n_keep = n_keep
        self.hydra, self.mode, self.T, self.residual = hydra, int(mode), float(temperature), residual
        self.eps, self.delta = eps, delta  # typical acceptance (mode 2)
        B, d, V = shape["B"], shape["d"], shape["V"]
        Hq, Hkv, D = shape["Hq"], shape["Hkv"], shape["D"]
        self.shape = dict(shape)
        dt = weights["W_t"].dtype
        self.dtype = dt
        code = H.HYDRA_F32 if dt == torch.float32 else H.HYDRA_BF16
        N, R, Dm, K = self.dplan.N, self.dplan.R, self.dplan.dmax, n_keep
        i32, f32 = torch.int32, torch.float32
        z = lambda *s, dtype=f32: torch.empty(*s, dtype=dtype, device=device)  # noqa: E731
        self.head_logits = z(B, R, V)
        self.head_lse = z(B, R)
        self.head_hidden = z(B, R, d, dtype=dt) if keep_hidden else None
        self.cand_tok = z(B, N, dtype=i32)
        self.cand_logp = z(B, N)
        self.tok, self.parent, self.depth = z(B, K, dtype=i32), z(B, K, dtype=i32), z(B, K, dtype=i32)
        self.q_row, self.src = z(B, K, dtype=i32), z(B, K, dtype=i32)
        self.anc = z(B, K, Dm + 1, dtype=i32)
        self.attn_out = z(B, K, Hq, D, dtype=dt)
        self.rope_theta = rope_theta
        self.q_rot = z(B, K, Hq, D, dtype=dt) if rope_theta else None
        self.k_rot = z(B, K, Hkv, D, dtype=dt) if rope_theta else None
        self.attn_lse = z(B, K, Hq)
        self.target_logits = z(B, K, V)
        self.target = weights.get("target")
        self.hidden = self.k_layers = self.v_layers = None
        if self.target is not None:
            n_layers, F = self.target["Wqkv"].shape[0], self.target["Wd"].shape[2]
            self.hidden = z(B, K, d, dtype=dt)
            self.k_layers = z(n_layers, B, K, Hkv, D, dtype=dt)
            self.v_layers = z(n_layers, B, K, Hkv, D, dtype=dt)
        self.n_accepted = z(B, dtype=i32)
        self.path = z(B, Dm + 1, dtype=i32)
        self.out_tok = z(B, Dm + 1, dtype=i32)
        # handed to the next round by the commit
        self.next_prefix_len = z(B, dtype=i32)
        self.next_root_tok = z(B, dtype=i32)
        self.next_h = z(B, Hq * D, dtype=dt)
        nb = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)  # noqa: E731
        self.sketch = weights.get("heads") is not None
        self.full_path = bool(full_path)
        self.attn = weights.get("attn")
        if self.attn is not None:
            self.ws_draft = nb(H.hydra_draft_heads_attn_workspace_size(code, B, d, V, self.dplan))
        elif self.sketch:
            hid = weights["heads"][1]["Wa"].shape[0] if len(weights["heads"]) > 1 else d
            self.ws_draft = nb(H.hydra_draft_heads_sketch_workspace_size(code, B, d, V, hid, self.dplan))
        else:
            self.ws_draft = nb(H.hydra_draft_heads_workspace_size(code, B, d, V, 2 if full_path else hydra,
                                                                  self.dplan))
        self.ws_build = nb(H.tree_build_workspace_size(B, N, K))
        self.ws_attn = nb(H.tree_attention_verify_workspace_size(code, B, K, Hq, Hkv, D,
                                                                 shape["max_prefix_len"]))
        self.ws_accept = nb(H.tree_accept_workspace_size(self.mode, B, K, V))
        if self.target is not None:
            self.ws_verify = nb(H.tree_verify_layers_workspace_size(code, B, K, d, Hq, Hkv, D, F,
                                                                    shape["max_prefix_len"]))
        if fold_embedding is None:
            fold_embedding = hydra and dt == torch.bfloat16 and not self.sketch and not self.full_path
            fold_embedding = fold_embedding and self.attn is None
        if pack_vocab is None:
            pack_vocab = dt == torch.bfloat16 and d % 256 == 0
        self.pack_vocab = bool(pack_vocab)
        pk = H.hydra_pack_weight if self.pack_vocab else (lambda W: W)  # noqa: E731
        self.W_t = pk(weights["W_t"])
        if self.target is not None and self.pack_vocab:
            # the decoder layers' products stream their weights the same way
            self.target = dict(self.target, **{n: H.hydra_pack_weight(self.target[n])
                                               for n in ("Wqkv", "Wo", "Wgu", "Wd")})
        if self.sketch:
            self.heads = [dict(hd, W2=pk(hd["W2"])) for hd in weights["heads"]]
        else:
            self.W2 = [pk(W) for W in weights["W2"]]
        self.emb_proj = None
        self.W1h = None
        if fold_embedding:
            self.emb_proj = [z(V, d) for _ in weights["W1"]]
            for w1, t in zip(weights["W1"], self.emb_proj):
                H.hydra_fold_embedding(weights["emb"], w1, t)
            # the folded round reads only the h halves of W1: packed, they
            # stream at the packed layout's rate
            # (only where the library takes the folded path: bf16, d % 256 == 0,
            # at most 16 sequences)
            if self.pack_vocab and d % 256 == 0 and shape["B"] <= 16:
                self.W1h = [H.hydra_pack_weight(w1[:, :d].contiguous()) for w1 in weights["W1"]]

    def draft(self, h, root_tok, stream=None):
        if self.attn is not None:
            H.hydra_draft_heads_attn(h, root_tok, self.w["emb"], self.attn["Wqkv"], self.attn["Wo"], self.w["W1"],
                                     self.w["b1"], self.W2, self.dplan, self.head_logits, self.head_lse,
                                     self.cand_tok, self.cand_logp, self.ws_draft, head_hidden=self.head_hidden,
                                     residual=self.residual, stream=stream)
            return
        if self.sketch:
            H.hydra_draft_heads_sketch(h, root_tok, self.w["emb"], self.heads, self.dplan, self.head_logits,
                                       self.head_lse, self.cand_tok, self.cand_logp, self.ws_draft,
                                       head_hidden=self.head_hidden, stream=stream)
            return
        H.hydra_draft_heads(h, root_tok, self.w.get("emb"), self.W1h or self.w["W1"], self.w["b1"], self.W2, self.dplan,
                            self.head_logits, self.head_lse, self.cand_tok, self.cand_logp, self.ws_draft,
                            head_hidden=self.head_hidden, residual=self.residual, emb_proj=self.emb_proj,
                            full_path=self.full_path, stream=stream)

    def build(self, stream=None):
        H.tree_build(self.dplan, self.cand_tok, self.cand_logp, self.n_keep, self.tok, self.parent, self.depth,
                     self.anc, self.q_row, self.src, self.ws_build, stream=stream)

    def attend(self, q, k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, stream=None):
        if self.rope_theta:
            H.tree_rope_qk(q, k_tree, self.depth, prefix_len, q_out=self.q_rot, k_out=self.k_rot,
                           theta=self.rope_theta, stream=stream)
            q, k_tree = self.q_rot, self.k_rot
        H.tree_attention_verify(q, k_tree, v_tree, k_pages, v_pages, block_table, prefix_len,
                                self.shape["max_prefix_len"], self.anc, self.depth, self.attn_out, self.attn_lse,
                                self.ws_attn, stream=stream)

    def verify(self, k_pages, v_pages, block_table, prefix_len, stream=None):
        """The target's forward pass over the tree tokens: every layer's
        rotated K/V into k_layers / v_layers, the final hidden states into
        hidden."""
        t = self.target
        H.tree_verify_layers(self.tok, t["emb"], t, t["ln_f"], self.shape["Hq"], self.shape["Hkv"], k_pages,
                             v_pages, block_table, prefix_len, self.shape["max_prefix_len"], self.anc, self.depth,
                             self.hidden, self.k_layers, self.v_layers, self.ws_verify, eps=t.get("eps", 1e-6),
                             theta=self.rope_theta or 10000.0, stream=stream)

    def rows(self):
        """[B, N, d] hidden states of the tree rows that the target projection
        reads: the final layer's output, or the attention output."""
        if self.target is not None:
            return self.hidden
        B, K = self.attn_out.shape[:2]
        return self.attn_out.view(B, K, -1)

    def accept(self, u_acc=None, u_res=None, stream=None):
        H.tree_accept(self.rows(), self.W_t, self.tok, self.parent, self.target_logits,
                      self.n_accepted, self.path, self.out_tok, self.ws_accept, mode=self.mode,
                      temperature=self.T, q_row=self.q_row, head_logits=self.head_logits, u_acc=u_acc,
                      u_res=u_res, eps=self.eps, delta=self.delta, stream=stream)

    def commit(self, k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, stream=None):
        """Root and accepted rows into the paged cache (in place); next
        prefix lengths, roots and hidden states into next_*."""
        if self.target is not None:
            k_tree, v_tree = self.k_layers, self.v_layers
        elif self.rope_theta:
            k_tree = self.k_rot  # the cache holds rotated keys
        H.tree_commit(k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, self.n_accepted, self.path,
                      self.out_tok, self.next_prefix_len, self.next_root_tok, hidden=self.rows(),
                      next_h=self.next_h, stream=stream)

    def run(self, h, root_tok, q, k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, u_acc=None,
            u_res=None, stream=None):
        self.draft(h, root_tok, stream)
        self.build(stream)
        if self.target is not None:
            self.verify(k_pages, v_pages, block_table, prefix_len, stream)
        else:
            self.attend(q, k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, stream)
        self.accept(u_acc, u_res, stream)
        self.commit(k_tree, v_tree, k_pages, v_pages, block_table, prefix_len, stream)


def round_from_inputs(inp, device="cuda", keep_hidden=True, fold_embedding=None, residual=True, pack_vocab=None):
    """HydraRound plus device copies of a dict of named input tensors.

    Keys: workload (sizes, tree, dtype, mode), root_tok, h, E, W1, b1, W2 (or
    heads, for two-layer heads), W_t,
    q_tree, k_tree, v_tree (or, with the target's layers, target and ln_f),
    k_pages, v_pages, block_table, prefix_len and, for the rejection and
    typical modes, u_acc and u_res. Returns (round, device tensors).
    """
    w = inp["workload"]
    to = lambda t: t.to(device).contiguous()  # noqa: E731
    weights = dict(emb=to(inp["E"]) if w.hydra else None, W_t=to(inp["W_t"]))
    if w.cond == "attn":
        weights["attn"] = {n: to(t) for n, t in inp["attn"].items()}
    if w.layers:
        weights["target"] = dict({n: to(t) for n, t in inp["target"].items()}, ln_f=to(inp["ln_f"]),
                                 emb=to(inp["E"]))
    if w.head == "sketch":
        weights["heads"] = [{n: to(t) for n, t in hd.items()} for hd in inp["heads"]]
    else:
        weights.update(W1=[to(x) for x in inp["W1"]], b1=[to(x) for x in inp["b1"]], W2=[to(x) for x in inp["W2"]])
    shape = dict(B=w.B, d=w.d, V=w.V, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                 max_prefix_len=int(inp["prefix_len"].max()))
    mode = {"greedy": 0, "stochastic": 1, "typical": 2}[w.mode]
    rnd = HydraRound(weights, w.tree, shape, hydra=w.hydra, mode=mode, temperature=w.T, residual=residual, keep_hidden=keep_hidden, device=device,
                     fold_embedding=fold_embedding, eps=w.eps, delta=w.delta, full_path=w.cond == "path",
                     pack_vocab=pack_vocab)
    dev = dict(h=to(inp["h"]), root_tok=to(inp["root_tok"]), k_pages=to(inp["k_pages"]), v_pages=to(inp["v_pages"]),
               block_table=to(inp["block_table"]), prefix_len=to(inp["prefix_len"]))
    if not w.layers:  # the target's layers make their own Q/K/V
        dev.update(q=to(inp["q_tree"]), k_tree=to(inp["k_tree"]), v_tree=to(inp["v_tree"]))
    if w.mode in ("stochastic", "typical"):
        dev["u_acc"], dev["u_res"] = to(inp["u_acc"]), to(inp["u_res"])
    return rnd, dev


def run_round(rnd, dev, stream=None):
    """One round on the device tensors returned by round_from_inputs."""
    rnd.run(dev["h"], dev["root_tok"], dev.get("q"), dev.get("k_tree"), dev.get("v_tree"), dev["k_pages"],
            dev["v_pages"], dev["block_table"], dev["prefix_len"], dev.get("u_acc"), dev.get("u_res"), stream=stream)
