"""Seeded synthetic inputs for one Hydra/Medusa draft-and-verify round.

This module is shared by the tests, the benchmark and the smoke check: it
feeds the same arrays to the device path and to the CPU oracle. It holds none
of the method's arithmetic, only random draws, the rounding of inputs to
bfloat16, and the placement of prefix K/V rows into a paged pool.

Workloads stand in for the pages' models (Vicuna-7B and LLaMA-2-70B layer
shapes, 64-node sparse and 256-node dense trees); no checkpoint or dataset is
used. Every tensor is drawn from one ``torch.Generator`` seeded per workload,
in this fixed order:

  1. root tokens [B] uniform in [0, V)
  2. h [B, d] ~ N(0, 1)
  3. embedding table E [V, d] ~ N(0, 1)
  4. per head k = 1..n_heads: W1 [d, in] ~ N(0, 0.02), b1 [d] ~ N(0, 0.02),
     W2 [V, d] ~ N(0, 0.02)      (in = 2 d for Hydra, d for Medusa, (k + 1) d
     for full-path conditioning)
  5. target vocabulary projection W_t [V, d] ~ N(0, 0.02)
  6. prefix lengths L_b (fixed, or uniform in [lo, hi])
  7. per sequence: prefix K [L_b, Hkv, D], then prefix V, ~ N(0, 1)
  8. page order: identity, or a random permutation of the pool (the pool
     holds each prefix plus a reserve of free positions after it)
  9. tree Q [B, N, Hq, D], tree K [B, N, Hkv, D], tree V ~ N(0, 1)
 10. uniforms u_acc [B, N], u_res [B, N] in [0, 1)  (stochastic and typical
     modes)
 11. two-layer heads only, per head k: Wa [d, d] (k = 1) or [H, 2d], ba, then
     (k > 1) Wb [d, H], bb, all ~ N(0, 0.02); LayerNorm gain 1 + N(0, 0.1) and
     bias N(0, 0.1) [d]; W2 [V, d] ~ N(0, 0.02)  (H = head_hidden, 1024)
 12. Hydra++ fusion only: Wqkv [3d, d], then Wo [d, d], ~ N(0, 0.02)

Draws are float32; bfloat16 workloads round them to bfloat16 (round to
nearest even, torch's conversion). ``generate(w, device="cuda")`` makes the
same draws in the same order from a generator on that device (same shapes,
distributions and seed, different numbers): the benchmark's extra workloads
use it to skip the host-side draws; parity tests use the host default.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

PAGE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str            # "fp32" | "bf16"
    B: int
    d: int
    V: int
    n_heads: int
    hydra: bool
    tree: tuple           # ("cartesian", b) | ("sparse", caps, n_nodes) | ("dense", b, n_keep)
    Hq: int
    Hkv: int
    D: int
    L: tuple              # (L,) fixed or (lo, hi) uniform per sequence
    mode: str = "greedy"  # "greedy" | "stochastic" | "typical"
    T: float = 1.0
    eps: float = 0.1      # typical acceptance: threshold min(eps, delta * exp(-H))
    delta: float = 0.3
    scattered: bool = False
    zero_init: bool = False
    head: str = "mlp"     # "mlp" (one SiLU layer) | "sketch" (two-layer LayerNorm heads)
    head_hidden: int = 1024
    cond: str = "parent"  # Hydra conditioning: "parent" token, the whole "path", or Hydra++ "attn" fusion
    layers: int = 0       # 0: one attention layer over given tree Q/K/V; n: the target's n decoder layers
    ffn: int = 0          # the decoder layers' feed-forward width
    extra: dict = field(default_factory=dict)

    @property
    def n_tree(self) -> int:
        kind = self.tree[0]
        if kind == "cartesian":
            n, f = 1, 1
            for b in self.tree[1]:
                f *= b
                n += f
            return n
        if kind == "sparse":
            return self.tree[2]
        return self.tree[2]

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


_7B = dict(dtype="bf16", d=4096, V=32000, n_heads=4, hydra=True, Hq=32, Hkv=32, D=128)
_SPARSE = ("sparse", (10, 4, 2, 1), 64)

WORKLOADS = {
    # hidden 256, vocab 1000, 3 heads, 2x3 Cartesian tree, 8 heads x 32, prefix 128
    "tiny": Workload("tiny", 0, "fp32", 1, 256, 1000, 3, True, ("cartesian", (2, 3)),
                     8, 8, 32, (128,)),
    "tiny_medusa": Workload("tiny_medusa", 0, "fp32", 1, 256, 1000, 3, False,
                            ("cartesian", (2, 3)), 8, 8, 32, (128,)),
    # Vicuna-7B-shaped layer, 64-node sparse tree, prefix 2048
    "7b_sparse64": Workload("7b_sparse64", 1, B=1, tree=_SPARSE, L=(2048,), **_7B),
    # dense 4-ary depth-4 tree pruned to 256 rows, prefix 8192 (and the sparse
    # tree on the same seed)
    "7b_dense256": Workload("7b_dense256", 2, B=1, tree=("dense", (4, 4, 4, 4), 256),
                            L=(8192,), **_7B),
    "7b_sparse64_L8192": Workload("7b_sparse64_L8192", 2, B=1, tree=_SPARSE, L=(8192,), **_7B),
    # 16 sequences, ragged prefixes in [512, 4096], scattered 16-token pages
    "7b_batched16": Workload("7b_batched16", 3, B=16, tree=_SPARSE, L=(512, 4096),
                             scattered=True, **_7B),
    # 70B-shaped GQA layer, stochastic acceptance at temperature 0.7
    # the two-layer LayerNorm heads of the Hydra guide's sketch (hidden 1024)
    "tiny_sketch": Workload("tiny_sketch", 5, "fp32", 1, 256, 1000, 3, True, ("cartesian", (2, 3)),
                            8, 8, 32, (128,), head="sketch"),
    "7b_sketch": Workload("7b_sketch", 6, B=1, tree=_SPARSE, L=(2048,), head="sketch", **_7B),
    # full-path conditioning: head k reads h and the embeddings of its whole path
    "tiny_path": Workload("tiny_path", 7, "fp32", 1, 256, 1000, 3, True, ("cartesian", (2, 3)),
                          8, 8, 32, (128,), cond="path"),
    "7b_path": Workload("7b_path", 8, B=1, tree=_SPARSE, L=(2048,), cond="path", **_7B),
    # Hydra++ self-attention fusion over the path embeddings
    "tiny_attn": Workload("tiny_attn", 9, "fp32", 1, 256, 1000, 3, True, ("cartesian", (2, 3)),
                          8, 8, 32, (128,), cond="attn"),
    "7b_attn": Workload("7b_attn", 10, B=1, tree=_SPARSE, L=(2048,), cond="attn", **_7B),
    "70b_gqa": Workload("70b_gqa", 4, "bf16", 4, 8192, 32000, 4, True, _SPARSE,
                        64, 8, 128, (16384,), mode="stochastic", T=0.7),
    # the verification pass through the target's decoder layers (embeddings of
    # the tree tokens, n LLaMA layers over per-layer paged prefixes, final
    # norm) instead of one attention layer over given Q/K/V
    "tiny_layers": Workload("tiny_layers", 11, "fp32", 2, 256, 1000, 3, True, ("cartesian", (2, 3)),
                            8, 4, 32, (40, 130), layers=3, ffn=512),
    "7b_layers": Workload("7b_layers", 12, B=1, tree=_SPARSE, L=(2048,), layers=32, ffn=11008, **_7B),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _normal(g, shape, std, dtype):
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=g.device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def generate(w: Workload, n_tree: int | None = None, reserve: int | None = None, device=None) -> dict:
    """Draw every input of one round for workload ``w`` (CPU tensors, or on
    ``device`` from a generator there).

    Each sequence's block table maps pages for its prefix plus ``reserve``
    more positions (default: one round's commit, n_heads + 1 rows), zeroed.
    """
    if reserve is None:
        reserve = w.n_heads + 1
    g = torch.Generator(device=device or "cpu").manual_seed(w.seed)
    on = g.device
    dt = w.torch_dtype
    N = w.n_tree if n_tree is None else n_tree
    out = {"workload": w, "N": N}
    out["root_tok"] = torch.randint(0, w.V, (w.B,), generator=g, dtype=torch.int64, device=on).to(torch.int32)
    out["h"] = _normal(g, (w.B, w.d), 1.0, dt)
    out["E"] = _normal(g, (w.V, w.d), 1.0, dt)
    in_dim = 2 * w.d if w.hydra else w.d
    W1, b1, W2 = [], [], []
    for k in range(1, w.n_heads + 1):
        if w.cond == "path":
            in_dim = (k + 1) * w.d
        W1.append(_normal(g, (w.d, in_dim), 0.02, dt))
        b1.append(_normal(g, (w.d,), 0.02, dt))
        W2.append(_normal(g, (w.V, w.d), 0.02, dt))
    out["W_t"] = _normal(g, (w.V, w.d), 0.02, dt)
    if w.zero_init:
        # every head starts as a copy of the base vocabulary projection with
        # a zero feed-forward layer; W_t plays the base projection
        W1 = [torch.zeros_like(x) for x in W1]
        b1 = [torch.zeros_like(x) for x in b1]
        W2 = [out["W_t"].clone() for _ in W2]
    out["W1"], out["b1"], out["W2"] = W1, b1, W2

    if len(w.L) == 1:
        lens = [w.L[0]] * w.B
    else:
        lens = torch.randint(w.L[0], w.L[1] + 1, (w.B,), generator=g, device=on).tolist()
    out["prefix_len"] = torch.tensor(lens, dtype=torch.int32, device=on)
    kp, vp = [], []
    for L in lens:
        kp.append(_normal(g, (L, w.Hkv, w.D), 1.0, dt))
        vp.append(_normal(g, (L, w.Hkv, w.D), 1.0, dt))
    out["k_prefix"], out["v_prefix"] = kp, vp
    pages_per = [math.ceil((L + reserve) / PAGE) for L in lens]
    n_pages = max(1, sum(pages_per))
    if w.scattered:
        order = torch.randperm(n_pages, generator=g, device=on).to(torch.int32).cpu()
    else:
        order = torch.arange(n_pages, dtype=torch.int32)
    max_pages = max(1, max(pages_per))
    block_table = torch.full((w.B, max_pages), -1, dtype=torch.int32)
    k_pages = torch.zeros((n_pages, w.Hkv, PAGE, w.D), dtype=dt, device=on)
    v_pages = torch.zeros((n_pages, w.Hkv, PAGE, w.D), dtype=dt, device=on)
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(pages_per[b]):
            pid = int(order[nxt])
            nxt += 1
            block_table[b, j] = pid
            lo, hi = j * PAGE, min(L, (j + 1) * PAGE)
            if hi > lo:  # pages past the prefix stay zero (the reserve)
                k_pages[pid, :, : hi - lo] = kp[b][lo:hi].transpose(0, 1)
                v_pages[pid, :, : hi - lo] = vp[b][lo:hi].transpose(0, 1)
    out["block_table"], out["k_pages"], out["v_pages"] = block_table.to(on), k_pages, v_pages
    out["page_size"] = PAGE

    out["q_tree"] = _normal(g, (w.B, N, w.Hq, w.D), 1.0, dt)
    out["k_tree"] = _normal(g, (w.B, N, w.Hkv, w.D), 1.0, dt)
    out["v_tree"] = _normal(g, (w.B, N, w.Hkv, w.D), 1.0, dt)
    if w.mode in ("stochastic", "typical"):
        out["u_acc"] = torch.rand((w.B, N), generator=g, dtype=torch.float32, device=on)
        out["u_res"] = torch.rand((w.B, N), generator=g, dtype=torch.float32, device=on)
    if w.head == "sketch":
        # drawn last so the other inputs of a seed do not move; LayerNorm gain
        # near 1 and bias near 0 (not exactly, so both take part)
        heads = []
        for k in range(1, w.n_heads + 1):
            width = w.d if k == 1 else w.head_hidden
            hd = {"Wa": _normal(g, (width, w.d if k == 1 else 2 * w.d), 0.02, dt),
                  "ba": _normal(g, (width,), 0.02, dt)}
            if k > 1:
                hd["Wb"] = _normal(g, (w.d, w.head_hidden), 0.02, dt)
                hd["bb"] = _normal(g, (w.d,), 0.02, dt)
            hd["ln_g"] = (1.0 + _normal(g, (w.d,), 0.1, torch.float32)).to(dt)
            hd["ln_b"] = _normal(g, (w.d,), 0.1, dt)
            hd["W2"] = _normal(g, (w.V, w.d), 0.02, dt)
            heads.append(hd)
        out["heads"] = heads
    if w.cond == "attn":
        out["attn"] = {"Wqkv": _normal(g, (3 * w.d, w.d), 0.02, dt), "Wo": _normal(g, (w.d, w.d), 0.02, dt)}
    if w.layers:
        # the target's layers, layer-stacked; norm gains near 1. Layer 0's
        # prefix is the one drawn above; each further layer draws its own
        # into pools that share the block table
        n, F, HD = w.layers, w.ffn, (w.Hq + 2 * w.Hkv) * w.D
        gain = lambda *shape: (1.0 + _normal(g, shape, 0.1, torch.float32)).to(dt)  # noqa: E731
        out["target"] = {"ln1": gain(n, w.d), "Wqkv": _normal(g, (n, HD, w.d), 0.02, dt),
                         "Wo": _normal(g, (n, w.d, w.Hq * w.D), 0.02, dt), "ln2": gain(n, w.d),
                         "Wgu": _normal(g, (n, 2 * F, w.d), 0.02, dt), "Wd": _normal(g, (n, w.d, F), 0.02, dt)}
        out["ln_f"] = gain(w.d)
        kpl, vpl = [kp], [vp]
        kps = torch.zeros((n,) + tuple(k_pages.shape), dtype=dt, device=on)
        vps = torch.zeros_like(kps)
        kps[0], vps[0] = k_pages, v_pages
        for layer in range(1, n):
            kl = [_normal(g, (L, w.Hkv, w.D), 1.0, dt) for L in lens]
            vl = [_normal(g, (L, w.Hkv, w.D), 1.0, dt) for L in lens]
            for b, L in enumerate(lens):
                for j in range(pages_per[b]):
                    pid, lo, hi = int(block_table[b, j]), j * PAGE, min(L, (j + 1) * PAGE)
                    if hi > lo:
                        kps[layer, pid, :, : hi - lo] = kl[b][lo:hi].transpose(0, 1)
                        vps[layer, pid, :, : hi - lo] = vl[b][lo:hi].transpose(0, 1)
            kpl.append(kl)
            vpl.append(vl)
        out["k_prefix_layers"], out["v_prefix_layers"] = kpl, vpl
        out["k_pages"], out["v_pages"] = kps, vps
    return out


def as_f64(t):
    """Host float64 numpy copy of a tensor (the oracle's input form)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
