"""Seeded synthetic inputs for the speculative-decoding verify step.

This module is shared by the tests, the benchmark, the oracle runs and the
GPU runs.  It holds none of the verify step's arithmetic: it makes logits,
draft tokens, tree shapes and KV buffers, nothing else.

* Verifier logits follow the five workloads of the build: Gaussian logits,
  Gaussian plus "peak" tokens, or Gaussian plus a Zipf log-prior over a
  seeded permutation of the vocabulary.  Draft logits are the verifier
  logits plus Gaussian noise.  bf16 workloads round both with
  round-to-nearest-even (torch's conversion).
* Draft tokens of a chain are drawn from p = softmax(draft / T) with the
  Gumbel-max construction (argmax of logits/T plus Gumbel noise), which
  samples the categorical law exactly without forming p.
* Static trees take, at every internal node, the top-k tokens of that node's
  draft logits (siblings in descending draft order).  Dynamic trees grow
  EAGLE-2 style ([ZH] "投机解码与 EAGLE", section 4 "eagle_round", step 2
  and section 5 on EAGLE-2): a node's path score is the product of draft
  probabilities along its path; each level expands the global top-k frontier
  and the tree keeps the global top-budget nodes by score.  The draft
  probabilities that rank candidates come from torch.log_softmax; they only
  shape the input and are never compared with anything.

All randomness comes from torch.Generator objects seeded from the arguments,
so a (config, seed, device) triple always gives the same tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# Parent array of the 26-node static tree (root + 25 drafts, depth 5, level
# sizes 4, 8, 8, 3, 2): level 1 = top-4 under the root, level 2 = top-2 under
# each level-1 node, level 3 = top-1 under each level-2 node, level 4 = top-1
# under the first three level-3 nodes, level 5 = top-1 under the first two
# level-4 nodes.
STATIC_TREE_PARENTS = [-1, 0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 21, 22]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # "chain", "tree_static", "tree_dynamic"
    B: int
    V: int
    dtype: str             # "f32" or "bf16"
    T: float = 1.0
    N: int = 0             # chain drafts
    sigma_q: float = 3.0
    sigma_noise: float = 0.5
    prior: str = "none"    # "none", "peaks", "zipf"
    zipf_s: float = 1.1
    peaks: int = 0
    peak_boost: float = 0.0
    depth: int = 0         # tree depth (max_depth)
    topk: int = 0
    budget: int = 0
    rounds: int = 0
    pool: int = 1
    L0: int = 0            # KV row of the root / pending token
    kv_heads: int = 0
    kv_dim: int = 0

    def with_sizes(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    # chain, B=1, N=4, V=32, fp32, q-logits N(0,2^2) fixed from seed 0, noise 0.5
    "chain_b1_v32": Workload("chain_b1_v32", "chain", B=1, N=4, V=32, dtype="f32", sigma_q=2.0, sigma_noise=0.5, rounds=10000),
    # chain, B=64, N=5, V=32000, fp32, N(0,3^2) + 8 peaks (+6), noise 0.7
    "chain_b64_v32000": Workload("chain_b64_v32000", "chain", B=64, N=5, V=32000, dtype="f32", sigma_q=3.0, sigma_noise=0.7, prior="peaks",
                   peaks=8, peak_boost=6.0, rounds=1000, pool=4),
    # chain, B=256, N=7, V=128256, bf16, N(0,3^2) - 1.1 ln rank, noise 0.4
    "chain_b256_v128256": Workload("chain_b256_v128256", "chain", B=256, N=7, V=128256, dtype="bf16", sigma_q=3.0, sigma_noise=0.4, prior="zipf",
                   rounds=500, pool=8),
    # static 26-node tree, B=32, V=128256, bf16, noise 0.5
    "tree_static_b32_v128256": Workload("tree_static_b32_v128256", "tree_static", B=32, V=128256, dtype="bf16", sigma_q=3.0, sigma_noise=0.5, prior="zipf",
                   depth=5, rounds=200, pool=8, L0=4095),
    # dynamic 60-node tree, depth 6, topk 10, B=128, V=152064, bf16, T=0.7, noise 0.3, KV [B, 4156, 8, 128]
    "tree_dynamic_b128_v152064": Workload("tree_dynamic_b128_v152064", "tree_dynamic", B=128, V=152064, dtype="bf16", T=0.7, sigma_q=3.0, sigma_noise=0.3,
                   prior="zipf", depth=6, topk=10, budget=60, rounds=200, pool=4, L0=4095, kv_heads=8, kv_dim=128),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _zipf_prior(w: Workload, device) -> torch.Tensor:
    """-s * ln(rank(t)) with rank a seeded permutation of 1..V, shared by all rows."""
    g = _gen(0x5EED0000 + w.V, "cpu")
    rank = torch.randperm(w.V, generator=g).to(torch.float64) + 1.0
    return (-w.zipf_s * torch.log(rank)).to(torch.float32).to(device)


def verifier_logits(w: Workload, rows: int, g: torch.Generator, device) -> torch.Tensor:
    """[rows, V] float32 verifier logits of workload w."""
    z = torch.randn((rows, w.V), generator=g, device=device, dtype=torch.float32) * w.sigma_q
    if w.prior == "peaks":
        scores = torch.rand((rows, w.V), generator=g, device=device)
        ids = torch.topk(scores, min(w.peaks, w.V), dim=1).indices  # distinct random ids per row
        z.scatter_add_(1, ids, torch.full(ids.shape, w.peak_boost, device=device))
    elif w.prior == "zipf":
        z += _zipf_prior(w, device)
    return z


def draft_from_verifier(w: Workload, zq: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    return zq + torch.randn(zq.shape, generator=g, device=zq.device, dtype=torch.float32) * w.sigma_noise


def _round(w: Workload, z: torch.Tensor) -> torch.Tensor:
    return z.to(w.torch_dtype)


def gumbel_max(logits: torch.Tensor, T: float, g: torch.Generator) -> torch.Tensor:
    """One draw from softmax(logits / T) per row (last axis), by Gumbel-max.

    Works in float64 so the Gumbel tail is resolved finely; -inf logits are
    never drawn."""
    x = logits.to(torch.float64) / T
    u = torch.rand(x.shape, generator=g, device=x.device, dtype=torch.float64)
    u = u.clamp_min(torch.finfo(torch.float64).tiny)
    gum = -torch.log(-torch.log(u))
    return torch.argmax(x + gum, dim=-1).to(torch.int32)


# --------------------------------------------------------------------------- #
# chains
# --------------------------------------------------------------------------- #
def chain_logits(w: Workload, seed: int, device="cpu", B: Optional[int] = None, N: Optional[int] = None):
    """(zq [B, N+1, V], zp [B, N, V]) in the workload's dtype."""
    B = w.B if B is None else B
    N = w.N if N is None else N
    g = _gen(seed, device)
    zq32 = verifier_logits(w, B * (N + 1), g, device).view(B, N + 1, w.V)
    zp32 = draft_from_verifier(w, zq32[:, :N, :], g)
    return _round(w, zq32).contiguous(), _round(w, zp32).contiguous()


def chain_draft_tokens(w: Workload, zp: torch.Tensor, seed: int) -> torch.Tensor:
    """d_i ~ p_i for every (sequence, position): [B, N] int32."""
    g = _gen(seed ^ 0xD7AF7, zp.device)
    if zp.shape[1] == 0:
        return torch.zeros((zp.shape[0], 0), dtype=torch.int32, device=zp.device)
    # chunk over rows to bound the float64 working set
    flat = zp.reshape(-1, zp.shape[-1])
    out = torch.empty(flat.shape[0], dtype=torch.int32, device=zp.device)
    step = max(1, (1 << 26) // max(1, flat.shape[1]))
    for i in range(0, flat.shape[0], step):
        out[i:i + step] = gumbel_max(flat[i:i + step], w.T, g)
    return out.view(zp.shape[0], zp.shape[1])


def chain_inputs(w: Workload, seed: int, device="cpu", B: Optional[int] = None, N: Optional[int] = None):
    zq, zp = chain_logits(w, seed, device, B, N)
    d = chain_draft_tokens(w, zp, seed)
    return {"zq": zq, "zp": zp, "d": d}


# --------------------------------------------------------------------------- #
# trees
# --------------------------------------------------------------------------- #
def static_tree_inputs(w: Workload, seed: int, device="cpu", B: Optional[int] = None, parents=None):
    """Static tree: shared parents; node tokens = top-k of the parent's draft
    logits, siblings in descending draft order."""
    B = w.B if B is None else B
    parents = list(STATIC_TREE_PARENTS if parents is None else parents)
    nn = len(parents)
    g = _gen(seed, device)
    zq32 = verifier_logits(w, B * nn, g, device).view(B, nn, w.V)
    zp32 = draft_from_verifier(w, zq32, g)
    zq, zp = _round(w, zq32).contiguous(), _round(w, zp32).contiguous()
    tokens = torch.zeros((B, nn), dtype=torch.int32, device=device)
    children = {}
    for n in range(1, nn):
        children.setdefault(parents[n], []).append(n)
    for par, kids in children.items():
        top = torch.topk(zp[:, par, :].float(), len(kids), dim=1).indices.to(torch.int32)
        for j, c in enumerate(kids):
            tokens[:, c] = top[:, j]
    return {"zq": zq, "zp": zp, "tokens": tokens,
            "parents": torch.tensor(parents, dtype=torch.int32, device=device)}


def dynamic_tree_inputs(w: Workload, seed: int, device="cpu", B: Optional[int] = None, depth: Optional[int] = None,
                        topk: Optional[int] = None, budget: Optional[int] = None):
    """EAGLE-2-style dynamic tree per sequence (see the module docstring).

    Returns zq, zp [B, budget+1, V], tokens [B, budget+1], parents
    [B, budget+1] (node 0 = root, nodes ordered by (depth, score desc,
    creation order)), depth_of [B, budget+1], and expanded_p
    [B, 1 + topk*(depth-1), V]: the draft rows the tree was grown from (the
    root's, then each level's frontier in rank order)."""
    B = w.B if B is None else B
    depth = w.depth if depth is None else depth
    topk = w.topk if topk is None else topk
    budget = w.budget if budget is None else budget
    V = w.V
    g = _gen(seed, device)
    ar = torch.arange(B, device=device)

    # rows of expanded nodes: expanded id 0 = root, then topk per level
    n_exp = 1 + topk * (depth - 1)
    exp_q = torch.empty((B, n_exp, V), dtype=w.torch_dtype, device=device)
    exp_p = torch.empty((B, n_exp, V), dtype=w.torch_dtype, device=device)

    def new_rows(count):
        zq32 = verifier_logits(w, B * count, g, device).view(B, count, V)
        zp32 = draft_from_verifier(w, zq32, g)
        return _round(w, zq32), _round(w, zp32)

    exp_q[:, :1], exp_p[:, :1] = new_rows(1)
    # candidate table (created order): parent (candidate id, -1 = root), token, logscore, level, expanded slot
    cand_parent, cand_token, cand_score, cand_level, cand_slot = [], [], [], [], []
    frontier_cand = torch.full((B, 1), -1, dtype=torch.long, device=device)       # candidate ids (-1 root)
    frontier_slot = torch.zeros((B, 1), dtype=torch.long, device=device)          # expanded-row slot
    frontier_score = torch.zeros((B, 1), dtype=torch.float64, device=device)
    n_cand = 0
    next_slot = 1
    for level in range(1, depth + 1):
        F = frontier_cand.shape[1]
        rows = exp_p[ar[:, None], frontier_slot].float() / w.T            # [B, F, V]
        logp = torch.log_softmax(rows.double(), dim=-1)
        top = torch.topk(logp, topk, dim=-1)                              # [B, F, topk]
        score = frontier_score[:, :, None] + top.values                   # [B, F, topk]
        par = frontier_cand[:, :, None].expand(B, F, topk)
        cand_parent.append(par.reshape(B, F * topk))
        cand_token.append(top.indices.reshape(B, F * topk).to(torch.int32))
        cand_score.append(score.reshape(B, F * topk))
        cand_level.append(torch.full((B, F * topk), level, dtype=torch.long, device=device))
        ids = torch.arange(n_cand, n_cand + F * topk, device=device)
        n_cand += F * topk
        slots = torch.full((B, F * topk), -1, dtype=torch.long, device=device)
        if level < depth:
            # global top-k of this level's candidates become the next frontier
            sel = _top_stable(score.reshape(B, F * topk), topk)
            frontier_cand = ids[sel]
            frontier_score = torch.gather(score.reshape(B, F * topk), 1, sel)
            frontier_slot = torch.arange(next_slot, next_slot + topk, device=device).expand(B, topk).contiguous()
            slots.scatter_(1, sel, frontier_slot)
            exp_q[:, next_slot:next_slot + topk], exp_p[:, next_slot:next_slot + topk] = new_rows(topk)
            next_slot += topk
        cand_slot.append(slots)
    cp = torch.cat(cand_parent, 1)
    ct = torch.cat(cand_token, 1)
    cs = torch.cat(cand_score, 1)
    cl = torch.cat(cand_level, 1)
    cslot = torch.cat(cand_slot, 1)
    # global top-budget by score, ties to the earlier-created candidate
    keep = _top_stable(cs, budget)                                        # [B, budget] candidate ids
    keep_level = torch.gather(cl, 1, keep)
    keep_score = torch.gather(cs, 1, keep)
    # flatten by (level, score desc, creation order)
    order_key = keep_level.double() * 1e6 - keep_score  # scores are log-probs >= -1e5 in practice
    order = _stable_argsort(order_key, keep)
    keep = torch.gather(keep, 1, order)
    keep_level = torch.gather(keep_level, 1, order)
    nn = budget + 1
    node_of_cand = torch.full((B, n_cand), -1, dtype=torch.long, device=device)
    node_of_cand.scatter_(1, keep, torch.arange(1, nn, device=device).expand(B, budget).contiguous())
    kp = torch.gather(cp, 1, keep)
    parents = torch.zeros((B, nn), dtype=torch.int32, device=device)
    parents[:, 0] = -1
    root_child = kp < 0
    mapped = torch.gather(node_of_cand, 1, kp.clamp_min(0))
    parents[:, 1:] = torch.where(root_child, torch.zeros_like(mapped), mapped).to(torch.int32)
    if bool((parents[:, 1:] < 0).any()):
        raise RuntimeError("kept set is not ancestor-closed")
    tokens = torch.zeros((B, nn), dtype=torch.int32, device=device)
    tokens[:, 1:] = torch.gather(ct, 1, keep)
    # rows: expanded nodes reuse their rows; others get fresh ones
    slot = torch.gather(cslot, 1, keep)                                   # [B, budget]
    zq = torch.empty((B, nn, V), dtype=w.torch_dtype, device=device)
    zp = torch.empty((B, nn, V), dtype=w.torch_dtype, device=device)
    zq[:, 0], zp[:, 0] = exp_q[:, 0], exp_p[:, 0]
    fq, fp = new_rows(budget)
    has = slot >= 0
    src_slot = slot.clamp_min(0)
    gq = exp_q[ar[:, None], src_slot]
    gp = exp_p[ar[:, None], src_slot]
    zq[:, 1:] = torch.where(has[:, :, None], gq, fq)
    zp[:, 1:] = torch.where(has[:, :, None], gp, fp)
    depth_of = torch.zeros((B, nn), dtype=torch.int32, device=device)
    depth_of[:, 1:] = keep_level.to(torch.int32)
    return {"zq": zq, "zp": zp, "tokens": tokens, "parents": parents, "depth_of": depth_of,
            "expanded_p": exp_p}


def _top_stable(score: torch.Tensor, k: int) -> torch.Tensor:
    """Indices of the k largest entries per row, ties to the lower index."""
    order = torch.argsort(-score, dim=1, stable=True)
    return order[:, :k]


def _stable_argsort(key: torch.Tensor, tiebreak: torch.Tensor) -> torch.Tensor:
    """argsort by key, ties by tiebreak (both [B, n])."""
    o1 = torch.argsort(tiebreak, dim=1, stable=True)
    k1 = torch.gather(key, 1, o1)
    o2 = torch.argsort(k1, dim=1, stable=True)
    return torch.gather(o1, 1, o2)


# --------------------------------------------------------------------------- #
# KV buffers
# --------------------------------------------------------------------------- #
def kv_buffer(B: int, L: int, heads: int, dim: int, seed: int, device="cpu", dtype=torch.bfloat16):
    g = _gen(seed ^ 0x4B56, device)
    return torch.randn((B, L, heads, dim), generator=g, device=device, dtype=torch.float32).to(dtype)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a bf16 tensor as a numpy uint16 array (for the oracle)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_oracle(t: torch.Tensor):
    """A logits tensor as the oracle's numpy input (float32 or raw bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy()


def algorithmic_bytes_chain(B: int, N: int, V: int, elem: int) -> int:
    """Every logit row the chain step can need, read once: B*(2N+1)*V*s."""
    return B * (2 * N + 1) * V * elem


def algorithmic_bytes_tree(parents, V: int, elem: int) -> int:
    """q at every node plus p at every internal node, per sequence, summed."""
    import numpy as np
    p = np.asarray(parents)
    if p.ndim == 1:
        p = p[None, :]
    total = 0
    for row in p:
        nn = row.shape[0]
        internal = len(set(int(x) for x in row[1:]))
        total += (nn + internal) * V * elem
    return total


__all__ = ["Workload", "WORKLOADS", "STATIC_TREE_PARENTS", "chain_inputs", "chain_logits", "chain_draft_tokens",
           "static_tree_inputs", "dynamic_tree_inputs", "kv_buffer", "to_oracle", "bf16_bits", "gumbel_max",
           "algorithmic_bytes_chain", "algorithmic_bytes_tree", "math"]
