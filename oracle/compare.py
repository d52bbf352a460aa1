"""GPU-vs-oracle comparison rules (test infrastructure).

The device path computes the row statistics of the accept test in fp32 and
the sampled row in fp64; the oracle works in fp64 throughout.  The rules:

* Accept decisions are identical, except a *band case*: the oracle's
  threshold min(1, q(d)/p(d)) lies within 1e-6 of the uniform.  A band case
  whose decisions differ is excused; if it sits on the decided prefix of the
  sequence (a position up to the oracle's first rejection, or a tree node
  whose decision the walk reads) the sequence's outcome is excluded from the
  exact comparisons below and counted.
* Accepted counts, accepted tokens, tree paths and KV indices are identical.
* Probabilities q(d), p(d) agree within 1e-5 relative (fp32 outputs; an
  absolute floor of 1e-37 covers values below the fp32 normal range), and the
  residual mass within 1e-5 relative.
* The sampled token is identical, except when u*W lies within 1e-6*W of the
  oracle's CDF edge of either token (the oracle's or the device's); such
  mismatches are excused and counted, and their count must stay below 1e-4
  of the samples compared.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

BAND = 1e-6
PROB_RTOL = 1e-5
PROB_ATOL = 1e-37
MASS_RTOL = 1e-5
MISMATCH_BUDGET = 1e-4


@dataclasses.dataclass
class Report:
    sequences: int = 0
    errors: int = 0                 # sequences both sides marked -1
    decisions: int = 0
    band_decisions: int = 0         # decisions inside the band (agreeing or not)
    band_flips: int = 0             # band decisions that differ
    excluded: int = 0               # sequences whose outcome was excluded
    samples: int = 0                # sampled tokens compared
    token_mismatch_excused: int = 0
    max_prob_rel: float = 0.0
    max_mass_rel: float = 0.0
    failures: List[str] = dataclasses.field(default_factory=list)

    def merge(self, other: "Report") -> "Report":
        for f in dataclasses.fields(self):
            if f.name == "failures":
                self.failures += other.failures
            elif f.name.startswith("max_"):
                setattr(self, f.name, max(getattr(self, f.name), getattr(other, f.name)))
            else:
                setattr(self, f.name, getattr(self, f.name) + getattr(other, f.name))
        return self

    def check(self) -> None:
        msgs = list(self.failures[:20])
        if self.token_mismatch_excused > 0 and self.token_mismatch_excused >= MISMATCH_BUDGET * self.samples:
            msgs.append(f"{self.token_mismatch_excused} excused token mismatches in {self.samples} samples "
                        f"exceed {MISMATCH_BUDGET:g} of the samples")
        if msgs:
            raise AssertionError("parity failures:\n  " + "\n  ".join(msgs) + f"\n{self.summary()}")

    def summary(self) -> str:
        return (f"seq={self.sequences} err={self.errors} decisions={self.decisions} band={self.band_decisions} "
                f"flips={self.band_flips} excluded={self.excluded} samples={self.samples} "
                f"excused_mismatch={self.token_mismatch_excused} max_prob_rel={self.max_prob_rel:.2e} "
                f"max_mass_rel={self.max_mass_rel:.2e}")


def _rel(a, b, floor):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), floor)


def _in_band(u, ratio):
    thr = np.minimum(1.0, ratio)
    return np.isfinite(ratio) & (np.abs(u - thr) < BAND)


def _token_excused(o, b) -> bool:
    W = o["weight_total"][b]
    t = o["target"][b]
    edges = [o["edge_lo"][b], o["edge_hi"][b]]
    if "qedge_lo" in o:
        edges += [o["qedge_lo"][b], o["qedge_hi"][b]]
    return min(abs(t - e) for e in edges) <= BAND * W


def compare_chain(g: dict, o: dict, b_range=None) -> Report:
    """g: device outputs as numpy (tokens, num_accepted, accept, probs,
    residual_mass); o: oracle outputs (queried with the device's sampled
    tokens)."""
    rep = Report()
    B = g["num_accepted"].shape[0]
    lo, hi = b_range if b_range is not None else (0, B)
    N = g["tokens"].shape[1] - 1
    for b in range(lo, hi):
        rep.sequences += 1
        kg, ko = int(g["num_accepted"][b]), int(o["num_accepted"][b])
        if ko < 0 or kg < 0:
            if ko != kg:
                rep.failures.append(f"b={b}: error flag device {kg} oracle {ko}")
            elif not (g["tokens"][b] == -1).all():
                rep.failures.append(f"b={b}: error sequence with tokens {g['tokens'][b]}")
            else:
                rep.errors += 1
            continue
        if N > 0:
            u, r = o["u_acc"][b], o["ratio"][b]
            band = _in_band(u, r)
            dg = g["accept"][b].astype(np.int32)
            do = o["accept"][b]
            flips = dg != do
            rep.decisions += N
            rep.band_decisions += int(band.sum())
            rep.band_flips += int((flips & band).sum())
            if (flips & ~band).any():
                i = int(np.argmax(flips & ~band))
                rep.failures.append(f"b={b}: decision {i} device {dg[i]} oracle {do[i]} u={u[i]:.17g} r={r[i]:.17g}")
                continue
            decided = np.arange(N) <= ko
            prel = max(float(_rel(g["probs"][b, :, 0], o["q_tok"][b], PROB_ATOL).max()),
                       float(_rel(g["probs"][b, :, 1], o["p_tok"][b], PROB_ATOL).max()))
            rep.max_prob_rel = max(rep.max_prob_rel, prel)
            if prel > PROB_RTOL:
                rep.failures.append(f"b={b}: probability rel error {prel:.3g}")
            if (flips & decided).any():
                rep.excluded += 1
                continue
        if kg != ko:
            rep.failures.append(f"b={b}: num_accepted device {kg} oracle {ko}")
            continue
        if not np.array_equal(g["tokens"][b, :kg], o["tokens"][b, :ko]):
            rep.failures.append(f"b={b}: accepted tokens differ")
            continue
        if not (g["tokens"][b, kg + 1:] == -1).all():
            rep.failures.append(f"b={b}: padding not -1")
        rep.samples += 1
        tg, to = int(g["tokens"][b, kg]), int(o["tokens"][b, ko])
        if tg != to:
            if _token_excused(o, b):
                rep.token_mismatch_excused += 1
            else:
                rep.failures.append(f"b={b}: token device {tg} oracle {to} target={o['target'][b]:.17g} "
                                    f"W={o['weight_total'][b]:.17g} edges=({o['edge_lo'][b]:.17g},"
                                    f"{o['edge_hi'][b]:.17g})")
        if "residual_mass" in g:
            mrel = float(_rel(g["residual_mass"][b], o["resid_mass"][b], 1e-300))
            if o["resid_mass"][b] == 0.0:
                mrel = abs(float(g["residual_mass"][b]))
            rep.max_mass_rel = max(rep.max_mass_rel, mrel)
            if mrel > MASS_RTOL:
                rep.failures.append(f"b={b}: residual mass device {g['residual_mass'][b]!r} "
                                    f"oracle {o['resid_mass'][b]!r}")
    return rep


def compare_tree(g: dict, o: dict, parents, b_range=None) -> Report:
    """Tree outputs (tokens, path_nodes, num_accepted, accept, probs,
    residual_mass) against the oracle's.  parents [T+1] or [B, T+1]."""
    rep = Report()
    B = g["num_accepted"].shape[0]
    lo, hi = b_range if b_range is not None else (0, B)
    par_all = np.asarray(parents)
    for b in range(lo, hi):
        rep.sequences += 1
        par = par_all if par_all.ndim == 1 else par_all[b]
        kg, ko = int(g["num_accepted"][b]), int(o["num_accepted"][b])
        if ko < 0 or kg < 0:
            if ko != kg:
                rep.failures.append(f"b={b}: error flag device {kg} oracle {ko}")
            elif not ((g["tokens"][b] == -1).all() and (g["path_nodes"][b] == -1).all()):
                rep.failures.append(f"b={b}: error sequence outputs not -1")
            else:
                rep.errors += 1
            continue
        nn = g["accept"].shape[1]
        u, r = o["u_acc"][b, 1:], o["ratio"][b, 1:]
        band = _in_band(u, r)
        dg = g["accept"][b, 1:].astype(np.int32)
        do = o["accept"][b, 1:]
        flips = dg != do
        rep.decisions += nn - 1
        rep.band_decisions += int(band.sum())
        rep.band_flips += int((flips & band).sum())
        if (flips & ~band).any():
            i = int(np.argmax(flips & ~band)) + 1
            rep.failures.append(f"b={b}: node {i} decision device {dg[i - 1]} oracle {do[i - 1]}")
            continue
        prel = max(float(_rel(g["probs"][b, 1:, 0], o["q_tok"][b, 1:], PROB_ATOL).max()),
                   float(_rel(g["probs"][b, 1:, 1], o["p_tok"][b, 1:], PROB_ATOL).max()))
        rep.max_prob_rel = max(rep.max_prob_rel, prel)
        if prel > PROB_RTOL:
            rep.failures.append(f"b={b}: probability rel error {prel:.3g}")
        # nodes whose decision the walk reads: children of nodes on either path
        on_path = set(int(x) for x in o["path_nodes"][b] if x >= 0) | set(int(x) for x in g["path_nodes"][b] if x >= 0)
        decided = np.array([int(par[n]) in on_path for n in range(1, nn)])
        if flips.any() and (flips & decided).any():
            rep.excluded += 1
            continue
        if kg != ko or not np.array_equal(g["path_nodes"][b], o["path_nodes"][b]):
            rep.failures.append(f"b={b}: path device {g['path_nodes'][b]} oracle {o['path_nodes'][b]}")
            continue
        if not np.array_equal(g["tokens"][b, :kg], o["tokens"][b, :ko]):
            rep.failures.append(f"b={b}: path tokens differ")
            continue
        if not (g["tokens"][b, kg + 1:] == -1).all():
            rep.failures.append(f"b={b}: padding not -1")
        rep.samples += 1
        tg, to = int(g["tokens"][b, kg]), int(o["tokens"][b, ko])
        if tg != to:
            if _token_excused(o, b):
                rep.token_mismatch_excused += 1
            else:
                rep.failures.append(f"b={b}: token device {tg} oracle {to}")
        if "residual_mass" in g:
            mrel = float(_rel(g["residual_mass"][b], o["resid_mass"][b], 1e-300))
            if o["resid_mass"][b] == 0.0:
                mrel = abs(float(g["residual_mass"][b]))
            rep.max_mass_rel = max(rep.max_mass_rel, mrel)
            if mrel > MASS_RTOL:
                rep.failures.append(f"b={b}: residual mass device {g['residual_mass'][b]!r} "
                                    f"oracle {o['resid_mass'][b]!r}")
    return rep


def sampled_tokens(g: dict) -> np.ndarray:
    """The device's sampled token per sequence (-1 on errors), for the
    oracle's query argument."""
    k = g["num_accepted"]
    B = k.shape[0]
    out = np.full(B, -1, np.int32)
    ok = k >= 0
    out[ok] = g["tokens"][np.arange(B)[ok], k[ok]]
    return out
