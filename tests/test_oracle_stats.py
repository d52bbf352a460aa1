"""Statistical and enumeration pins of the fp64 oracle (no GPU).

Every random quantity is seeded, so each test is deterministic.  The laws the
oracle is compared with are computed here from the pages' definitions with
scipy's softmax, by brute-force enumeration, or from closed forms; none of
them calls the oracle's arithmetic.

Pages: [PT] "Decodificacao Especulativa e EAGLE-3" (ai-engineering.academy),
sections "O Conceito" (the invariant), "O que determina a aceleracao",
"Implementando" Passo 5 (the chi-square check) and "Exercicios" 1.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import chi2

import synth
from oracle import analytic

from _stats import chi2_pooled as _chi2_stat


def _broadcast(z, R):
    """[1, rows, V] -> a stride-0 view [R, rows, V]."""
    assert z.ndim == 3 and z.shape[0] == 1
    return np.broadcast_to(z, (R,) + z.shape[1:])


def _c1_runs(orc, R, seed):
    w = synth.WORKLOADS["chain_b1_v32"]
    zq, zp = synth.chain_logits(w, 0, "cpu")           # fixed logits (seed 0)
    d = synth.chain_draft_tokens(w, zp.expand(R, -1, -1).contiguous(), seed).numpy()
    q = softmax(zq[0].double().numpy(), axis=1)
    Q = np.broadcast_to(zq.numpy(), (R,) + tuple(zq.shape[1:]))
    P = np.broadcast_to(zp.numpy(), (R,) + tuple(zp.shape[1:]))
    out = orc.verify_chain(Q, P, d, seed=seed, rnd=0, T=w.T)
    return out, q, w


def test_pages_chi_square_50000_steps(orc):
    """[PT] Implementando, Passo 5 and Exercicios 1: 50,000 speculative steps
    against 50,000 direct draws from q; the two-sample chi-square statistic of
    the first emitted token is below the 95% critical value.  The B=1, N=4, V=32 chain workload
    (B=1, N=4, V=32, fp32, q-logits N(0, 2^2) from seed 0, draft noise 0.5)."""
    R = 50000
    out, q, w = _c1_runs(orc, R, seed=20240101)
    spec = np.bincount(out["tokens"][:, 0], minlength=w.V)
    rng = np.random.default_rng(20240102)
    direct = np.bincount(rng.choice(w.V, size=R, p=q[0]), minlength=w.V)
    keep = (spec + direct) > 0
    a, b = spec[keep].astype(float), direct[keep].astype(float)
    # two-sample test of homogeneity with equal sample sizes
    stat = float((((a - b) ** 2) / (a + b)).sum())
    df = int(keep.sum()) - 1
    assert stat < chi2.ppf(0.95, df), (stat, df)


def test_chain_b1_every_slot_is_distributed_as_q(orc):
    """The B=1, N=4, V=32 chain, 10,000 rounds: conditional on reaching slot s (s = 1..N+1), the
    token emitted there is distributed as q_s ([PT] O Conceito: the output is
    distributed as q whatever p is); acceptance of slot s matches
    alpha_s = sum min(p_s, q_s)."""
    R = 10000
    out, q, w = _c1_runs(orc, R, seed=77)
    zp = synth.chain_logits(w, 0, "cpu")[1][0].double().numpy()
    p = softmax(zp, axis=1)
    k = out["num_accepted"]
    for s in range(w.N + 1):
        reached = k >= s
        toks = out["tokens"][reached, s]
        stat, df = _chi2_stat(np.bincount(toks, minlength=w.V).astype(float), q[s])
        assert stat < chi2.ppf(0.999, df), (s, stat, df)
        if s < w.N:
            alpha = np.minimum(p[s], q[s]).sum()
            acc = (k[reached] > s).mean()
            n = reached.sum()
            assert abs(acc - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / n)


def _exact_chain_law(zq, zp):
    """Exact law of (k, tokens) of a chain with N = 2, enumerated from the
    pages' definitions: accept d with min(1, q/p), first rejection samples
    (q-p)_+ normalised, all accepted -> bonus from q_{N+1}."""
    q = softmax(zq, axis=1)
    p = softmax(zp, axis=1)
    V = q.shape[1]
    a = np.minimum(1.0, q[:2] / p[:2])
    res = []
    for s in range(2):
        r = np.maximum(q[s] - p[s], 0.0)
        res.append(r / r.sum() if r.sum() > 0 else q[s])
    alpha = (p[:2] * a).sum(axis=1)
    law = {}
    for t in range(V):
        law[(0, t)] = (1 - alpha[0]) * res[0][t]
    for d1 in range(V):
        g1 = p[0, d1] * a[0, d1]
        for t in range(V):
            law[(1, d1, t)] = g1 * (1 - alpha[1]) * res[1][t]
        for d2 in range(V):
            g2 = g1 * p[1, d2] * a[1, d2]
            for t in range(V):
                law[(2, d1, d2, t)] = g2 * q[2, t]
    return law


@pytest.mark.parametrize("V", [3, 8])
def test_exact_joint_law_n2(orc, V):
    """Exhaustive enumeration (V <= 8, N = 2): the law of (k, emitted tokens)
    sums to one, P(k >= i) = prod_{j<=i} alpha_j, every slot's conditional law
    is q_s to 1e-12; then 10^6 Philox-driven oracle rounds (d ~ p by
    Gumbel-max) fit that law (chi-square below the 99.9% point over up to
    584 cells)."""
    rng = np.random.default_rng(900 + V)
    zq = rng.normal(0, 1.5, size=(3, V))
    zp = zq[:2] + rng.normal(0, 1.0, size=(2, V))
    law = _exact_chain_law(zq, zp)
    probs = np.array(list(law.values()))
    assert abs(probs.sum() - 1) < 1e-12
    q = softmax(zq, axis=1)
    p = softmax(zp, axis=1)
    alpha = np.minimum(p[:2], q[:2]).sum(axis=1)
    pk1 = sum(v for key, v in law.items() if key[0] >= 1)
    pk2 = sum(v for key, v in law.items() if key[0] == 2)
    assert abs(pk1 - alpha[0]) < 1e-12 and abs(pk2 - alpha[0] * alpha[1]) < 1e-12
    R = 1_000_000
    w = synth.Workload("tiny", "chain", B=R, N=2, V=V, dtype="f32", T=1.0)
    zpt = torch.tensor(zp)[None].expand(R, -1, -1).contiguous()
    d = synth.chain_draft_tokens(w, zpt, seed=31 + V).numpy()
    out = orc.verify_chain(_broadcast(zq[None], R), _broadcast(zp[None], R), d, seed=5 + V, rnd=3)
    keys = list(law.keys())
    index = {kk: i for i, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    k = out["num_accepted"]
    toks = out["tokens"]
    for kk in range(3):
        sel = k == kk
        if kk == 0:
            ids = [index[(0, t)] for t in toks[sel, 0]]
        elif kk == 1:
            ids = [index[(1, a, t)] for a, t in zip(toks[sel, 0], toks[sel, 1])]
        else:
            ids = [index[(2, a, b, t)] for a, b, t in zip(toks[sel, 0], toks[sel, 1], toks[sel, 2])]
        np.add.at(counts, ids, 1)
    stat, df = _chi2_stat(counts, probs)
    assert stat < chi2.ppf(0.999, df), (stat, df)


@pytest.mark.parametrize("alpha_noise,N", [(0.6, 5), (1.5, 7), (0.3, 3)])
def test_expected_accepted_closed_form(orc, alpha_noise, N):
    """[PT] O que determina a aceleracao: with the same overlap alpha at every
    position, tokens per verifier pass (k+1) average
    (1 - alpha^(N+1)) / (1 - alpha), and P(k >= i) = alpha^i.  z-test with
    the exact variance of the truncated geometric, |z| < 4."""
    rng = np.random.default_rng(int(alpha_noise * 100) + N)
    V, R = 64, 200_000
    zrow = rng.normal(0, 2.0, size=V)
    prow = zrow + rng.normal(0, alpha_noise, size=V)
    alpha = float(np.minimum(softmax(zrow), softmax(prow)).sum())
    zq = np.tile(zrow, (N + 1, 1))
    zp = np.tile(prow, (N, 1))
    w = synth.Workload("const", "chain", B=R, N=N, V=V, dtype="f32")
    d = synth.chain_draft_tokens(w, torch.tensor(zp)[None].expand(R, -1, -1).contiguous(), seed=N).numpy()
    out = orc.verify_chain(_broadcast(zq[None], R), _broadcast(zp[None], R), d, seed=11, rnd=N)
    k = out["num_accepted"].astype(float)
    mean = (k + 1).mean()
    expect = analytic.expected_tokens(alpha, N)
    z = (mean - expect) / np.sqrt(analytic.truncated_geometric_var(alpha, N) / R)
    assert abs(z) < 4, (mean, expect, z)
    for i in range(1, N + 1):
        pk = (k >= i).mean()
        ai = alpha ** i
        assert abs(pk - ai) < 4 * np.sqrt(ai * (1 - ai) / R) + 1e-12


@pytest.mark.parametrize("V", [4, 7])
def test_stratified_sampling_sweep(orc, V):
    """Inverse CDF ([PT] Implementando, Passo 2 + sample): sweeping the
    sampling uniform over 2^16 stratified points of a rejected slot, the
    share of points that give token t equals the residual mass of t within
    2^-16 (deterministic)."""
    rng = np.random.default_rng(40 + V)
    zq = rng.normal(0, 1.5, size=(2, V))
    zp = zq[:1] + rng.normal(0, 1.0, size=(1, V))
    q, p = softmax(zq, axis=1), softmax(zp, axis=1)
    a = np.minimum(1.0, q[0] / p[0])
    d = int(np.argmin(a))  # a token that can be rejected
    assert a[d] < 1
    M = 1 << 16
    u = np.zeros((M, 3))
    u[:, 0] = 1.0 - 2.0 ** -53  # force the rejection
    u[:, 1] = (np.arange(M) + 0.5) / M
    out = orc.verify_chain(_broadcast(zq[None], M), _broadcast(zp[None], M), np.full((M, 1), d, np.int32),
                           0, 0, u=u)
    assert (out["num_accepted"] == 0).all()
    share = np.bincount(out["tokens"][:, 0], minlength=V) / M
    r = np.maximum(q[0] - p[0], 0.0)
    assert np.max(np.abs(share - r / r.sum())) <= 1.0 / M
