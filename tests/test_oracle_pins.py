"""Deterministic pins of the fp64 oracle against what the pages and the
mathematics fix (no GPU).

Pages: [PT] "Decodificacao Especulativa e EAGLE-3" (ai-engineering.academy);
[ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异" (caijizhuo.github.io).
"""
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOP = 1.0 - 2.0 ** -53  # largest u53 value: rejects every threshold below 1


def _read_kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                v = [int(x, 16) for x in line.split()]
                rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


def test_philox_known_answers(orc):
    """Philox4x32-10 reproduces the published Random123 known-answer vectors."""
    kat = _read_kat()
    assert len(kat) == 3
    for ctr, key, expect in kat:
        assert orc.philox4x32_10(ctr, key) == expect


def test_u53_is_exact_dyadic(orc):
    """u53 maps (a, b) to (a>>5 * 2^26 + b>>6) / 2^53 exactly: 0 at the bottom,
    1 - 2^-53 at the top, every value a multiple of 2^-53."""
    assert orc.u53(0, 0) == 0.0
    assert orc.u53(0xFFFFFFFF, 0xFFFFFFFF) == TOP
    rng = np.random.default_rng(1)
    for a, b in rng.integers(0, 2 ** 32, size=(500, 2)):
        v = orc.u53(int(a), int(b))
        assert v * 2.0 ** 53 == float((int(a) >> 5) * 2 ** 26 + (int(b) >> 6))


def test_uniforms_layout(orc):
    """The accept and sampling uniforms of a position come from words (0,1)
    and (2,3) of one Philox block keyed by (seed) and countered by
    (position, sequence, round, stream 0)."""
    seed, rnd = 0x1234_5678_9ABC, 0x1_0000_0007
    for seq, pos in [(0, 1), (3, 7), (255, 8)]:
        w = orc.philox4x32_10([pos, seq, rnd & 0xFFFFFFFF, ((rnd >> 32) << 4) | 0],
                              [seed & 0xFFFFFFFF, seed >> 32])
        ua, us = orc.uniforms(seed, rnd, seq, pos)
        assert ua == orc.u53(w[0], w[1]) and us == orc.u53(w[2], w[3])
    a, s = orc.uniform_grid(seed, rnd, 4, 3)
    assert a[2, 1] == orc.uniforms(seed, rnd, 2, 2)[0]
    assert s[3, 2] == orc.uniforms(seed, rnd, 3, 3)[1]


def test_uniforms_are_uniform(orc):
    """Chi-square over 4096 bins of 2^20 uniforms (both words) is below the
    99.9% point, and the mean/variance match U(0,1)."""
    from scipy.stats import chi2
    a, s = orc.uniform_grid(7, 11, 1024, 512)
    for u in (a.ravel(), s.ravel()):
        assert u.min() >= 0.0 and u.max() < 1.0
        counts = np.bincount((u * 4096).astype(np.int64), minlength=4096)
        e = u.size / 4096
        stat = float(((counts - e) ** 2 / e).sum())
        assert stat < chi2.ppf(0.999, 4095)
        assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)
        assert abs(u.var() - 1 / 12) < 1e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
@pytest.mark.parametrize("T", [1.0, 0.7, 1.9])
def test_row_lse_matches_logsumexp(orc, dtype, T):
    """lse(z/T) equals scipy.special.logsumexp to 1e-13 (a library routine)."""
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, size=5003) - 1.1 * np.log(rng.permutation(5003) + 1.0)
    z[17] = -np.inf
    if dtype == "f32":
        arr = z.astype(np.float32)
        zz = arr.astype(np.float64)
    elif dtype == "bf16":
        import torch
        t = torch.tensor(z, dtype=torch.float32).to(torch.bfloat16)
        arr = t.view(torch.int16).numpy().view(np.uint16)
        zz = t.float().double().numpy()
    else:
        arr = z
        zz = z
    m, lse = orc.row_lse(arr, T)
    assert m == np.max(zz / T)
    assert abs(lse - logsumexp(zz / T)) <= 1e-13 * max(1.0, abs(lse))


def test_row_lse_errors(orc):
    """NaN, +inf and all -inf rows are data errors; a partly -inf row is not."""
    z = np.zeros(8)
    assert orc.row_lse(z) is not None
    for bad in (np.nan, np.inf):
        y = z.copy()
        y[3] = bad
        assert orc.row_lse(y) is None
    assert orc.row_lse(np.full(8, -np.inf)) is None
    y = np.full(8, -np.inf)
    y[5] = 2.0
    m, l = orc.row_lse(y)
    assert m == 2.0 and l == 2.0


def test_n0_is_plain_categorical_sampling(orc):
    """With no drafts the step samples q_1 by inverse CDF: identical to
    np.searchsorted(cumsum(q), u * sum(q), 'right') on the same uniform."""
    rng = np.random.default_rng(5)
    B, V, T = 300, 1000, 0.8125  # exactly representable in fp32, as the ABI passes T
    zq = rng.normal(0, 3, size=(B, 1, V))
    zp = np.zeros((B, 0, V))
    out = orc.verify_chain(zq, zp, np.zeros((B, 0), np.int32), seed=9, rnd=4, T=T)
    assert (out["num_accepted"] == 0).all()
    for b in range(B):
        q = softmax(zq[b, 0] / T)
        u = orc.uniforms(9, 4, b, 1)[1]
        c = np.cumsum(q)
        expect = int(np.searchsorted(c, u * c[-1], side="right"))
        assert out["tokens"][b, 0] == expect
        assert out["sample_kind"][b] == orc.KIND_BONUS


def _law_rows(rng, V, N, scale=1.5):
    zq = rng.normal(0, scale, size=(N + 1, V))
    zp = zq[:N] + rng.normal(0, 1.0, size=(N, V))
    return zq, zp


@pytest.mark.parametrize("V,N", [(2, 1), (3, 2), (5, 2), (8, 2), (8, 1)])
def test_theorem_on_oracle_primitives(orc, V, N):
    """Per slot, the oracle's accept probability and residual compose to
    exactly q ([PT] O Conceito, the invariant): for every token t,
    p(t) a(t) + (1 - sum_d p(d) a(d)) res(t) = q(t), and the acceptance
    sum_d p(d) a(d) = sum_t min(p, q).  Exact to 1e-12."""
    rng = np.random.default_rng(V * 10 + N)
    for trial in range(20):
        zq, zp = _law_rows(rng, V, N)
        for s in range(N):
            q, p = softmax(zq[s]), softmax(zp[s])
            a = np.array([orc.accept_prob(zq[s], zp[s], d) for d in range(V)])
            res, kind = orc.residual_probs(zq[s], zp[s])
            alpha = float((p * a).sum())
            assert abs(alpha - np.minimum(p, q).sum()) < 1e-12
            law = p * a + (1 - alpha) * res
            assert np.max(np.abs(law - q)) < 1e-12
            assert abs(res.sum() - 1) < 1e-12 and (res >= 0).all()


def test_accept_rule_edges(orc):
    """[PT] Implementando, Passo 1: accept iff u < min(1, q(d)/p(d)); a draft
    token of zero draft probability is accepted; q(d) = 0 never is."""
    zq = np.array([[0.0, 1.0, -np.inf, 0.5], [0.0, 0.0, 0.0, 0.0]])
    zp = np.array([[0.5, 0.0, 0.0, -np.inf]])
    B = 4
    Q = np.broadcast_to(zq[None], (B, 2, 4))
    P = np.broadcast_to(zp[None], (B, 1, 4))
    d = np.array([[0], [1], [2], [3]], np.int32)
    r0 = np.exp((0.0 - logsumexp(zq[0])) - (0.5 - logsumexp(zp[0])))
    # u just below and at the threshold
    u = np.zeros((B, 3))
    u[:, 0] = [np.nextafter(r0, 0), TOP, 0.0, TOP]
    out = orc.verify_chain(Q, P, d, 0, 0, u=u)
    # token 1 has q/p > 1 (min(1, r) = 1), so even the top uniform accepts it
    r1 = np.exp((1.0 - logsumexp(zq[0])) - (0.0 - logsumexp(zp[0])))
    assert r1 > 1.0
    assert out["accept"][:, 0].tolist() == [1, 1, 0, 1]
    assert abs(out["ratio"][0, 0] - r0) < 1e-15
    u[0, 0] = r0
    out = orc.verify_chain(Q, P, d, 0, 0, u=u)
    assert out["accept"][0, 0] == 0  # strict <
    assert np.isinf(out["ratio"][3, 0])  # p(d) = 0


@pytest.mark.parametrize("V,N,T", [(4, 1, 1.0), (5, 2, 1.0), (8, 2, 1.0), (5, 2, 0.75), (6, 1, 1.625)])
def test_chain_structure_under_forced_uniforms(orc, V, N, T):
    """For every draft vector and every forced accept/reject pattern, the
    chain keeps d_1..d_k up to the first rejection k+1, then emits one token
    drawn from residual(q_{k+1}, p_{k+1}), or from q_{N+1} when all N are
    accepted ([PT] O Conceito; [ZH] section 2, the three steps).  The
    sampling interval the oracle reports for its token carries exactly the
    residual (resp. q) mass of that token."""
    rng = np.random.default_rng(100 + V + N)
    zq, zp = _law_rows(rng, V, N)
    ds = np.array(np.meshgrid(*[np.arange(V)] * N, indexing="ij")).reshape(N, -1).T
    pats = np.array(np.meshgrid(*[[0, 1]] * N, indexing="ij")).reshape(N, -1).T
    B = len(ds) * len(pats) * 3
    d = np.repeat(ds, len(pats) * 3, axis=0).astype(np.int32)
    pat = np.tile(np.repeat(pats, 3, axis=0), (len(ds), 1))
    us = np.tile(np.array([0.0, 0.37, TOP]), len(ds) * len(pats))
    u = np.zeros((B, 2 * N + 1))
    u[:, :N] = np.where(pat == 1, 0.0, TOP)
    u[:, N:] = us[:, None]
    Q = np.broadcast_to(zq[None], (B, N + 1, V))
    P = np.broadcast_to(zp[None], (B, N, V))
    out = orc.verify_chain(Q, P, d, 0, 0, T=T, u=u)
    q = softmax(zq / T, axis=1)
    p = softmax(zp / T, axis=1)
    for b in range(B):
        a = np.array([min(1.0, q[i, d[b, i]] / p[i, d[b, i]]) for i in range(N)])
        forced = np.where(pat[b] == 1, a > 0, a >= 1.0).astype(int)  # what u forces
        k = N if forced.all() else int(np.argmin(forced))
        assert out["num_accepted"][b] == k
        assert out["tokens"][b, :k].tolist() == d[b, :k].tolist()
        assert (out["tokens"][b, k + 1:] == -1).all()
        t = out["tokens"][b, k]
        if k < N:
            w = np.maximum(q[k] - p[k], 0.0)
            law = w / w.sum()
        else:
            law = q[N]
        mass = (out["edge_hi"][b] - out["edge_lo"][b]) / out["weight_total"][b]
        assert abs(mass - law[t]) < 1e-12
        lo = out["edge_lo"][b] / out["weight_total"][b]
        assert abs(lo - law[:t].sum()) < 1e-12
        assert lo <= u[b, N + k] < lo + mass + 1e-15


def test_p_equals_q_accepts_everything(orc):
    """p == q gives ratio 1, so every draft is accepted and the bonus is drawn."""
    rng = np.random.default_rng(8)
    B, N, V = 64, 6, 100
    zq = rng.normal(0, 2, size=(B, N + 1, V)).astype(np.float32)
    zp = zq[:, :N].copy()
    d = rng.integers(0, V, size=(B, N)).astype(np.int32)
    out = orc.verify_chain(zq, zp, d, 3, 1)
    assert (out["num_accepted"] == N).all()
    assert (out["sample_kind"] == orc.KIND_BONUS).all()
    assert np.allclose(out["ratio"], 1.0, rtol=0, atol=1e-15)


def test_disjoint_supports_reject_first_and_sample_q(orc):
    """Disjoint supports: q(d) = 0 for every draft, so k = 0 and the residual
    is q itself (mass 1)."""
    B, N, V = 50, 3, 10
    zq = np.full((B, N + 1, V), -np.inf)
    zp = np.full((B, N, V), -np.inf)
    zq[:, :, :5] = 0.0
    zp[:, :, 5:] = 0.0
    d = np.full((B, N), 7, np.int32)
    out = orc.verify_chain(zq, zp, d, 4, 2)
    assert (out["num_accepted"] == 0).all()
    assert np.allclose(out["resid_mass"], 1.0)
    assert ((out["tokens"][:, 0] >= 0) & (out["tokens"][:, 0] < 5)).all()


def test_worked_example_three_tokens(orc):
    """[ZH] section 2 worked example: 4 drafts, the first two accepted, the
    third rejected -> 3 tokens from one verifier pass (2 drafts + 1
    correction).  Drafts 1-2 have q >= p (always accepted), draft 3 has
    q = 0 (always rejected)."""
    V, N = 16, 4
    rng = np.random.default_rng(2)
    zq = rng.normal(0, 1, size=(1, N + 1, V))
    zp = zq[:, :N].copy()
    d = np.array([[3, 9, 12, 1]], np.int32)
    zq[0, 2, 12] = -np.inf  # q_3(d_3) = 0
    out = orc.verify_chain(zq, zp, d, 1, 1)
    assert out["num_accepted"][0] == 2
    toks = out["tokens"][0]
    assert toks[:2].tolist() == [3, 9] and toks[2] not in (-1, 12) and toks[3] == -1
    assert int((toks >= 0).sum()) == 3


def test_exercise4_batched_kv_length(orc):
    """[PT] Exercicios, 4 / Passo 4: two sequences in one batch; A accepts all
    N drafts, B rejects at (1-based) position 2.  With L0 the KV row of the
    pending token, kv_len = L0 + k + 1: A -> L0 + N + 1, B -> L0 + 2, and the
    kept rows are the identity prefix."""
    V, N = 12, 5
    rng = np.random.default_rng(4)
    zq = rng.normal(0, 1, size=(2, N + 1, V))
    zp = zq[:, :N].copy()
    d = np.array([[1, 2, 3, 4, 5], [6, 7, 8, 9, 10]], np.int32)
    zq[1, 1, 7] = -np.inf  # B: q_2(d_2) = 0 -> reject at position 2
    out = orc.verify_chain(zq, zp, d, 6, 0)
    assert out["num_accepted"].tolist() == [N, 1]
    L0 = np.array([100, 250], np.int32)
    src, kvl = orc.kv_compact(None, out["num_accepted"], L0, max_depth=N)
    assert kvl.tolist() == [100 + N + 1, 250 + 2]
    assert src[0].tolist() == list(range(100, 100 + N + 1))
    assert src[1].tolist() == [250, 251] + [-1] * (N - 1)


def test_data_errors_mark_sequence(orc):
    """NaN / +inf in a row the outcome reads, an all -inf row, or a draft
    token outside [0, V) gives num_accepted = -1 for that sequence only."""
    rng = np.random.default_rng(12)
    B, N, V = 6, 3, 20
    zq = rng.normal(size=(B, N + 1, V)).astype(np.float32)
    zp = (zq[:, :N] + 0.1).astype(np.float32)
    d = rng.integers(0, V, size=(B, N)).astype(np.int32)
    zq[1, 2, 4] = np.nan
    zp[2, 0, 0] = np.inf
    zq[3, 1, :] = -np.inf
    d[4, 2] = V
    out = orc.verify_chain(zq, zp, d, 0, 0)
    assert out["num_accepted"].tolist()[:5] == [out["num_accepted"][0], -1, -1, -1, -1]
    assert out["num_accepted"][0] >= 0 and out["num_accepted"][5] >= 0
    assert (out["tokens"][1:5] == -1).all()


def test_chain_uses_documented_uniforms(orc):
    """Position i's decision uses the accept uniform of position i and the
    emitted token uses the sampling uniform of slot k+1, both from the Philox
    layout (seed; position, sequence, round)."""
    rng = np.random.default_rng(21)
    B, N, V, seed, rnd = 40, 4, 50, 0xABCDEF, 12
    zq = rng.normal(0, 2, size=(B, N + 1, V))
    zp = zq[:, :N] + rng.normal(0, 1, size=(B, N, V))
    d = rng.integers(0, V, size=(B, N)).astype(np.int32)
    out = orc.verify_chain(zq, zp, d, seed, rnd, T=1.3)
    for b in range(B):
        for i in range(N):
            assert out["u_acc"][b, i] == orc.uniforms(seed, rnd, b, i + 1)[0]
        k = out["num_accepted"][b]
        assert out["u_samp"][b] == orc.uniforms(seed, rnd, b, k + 1)[1]
        assert out["target"][b] == out["u_samp"][b] * out["weight_total"][b]


def test_residual_of_equal_rows_falls_back_to_q(orc):
    """[PT] Implementando, Passo 2: when (q - p)_+ sums to zero the residual
    is q itself."""
    z = np.array([0.3, -1.0, 2.0, 0.0, 0.5])
    res, kind = orc.residual_probs(z, z.copy(), T=0.8)
    assert kind == orc.KIND_RESIDUAL_WAS_ZERO
    assert np.allclose(res, softmax(z / 0.8), rtol=0, atol=1e-15)
    res, kind = orc.residual_probs(z, z[::-1].copy())
    assert kind == orc.KIND_RESIDUAL


def test_inverse_cdf_edges_are_strict(orc):
    """The inverse CDF takes the first token whose running sum is strictly
    above u*W, so a threshold that lands exactly on an edge belongs to the
    next token, zero-weight tokens are never chosen, and u = 0 gives the
    first positive-weight token."""
    assert orc.inverse_cdf([1.0, 1.0, 2.0], 0.5) == 2  # u*W = 2 = running sum at t=1
    assert orc.inverse_cdf([1.0, 1.0, 2.0], 0.0) == 0
    assert orc.inverse_cdf([0.0, 1.0, 0.0, 1.0], 0.0) == 1
    assert orc.inverse_cdf([0.0, 1.0, 0.0, 1.0], 0.5) == 3
    assert orc.inverse_cdf([3.0, 0.0, 0.0], TOP) == 0


def test_cdf_edges_of_queried_tokens(orc):
    """The CDF edges the oracle reports for a queried token (used to excuse a
    device token that differs from the oracle's) are the running sums of the
    distribution sampled from, just before and just after that token: for
    the bonus (N = 0) against np.cumsum of scipy's softmax, for a rejection
    against np.cumsum of max(0, q - p) from scipy's softmaxes, and for the
    draft sampler against np.cumsum of softmax(z / T).  Querying the oracle's
    own token returns its (edge_lo, edge_hi) exactly."""
    rng = np.random.default_rng(41)
    B, V, T = 64, 700, 0.8125
    # bonus: q_1 sampled directly
    zq = rng.normal(0, 3, size=(B, 1, V))
    d0 = np.zeros((B, 0), np.int32)
    own = orc.verify_chain(zq, np.zeros((B, 0, V)), d0, seed=3, rnd=1, T=T)
    assert (own["sample_kind"] == orc.KIND_BONUS).all()
    same = orc.verify_chain(zq, np.zeros((B, 0, V)), d0, seed=3, rnd=1, T=T, query=own["tokens"][:, 0])
    assert np.array_equal(same["qedge_lo"], own["edge_lo"]) and np.array_equal(same["qedge_hi"], own["edge_hi"])
    query = rng.integers(0, V, size=B).astype(np.int32)
    out = orc.verify_chain(zq, np.zeros((B, 0, V)), d0, seed=3, rnd=1, T=T, query=query)
    for b in range(B):
        c = np.concatenate([[0.0], np.cumsum(softmax(zq[b, 0] / T))])
        g = query[b]
        assert abs(out["qedge_lo"][b] - c[g]) <= 1e-13 and abs(out["qedge_hi"][b] - c[g + 1]) <= 1e-13
    # residual: one draft, rejected (the largest uniform rejects every ratio below 1)
    zq = rng.normal(0, 2, size=(B, 2, V))
    zp = zq[:, :1] + rng.normal(0, 1.5, size=(B, 1, V))
    d = np.array([[int(np.argmax(zp[b, 0] - zq[b, 0]))] for b in range(B)], np.int32)  # q(d) < p(d)
    u = np.zeros((B, 3))
    u[:, 0] = TOP
    u[:, 1] = rng.random(B)
    query = rng.integers(0, V, size=B).astype(np.int32)
    out = orc.verify_chain(zq, zp, d, seed=0, rnd=0, T=T, u=u, query=query)
    assert (out["num_accepted"] == 0).all() and (out["sample_kind"] == orc.KIND_RESIDUAL).all()
    for b in range(B):
        w = np.maximum(0.0, softmax(zq[b, 0] / T) - softmax(zp[b, 0] / T))
        c = np.concatenate([[0.0], np.cumsum(w)])
        g = query[b]
        assert abs(out["qedge_lo"][b] - c[g]) <= 1e-13 and abs(out["qedge_hi"][b] - c[g + 1]) <= 1e-13
        assert abs(out["weight_total"][b] - c[-1]) <= 1e-13
    # draft sampler
    zd = rng.normal(0, 3, size=(8, 3, V))
    query = rng.integers(0, V, size=(8, 3)).astype(np.int32)
    o = orc.sample_draft(zd, seed=11, rnd=2, T=T, query=query)
    for b in range(8):
        for r in range(3):
            c = np.concatenate([[0.0], np.cumsum(softmax(zd[b, r] / T))])
            g = query[b, r]
            assert abs(o["qedge_lo"][b, r] - c[g]) <= 1e-13 and abs(o["qedge_hi"][b, r] - c[g + 1]) <= 1e-13
