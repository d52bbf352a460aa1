"""Pins of the oracle's tree walk and KV compaction (no GPU).

Pages: [ZH] "投机解码与 EAGLE：步骤、发展历史与三代差异" (caijizhuo.github.io),
section 3 (the flattened tree and its mask; KV rows of the accepted path are
copied together after acceptance) and section 4 ("eagle_round", step 4, the
walk from the root); [PT] "Decodificacao Especulativa e EAGLE-3", "Reversao
de KV cache" and Implementando, Passo 4.

The walk reading (tested here): node n >= 1 is tested with q/p of its parent;
from the root, descend into the lowest-index accepted child; stop at a leaf
(bonus from the leaf's q) or where no child is accepted (residual of that
node's q and p); no bonus after a rejection.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import chi2

import synth
from _stats import chi2_pooled

TOP = 1.0 - 2.0 ** -53


def _walk(parents, flags):
    """Brute-force walk over accept flags (flags[0] unused)."""
    nn = len(parents)
    kids = {n: [c for c in range(1, nn) if parents[c] == n] for n in range(nn)}
    path, cur = [0], 0
    while True:
        if not kids[cur]:
            return path, cur, "bonus"
        nxt = [c for c in kids[cur] if flags[c]]
        if not nxt:
            return path, cur, "residual"
        cur = nxt[0]
        path.append(cur)


def _random_tree(rng, nn):
    return [-1] + [int(rng.integers(0, n)) for n in range(1, nn)]


def _depth(parents):
    d = [0] * len(parents)
    for n in range(1, len(parents)):
        d[n] = d[parents[n]] + 1
    return max(d)


def _chain_as_tree(zq, zp, d):
    B, N1, V = zq.shape
    N = N1 - 1
    zpt = np.concatenate([zp, zq[:, N:N + 1]], axis=1)  # leaf p row never read
    tok = np.concatenate([np.zeros((B, 1), np.int32), d], axis=1)
    parents = np.arange(-1, N, dtype=np.int32)
    return zpt, tok, parents


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_path_tree_equals_chain_bit_for_bit(orc, dtype):
    """A path-shaped tree (parent[n] = n-1) is the chain: same decisions,
    tokens, ratios and uniforms, bit for bit (independent code paths)."""
    w = synth.WORKLOADS["chain_b256_v128256"].with_sizes(V=3001, dtype=dtype, B=40, N=6)
    inp = synth.chain_inputs(w, seed=3, device="cpu")
    zq, zp, d = synth.to_oracle(inp["zq"]), synth.to_oracle(inp["zp"]), inp["d"].numpy()
    ch = orc.verify_chain(zq, zp, d, seed=17, rnd=5, T=0.9)
    zpt, tok, parents = _chain_as_tree(zq, zp, d)
    tr = orc.verify_tree(zq, np.ascontiguousarray(zpt), tok, parents, seed=17, rnd=5, T=0.9, max_depth=w.N)
    assert (ch["num_accepted"] == tr["num_accepted"]).all()
    assert (ch["tokens"] == tr["tokens"]).all()
    assert (ch["accept"] == tr["accept"][:, 1:]).all()
    assert np.array_equal(ch["ratio"], tr["ratio"][:, 1:])
    assert np.array_equal(ch["q_tok"], tr["q_tok"][:, 1:])
    assert np.array_equal(ch["weight_total"], tr["weight_total"])
    k = ch["num_accepted"]
    for b in range(w.B):
        assert tr["path_nodes"][b, :k[b] + 1].tolist() == list(range(k[b] + 1))
    assert 0 < (k == w.N).sum() < w.B and (k < w.N).sum() > 0  # both branches exercised


@pytest.mark.parametrize("nn", [2, 4, 7])
def test_tree_walk_under_forced_flags(orc, nn):
    """For random tiny trees and every accept-flag pattern that the rows
    allow, the oracle's path, stop node and sample kind equal a brute-force
    walk, and its token's sampling interval carries exactly the residual
    (or, at a leaf, q) mass."""
    rng = np.random.default_rng(nn)
    V = 6
    for trial in range(6):
        parents = _random_tree(rng, nn)
        md = _depth(parents)
        zq = rng.normal(0, 1.5, size=(nn, V))
        zp = zq + rng.normal(0, 1.0, size=(nn, V))
        tok = [0] + [int(rng.integers(0, V)) for _ in range(1, nn)]
        q, p = softmax(zq, axis=1), softmax(zp, axis=1)
        a = np.array([1.0] + [min(1.0, q[parents[n], tok[n]] / p[parents[n], tok[n]]) for n in range(1, nn)])
        pats = [f for f in itertools.product([0, 1], repeat=nn - 1)
                if all((fl == 1 and a[n + 1] > 0) or (fl == 0 and a[n + 1] < 1) for n, fl in enumerate(f))]
        B = len(pats)
        u = np.zeros((B, nn - 1 + md + 1))
        for i, f in enumerate(pats):
            u[i, :nn - 1] = [0.0 if fl else TOP for fl in f]
        u[:, nn - 1:] = 0.61
        out = orc.verify_tree(np.broadcast_to(zq[None], (B, nn, V)), np.broadcast_to(zp[None], (B, nn, V)),
                              np.tile(np.array(tok, np.int32), (B, 1)), np.array(parents, np.int32), 0, 0,
                              max_depth=md, u=u)
        for i, f in enumerate(pats):
            path, stop, kind = _walk(parents, (1,) + f)
            k = len(path) - 1
            assert out["num_accepted"][i] == k
            assert out["path_nodes"][i, :k + 1].tolist() == path
            assert out["stop_node"][i] == stop
            assert out["tokens"][i, :k].tolist() == [tok[n] for n in path[1:]]
            assert out["accept"][i, 1:].tolist() == list(f)
            if kind == "bonus":
                law = q[stop]
                assert out["sample_kind"][i] == orc.KIND_BONUS
            else:
                r = np.maximum(q[stop] - p[stop], 0.0)
                law = r / r.sum()
                assert out["sample_kind"][i] == orc.KIND_RESIDUAL
            t = out["tokens"][i, k]
            mass = (out["edge_hi"][i] - out["edge_lo"][i]) / out["weight_total"][i]
            assert abs(mass - law[t]) < 1e-12


def _walk_best(parents, flags):
    """Brute-force literal walk: only the lowest-index child is tried."""
    nn = len(parents)
    kids = {n: [c for c in range(1, nn) if parents[c] == n] for n in range(nn)}
    path, cur = [0], 0
    while True:
        if not kids[cur]:
            return path, cur, "bonus"
        if not flags[kids[cur][0]]:
            return path, cur, "residual"
        cur = kids[cur][0]
        path.append(cur)


@pytest.mark.parametrize("nn", [3, 5, 8])
def test_best_child_walk_under_forced_flags(orc, nn):
    """walk = 1 (the pages' literal walk): for random tiny trees and every
    accept-flag pattern the rows allow, path, stop node and sample kind equal
    a brute-force walk that only tries each node's first child."""
    rng = np.random.default_rng(100 + nn)
    V = 6
    for trial in range(6):
        parents = _random_tree(rng, nn)
        md = _depth(parents)
        zq = rng.normal(0, 1.5, size=(nn, V))
        zp = zq + rng.normal(0, 1.0, size=(nn, V))
        tok = [0] + [int(rng.integers(0, V)) for _ in range(1, nn)]
        q, p = softmax(zq, axis=1), softmax(zp, axis=1)
        a = np.array([1.0] + [min(1.0, q[parents[n], tok[n]] / p[parents[n], tok[n]]) for n in range(1, nn)])
        pats = [f for f in itertools.product([0, 1], repeat=nn - 1)
                if all((fl == 1 and a[n + 1] > 0) or (fl == 0 and a[n + 1] < 1) for n, fl in enumerate(f))]
        B = len(pats)
        u = np.zeros((B, nn - 1 + md + 1))
        for i, f in enumerate(pats):
            u[i, :nn - 1] = [0.0 if fl else TOP for fl in f]
        u[:, nn - 1:] = 0.37
        out = orc.verify_tree(np.broadcast_to(zq[None], (B, nn, V)), np.broadcast_to(zp[None], (B, nn, V)),
                              np.tile(np.array(tok, np.int32), (B, 1)), np.array(parents, np.int32), 0, 0,
                              max_depth=md, u=u, walk=1)
        for i, f in enumerate(pats):
            path, stop, kind = _walk_best(parents, (1,) + f)
            k = len(path) - 1
            assert out["num_accepted"][i] == k
            assert out["path_nodes"][i, :k + 1].tolist() == path
            assert out["stop_node"][i] == stop
            assert out["accept"][i, 1:].tolist() == list(f)  # every node is still decided
            want = orc.KIND_BONUS if kind == "bonus" else orc.KIND_RESIDUAL
            assert out["sample_kind"][i] == want


def test_best_child_walk_ignores_an_accepted_sibling(orc):
    """Root with two children: the first rejected, the second accepted.
    The default walk takes the second; the literal walk stops at the root
    and resamples from the root's residual."""
    V = 5
    zq = np.log(np.array([[0.05, 0.60, 0.15, 0.10, 0.10]] * 3))
    zp = np.log(np.array([[0.60, 0.05, 0.15, 0.10, 0.10]] * 3))
    tok = np.array([[0, 0, 1]], np.int32)                      # child 1: a = 1/12, child 2: a = 1
    parents = np.array([-1, 0, 0], np.int32)
    u = np.array([[0.5, 0.5, 0.3, 0.3]])                       # child 1 rejected (0.5 > 1/12), child 2 accepted
    d0 = orc.verify_tree(zq[None], zp[None], tok, parents, 0, 0, max_depth=1, u=u, walk=0)
    d1 = orc.verify_tree(zq[None], zp[None], tok, parents, 0, 0, max_depth=1, u=u, walk=1)
    assert d0["num_accepted"][0] == 1 and d0["path_nodes"][0].tolist() == [0, 2]
    assert d0["sample_kind"][0] == orc.KIND_BONUS
    assert d1["num_accepted"][0] == 0 and d1["path_nodes"][0, 0] == 0 and d1["stop_node"][0] == 0
    assert d1["sample_kind"][0] == orc.KIND_RESIDUAL
    # residual of the root: (q - p)_+ = 0.55 on token 1 only
    assert d1["tokens"][0, 0] == 1 and abs(d1["resid_mass"][0] - 0.55) < 1e-12


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_best_child_walk_is_the_chain_on_the_best_child_path(orc, seed):
    """walk = 1 on any tree equals the chain verify (a separate code path)
    run on the tree's best-child path: the chain's rows are those of the path
    nodes, its drafts their tokens, its uniforms the path nodes' accept
    uniforms and the tree's sampling uniforms."""
    rng = np.random.default_rng(seed)
    nn, V, B = 14, 700, 96
    parents = _random_tree(rng, nn)
    md = _depth(parents)
    zq = rng.normal(0, 2.0, size=(B, nn, V))
    zp = zq + rng.normal(0, 0.7, size=(B, nn, V))
    tok = np.concatenate([np.zeros((B, 1), np.int32),
                          rng.integers(0, V, size=(B, nn - 1)).astype(np.int32)], axis=1)
    # the best-child path, and drafts that are likely enough to be accepted
    path = [0]
    while True:
        kids = [c for c in range(1, nn) if parents[c] == path[-1]]
        if not kids:
            break
        path.append(kids[0])
    for i, n in enumerate(path[1:]):
        tok[:, n] = np.argsort(-zp[:, path[i]], axis=1)[:, rng.integers(0, 3)]
    u = rng.random((B, nn - 1 + md + 1))
    tr = orc.verify_tree(zq, zp, tok, np.array(parents, np.int32), 0, 0, max_depth=md, u=u, walk=1)
    N = len(path) - 1
    cq = np.ascontiguousarray(zq[:, path])
    cp = np.ascontiguousarray(zp[:, path[:-1]])
    d = np.ascontiguousarray(tok[:, path[1:]])
    cu = np.concatenate([u[:, [n - 1 for n in path[1:]]], u[:, nn - 1:nn - 1 + N + 1]], axis=1)
    ch = orc.verify_chain(cq, cp, d, 0, 0, u=cu)
    k = ch["num_accepted"]
    assert np.array_equal(k, tr["num_accepted"])
    assert np.array_equal(ch["tokens"], tr["tokens"][:, :N + 1])
    assert np.array_equal(ch["weight_total"], tr["weight_total"])
    assert np.array_equal(ch["sample_kind"], tr["sample_kind"])
    for b in range(B):
        assert tr["path_nodes"][b, :k[b] + 1].tolist() == path[:k[b] + 1]
    assert (k == N).any() and (k < N).any()  # both ends of the walk exercised


def test_tree_law_chi_square(orc):
    """Philox-driven tree rounds fit the exact law of (stop node, token)
    obtained by enumerating all 2^T accept patterns with weights
    prod a_n or (1 - a_n) and the brute-force walk (chi-square < 99.9%)."""
    rng = np.random.default_rng(2024)
    nn, V, R = 6, 5, 300_000
    parents = [-1, 0, 0, 1, 1, 2]
    zq = rng.normal(0, 1.2, size=(nn, V))
    zp = zq + rng.normal(0, 0.8, size=(nn, V))
    tok = [0, 1, 3, 0, 2, 4]
    q, p = softmax(zq, axis=1), softmax(zp, axis=1)
    a = np.array([1.0] + [min(1.0, q[parents[n], tok[n]] / p[parents[n], tok[n]]) for n in range(1, nn)])
    law = {}
    for f in itertools.product([0, 1], repeat=nn - 1):
        wgt = np.prod([a[n + 1] if fl else 1 - a[n + 1] for n, fl in enumerate(f)])
        if wgt == 0:
            continue
        path, stop, kind = _walk(parents, (1,) + f)
        if kind == "bonus":
            dist = q[stop]
        else:
            r = np.maximum(q[stop] - p[stop], 0.0)
            dist = r / r.sum()
        for t in range(V):
            law[(stop, t)] = law.get((stop, t), 0.0) + wgt * dist[t]
    keys = sorted(law)
    probs = np.array([law[kk] for kk in keys])
    assert abs(probs.sum() - 1) < 1e-12
    out = orc.verify_tree(np.broadcast_to(zq[None], (R, nn, V)), np.broadcast_to(zp[None], (R, nn, V)),
                          np.tile(np.array(tok, np.int32), (R, 1)), np.array(parents, np.int32), seed=99, rnd=1,
                          max_depth=_depth(parents))
    k = out["num_accepted"]
    last = out["tokens"][np.arange(R), k]
    idx = {kk: i for i, kk in enumerate(keys)}
    counts = np.zeros(len(keys))
    np.add.at(counts, [idx[(s, t)] for s, t in zip(out["stop_node"], last)], 1)
    stat, df = chi2_pooled(counts, probs)
    assert stat < chi2.ppf(0.999, df), (stat, df)


def test_tree_data_errors(orc):
    """A parent outside [0, n) or a walk deeper than max_depth marks the
    sequence (-1); the other sequences are unaffected."""
    rng = np.random.default_rng(5)
    B, nn, V = 3, 5, 7
    zq = rng.normal(size=(B, nn, V))
    zp = zq.copy()  # everything accepted -> the walk reaches a leaf
    tok = rng.integers(0, V, size=(B, nn)).astype(np.int32)
    parents = np.tile(np.array([-1, 0, 1, 2, 3], np.int32), (B, 1))
    parents[1, 3] = 3  # not < 3
    out = orc.verify_tree(zq, zp, tok, parents, 0, 0, max_depth=4)
    assert out["num_accepted"].tolist() == [4, -1, 4]
    out = orc.verify_tree(zq, zp, tok, np.array([-1, 0, 1, 2, 3], np.int32), 0, 0, max_depth=3)
    assert (out["num_accepted"] == -1).all()


def test_static_tree_shape():
    """The 26-node static tree: level sizes 4, 8, 8, 3, 2; 18 internal nodes;
    depth 5; siblings in descending draft order."""
    par = synth.STATIC_TREE_PARENTS
    depth = [0] * len(par)
    for n in range(1, len(par)):
        assert 0 <= par[n] < n
        depth[n] = depth[par[n]] + 1
    assert len(par) == 26 and max(depth) == 5
    assert [depth.count(L) for L in range(1, 6)] == [4, 8, 8, 3, 2]
    assert len(set(par[1:])) == 18
    w = synth.WORKLOADS["tree_static_b32_v128256"].with_sizes(V=500, B=3)
    inp = synth.static_tree_inputs(w, seed=1)
    for n in range(len(par)):
        kids = [c for c in range(1, len(par)) if par[c] == n]
        if len(kids) > 1:
            vals = inp["zp"][:, n, :].float().gather(1, inp["tokens"][:, kids].long())
            assert (vals[:, :-1] >= vals[:, 1:]).all()


def test_dynamic_tree_shape():
    """Dynamic trees: budget+1 nodes, parents before children, depth <= 6,
    siblings by descending path score, and every kept node's ancestors kept."""
    w = synth.WORKLOADS["tree_dynamic_b128_v152064"].with_sizes(V=400, B=4)
    inp = synth.dynamic_tree_inputs(w, seed=2)
    par = inp["parents"].numpy()
    assert par.shape == (4, 61)
    for b in range(4):
        depth = [0] * 61
        for n in range(1, 61):
            assert 0 <= par[b, n] < n
            depth[n] = depth[par[b, n]] + 1
        assert max(depth) <= 6
        assert depth == inp["depth_of"][b].tolist()


@pytest.mark.parametrize("chain", [True, False])
def test_kv_gather_matches_fancy_indexing(orc, chain):
    """KV compaction ([ZH] section 3; [PT] Passo 4): rows L0+path[i] move to
    L0+i for i <= k in every plane (the gather equals numpy fancy indexing
    on a copy); kv_len = L0 + k + 1; a failed sequence (k = -1) keeps its
    length and its rows."""
    rng = np.random.default_rng(7)
    P, B, L, rb, md = 3, 5, 40, 48, 6
    kv = rng.integers(0, 256, size=(P, B, L, rb), dtype=np.uint8)
    orig = kv.copy()
    k = np.array([6, 0, 3, -1, 2], np.int32)
    L0 = np.array([10, 3, 20, 5, 30], np.int32)
    path = np.full((B, md + 1), -1, np.int32)
    for b in range(B):
        if k[b] >= 0:
            nodes = [0] if chain else [0] + sorted(rng.choice(np.arange(1, 9), size=k[b], replace=False).tolist())
            path[b, :k[b] + 1] = list(range(k[b] + 1)) if chain else nodes
    src, kvl = orc.kv_compact(None if chain else path, k, L0, md, kv=kv)
    expect = orig.copy()
    for b in range(B):
        if k[b] < 0:
            assert kvl[b] == L0[b] and (src[b] == -1).all()
            continue
        assert kvl[b] == L0[b] + k[b] + 1
        rows = L0[b] + path[b, :k[b] + 1]
        assert src[b, :k[b] + 1].tolist() == rows.tolist() and (src[b, k[b] + 1:] == -1).all()
        expect[:, b, L0[b]:L0[b] + k[b] + 1] = orig[:, b, rows]
    assert np.array_equal(kv, expect)
