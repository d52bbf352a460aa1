"""Pins of the oracle's draft-token sampler (no GPU).

Pages: [PT] "Decodificacao Especulativa e EAGLE-3", O Conceito and
Implementando, Passo 1 (the draft proposes d ~ p); [ZH] "投机解码与 EAGLE"
section 2 (each draft token drawn from the draft model's softmax in turn).
Readings: R3 (inverse CDF in token order, threshold u*W, strict >,
fallback to the last positive-weight token) and R4 (Philox uniforms; the
draft draws use stream 1).  Each pin checks the oracle against something it
does not compute itself: scipy's softmax / log-softmax, numpy's
searchsorted over a cumulative sum, stratified uniforms, and the Philox
known answers pinned elsewhere.
"""
import numpy as np
import pytest
from scipy.special import log_softmax, softmax

import oracle


def _rows(B, R, V, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, R, V)) * scale).astype(np.float32)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_stratified_uniforms_give_the_softmax_law(T):
    """n stratified uniforms (i + 1/2)/n on one row: token counts equal n*p
    within one count (p = scipy softmax(z / T))."""
    V, n = 9, 20000
    z = _rows(1, 1, V, 3)[0, 0]
    zp = np.broadcast_to(z, (n, 1, V))
    u = ((np.arange(n) + 0.5) / n).reshape(n, 1)
    o = oracle.sample_draft(np.ascontiguousarray(zp), 0, 0, T, u=u)
    counts = np.bincount(o["tokens"][:, 0], minlength=V)
    p = softmax(z.astype(np.float64) / np.float32(T))
    assert np.abs(counts - n * p).max() <= 1.0 + 1e-9


def test_uniform_source_and_token_by_searchsorted():
    """The uniform is Philox stream 1 at (b, pos0 + r), words 0 and 1; the
    token is numpy's searchsorted of u*W in the cumulative softmax."""
    B, R, V = 5, 4, 300
    zp = _rows(B, R, V, 7)
    o = oracle.sample_draft(zp, seed=99, rnd=12, T=0.9, pos0=3)
    L = oracle.lib()
    import ctypes
    for b in range(B):
        for r in range(R):
            w = (ctypes.c_uint32 * 4)()
            L.orc_philox_block(99, 12, b, 3 + r, 1, w)
            u = L.orc_u53(w[0], w[1])
            assert o["u"][b, r] == u
            p = softmax(zp[b, r].astype(np.float64) / np.float32(0.9))
            c = np.cumsum(p)
            assert o["tokens"][b, r] == int(np.searchsorted(c, u * c[-1], side="right"))


def test_verify_stream_differs_from_draft_stream():
    """Stream 1 is not the verify stream: the draft's uniform differs from
    the verify accept uniform of the same (sequence, position)."""
    zp = _rows(3, 2, 50, 1)
    o = oracle.sample_draft(zp, seed=5, rnd=1, pos0=1)
    ua = np.empty((3, 2))
    us = np.empty((3, 2))
    oracle.lib().orc_uniform_grid(5, 1, 3, 2, ua.ctypes.data_as(oracle.ctypes.c_void_p),
                                  us.ctypes.data_as(oracle.ctypes.c_void_p))
    assert not np.isin(o["u"], ua).any() and not np.isin(o["u"], us).any()


def test_logprob_is_log_softmax():
    B, R, V = 4, 3, 1000
    zp = _rows(B, R, V, 11)
    o = oracle.sample_draft(zp, 1, 2, T=0.7)
    for b in range(B):
        for r in range(R):
            lp = log_softmax(zp[b, r].astype(np.float64) / np.float32(0.7))
            assert abs(o["logprob"][b, r] - lp[o["tokens"][b, r]]) < 1e-12


def test_edges_and_masked_tokens():
    """u = 0 gives the first token of positive weight; u just below 1 the
    last; -inf logits are never drawn; the edges bracket u*W."""
    V = 12
    z = np.full((1, 1, V), -np.inf, np.float32)
    z[0, 0, [2, 5, 9]] = [0.0, 1.0, -1.0]
    zp = np.ascontiguousarray(np.broadcast_to(z, (3, 1, V)))
    u = np.array([[0.0], [0.5], [1.0 - 2.0 ** -53]])
    o = oracle.sample_draft(zp, 0, 0, u=u)
    assert o["tokens"][:, 0].tolist()[0] == 2 and o["tokens"][2, 0] == 9
    assert set(o["tokens"][:, 0].tolist()) <= {2, 5, 9}
    assert (o["edge_lo"] <= o["target"]).all() and (o["target"] < o["edge_hi"]).all()


def test_bad_rows_give_minus_one():
    V = 40
    zp = _rows(4, 1, V, 2)
    zp[0, 0, 3] = np.nan
    zp[1, 0, 7] = np.inf
    zp[2, 0, :] = -np.inf
    o = oracle.sample_draft(zp, 0, 0)
    assert o["tokens"][:3, 0].tolist() == [-1, -1, -1] and np.isnan(o["logprob"][:3, 0]).all()
    assert 0 <= o["tokens"][3, 0] < V


def test_bf16_rows_read_as_their_float_values():
    """bf16 bits (uint16) sample exactly as the float32 values they encode."""
    zp = _rows(3, 2, 257, 4)
    bits = (zp.view(np.uint32) >> 16).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    a = oracle.sample_draft(bits, 8, 8, T=0.8)
    b = oracle.sample_draft(np.ascontiguousarray(f), 8, 8, T=0.8)
    assert np.array_equal(a["tokens"], b["tokens"]) and np.allclose(a["logprob"], b["logprob"], rtol=0, atol=1e-13)
