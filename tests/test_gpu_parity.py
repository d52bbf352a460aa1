"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name before it runs.  Sizes: reduced cases span
several 2048-element chunks and a ragged tail and run the oracle on every
sequence; the full-size workloads (chains of B=1, 64, 256 sequences, static and dynamic trees) run the device path in the launch
configuration the benchmark times and the oracle on a window of sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import log, run_chain, run_tree
from oracle import compare

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_14_amd as sv
    sv.library()
    oracle.lib()


def _done(name, rep):
    log(f"[parity] {name}: {rep.summary()}")
    rep.check()


# --------------------------------------------------------------------------- #
# Philox
# --------------------------------------------------------------------------- #
def test_device_philox_matches_oracle():
    """10^7 counters (10 seeds/rounds x 1000 sequences x 1000 positions):
    the device uniforms equal the oracle's bit for bit."""
    import rejection_sampling_verify_14_amd as sv
    for i, (seed, rnd) in enumerate([(0, 0), (1, 7), (2 ** 40 + 3, 2 ** 33 + 9), (123456789, 499), (7, 2 ** 32),
                                     (2 ** 64 - 1, 2 ** 60 - 1), (42, 1), (99, 12), (5, 6), (31337, 0)]):
        log(f"[philox] seed={seed} round={rnd}")
        a, s = sv.sv_philox_uniforms(seed, rnd, 1000, 1000)
        ea, es = oracle.uniform_grid(seed, rnd, 1000, 1000)
        assert np.array_equal(a.cpu().numpy(), ea)
        assert np.array_equal(s.cpu().numpy(), es)


# --------------------------------------------------------------------------- #
# Chains, reduced sizes (oracle on every sequence)
# --------------------------------------------------------------------------- #
CHAIN_CASES = [
    # name, workload, overrides (B, N, V, T, dtype)
    ("chain_b64_small_ragged", "chain_b64_v32000", dict(B=16, N=5, V=9001)),
    ("chain_b256_small_bf16", "chain_b256_v128256", dict(B=24, N=7, V=20011)),
    ("chain_b256_temp07", "chain_b256_v128256", dict(B=16, N=4, V=12289, T=0.7)),
    ("chain_b256_n1", "chain_b256_v128256", dict(B=40, N=1, V=5000)),
    ("chain_b256_n64", "chain_b256_v128256", dict(B=4, N=64, V=3001)),
    ("chain_b1_tiny_v", "chain_b1_v32", dict(B=50, N=4, V=32)),
    ("v_tail_only", "chain_b64_v32000", dict(B=8, N=3, V=7)),
    ("v_one_token", "chain_b64_v32000", dict(B=4, N=2, V=1)),
    ("f32_temp19", "chain_b64_v32000", dict(B=12, N=6, V=4097, T=1.9)),
]


@pytest.mark.parametrize("name,wl,ov", CHAIN_CASES, ids=[c[0] for c in CHAIN_CASES])
def test_chain_parity_reduced(name, wl, ov):
    log(f"[case] {name}")
    w = W[wl].with_sizes(**{k: v for k, v in ov.items() if k in ("V", "T")})
    rep = compare.Report()
    for rnd in range(3):
        r, g, _ = run_chain(w, seed=1000 + rnd, rnd=rnd, B=ov.get("B"), N=ov.get("N"))
        rep.merge(r)
    _done(name, rep)


# --------------------------------------------------------------------------- #
# Chains of bf16 logits in 16-byte aligned rows (V a multiple of 8): the
# sample step that reads exp(z/T) from the bf16-grid table
# --------------------------------------------------------------------------- #
TABLE_CASES = [
    # name, overrides: less than one chunk, whole chunks only, several
    # temperatures (each moves the table's binades)
    ("tab_v1504", dict(B=16, N=3, V=1504, T=1.0)),
    ("tab_v2048", dict(B=16, N=5, V=2048, T=1.0)),
    ("tab_v6144_t07", dict(B=16, N=4, V=6144, T=0.7)),
    ("tab_v10008_t33", dict(B=16, N=7, V=10008, T=3.3)),
    ("tab_v8000_t013", dict(B=12, N=2, V=8000, T=0.13)),
    # which wave forms the partial last chunk: a full last block of four
    # one-chunk waves (wave 0 of the first block takes it), a last block of
    # three (its idle fourth wave), and 80 sequences, whose first groups use
    # blocks of eight chunks (two per wave; a full last block)
    ("tab_v16904_last_full", dict(B=16, N=3, V=16904, T=1.0)),
    ("tab_v18440_last_three", dict(B=16, N=3, V=18440, T=1.0)),
    ("tab_v33768_b80", dict(B=80, N=2, V=33768, T=1.0)),
]


@pytest.mark.parametrize("name,ov", TABLE_CASES, ids=[c[0] for c in TABLE_CASES])
def test_chain_parity_table_path(name, ov):
    log(f"[case] {name}")
    w = W["chain_b256_v128256"].with_sizes(V=ov["V"], T=ov["T"])
    rep = compare.Report()
    for rnd in range(3):
        r, g, _ = run_chain(w, seed=4000 + rnd, rnd=rnd, B=ov["B"], N=ov["N"])
        rep.merge(r)
    _done(name, rep)


def test_chain_table_path_logits_outside_table():
    """bf16 rows with logits the table does not hold: zeros, tiny
    magnitudes (below 2^-12 T), large ones (at and above 2^7 T), -inf
    entries, subnormals; and whole sequences whose reference is beyond
    512 T (their rows take exp_rel throughout)."""
    log("[case] tab_outside")
    w = W["chain_b256_v128256"].with_sizes(V=8000)
    B, N = 16, 4

    def plant(inp):
        zq, zp = inp["zq"], inp["zp"]
        g = torch.Generator(device="cuda").manual_seed(5)
        V = w.V
        for t, v in [(0.0, 11), (-0.0, 12), (1e-6, 13), (-3e-5, 14), (2.0 ** -13, 15), (128.0, 16), (-200.0, 17),
                     (1e-40, 18), (-1e-39, 19)]:
            idx = torch.randint(0, V, (B, 64), generator=g, device="cuda")
            zq[:, :, :].scatter_(2, idx[:, None, :].expand(B, N + 1, 64), torch.full((B, N + 1, 64), t,
                                                                                  device="cuda", dtype=zq.dtype))
            idx2 = torch.randint(0, V, (B, 64), generator=g, device="cuda")
            zp[:, :, :].scatter_(2, idx2[:, None, :].expand(B, N, 64), torch.full((B, N, 64), -t if v % 2 else t,
                                                                               device="cuda", dtype=zp.dtype))
        zq[:, :, 100:160] = float("-inf")
        zp[:, :, 130:190] = float("-inf")
        zq[3] += 600.0      # reference beyond 512 T: no table for these rows
        zp[3] += 600.0
        zq[5] -= 700.0
        zp[5] -= 700.0
    rep = compare.Report()
    for rnd in range(3):
        r, g, _ = run_chain(w, seed=61 + rnd, rnd=rnd, B=B, N=N, modify=plant)
        rep.merge(r)
    _done("tab_outside", rep)


def test_chain_bonus_row_read_only_when_sampled():
    """bf16 chains whose bonus row q_{N+1} is read only by the bonus sample
    (it has no row statistics): all-accepted sequences with a NaN, a +inf,
    an all -inf bonus row (each -1), logits far outside the table (1000 and
    900 at T = 1, beyond exp's range in units of exp(z/T)), large ones
    (300), only tiny ones (below 2^-12 T), a single finite logit; and a
    rejected sequence whose bonus row holds a NaN (it is never read: valid)."""
    log("[case] bonus_lazy")
    w = W["chain_b256_v128256"].with_sizes(V=8000)
    B, N = 12, 3

    def plant(inp):
        zq, zp, d = inp["zq"], inp["zp"], inp["d"]
        for b in range(B):
            if b != 6:
                zp[b] = zq[b, :N]          # p == q: every draft accepted
        zq[0, N, 17] = float("nan")
        zq[1, N, 4000] = float("inf")
        zq[2, N, :] = float("-inf")
        zq[3, N, 100] = 1000.0
        zq[3, N, 7999] = 900.0
        zq[4, N, 50:70] = 300.0
        zq[5, N, :] = 1e-5 * torch.randn(w.V, device="cuda").to(zq.dtype)
        zq[7, N, :] = float("-inf")
        zq[7, N, 5555] = 2.5
        zq[6, 0, int(d[6, 0])] = float("-inf")   # rejected at once ...
        zq[6, N, 3] = float("nan")                # ... so its bonus row is never read
        zq[8, N, ::2] = float("-inf")
        zq[9, N, 2048:4096] = 40.0
    rep, g, _ = run_chain(w, seed=23, rnd=4, B=B, N=N, modify=plant)
    k = g["num_accepted"]
    assert k[0] == -1 and k[1] == -1 and k[2] == -1
    assert k[6] == 0 and all(int(k[b]) == N for b in (3, 4, 5, 7, 8, 9, 10, 11))
    assert int(g["tokens"][7, N]) == 5555
    _done("bonus_lazy", rep)


def test_chain_n0_plain_sampling():
    """N = 0: the step samples q_1 directly (no drafts)."""
    log("[case] chain_n0")
    w = W["chain_b256_v128256"].with_sizes(V=30001)
    rep, g, _ = run_chain(w, seed=3, rnd=3, B=32, N=0)
    assert (g["num_accepted"] == 0).all()
    _done("chain_n0", rep)


def test_chain_edge_cases():
    """NaN / +inf / all -inf rows, out-of-range tokens, -inf draft logit at d
    (accepted), q(d) = -inf (rejected), p == q (all accepted), and masked
    vocab entries, all in one batch."""
    log("[case] chain_edges")
    w = W["chain_b64_v32000"].with_sizes(V=6007)
    B, N = 12, 4

    def plant(inp):
        zq, zp, d = inp["zq"], inp["zp"], inp["d"]
        zq[1, 2, 100] = float("nan")
        zp[2, 0, 5] = float("inf")
        zq[3, 1, :] = float("-inf")
        d[4, 3] = w.V
        d[5, 0] = -1
        zp[6, 0, int(d[6, 0])] = float("-inf")
        zq[7, 0, int(d[7, 0])] = float("-inf")
        zp[8] = zq[8, :N]
        zq[9, :, ::3] = float("-inf")
        zp[9, :, ::3] = float("-inf")
        d[9] = ((d[9] // 3) * 3 + 1).clamp(max=w.V - 2)  # unmasked ids (V - 2 = 2 mod 3)
        zq[10, N, 7] = float("nan")   # bonus row: matters only if all are accepted
        zp[10] = zq[10, :N]          # ... which they are
    rep, g, _ = run_chain(w, seed=11, rnd=2, B=B, N=N, modify=plant)
    k = g["num_accepted"]
    assert k[1] == -1 and k[2] == -1 and k[3] == -1 and k[4] == -1 and k[5] == -1 and k[10] == -1
    assert g["accept"][6, 0] == 1 and g["accept"][7, 0] == 0 and k[8] == N
    _done("chain_edges", rep)


@pytest.mark.parametrize("dtype,noise", [("bf16", 0.0), ("f32", 1e-7), ("f32", 0.0)])
def test_residual_near_threshold_exact(dtype, noise):
    """Rows where q and p agree on almost every token (identical logits, or
    logits 1e-7 apart): many tokens sit at the q > p threshold.  The
    residual mass and the sampled token must still match the oracle."""
    log(f"[case] near_threshold {dtype} noise={noise}")
    w = W["chain_b256_v128256"].with_sizes(V=20000, dtype=dtype)
    B, N = 24, 3

    def plant(inp):
        g = torch.Generator(device="cuda").manual_seed(17)
        zq, zp = inp["zq"], inp["zp"]
        base = zq[:, :N].float()
        pert = base + noise * torch.randn(base.shape, generator=g, device="cuda")
        pert[:, :, :40] += torch.randn((B, N, 40), generator=g, device="cuda")  # a few real differences
        zp.copy_(pert.to(zp.dtype))
    rep = compare.Report()
    for rnd in range(3):
        r, g, _ = run_chain(w, seed=77 + rnd, rnd=rnd, B=B, N=N, modify=plant)
        rep.merge(r)
    _done(f"near_threshold_{dtype}_{noise}", rep)
    assert rep.max_mass_rel < 1e-9


def test_chain_strided_inputs():
    """Sequence and row strides larger than the packed layout."""
    log("[case] chain_strided")
    w = W["chain_b256_v128256"].with_sizes(V=8000)
    B, N = 10, 3
    inp = synth.chain_inputs(w, 5, "cuda", B=B, N=N)
    bigq = torch.zeros((B, N + 3, w.V + 24), dtype=inp["zq"].dtype, device="cuda")
    bigp = torch.zeros((B, N + 2, w.V + 40), dtype=inp["zp"].dtype, device="cuda")
    bigq[:, :N + 1, :w.V] = inp["zq"]
    bigp[:, :N, :w.V] = inp["zp"]
    inp2 = {"zq": bigq[:, :N + 1, :w.V], "zp": bigp[:, :N, :w.V], "d": inp["d"]}
    rep, g, _ = run_chain(w, seed=5, rnd=0, inputs=inp2)
    _done("chain_strided", rep)


# --------------------------------------------------------------------------- #
# Chains, full sizes
# --------------------------------------------------------------------------- #
def test_chain_b1_full_10000_rounds():
    """Chains of B=1, N=4, V=32 fp32, 10,000 rounds with Philox keyed by
    (seed, round, position); fixed logits, fresh d ~ p each round."""
    import rejection_sampling_verify_14_amd as sv
    log("[case] chain_b1_full")
    w = W["chain_b1_v32"]
    zq, zp = synth.chain_logits(w, 0, "cuda")
    R = w.rounds
    d_all = synth.chain_draft_tokens(w, zp.expand(R, -1, -1).contiguous(), seed=77)
    outs = sv.alloc_chain_outputs(1, w.N, "cuda")
    ws = sv.alloc_workspace(sv.chain_workspace_bytes(1, w.N, w.V), "cuda")
    toks, ks, accs, probs, mass = [], [], [], [], []
    for r in range(R):
        sv.spec_verify_chain(zq, zp, d_all[r:r + 1], seed=0, round=r, temperature=w.T, out=outs, workspace=ws)
        toks.append(outs["tokens"].clone())
        ks.append(outs["num_accepted"].clone())
        accs.append(outs["accept"].clone())
        probs.append(outs["probs"].clone())
        mass.append(outs["residual_mass"].clone())
    torch.cuda.synchronize()
    g = {"tokens": torch.cat(toks).cpu().numpy(), "num_accepted": torch.cat(ks).cpu().numpy(),
         "accept": torch.cat(accs).cpu().numpy(), "probs": torch.cat(probs).cpu().numpy(),
         "residual_mass": torch.cat(mass).cpu().numpy()}
    rep = compare.Report()
    zqn, zpn, dn = synth.to_oracle(zq), synth.to_oracle(zp), d_all.cpu().numpy()
    for r in range(R):
        o = oracle.verify_chain(zqn, zpn, dn[r:r + 1], 0, r, w.T, nthreads=1,
                                query=compare.sampled_tokens({k: v[r:r + 1] for k, v in g.items()}))
        rep.merge(compare.compare_chain({k: v[r:r + 1] for k, v in g.items()}, o))
    _done("chain_b1_full", rep)


@pytest.mark.parametrize("wl,rounds,window", [("chain_b64_v32000", 3, 64), ("chain_b256_v128256", 2, 24)])
def test_chain_full_size(wl, rounds, window):
    """Chains of B=64 (all 64 sequences) and B=256 (a window of sequences per round) at full
    size, in the benchmark's launch configuration."""
    w = W[wl]
    rep = compare.Report()
    for rnd in range(rounds):
        lo = (rnd * 97) % (w.B - window + 1)
        log(f"[case] {wl}_full round={rnd} window=({lo},{lo + window})")
        r, g, _ = run_chain(w, seed=500 + rnd, rnd=rnd, b_range=(lo, lo + window))
        log(f"   mean accepted {g['num_accepted'].mean():.3f} of {w.N}")
        rep.merge(r)
    _done(f"{wl}_full", rep)


def test_chain_b256_full_all_sequences_20_rounds():
    """Chains at full size (B=256, N=7, V=128256 bf16) in the benchmark's launch
    configuration: every sequence of 20 rounds (4 logit sets x 5 rounds)
    against the oracle.  Logs the decision band, flip, exclusion and excused
    mismatch counts; the comparison rules bound the excused mismatches."""
    w = W["chain_b256_v128256"]
    rep = compare.Report()
    for s in range(4):
        inp = synth.chain_inputs(w, 7000 + s, "cuda")
        for r in range(5):
            rnd = 5 * s + r
            log(f"[case] chain_b256_all set={s} round={rnd}")
            rr, g, _ = run_chain(w, seed=7000 + s, rnd=rnd, inputs=inp)
            rep.merge(rr)
        del inp
        torch.cuda.empty_cache()
    log(f"[rates] chain_b256_all: {rep.summary()} band_rate={rep.band_decisions / max(rep.decisions, 1):.3e} "
        f"excused_rate={rep.token_mismatch_excused / max(rep.samples, 1):.3e}")
    _done("chain_b256_all", rep)


# --------------------------------------------------------------------------- #
# Trees
# --------------------------------------------------------------------------- #
def test_path_tree_equals_chain_on_device():
    """A path-shaped tree gives the chain's decisions, path and tokens on the
    device.  The two split pass-1 rows differently (chains into equal wave
    ranges of all rows, trees into per-row segments), so the row sums may
    differ in their last bits: probabilities and residual mass agree to
    1e-9 relative."""
    import rejection_sampling_verify_14_amd as sv
    log("[case] path_tree_eq_chain")
    w = W["chain_b256_v128256"].with_sizes(V=10008)
    B, N = 20, 6
    inp = synth.chain_inputs(w, 8, "cuda", B=B, N=N)
    ch = sv.spec_verify_chain(inp["zq"], inp["zp"], inp["d"], seed=4, round=9, temperature=0.9)
    zpt = torch.cat([inp["zp"], inp["zq"][:, N:N + 1]], dim=1).contiguous()
    tok = torch.cat([torch.zeros((B, 1), dtype=torch.int32, device="cuda"), inp["d"]], dim=1).contiguous()
    par = torch.arange(-1, N, dtype=torch.int32, device="cuda")
    tr = sv.spec_verify_tree(inp["zq"], zpt, tok, par, seed=4, round=9, temperature=0.9, max_depth=N)
    torch.cuda.synchronize()
    assert torch.equal(ch["num_accepted"], tr["num_accepted"])
    assert torch.equal(ch["tokens"], tr["tokens"])
    assert torch.equal(ch["accept"], tr["accept"][:, 1:])
    torch.testing.assert_close(ch["probs"], tr["probs"][:, 1:], rtol=1e-6, atol=1e-37)
    torch.testing.assert_close(ch["residual_mass"], tr["residual_mass"], rtol=1e-9, atol=0.0)


def test_static_tree_reduced():
    log("[case] static_tree_reduced")
    w = W["tree_static_b32_v128256"].with_sizes(V=9001)
    rep = compare.Report()
    for rnd in range(3):
        inp = synth.static_tree_inputs(w, 40 + rnd, "cuda", B=12)
        r, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 40 + rnd, rnd, w.T, w.depth)
        rep.merge(r)
    _done("static_tree_reduced", rep)


def test_dynamic_tree_reduced():
    log("[case] dynamic_tree_reduced")
    w = W["tree_dynamic_b128_v152064"].with_sizes(V=7001)
    rep = compare.Report()
    for rnd in range(2):
        inp = synth.dynamic_tree_inputs(w, 60 + rnd, "cuda", B=10)
        r, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 60 + rnd, rnd, w.T, w.depth)
        rep.merge(r)
    _done("dynamic_tree_reduced", rep)


@pytest.mark.parametrize("wl", ["tree_static_b32_v128256", "tree_dynamic_b128_v152064"])
def test_best_child_walk_reduced(wl):
    """The pages' literal walk (walk = 1) on the static 26-node tree and
    the dynamic 61-node trees, reduced V: device vs oracle with walk = 1."""
    log(f"[case] best_child_walk_{wl}")
    w = W[wl].with_sizes(V=9001 if wl == "tree_static_b32_v128256" else 7001)
    rep = compare.Report()
    kd, ks = [], []
    for rnd in range(2):
        if wl == "tree_static_b32_v128256":
            inp = synth.static_tree_inputs(w, 70 + rnd, "cuda", B=16)
        else:
            inp = synth.dynamic_tree_inputs(w, 70 + rnd, "cuda", B=12)
        r, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 70 + rnd, rnd, w.T, w.depth, walk=1)
        rep.merge(r)
        r0, g0 = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 70 + rnd, rnd, w.T, w.depth, walk=0)
        rep.merge(r0)
        # same decisions, and the literal walk never goes deeper than the default one
        assert np.array_equal(g["accept"], g0["accept"])
        assert (g["num_accepted"] <= g0["num_accepted"]).all()
        kd.append(g0["num_accepted"].mean())
        ks.append(g["num_accepted"].mean())
    log(f"   mean accepted depth: first accepted child {np.mean(kd):.3f}, best child only {np.mean(ks):.3f}")
    _done(f"best_child_walk_{wl}", rep)


def test_walk_compare_matches_its_expectations():
    """Exercise 3's experiment (bench.py --walk-compare) at a reduced V: the
    device's tokens per verifier call for both walks and the chain lie within
    5 standard errors of their exact expectations from the same logits, and
    each leaf's reach rate within 5 binomial standard errors."""
    import importlib.util
    import os
    log("[case] walk_compare")
    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    res = bench.walk_compare(rounds=4, B=256, V=16384, seed=5)
    log(f"   {res}")
    for k in ("tree_first_accepted", "tree_best_child", "chain"):
        r = res[k]
        assert abs(r["tokens_per_call"] - r["expected"]) < 5 * r["std_err"] + 1e-3, (k, r)
    n = res["samples"]
    for m, e in zip(res["alpha_per_leaf"], res["alpha_per_leaf_expected"]):
        assert abs(m - e) < 5 * np.sqrt(max(e * (1 - e), 1e-4) / n) + 1e-3, (m, e)
    assert res["tree_first_accepted"]["expected"] >= res["tree_best_child"]["expected"]
    log("[done] walk_compare")


def _draft_case(name, rows, T, seed, rnd, pos0=0, b_sel=None):
    """Device draft draws vs the oracle: every device token's CDF interval
    holds the oracle's u*W, up to a band of 1e-6 W (draws decided inside the
    band are excused and counted; the device's weights are double, so none
    is expected), and ln p of the draws both sides make within 1e-6."""
    import rejection_sampling_verify_14_amd as sv
    log(f"[case] draft {name} rows={tuple(rows.shape)} T={T}")
    tok, lp = sv.sample_draft(rows, seed, rnd, T, pos0=pos0)
    torch.cuda.synchronize()
    tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
    if b_sel is None:
        o = oracle.sample_draft(synth.to_oracle(rows.contiguous()), seed, rnd, T, pos0=pos0, query=tok)
    else:
        # a sample of sequences: the oracle numbers them 0.., so it gets
        # their own uniforms (Philox stream 1 at (b, pos0 + r), words 0, 1)
        import ctypes
        tok, lp = tok[b_sel], lp[b_sel]
        L = oracle.lib()
        u = np.empty(tok.shape)
        for i, b in enumerate(b_sel):
            for r in range(tok.shape[1]):
                w4 = (ctypes.c_uint32 * 4)()
                L.orc_philox_block(seed, rnd, int(b), pos0 + r, 1, w4)
                u[i, r] = L.orc_u53(w4[0], w4[1])
        o = oracle.sample_draft(synth.to_oracle(rows[b_sel].contiguous()), seed, rnd, T, u=u, query=tok)
    bad = o["tokens"] < 0
    assert np.array_equal(tok[bad], o["tokens"][bad]) and np.isnan(lp[bad]).all(), f"{name}: bad rows"
    ok = ~bad
    band = 1e-6 * o["W"][ok]
    inside = (o["qedge_lo"][ok] - band <= o["target"][ok]) & (o["target"][ok] < o["qedge_hi"][ok] + band)
    assert inside.all(), f"{name}: {int((~inside).sum())} draws outside their CDF interval"
    exact = (tok[ok] == o["tokens"][ok])
    d = np.abs(lp[ok][exact] - o["logprob"][ok][exact])
    assert d.max(initial=0.0) < 1e-6, f"{name}: logprob error {d.max()}"
    excused = int((~exact).sum())
    log(f"[parity] draft {name}: draws={int(ok.sum())} exact={int(exact.sum())} excused={excused} "
        f"bad_rows={int(bad.sum())} max_logprob_err={d.max(initial=0.0):.2e}")
    # the budget of the comparison rules: excused mismatches below 1e-4 of the draws
    assert excused == 0 or excused < compare.MISMATCH_BUDGET * int(ok.sum()), \
        f"{name}: {excused} excused draws in {int(ok.sum())}"
    return tok, lp


def test_draft_sampler_parity():
    """Reduced sizes: ragged V (not a multiple of the 2048-logit chunk, nor
    of the 16-byte vector), unaligned rows, both dtypes, two temperatures,
    and bad rows."""
    g = torch.Generator(device="cuda").manual_seed(5)
    w = W["chain_b256_v128256"]
    for dt, V, T in (("bf16", 30001, 1.0), ("f32", 4097, 0.7), ("bf16", 2048, 0.8), ("bf16", 5, 1.0)):
        zq = synth.verifier_logits(w.with_sizes(V=V), 24 * 3, g, "cuda").view(24, 3, V)
        rows = zq.to(torch.bfloat16 if dt == "bf16" else torch.float32)
        _draft_case(f"{dt}_V{V}_T{T}", rows, T, seed=31, rnd=4, pos0=2)
    # unaligned rows: a bf16 row stride of V + 1 elements
    V = 3001
    big = synth.verifier_logits(w.with_sizes(V=V + 1), 16 * 2, g, "cuda").view(16, 2, V + 1).to(torch.bfloat16)
    _draft_case("bf16_unaligned", big[:, :, 1:], 1.0, seed=2, rnd=9)
    # bad rows
    rows = synth.verifier_logits(w.with_sizes(V=4096), 6, g, "cuda").view(3, 2, 4096).to(torch.bfloat16)
    rows[0, 1, 17] = float("nan")
    rows[1, 0, 4000] = float("inf")
    rows[2, 1, :] = float("-inf")
    tok, _ = _draft_case("bad_rows", rows, 1.0, seed=3, rnd=3)
    assert tok[0, 1] == -1 and tok[1, 0] == -1 and tok[2, 1] == -1 and (tok[[0, 1, 2], [0, 1, 0]] >= 0).all()
    # a NaN inside a stretch of -inf that one wave reads alone (its chunk
    # has nothing above -inf), the row finite elsewhere
    rows = synth.verifier_logits(w.with_sizes(V=4096), 4, g, "cuda").view(2, 2, 4096).to(torch.bfloat16)
    rows[1, 0, 1024:] = float("-inf")
    rows[1, 0, 2500] = float("nan")
    tok, _ = _draft_case("nan_in_neg_inf", rows, 1.0, seed=4, rnd=1)
    assert tok[1, 0] == -1 and (tok[0] >= 0).all() and tok[1, 1] >= 0
    log("[done] draft parity")


def test_draft_sampler_mismatch_rate_chain_b256():
    """The draft rows of B=256 chains (B=256, 7 positions, V=128256 bf16) over 60
    rounds: 107,520 draws, every one against the oracle.  No draw may fall
    outside its token's CDF interval widened by the 1e-6 W band, and the
    excused draws (inside the band, other token) stay below 1e-4 of all."""
    w = W["chain_b256_v128256"]
    inp = synth.chain_inputs(w, seed=31, device="cuda")
    rows = inp["zp"]
    host = synth.to_oracle(rows.contiguous())
    import rejection_sampling_verify_14_amd as sv
    draws = excused = 0
    worst = 0.0
    for rnd in range(60):
        if rnd % 10 == 0:
            log(f"[case] draft_rate round={rnd}")
        tok, lp = sv.sample_draft(rows, 4242, rnd, w.T)
        torch.cuda.synchronize()
        tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
        o = oracle.sample_draft(host, 4242, rnd, w.T, query=tok)
        ok = o["tokens"] >= 0
        assert np.array_equal(tok[~ok], o["tokens"][~ok])
        band = 1e-6 * o["W"][ok]
        inside = (o["qedge_lo"][ok] - band <= o["target"][ok]) & (o["target"][ok] < o["qedge_hi"][ok] + band)
        assert inside.all(), f"round {rnd}: {int((~inside).sum())} draws outside their CDF interval"
        draws += int(ok.sum())
        same = tok[ok] == o["tokens"][ok]
        excused += int((~same).sum())
        worst = max(worst, float(np.abs(lp[ok][same] - o["logprob"][ok][same]).max(initial=0.0)))
    log(f"[rates] draft_chain_b256: draws={draws} excused={excused} rate={excused / draws:.3e} "
        f"max_logprob_err={worst:.2e}")
    assert worst < 1e-6
    assert excused < compare.MISMATCH_BUDGET * draws, f"{excused} excused draws in {draws}"


def test_draft_sampler_full_size_sampled():
    """The draft rows of B=256 chains at full size (B=256, 7 positions, V=128256
    bf16): every draw in range, and the oracle checks 48 sequences."""
    w = W["chain_b256_v128256"]
    inp = synth.chain_inputs(w, seed=12, device="cuda")
    rows = inp["zp"]
    sel = np.arange(0, w.B, w.B // 48)[:48]
    tok, lp = _draft_case("chain_b256_full", rows, w.T, seed=77, rnd=1, b_sel=sel)
    log("[done] draft full size")


def test_draft_sampler_law():
    """One row repeated over 8192 sequences (sequence stride 0), 4 rounds:
    the device's draws fit softmax(z/T) (chi-square, p > 1e-4)."""
    import rejection_sampling_verify_14_amd as sv
    from scipy.stats import chisquare
    V, n = 6, 8192
    z = torch.tensor([[0.3, -1.0, 2.0, 0.0, 1.2, -0.4]], device="cuda").to(torch.bfloat16)
    rows = z.view(1, 1, V).expand(n, 1, V)
    counts = np.zeros(V)
    for rnd in range(4):
        tok, _ = sv.sample_draft(rows, 123, rnd, 0.9, logprob=False)
        counts += np.bincount(tok.cpu().numpy().ravel(), minlength=V)
    p = torch.softmax(z.double().cpu().view(-1) / float(np.float32(0.9)), dim=0).numpy()
    stat, pv = chisquare(counts, counts.sum() * p)
    log(f"[law] draft sampler chi2={stat:.2f} p={pv:.3g}")
    assert pv > 1e-4


def test_tree_edge_cases():
    """Root-only tree (bonus from q_root), a bad parent, a walk deeper than
    max_depth, NaN in an internal row -- per-sequence -1 flags."""
    import rejection_sampling_verify_14_amd as sv
    log("[case] tree_edges")
    w = W["tree_static_b32_v128256"].with_sizes(V=3000)
    inp = synth.static_tree_inputs(w, 3, "cuda", B=6)
    zq, zp, tok = inp["zq"], inp["zp"], inp["tokens"]
    par = inp["parents"].expand(6, -1).contiguous().clone()
    par[1, 7] = 9           # parent not below the node
    zq[2, 3, 11] = float("nan")
    tok[3, 5] = w.V
    rep, g = run_tree(zq, zp, tok, par, 3, 1, w.T, w.depth)
    assert g["num_accepted"][1] == -1 and g["num_accepted"][2] == -1 and g["num_accepted"][3] == -1
    _done("tree_edges", rep)
    # a single-node tree: bonus straight from the root
    one = sv.spec_verify_tree(zq[:, :1].contiguous(), zp[:, :1].contiguous(), tok[:, :1].contiguous(),
                              torch.tensor([-1], dtype=torch.int32, device="cuda"), seed=1, round=1,
                              temperature=1.0, max_depth=0)
    torch.cuda.synchronize()
    assert (one["num_accepted"] == 0).all()
    o = oracle.verify_tree(synth.to_oracle(zq[:, :1].contiguous()), synth.to_oracle(zp[:, :1].contiguous()),
                           tok[:, :1].cpu().numpy(), np.array([-1], np.int32), 1, 1, 1.0, max_depth=0)
    assert np.array_equal(one["tokens"].cpu().numpy(), o["tokens"])
    # walk deeper than max_depth on an all-accepting path tree
    B, D = 3, 5
    zq2 = zq[:B, :D + 1].contiguous()
    zp2 = zq2.clone()
    tok2 = torch.zeros((B, D + 1), dtype=torch.int32, device="cuda")
    par2 = torch.arange(-1, D, dtype=torch.int32, device="cuda")
    deep = sv.spec_verify_tree(zq2, zp2, tok2, par2, seed=0, round=0, temperature=1.0, max_depth=D - 1)
    torch.cuda.synchronize()
    assert (deep["num_accepted"] == -1).all()


def test_tree_deep_residual():
    """Path-shaped trees of 100 nodes with near-identical draft and verifier
    logits, tokens the draft row's argmax: walks go deep, and some end with a
    residual at a node of index >= 64 (whose row statistics the walk loads
    again rather than reading them from the node tests' LDS copy)."""
    log("[case] tree_deep_residual")
    w = W["tree_static_b32_v128256"].with_sizes(V=3000, sigma_noise=0.05)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    nn, B = 100, 96
    zq = synth.verifier_logits(w, B * nn, g, "cuda").view(B, nn, w.V)
    zp = synth.draft_from_verifier(w, zq, g)
    zq, zp = zq.to(w.torch_dtype), zp.to(w.torch_dtype)
    par = torch.arange(-1, nn - 1, dtype=torch.int32, device="cuda")
    tok = torch.zeros((B, nn), dtype=torch.int32, device="cuda")
    tok[:, 1:] = torch.argmax(zp[:, :-1].float(), dim=-1).to(torch.int32)
    rep, out = run_tree(zq, zp, tok, par, 5, 2, w.T, nn - 1)
    k = out["num_accepted"]
    log(f"   residuals past node 63: {int(((k >= 64) & (k < nn - 1)).sum())}, bonus at the leaf: {int((k == nn - 1).sum())}")
    assert ((k >= 64) & (k < nn - 1)).any()
    _done("tree_deep_residual", rep)


@pytest.mark.parametrize("wl", ["tree_static_b32_v128256", "tree_dynamic_b128_v152064"])
def test_tree_full_size(wl):
    """The static 26-node tree (B=32) and the dynamic 61-node trees (B=128,
    T=0.7) at full size; the oracle checks a window of sequences."""
    w = W[wl]
    log(f"[case] {wl}_full")
    if wl == "tree_static_b32_v128256":
        inp = synth.static_tree_inputs(w, 900, "cuda")
        rng = (0, w.B)
    else:
        inp = synth.dynamic_tree_inputs(w, 901, "cuda")
        rng = (40, 56)
    rep, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 900, 3, w.T, w.depth, b_range=rng)
    log(f"   mean accepted depth {g['num_accepted'].mean():.3f}")
    _done(f"{wl}_full", rep)
    rep, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 900, 3, w.T, w.depth, b_range=rng,
                      walk=1)
    log(f"   best-child walk: mean accepted depth {g['num_accepted'].mean():.3f}")
    _done(f"{wl}_full_best_child", rep)


def test_tree_dynamic_full_all_sequences():
    """Dynamic trees at full size (B=128 dynamic 61-node trees, V=152064 bf16, T=0.7):
    every sequence against the oracle, both walks, two rounds."""
    w = W["tree_dynamic_b128_v152064"]
    rep = compare.Report()
    inp = synth.dynamic_tree_inputs(w, 905, "cuda")
    for rnd in range(2):
        for walk in (0, 1):
            log(f"[case] tree_dynamic_all round={rnd} walk={walk}")
            r, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 905, rnd, w.T, w.depth, walk=walk)
            rep.merge(r)
    log(f"[rates] tree_dynamic_all: {rep.summary()} band_rate={rep.band_decisions / max(rep.decisions, 1):.3e} "
        f"excused_rate={rep.token_mismatch_excused / max(rep.samples, 1):.3e}")
    _done("tree_dynamic_all", rep)


# --------------------------------------------------------------------------- #
# KV compaction
# --------------------------------------------------------------------------- #
def test_kv_compaction_full_tree_dynamic():
    """The dynamic-tree workload's KV buffer [B=128, 4096+60, 8, 128] bf16 (two planes): the
    in-place gather equals torch.index_select on a copy, the indices and
    lengths equal the oracle's, and rows outside the kept path are
    untouched."""
    import rejection_sampling_verify_14_amd as sv
    log("[case] kv_c5_full")
    w = W["tree_dynamic_b128_v152064"]
    B, L = w.B, 4096 + w.budget
    rng = np.random.default_rng(0)
    # a valid random path per sequence (strictly increasing from node 0)
    k = rng.integers(0, w.depth + 1, size=B).astype(np.int32)
    k[5] = -1
    path = np.full((B, w.depth + 1), -1, np.int32)
    for b in range(B):
        if k[b] >= 0:
            path[b, :k[b] + 1] = [0] + sorted(rng.choice(np.arange(1, w.budget + 1), size=k[b], replace=False))
    L0 = np.full(B, w.L0, np.int32)
    kv = torch.stack([synth.kv_buffer(B, L, w.kv_heads, w.kv_dim, seed=s, device="cuda") for s in (1, 2)])
    orig = kv.clone()
    out = sv.kv_compact_indices(torch.tensor(path, device="cuda"), torch.tensor(k, device="cuda"),
                                torch.tensor(L0, device="cuda"), w.depth, kv=kv, stacked_planes=True)
    torch.cuda.synchronize()
    src_o, len_o = oracle.kv_compact(path, k, L0, w.depth)
    assert np.array_equal(out["src_rows"].cpu().numpy(), src_o)
    assert np.array_equal(out["kv_len"].cpu().numpy(), len_o)
    expect = orig.clone()
    for b in range(B):
        if k[b] > 0:
            rows = torch.tensor(src_o[b, :k[b] + 1], device="cuda", dtype=torch.long)
            expect[:, b, w.L0:w.L0 + k[b] + 1] = torch.index_select(orig[:, b], 1, rows)
    assert torch.equal(kv, expect)


def test_kv_chain_indices_and_invalid_paths():
    import rejection_sampling_verify_14_amd as sv
    log("[case] kv_chain_invalid")
    k = torch.tensor([3, 0, -1, 2, 2], dtype=torch.int32, device="cuda")
    L0 = torch.tensor([10, 20, 30, 40, 50], dtype=torch.int32, device="cuda")
    out = sv.kv_compact_indices(None, k, L0, 4)
    torch.cuda.synchronize()
    src_o, len_o = oracle.kv_compact(None, k.cpu().numpy(), L0.cpu().numpy(), 4)
    assert np.array_equal(out["src_rows"].cpu().numpy(), src_o)
    assert np.array_equal(out["kv_len"].cpu().numpy(), len_o)
    # a path that is not strictly increasing, and one past kv_rows
    path = torch.tensor([[0, 2, 1, -1, -1], [0, 3, 60, -1, -1]], dtype=torch.int32, device="cuda")
    kv = torch.zeros((2, 64, 16), dtype=torch.bfloat16, device="cuda")
    before = kv.clone()
    out = sv.kv_compact_indices(path, torch.tensor([2, 2], dtype=torch.int32, device="cuda"),
                                torch.tensor([0, 10], dtype=torch.int32, device="cuda"), 4, kv=kv)
    torch.cuda.synchronize()
    assert out["kv_len"].tolist() == [-1, -1]
    assert torch.equal(kv, before)


def test_tree_attention_mask_parity():
    """Ancestor masks and position ids of flattened trees, bit-exact against the
    oracle: the static 26-node tree (shared parents), the dynamic 61-node trees,
    random trees of 1..1024 nodes (one to sixteen 64-bit words per row), a
    1024-node chain (the deepest walk) and sequences with broken parents."""
    import rejection_sampling_verify_14_amd as sv
    rng = np.random.default_rng(5)

    def random_trees(nn, B):
        return np.stack([np.concatenate([[-1], rng.integers(0, np.arange(1, nn))]).astype(np.int32)
                         if nn > 1 else np.array([-1], np.int32) for _ in range(B)])

    w5 = synth.WORKLOADS["tree_dynamic_b128_v152064"].with_sizes(V=512)
    cases = [("tree_static_static", np.array(synth.STATIC_TREE_PARENTS, np.int32), 32),
             ("tree_dynamic_dynamic", synth.dynamic_tree_inputs(w5, seed=4, B=16)["parents"].numpy(), None)]
    for nn in (1, 2, 63, 64, 65, 200, 1024):
        cases.append((f"random_{nn}", random_trees(nn, 5), None))
    cases.append(("chain_1024", np.array([[-1] + list(range(1023))], np.int32), None))
    broken = random_trees(40, 6)
    broken[1, 0] = 0
    broken[3, 17] = 17
    broken[4, 30] = -3
    cases.append(("broken", broken, None))
    for name, P, B in cases:
        Bn = B if P.ndim == 1 else P.shape[0]
        L0 = rng.integers(0, 5000, Bn).astype(np.int32)
        for with_len in (True, False):
            log(f"[case] tree_mask {name} kv_len={with_len}")
            kv_len = torch.tensor(L0, device="cuda") if with_len else None
            out = sv.tree_attention_mask(torch.tensor(P, device="cuda"), kv_len_in=kv_len, B=B)
            torch.cuda.synchronize()
            m_o, p_o = oracle.tree_mask(P, L0 if with_len else None, B=B)
            assert np.array_equal(out["mask"].cpu().numpy().view(np.uint64), m_o), name
            assert np.array_equal(out["positions"].cpu().numpy(), p_o), name
    log("[done] tree_mask parity")


def _tree_build_case(name, rows, depth, topk, budget, T):
    import rejection_sampling_verify_14_amd as sv
    log(f"[case] tree_build {name} rows={tuple(rows.shape)} depth={depth} topk={topk} budget={budget} T={T}")
    out = sv.tree_build(rows, depth=depth, topk=topk, budget=budget, temperature=T)
    torch.cuda.synchronize()
    o = oracle.tree_build(synth.to_oracle(rows), depth, topk, budget, T)
    for key in ("parents", "tokens", "depth", "frontier"):
        g = out[key].cpu().numpy()
        bad = np.where((g != o[key]).reshape(g.shape[0], -1).any(axis=1))[0]
        assert bad.size == 0, f"{name}: {key} differs in sequences {bad[:8].tolist()}"
    ok = o["parents"][:, 0] == -1
    d = np.abs(out["score"].cpu().numpy() - o["score"])[ok]
    assert d.max(initial=0.0) < 1e-6, f"{name}: score error {d.max()}"
    return out


def test_tree_build_parity():
    """EAGLE-2 dynamic trees grown on the device level by level (tree_expand,
    tree_select, tree_finalize) against the oracle's construction: exact
    trees and frontiers, scores within 1e-6 (the device's row log-sum-exp is
    accurate to ~1e-8).  The dynamic-tree recipe at a reduced V in bf16 and fp32,
    other top-k / depth settings, and a sequence with a NaN row."""
    w = synth.WORKLOADS["tree_dynamic_b128_v152064"]
    for dt, T in (("bf16", 0.7), ("f32", 1.0)):
        wr = w.with_sizes(V=4096, dtype=dt, T=T)
        rows = synth.dynamic_tree_inputs(wr, seed=21, B=24, device="cuda")["expanded_p"]
        _tree_build_case(f"tree_dynamic_reduced_{dt}", rows, w.depth, w.topk, w.budget, T)
    g = torch.Generator(device="cuda").manual_seed(3)
    for depth, topk, budget, V in ((3, 16, 100, 1000), (4, 1, 4, 777), (2, 5, 30, 64)):
        rows = (torch.randn((8, 1 + topk * (depth - 1), V), generator=g, device="cuda") * 3).to(torch.bfloat16)
        _tree_build_case(f"d{depth}_k{topk}", rows, depth, topk, budget, 1.0)
    rows = (torch.randn((4, 1 + 3 * 2, 500), generator=g, device="cuda") * 3).to(torch.bfloat16)
    rows[2, 4, 100] = float("nan")
    rows[0, 0, 7] = float("inf")
    out = _tree_build_case("nan_row", rows, 3, 3, 10, 1.0)
    assert (out["parents"][2] == -1).all().item() and (out["parents"][0] == -1).all().item()
    # a NaN inside a stretch of -inf that one wave reads alone (its running
    # maximum never leaves -inf), the rest of the row finite elsewhere; row
    # lengths that end in the one-vector loop and in whole batches
    for V in (4096, 16384):
        rows = (torch.randn((3, 1 + 2 * 1, V), generator=g, device="cuda") * 3).to(torch.bfloat16)
        rows[1, 1, :] = float("-inf")
        rows[1, 1, :8] = 1.0
        rows[1, 1, 200 * 8 + 3] = float("nan")  # vector 200: lane 200 of the block, its fourth wave
        out = _tree_build_case(f"nan_in_neg_inf_V{V}", rows, 2, 2, 4, 1.0)
        assert (out["parents"][1] == -1).all().item() and (out["parents"][0, 1:] >= 0).all().item()
    log("[done] tree_build parity")


def test_tree_build_full_size_sampled():
    """The dynamic-tree workload's full vocabulary (V = 152064, bf16, T = 0.7) for 16 sequences."""
    w = synth.WORKLOADS["tree_dynamic_b128_v152064"]
    rows = synth.dynamic_tree_inputs(w, seed=22, B=16, device="cuda")["expanded_p"]
    _tree_build_case("tree_dynamic_full", rows, w.depth, w.topk, w.budget, w.T)
    log("[done] tree_build full size")


def test_wait_timeouts_report_minus_two(monkeypatch):
    """The timeout path, forced from the host: with SV_TEST_SPIN_LIMIT=0 every
    wait for another block's record polls once.  A chain sequence whose
    records were not there at that poll reports num_accepted = -2 (a timeout,
    not a data error: never -1 on clean data) with its token row all -1; every
    other sequence is unchanged.  Tree verify (one launch as well) obeys the
    same rule.  The next calls, with the normal bound, are exact again on the
    same workspace."""
    import rejection_sampling_verify_14_amd as sv
    log("[case] wait_timeouts")
    B, N = 64, 7
    for name, ov in [("bf16", dict(V=20008)), ("f32", dict(V=9001, dtype="f32"))]:
        w = W["chain_b256_v128256"].with_sizes(**ov)
        inp = synth.chain_inputs(w, 31, "cuda", B=B, N=N)
        ws = sv.alloc_workspace(sv.chain_workspace_bytes(B, N, w.V), "cuda")

        def call():
            out = sv.spec_verify_chain(inp["zq"], inp["zp"], inp["d"], seed=3, round=5, temperature=1.0,
                                       workspace=ws)
            torch.cuda.synchronize()
            return {k: v.cpu() for k, v in out.items()}

        ref = call()
        assert bool((ref["num_accepted"] >= 0).all())
        monkeypatch.setenv("SV_TEST_SPIN_LIMIT", "0")
        got = call()
        monkeypatch.delenv("SV_TEST_SPIN_LIMIT")
        k = got["num_accepted"]
        assert set(k.tolist()) <= {-2} | set(range(N + 1)), name
        assert bool((k == -2).any()), f"{name}: the one-poll bound never ran out"
        ok = k >= 0
        assert torch.equal(k[ok], ref["num_accepted"][ok])
        assert torch.equal(got["tokens"][ok], ref["tokens"][ok])
        assert bool((got["tokens"][~ok] == -1).all())
        again = call()
        for key in ("num_accepted", "tokens", "accept", "probs", "residual_mass"):
            assert torch.equal(again[key], ref[key]), (name, key)
        log(f"[case] wait_timeouts {name}: {int((k == -2).sum())} of {B} timed out")
    tw = W["tree_static_b32_v128256"].with_sizes(V=9001)
    tin = synth.static_tree_inputs(tw, 7, "cuda", B=8)

    def tcall():
        out = sv.spec_verify_tree(tin["zq"], tin["zp"], tin["tokens"], tin["parents"], seed=7, round=2,
                                  temperature=1.0, max_depth=tw.depth)
        torch.cuda.synchronize()
        return {k: v.cpu() for k, v in out.items()}

    tref = tcall()
    assert bool((tref["num_accepted"] >= 0).all())
    monkeypatch.setenv("SV_TEST_SPIN_LIMIT", "0")
    tgot = tcall()
    monkeypatch.delenv("SV_TEST_SPIN_LIMIT")
    tk = tgot["num_accepted"]
    assert set(tk.tolist()) <= {-2} | set(range(tw.depth + 1))
    tok_ = tk >= 0
    for key in ("num_accepted", "tokens", "path_nodes"):
        assert torch.equal(tgot[key][tok_], tref[key][tok_]), key
    assert bool((tgot["tokens"][~tok_] == -1).all())
    tagain = tcall()
    for key in ("num_accepted", "tokens", "path_nodes", "accept", "probs", "residual_mass"):
        assert torch.equal(tagain[key], tref[key]), key
    log(f"[case] wait_timeouts trees: {int((tk == -2).sum())} of {tk.numel()} timed out")
    log("[done] wait_timeouts")


def test_workspace_reused_across_calls_and_shapes():
    """One workspace serves a run of chain and tree calls of different sizes
    (records and counters carry each call's number): every call matches the
    oracle, including calls whose records sit where a larger earlier call
    left its own."""
    import rejection_sampling_verify_14_amd as sv
    log("[case] workspace_reuse")
    wc, wt = W["chain_b256_v128256"].with_sizes(V=9001), W["tree_static_b32_v128256"].with_sizes(V=6007)
    nbytes = max(sv.chain_workspace_bytes(24, 7, 9001), sv.tree_workspace_bytes(12, 25, 9001))
    ws = sv.alloc_workspace(nbytes, "cuda")
    rep = compare.Report()
    for i, (kind, B) in enumerate([("chain", 24), ("tree", 12), ("chain", 5), ("chain", 24), ("tree", 3),
                                   ("chain", 17)]):
        log(f"   call {i}: {kind} B={B}")
        if kind == "chain":
            r, g, _ = run_chain(wc, seed=70 + i, rnd=i, B=B, workspace=ws)
        else:
            inp = synth.static_tree_inputs(wt, 80 + i, "cuda", B=B)
            r, g = run_tree(inp["zq"], inp["zp"], inp["tokens"], inp["parents"], 80 + i, i, wt.T, wt.depth,
                            workspace=ws)
        rep.merge(r)
    _done("workspace_reuse", rep)
