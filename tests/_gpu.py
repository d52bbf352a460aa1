"""Harness of the GPU parity tests: run the device path and the oracle on the
same seeded inputs and compare them with oracle.compare's rules."""
import os
import sys

import numpy as np
import torch

import oracle
import synth
from oracle import compare

ORACLE_THREADS = min(16, os.cpu_count() or 1)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _np(d: dict) -> dict:
    return {k: v.detach().cpu().numpy() for k, v in d.items()}


def kv_rows_in(B: int, seed: int) -> torch.Tensor:
    """KV rows of the pending token, L0 [B] int32 (seeded, varied)."""
    rng = np.random.default_rng(seed + 17)
    return torch.tensor(rng.integers(0, 5000, size=B), dtype=torch.int32, device="cuda")


def check_kv_outputs(g: dict, L0: torch.Tensor, max_depth: int, tree: bool) -> None:
    """The verify call's KV outputs equal the oracle's KV indices for the
    call's own path and count (bit-exact): L0 + path[i] up to k, -1 after,
    length L0 + k + 1; a failed sequence keeps L0 and gets -1 rows."""
    path = g["path_nodes"] if tree else None
    src, kvl = oracle.kv_compact(path, g["num_accepted"], L0.cpu().numpy(), max_depth)
    assert np.array_equal(g["src_rows"], src), "KV source rows differ"
    assert np.array_equal(g["kv_len"], kvl), "KV lengths differ"


def run_chain(w, seed: int, rnd: int, *, B=None, N=None, T=None, b_range=None, modify=None, inputs=None,
              workspace=None):
    """Device chain verify vs oracle.  Returns (report, device outputs, inputs)."""
    import rejection_sampling_verify_14_amd as sv
    T = w.T if T is None else T
    inp = inputs if inputs is not None else synth.chain_inputs(w, seed, "cuda", B=B, N=N)
    if modify is not None:
        modify(inp)
    L0 = kv_rows_in(inp["zq"].shape[0], seed)
    out = sv.spec_verify_chain(inp["zq"], inp["zp"], inp["d"], seed=seed, round=rnd, temperature=T, kv_len_in=L0,
                               workspace=workspace)
    torch.cuda.synchronize()
    g = _np(out)
    check_kv_outputs(g, L0, inp["zq"].shape[1] - 1, False)
    zq, zp = synth.to_oracle(inp["zq"]), synth.to_oracle(inp["zp"])
    o = oracle.verify_chain(zq, zp, inp["d"].cpu().numpy(), seed, rnd, T, b_range=b_range,
                            nthreads=ORACLE_THREADS, query=compare.sampled_tokens(g))
    rep = compare.compare_chain(g, o, b_range)
    return rep, g, inp


def run_tree(zq, zp, tokens, parents, seed: int, rnd: int, T: float, max_depth: int, *, b_range=None, walk=0,
             workspace=None):
    import rejection_sampling_verify_14_amd as sv
    L0 = kv_rows_in(zq.shape[0], seed)
    out = sv.spec_verify_tree(zq, zp, tokens, parents, seed=seed, round=rnd, temperature=T, max_depth=max_depth,
                              walk=walk, kv_len_in=L0, workspace=workspace)
    torch.cuda.synchronize()
    g = _np(out)
    check_kv_outputs(g, L0, max_depth, True)
    par = parents.cpu().numpy()
    o = oracle.verify_tree(synth.to_oracle(zq), synth.to_oracle(zp), tokens.cpu().numpy(), par, seed, rnd, T,
                           max_depth=max_depth, b_range=b_range, nthreads=ORACLE_THREADS,
                           query=compare.sampled_tokens(g), walk=walk)
    rep = compare.compare_tree(g, o, par, b_range)
    return rep, g


def accept_rate(g: dict, N: int) -> float:
    k = g["num_accepted"]
    k = k[k >= 0]
    return float(k.mean()) / max(N, 1)
