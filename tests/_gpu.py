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


def run_chain(w, seed: int, rnd: int, *, B=None, N=None, T=None, b_range=None, modify=None, inputs=None):
    """Device chain verify vs oracle.  Returns (report, device outputs, inputs)."""
    import rejection_sampling_verify_14_amd as sv
    T = w.T if T is None else T
    inp = inputs if inputs is not None else synth.chain_inputs(w, seed, "cuda", B=B, N=N)
    if modify is not None:
        modify(inp)
    out = sv.spec_verify_chain(inp["zq"], inp["zp"], inp["d"], seed=seed, round=rnd, temperature=T)
    torch.cuda.synchronize()
    g = _np(out)
    zq, zp = synth.to_oracle(inp["zq"]), synth.to_oracle(inp["zp"])
    o = oracle.verify_chain(zq, zp, inp["d"].cpu().numpy(), seed, rnd, T, b_range=b_range,
                            nthreads=ORACLE_THREADS, query=compare.sampled_tokens(g))
    rep = compare.compare_chain(g, o, b_range)
    return rep, g, inp


def run_tree(zq, zp, tokens, parents, seed: int, rnd: int, T: float, max_depth: int, *, b_range=None, walk=0):
    import rejection_sampling_verify_14_amd as sv
    out = sv.spec_verify_tree(zq, zp, tokens, parents, seed=seed, round=rnd, temperature=T, max_depth=max_depth,
                              walk=walk)
    torch.cuda.synchronize()
    g = _np(out)
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
