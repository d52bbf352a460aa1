"""Benchmark of the speculative-decoding verify step on one MI355X.

A step is one verify round over one batch of synthetic inputs: for the chain
workload (default, B=256 sequences, N=7 drafts, V=128256, bf16 logits, T=1)
one spec_verify_chain call, which also writes the KV rows kept; tree
workloads call spec_verify_tree (the dynamic-tree workload adds the in-place KV gather of
kv_compact_indices).  Inputs are resident in HBM before the timed region;
the step cycles through a pool of distinct logit sets (8 x 0.99 GB for the
chain workload, far beyond the 256 MB Infinity Cache) and uses a fresh
Philox round per step.

Timing: W untimed warm-up steps, then 5 blocks of exactly K steps, each
bracketed by a device synchronize and HIP events on the stream the library
launches on; the median block gives ms_per_step and every block's time is
in the line.  One more block of K steps takes the verify kernel's own
start/stop events (stamped by its launch) for the roofline line.

Output: one JSON line (see the keys below); also the oracle timed on this
host's cores on a bounded sample (cpu_baseline).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload chain_b256_v128256]
  python bench.py --copy-calibration     # plain copy of known size, for PMC scaling
  python bench.py --tree-mask | --tree-build   # the tree kernels on the dynamic trees (B=128, 61 nodes)
  python bench.py --walk-compare          # exercise 3: [2,2,2] tree vs 14-draft chain
  python bench.py --draft-sample          # sv_sample_draft on the draft rows of B=256 chains (V=128256 bf16)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak, 8 TB/s
REPEATS = 5             # timed blocks of K steps; the median is reported
RAMP_S = 0.5            # untimed seconds of steps after the warm-up steps
PRE_STEPS = 10          # untimed steps queued before each timed block's begin event
PROFILE_PMC = os.path.join(ROOT, "profiles", "{kernel}_{workload}_pmc.json")
KERNEL_SOURCES = [os.path.join(ROOT, "rejection_sampling_verify_14_amd", "csrc", f)
                  for f in ("specverify.hip", "sv_device.h", "sv_exp_table.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the timing needs (events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """The source with comments removed and white space collapsed: what the
    compiler sees, so that a change of comments alone keeps the hash."""
    out = _CODE_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(out.split())


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def one_launch(w) -> bool:
    """Whether the library runs this workload's step as the single chain
    launch (k_chain_tab): chains of fp32 logits, and of bf16 logits in
    16-byte aligned rows at a temperature whose bf16-grid table fits (every
    benchmark chain)."""
    return w.kind == "chain"


def dominant_kernel(w) -> str:
    return "k_chain_tab" if one_launch(w) else "k_rows"


def load_traffic(w):
    """HBM bytes per launch of the dominant kernel on this workload from the
    committed rocprofv3 PMC summary, if it was taken on the current kernel
    source (else None: the counters no longer describe the kernel)."""
    try:
        with open(PROFILE_PMC.format(kernel=dominant_kernel(w), workload=w.name)) as f:
            p = json.load(f)
    except (OSError, ValueError):
        return None, None
    if p.get("kernel_hash") != kernel_hash():
        return None, "stale"
    return int(p["hbm_bytes_per_launch"]), p


def _pmc_per_dispatch(csv_path: str, name_part: str, counter: str) -> float:
    """Mean per dispatch of a rocprofv3 counter over the dispatches of the
    kernels whose name contains name_part (values of one dispatch summed)."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} for {name_part} in {csv_path}")
    return sum(per.values()) / len(per)


def pmc_summary(workload: str, fetch_csv: str, write_csv: str, cfetch_csv: str, cwrite_csv: str, commands,
                bench_json: str = None):
    """The dominant kernel's HBM bytes per launch from two rocprofv3 --pmc
    runs of this bench (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each
    scaled by what the same counter reads for a plain 1 GiB device copy
    (--copy-calibration); written to profiles/<kernel>_<workload>_pmc.json
    with the hash of the kernel sources it was taken on.  For the one-launch
    chain step the algorithmic bytes depend on the sampled rows: they are
    taken from the JSON line of the profiled bench run (bench_json)."""
    import synth
    w = synth.WORKLOADS[workload]
    kern = dominant_kernel(w)
    name = "k_chain_tab" if one_launch(w) else "k_rows<"
    fk = _pmc_per_dispatch(fetch_csv, name, "FETCH_SIZE")
    wk = _pmc_per_dispatch(write_csv, name, "WRITE_SIZE")
    copy_k_f = _pmc_per_dispatch(cfetch_csv, "copy", "FETCH_SIZE")
    copy_k_w = _pmc_per_dispatch(cwrite_csv, "copy", "WRITE_SIZE")
    n = 1 << 30
    fs, ws = n / (copy_k_f * 1024.0), n / (copy_k_w * 1024.0)
    hbm = fk * 1024.0 * fs + wk * 1024.0 * ws
    if bench_json:
        with open(bench_json) as f:
            line = [ln for ln in f if ln.startswith("{")][-1]
        alg = json.loads(line)["roofline"]["algorithmic_bytes_per_launch"]
    else:
        sets = build_pool(w, 1, "cpu") if w.kind != "chain" else [None]
        alg = row_kernel_bytes(w, sets[0])
    out = {"kernel": "sv::" + kern, "workload": workload, "kernel_hash": kernel_hash(),
           "fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
           "calibration": {"copy_bytes": n, "copy_fetch_kib": round(copy_k_f, 1), "copy_write_kib": round(copy_k_w, 1),
                           "fetch_scale": fs, "write_scale": ws,
                           "note": "scale = bytes of a plain 1 GiB device copy / (counter KiB x 1024) for that copy"},
           "hbm_bytes_per_launch": int(hbm), "algorithmic_bytes_per_launch": int(alg),
           "traffic_over_algorithmic": hbm / alg, "commands": list(commands)}
    path = PROFILE_PMC.format(kernel=kern, workload=workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def build_pool(w, pool: int, device: str):
    import synth
    sets = []
    for i in range(pool):
        log(f"[bench] generating logit set {i + 1}/{pool} ({w.name})")
        if w.kind == "chain":
            sets.append(synth.chain_inputs(w, seed=9000 + i, device=device))
        elif w.kind == "tree_static":
            sets.append(synth.static_tree_inputs(w, seed=9000 + i, device=device))
        else:
            sets.append(synth.dynamic_tree_inputs(w, seed=9000 + i, device=device))
    return sets


def algorithmic_bytes(w, s) -> int:
    """Bytes of every logit row one step can need, each read once (chain:
    B*(2N+1)*V*s; tree: q at every node plus p at every internal node)."""
    import numpy as np

    import synth
    if w.kind == "chain":
        return synth.algorithmic_bytes_chain(w.B, w.N, w.V, w.elem_bytes)
    par = s["parents"].cpu().numpy()
    p2 = par if par.ndim == 2 else np.repeat(par[None], w.B, 0)
    return synth.algorithmic_bytes_tree(p2, w.V, w.elem_bytes)


def row_kernel_bytes(w, s) -> int:
    """Bytes the row-statistics kernel must read once: every q/p row an
    accept test or the bonus uses (chain: B*(2N+1)*V*s; tree: q and p of
    every internal node)."""
    import numpy as np
    if w.kind == "chain":
        return w.B * (2 * w.N + 1) * w.V * w.elem_bytes
    par = s["parents"].cpu().numpy()
    p2 = par if par.ndim == 2 else np.repeat(par[None], w.B, 0)
    internal = 0
    for row in p2:
        internal += len(set(int(x) for x in row[1:] if x >= 0))
    return internal * 2 * w.V * w.elem_bytes


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Host threads the oracle may use: the job's allotment when the
    environment states one (OMP_NUM_THREADS; a one-GPU job on the GPU machine is
    allotted 16 host threads), else every core this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS")
    try:
        n = int(env) if env else 0
    except ValueError:
        n = 0
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, cores) if n > 0 else cores)


def _oracle_rate(w, s, threads: int, budget_s: float, chunk: int):
    """Sequences per second of the oracle over the first sequences of logit
    set s, in calls of `chunk` sequences, for about budget_s seconds."""
    import oracle
    import synth
    zq, zp = synth.to_oracle(s["zq"]), synth.to_oracle(s["zp"])
    done_seq, t_total, reps = 0, 0.0, 0
    B = w.B
    d = s["d"].cpu().numpy() if w.kind == "chain" else None
    if w.kind != "chain":
        tok, par = s["tokens"].cpu().numpy(), s["parents"].cpu().numpy()
    while t_total < budget_s:
        lo = (reps * chunk) % B
        hi = min(B, lo + chunk)
        t0 = time.perf_counter()
        if w.kind == "chain":
            oracle.verify_chain(zq, zp, d, 1, reps, w.T, b_range=(lo, hi), nthreads=threads)
        else:
            oracle.verify_tree(zq, zp, tok, par, 1, reps, w.T, max_depth=w.depth, b_range=(lo, hi), nthreads=threads)
        t_total += time.perf_counter() - t0
        done_seq += hi - lo
        reps += 1
    return done_seq, t_total


def cpu_baseline(w, sets, budget_s: float):
    """The oracle, as it stands, on this host's cores over a bounded sample of
    the same workload (logit set 0); rounds/s scaled from sequences/s.  Also
    a one-thread figure on a shorter sample."""
    threads = host_threads()
    B = w.B
    n_all, t_all = _oracle_rate(w, sets[0], threads, budget_s, min(B, max(2 * threads, 8)))
    n_one, t_one = _oracle_rate(w, sets[0], 1, min(5.0, budget_s / 3), 1)
    return {"value": (n_all / B) / t_all, "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "one_thread_rounds_per_s": (n_one / B) / t_one,
            "sample": f"{n_all} sequences ({n_all / B:.3g} rounds of B={B}) of logit set 0 in {t_all:.1f} s on "
                      f"{threads} OpenMP threads (the host threads allotted to this job); one thread: {n_one} "
                      f"sequences in {t_one:.1f} s; rounds/s = sequences/s / B"}


def copy_calibration():
    """A plain device copy of known size (for scaling PMC byte counters)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def tree_mask_bench(steps: int, warmup: int):
    """tree_attention_mask on the dynamic trees (B=128, 61 nodes, per-sequence
    parents from the dynamic-tree recipe; the logits only shape the trees, so
    they are drawn at a small V).  One JSON line of its own."""
    import torch

    import rejection_sampling_verify_14_amd as sv
    import synth

    w = synth.WORKLOADS["tree_dynamic_b128_v152064"]
    parents = synth.dynamic_tree_inputs(w.with_sizes(V=1024), seed=7, B=w.B)["parents"].to("cuda")
    B, nn = parents.shape
    L0 = torch.full((B,), w.L0, dtype=torch.int32, device="cuda")
    out = sv.tree_attention_mask(parents, kv_len_in=L0)
    for _ in range(warmup):
        sv.tree_attention_mask(parents, kv_len_in=L0, out=out)
    torch.cuda.synchronize()
    # a call takes less GPU time than its Python launch, so the calls are
    # captured in a graph of `per_graph` launches and the graph is replayed
    per_graph = 50
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            sv.tree_attention_mask(parents, kv_len_in=L0, out=out)
    reps = max(1, steps // per_graph)
    graph.replay()
    hip = Hip()
    stream = torch.cuda.current_stream()
    a, b = hip.event(), hip.event()
    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(a), ctypes.c_void_p(stream.cuda_stream))
    for _ in range(reps):
        graph.replay()
    hip.lib.hipEventRecord(ctypes.c_void_p(b), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    steps = reps * per_graph
    us = hip.elapsed_ms(a, b) * 1000.0 / steps
    W = (nn + 63) // 64
    nbytes = B * nn * 4 + B * 4 + B * nn * (8 * W + 4)   # parents + kv_len read, mask + positions written
    print(json.dumps({
        "metric": "tree attention mask builds/s (B=128 dynamic 61-node trees)", "value": round(1e6 / us, 1), "unit": "calls/s",
        "us_per_call": round(us, 3), "steps": steps, "warmup": warmup, "higher_is_better": True,
        "data": "synthetic", "config": {"workload": f"tree mask B={B} nodes={nn} (dynamic trees)"},
        "roofline": {"bound": "latency", "bytes_per_call": nbytes, "achieved": round(nbytes / us / 1e3, 2),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(nbytes / us / 1e3 / 8000.0, 6)}}), flush=True)


def tree_build_bench(steps: int, warmup: int):
    """The EAGLE-2 dynamic tree grown on the device (tree_expand per level,
    tree_select between levels, tree_finalize) over the dynamic-tree draft rows (B=128, V=152064 bf16):
    B=128, depth 6, top-10, budget 60, V=152064 bf16, T=0.7.  One JSON line
    of its own; the HBM roofline counts every expanded row read once."""
    import torch

    import rejection_sampling_verify_14_amd as sv
    import synth

    w = synth.WORKLOADS["tree_dynamic_b128_v152064"]
    rows = synth.dynamic_tree_inputs(w, seed=7, device="cuda")["expanded_p"]
    B, n_exp, V = rows.shape
    for _ in range(warmup):
        sv.tree_build(rows, depth=w.depth, topk=w.topk, budget=w.budget, temperature=w.T)
    hip = Hip()
    stream = torch.cuda.current_stream()
    a, b = hip.event(), hip.event()
    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(a), ctypes.c_void_p(stream.cuda_stream))
    for _ in range(steps):
        sv.tree_build(rows, depth=w.depth, topk=w.topk, budget=w.budget, temperature=w.T)
    hip.lib.hipEventRecord(ctypes.c_void_p(b), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    us = hip.elapsed_ms(a, b) * 1000.0 / steps
    nbytes = B * n_exp * V * rows.element_size()
    gbps = nbytes / us / 1e3
    print(json.dumps({
        "metric": "dynamic draft trees built/s (B=128, depth 6, top-10, budget 60)", "value": round(1e6 / us * B, 1), "unit": "trees/s",
        "us_per_batch": round(us, 2), "steps": steps, "warmup": warmup, "higher_is_better": True, "data": "synthetic",
        "config": {"workload": f"EAGLE-2 tree build B={B} depth={w.depth} topk={w.topk} budget={w.budget} "
                               f"V={V} bf16 T={w.T}"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbps / 8000.0, 4), "bytes_per_batch": nbytes}}), flush=True)


TREE_222 = [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6]  # [2, 2, 2]: 14 drafts, 8 leaves


def _accept_probs(zq, zp, par, tok, T):
    """a_n = min(1, q_par(t_n) / p_par(t_n)) in fp64, [B, nodes-1]."""
    import torch
    lq = torch.log_softmax(zq.double() / T, dim=-1)
    lp = torch.log_softmax(zp.double() / T, dim=-1)
    pa = torch.tensor(par[1:], device=zq.device, dtype=torch.long)
    t = tok[:, 1:].long()
    ar = torch.arange(zq.shape[0], device=zq.device)[:, None]
    return torch.clamp(torch.exp(lq[ar, pa[None, :], t] - lp[ar, pa[None, :], t]), max=1.0)


def _tree_expectations(a, par):
    """Exact expected accepted depth of both walks and the probability that
    the first-accepted-child walk reaches each node, from the per-node
    accept probabilities a [B, nodes-1] (decisions are independent)."""
    import torch
    nn = len(par)
    kids = [[c for c in range(1, nn) if par[c] == n] for n in range(nn)]
    B = a.shape[0]
    e0 = [None] * nn
    e1 = [None] * nn
    for n in reversed(range(nn)):
        if not kids[n]:
            e0[n] = e1[n] = torch.zeros(B, dtype=torch.float64, device=a.device)
            continue
        none_yet = torch.ones(B, dtype=torch.float64, device=a.device)
        acc = torch.zeros(B, dtype=torch.float64, device=a.device)
        for c in kids[n]:
            acc = acc + none_yet * a[:, c - 1] * (1.0 + e0[c])
            none_yet = none_yet * (1.0 - a[:, c - 1])
        e0[n] = acc
        c = kids[n][0]
        e1[n] = a[:, c - 1] * (1.0 + e1[c])
    reach = [None] * nn
    reach[0] = torch.ones(B, dtype=torch.float64, device=a.device)
    for n in range(nn):
        none_yet = torch.ones(B, dtype=torch.float64, device=a.device)
        for c in kids[n]:
            reach[c] = reach[n] * none_yet * a[:, c - 1]
            none_yet = none_yet * (1.0 - a[:, c - 1])
    return e0[0], e1[0], torch.stack(reach, 1)


def walk_compare(rounds: int = 8, B: int = 256, V: int = 128256, seed: int = 11, sigma_noise=None) -> dict:
    """[PT] / [FA] exercise 3: a [2, 2, 2] draft tree (children = the draft's
    top-2 at each node, 8 candidate paths) against a chain of equal verifier
    compute (14 drafts, d_i ~ p_i), on the B=256 chain logit recipe (sigma_noise,
    the draft's distance from the verifier, may be overridden).  For both
    tree walks and the chain: tokens per verifier call (accepted + 1) from the
    device verify, and its exact expectation from the same logits (fp64); and
    per leaf, the rate at which the first-accepted-child walk reaches it."""
    import numpy as np
    import torch

    import rejection_sampling_verify_14_amd as sv
    import synth

    w = synth.WORKLOADS["chain_b256_v128256"].with_sizes(V=V, B=B)
    if sigma_noise is not None:
        w = w.with_sizes(sigma_noise=float(sigma_noise))
    T = w.T
    par = TREE_222
    nn = len(par)
    N = nn - 1
    parents = torch.tensor(par, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    mc = {"tree_first_accepted": [], "tree_best_child": [], "chain": []}
    ex = {"tree_first_accepted": [], "tree_best_child": [], "chain": []}
    leaf_mc, leaf_ex = [], []
    for r in range(rounds):
        zq = synth.verifier_logits(w, B * nn, g, "cuda").view(B, nn, V)
        zp = synth.draft_from_verifier(w, zq, g)
        zq, zp = zq.to(w.torch_dtype), zp.to(w.torch_dtype)
        tok = torch.zeros((B, nn), dtype=torch.int32, device="cuda")
        for n in range(nn):
            kids = [c for c in range(1, nn) if par[c] == n]
            if kids:
                top = torch.topk(zp[:, n].float(), len(kids), dim=-1).indices.to(torch.int32)
                for j, c in enumerate(kids):
                    tok[:, c] = top[:, j]
        t0 = sv.spec_verify_tree(zq, zp, tok, parents, seed=seed, round=r, temperature=T, max_depth=3, walk=0)
        t1 = sv.spec_verify_tree(zq, zp, tok, parents, seed=seed, round=r, temperature=T, max_depth=3, walk=1)
        a = _accept_probs(zq, zp, par, tok, T)
        e0, e1, reach = _tree_expectations(a, par)
        mc["tree_first_accepted"].append(t0["num_accepted"].double() + 1)
        mc["tree_best_child"].append(t1["num_accepted"].double() + 1)
        ex["tree_first_accepted"].append(e0 + 1)
        ex["tree_best_child"].append(e1 + 1)
        path = t0["path_nodes"].long()
        hit = torch.zeros((B, nn), dtype=torch.float64, device="cuda")
        hit.scatter_(1, path.clamp_min(0), (path >= 0).double())
        leaf_mc.append(hit[:, 7:])
        leaf_ex.append(reach[:, 7:])
        del zq, zp
        # the chain: fresh rows, drafts sampled from the draft
        cq = synth.verifier_logits(w, B * (N + 1), g, "cuda").view(B, N + 1, V)
        cp = synth.draft_from_verifier(w, cq[:, :N], g)
        cq, cp = cq.to(w.torch_dtype), cp.to(w.torch_dtype)
        d = synth.gumbel_max(cp.float(), T, g)
        ch = sv.spec_verify_chain(cq, cp, d, seed=seed, round=r, temperature=T)
        q = torch.softmax(cq[:, :N].double() / T, dim=-1)
        p = torch.softmax(cp.double() / T, dim=-1)
        alpha = torch.minimum(q, p).sum(-1)          # [B, N]: P(accept) of a draft drawn from p
        mc["chain"].append(ch["num_accepted"].double() + 1)
        ex["chain"].append(1.0 + torch.cumprod(alpha, dim=1).sum(1))
        del cq, cp, q, p
    out = {}
    for k in mc:
        m = torch.cat(mc[k]).cpu().numpy()
        e = torch.cat(ex[k]).cpu().numpy()
        out[k] = {"tokens_per_call": round(float(m.mean()), 4), "expected": round(float(e.mean()), 4),
                  "std_err": round(float(m.std(ddof=1) / np.sqrt(m.size)), 4)}
    lm = torch.cat(leaf_mc).mean(0).cpu().numpy()
    le = torch.cat(leaf_ex).mean(0).cpu().numpy()
    out["alpha_per_leaf"] = [round(float(x), 4) for x in lm]
    out["alpha_per_leaf_expected"] = [round(float(x), 4) for x in le]
    out["samples"] = rounds * B
    return out


def walk_compare_bench(rounds: int):
    """One JSON line per draft quality: the B=256 chain recipe (the draft close
    to the verifier, sigma_noise 0.4) and a far draft (sigma_noise 3.0)."""
    for noise in (None, 3.0):
        res = walk_compare(rounds=rounds, sigma_noise=noise)
        print(json.dumps({
            "metric": "tokens per verifier call: [2,2,2] tree vs 14-draft chain (exercise 3)",
            "value": res["tree_first_accepted"]["tokens_per_call"], "unit": "tokens/call", "higher_is_better": True,
            "data": "synthetic",
            "config": {"workload": "chain logit recipe, B=256, V=128256 bf16, T=1.0; tree [2,2,2] (draft top-2 "
                                   "per node); chain N=14 (d ~ p)",
                       "sigma_noise": 0.4 if noise is None else noise},
            **res}), flush=True)


def draft_sample_bench(steps: int, warmup: int):
    """sv_sample_draft on the draft rows of B=256 chains (V=128256 bf16) (B=256, V=128256 bf16, T=1):
    all 7 positions in one call, and one position (the autoregressive
    step).  One JSON line each; the HBM roofline counts every row read once."""
    import torch

    import rejection_sampling_verify_14_amd as sv
    import synth

    w = synth.WORKLOADS["chain_b256_v128256"]
    rows = synth.chain_inputs(w, seed=5, device="cuda")["zp"]
    hip = Hip()
    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    for R in (w.N, 1):
        # one position: the calls cycle through the 7 positions' rows (460 MB
        # together, beyond the 256 MB Infinity Cache), so every call streams
        # its rows from HBM
        xs = [rows[:, :R]] if R == w.N else [rows[:, p:p + 1] for p in range(w.N)]
        for i in range(warmup):
            sv.sample_draft(xs[i % len(xs)], 1, 0, w.T)
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.lib.hipEventRecord(ctypes.c_void_p(a), ctypes.c_void_p(stream.cuda_stream))
        for i in range(steps):
            sv.sample_draft(xs[i % len(xs)], 1, i, w.T)
        hip.lib.hipEventRecord(ctypes.c_void_p(b), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        us = hip.elapsed_ms(a, b) * 1000.0 / steps
        nbytes = w.B * R * w.V * rows.element_size()
        gbps = nbytes / us / 1e3
        print(json.dumps({
            "metric": "draft tokens sampled/s", "value": round(w.B * R / us * 1e6, 1), "unit": "tokens/s",
            "us_per_call": round(us, 2), "steps": steps, "warmup": warmup, "higher_is_better": True,
            "data": "synthetic",
            "config": {"workload": f"draft sampling B={w.B} positions={R} V={w.V} bf16 T={w.T}"},
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(gbps / 8000.0, 4), "bytes_per_call": nbytes}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="chain_b256_v128256", choices=["chain_b64_v32000", "chain_b256_v128256", "tree_static_b32_v128256", "tree_dynamic_b128_v152064"])
    ap.add_argument("--pool", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the row kernel's PMC summary for --workload from rocprofv3 counter CSVs")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help="the commands that made the CSVs (recorded)")
    ap.add_argument("--pmc-bench-json", default=None,
                    help="the JSON line of the profiled run (algorithmic bytes of the one-launch chain step)")
    ap.add_argument("--tree-mask", action="store_true", help="time tree_attention_mask on the dynamic trees (B=128, 61 nodes) instead")
    ap.add_argument("--tree-build", action="store_true", help="time the dynamic tree build on the dynamic-tree rows (B=128, V=152064) instead")
    ap.add_argument("--draft-sample", action="store_true", help="time sv_sample_draft on the draft rows of B=256 chains (V=128256 bf16)")
    ap.add_argument("--walk-compare", action="store_true",
                    help="exercise 3: [2,2,2] tree (both walks) vs a 14-draft chain, tokens per verifier call")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (sequences are independent; "
              "a multi-GPU run would split the batch of sequences across GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rejection_sampling_verify_14_amd as sv
    import synth

    if args.copy_calibration:
        copy_calibration()
        return
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary, args.pmc_commands, args.pmc_bench_json)
        return
    if args.tree_mask:
        tree_mask_bench(args.steps, args.warmup)
        return
    if args.tree_build:
        tree_build_bench(args.steps, args.warmup)
        return
    if args.draft_sample:
        draft_sample_bench(args.steps, args.warmup)
        return
    if args.walk_compare:
        walk_compare_bench(rounds=8)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    pool = args.pool or w.pool
    sets = build_pool(w, pool, "cuda")
    hip = Hip()
    dev = "cuda"
    B = w.B
    if w.kind == "chain":
        outs = sv.alloc_chain_outputs(B, w.N, dev, kv=True)
        ws = sv.alloc_workspace(sv.chain_workspace_bytes(B, w.N, w.V), dev)
        width = w.N + 1
    else:
        T = sets[0]["zq"].shape[1] - 1
        outs = sv.alloc_tree_outputs(B, T, w.depth, dev, kv=True)
        ws = sv.alloc_workspace(sv.tree_workspace_bytes(B, T, w.V), dev)
        width = w.depth + 1
    kv_out = {"src_rows": torch.empty((B, width), dtype=torch.int32, device=dev),
              "kv_len": torch.empty(B, dtype=torch.int32, device=dev)}
    kv_len_in = torch.full((B,), max(w.L0, 0), dtype=torch.int32, device=dev)
    kv = None
    if w.kind == "tree_dynamic":
        kv = synth.kv_buffer(B, 4096 + w.budget, w.kv_heads, w.kv_dim, seed=5, device=dev)

    def step(i, timing=None):
        s = sets[i % pool]
        if w.kind == "chain":
            sv.spec_verify_chain(s["zq"], s["zp"], s["d"], seed=2026, round=i, temperature=w.T,
                                 kv_len_in=kv_len_in, out=outs, workspace=ws, timing=timing)
        else:
            sv.spec_verify_tree(s["zq"], s["zp"], s["tokens"], s["parents"], seed=2026, round=i, temperature=w.T,
                                max_depth=w.depth, kv_len_in=kv_len_in, out=outs, workspace=ws, timing=timing)
            if kv is not None:
                sv.kv_compact_indices(outs["path_nodes"], outs["num_accepted"], kv_len_in, w.depth, kv=kv,
                                      out=kv_out)

    log(f"[bench] warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # then untimed steps until the GPU has run this work for RAMP_S seconds
    # (a short warm-up leaves the clocks below their sustained level, and the
    # first timed blocks would measure the ramp)
    ramp_steps, t_ramp = 0, time.perf_counter()
    while time.perf_counter() - t_ramp < RAMP_S:
        for i in range(50):
            step(args.warmup + ramp_steps + i)
        torch.cuda.synchronize()
        ramp_steps += 50
    log(f"[bench] {ramp_steps} more untimed steps ({RAMP_S} s of clock ramp)")
    K = args.steps
    stream = torch.cuda.current_stream()
    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    t_begin, t_end = hip.event(), hip.event()
    # REPEATS blocks of exactly K steps, each bracketed by a synchronize and
    # events on the library's stream; the timed steps carry no per-step
    # events.  The reported time is the median block.
    blocks_ms, walls = [], []
    acc_sum = acc_n = tok_sum = tok_n = 0.0
    nxt = args.warmup + ramp_steps
    for rep in range(REPEATS):
        log(f"[bench] timing block {rep + 1}/{REPEATS} of {K} steps")
        torch.cuda.synchronize()
        # a few untimed steps queued ahead of the block's begin event, so the
        # block starts on a busy GPU rather than one just idled by the sync
        for i in range(PRE_STEPS):
            step(nxt + i)
        nxt += PRE_STEPS
        hip.lib.hipEventRecord(ctypes.c_void_p(t_begin), ctypes.c_void_p(stream.cuda_stream))
        wall0 = time.perf_counter()
        for i in range(K):
            step(nxt + i)
        hip.lib.hipEventRecord(ctypes.c_void_p(t_end), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - wall0)
        blocks_ms.append(hip.elapsed_ms(t_begin, t_end))
        nxt += K
        # acceptance of the block's last step (outputs are overwritten every
        # step), copied out as plain host arrays: no device work between
        # the timed blocks
        a8 = outs["accept"].cpu().numpy().astype("float64")
        if w.kind != "chain":
            a8 = a8[:, 1:]
        acc_sum += float(a8.sum())
        acc_n += a8.size
        k = outs["num_accepted"].cpu().numpy()
        tok_sum += float((k[k >= 0] + 1).sum())
        tok_n += int((k >= 0).sum())
    ms_step = statistics.median(blocks_ms) / K
    # the row kernel's own duration (the step's dominant kernel) and the
    # call's: one more block of K steps whose events are stamped by the
    # kernels' own starts and ends (no event between a call's kernels)
    log(f"[bench] timing the kernels of {K} more steps")
    ev = [(hip.event(), hip.event(), hip.event()) for _ in range(K)]
    nacc = torch.empty((K, B), dtype=torch.int32, device=dev)
    nres = torch.empty((K, B), dtype=torch.float64, device=dev)
    for i in range(K):
        step(nxt + i, timing=ev[i])
        nacc[i].copy_(outs["num_accepted"])
        nres[i].copy_(outs["residual_mass"])
    torch.cuda.synchronize()
    rows_ms = [hip.elapsed_ms(a, m) for a, m, _ in ev]
    call_ms = [hip.elapsed_ms(a, b) for a, _, b in ev]
    k_mean = sum(rows_ms) / K
    call_mean = sum(call_ms) / K
    per_set = [algorithmic_bytes(w, s) for s in sets]
    full_bytes = sum(per_set) / len(per_set)
    row_set = [row_kernel_bytes(w, s) for s in sets]
    row_bytes = sum(row_set) / len(row_set)
    if one_launch(w):
        # the one launch reads the 2N draft-position rows of every sequence
        # once, then the row(s) each sequence samples from: both rows of the
        # rejected position, or the bonus row (read only when sampled)
        k = nacc.long()
        nrows = torch.where(k < 0, 0, torch.where(k < w.N, 2, 1)).sum(dim=1).double()
        row_bytes = w.B * 2 * w.N * w.V * w.elem_bytes + float(nrows.mean()) * w.V * w.elem_bytes
    step_bytes = full_bytes
    if w.kind != "chain":
        # a tree step reads q and p of every node with children once, and
        # the q row of the leaf where a walk ends with a bonus (residual mass
        # 0); the q rows of the other leaves are never read
        nbonus = ((nres == 0.0) & (nacc >= 0)).sum(dim=1).double().cpu()
        step_bytes = sum(row_set[(nxt + i) % pool] + float(nbonus[i]) * w.V * w.elem_bytes for i in range(K)) / K
    rounds_per_s = 1000.0 / ms_step
    eff_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    k_gbps = row_bytes / (k_mean * 1e-3) / 1e9
    traffic, pmc = load_traffic(w)
    result = {
        "metric": "verified rounds/s + achieved HBM GB/s (% peak), " + {
            "chain_b256_v128256": "B=256 N=7 V=128256",
            "chain_b64_v32000": "B=64 N=5 V=32000",
            "tree_static_b32_v128256": "static 26-node trees B=32 V=128256",
            "tree_dynamic_b128_v152064": "dynamic 61-node trees B=128 V=152064"}[w.name],
        "value": round(rounds_per_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ramp_steps_untimed": ramp_steps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": {"chain_b256_v128256": "chain verify B=256 N=7 V=128256 bf16 logits T=1.0",
                         "chain_b64_v32000": "chain verify B=64 N=5 V=32000 fp32 logits T=1.0",
                         "tree_static_b32_v128256": "static 26-node tree verify B=32 V=128256 bf16 logits T=1.0",
                         "tree_dynamic_b128_v152064": "dynamic 61-node tree verify B=128 V=152064 bf16 T=0.7 + KV gather"}[w.name],
            "logits": w.dtype, "B": B, "V": w.V, "pool_sets": pool,
            "arithmetic": "row statistics f32 exp2 summed in f64; accept ratio and sampled rows f64",
            "step": "one spec_verify_* launch (KV rows included)" + (" + the in-place KV gather" if kv is not None
                                                                      else ""),
        },
        "effective_GBps": round(eff_gbps, 1),
        "effective_frac_of_peak": round(eff_gbps / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_step": int(full_bytes),
        "effective_bytes": ("algorithmic bytes: every logit row of the round once, B x (2N+1) x V x e" if w.kind == "chain"
                            else "bytes a step reads: q and p of every node with children once, plus the q row of "
                                 "the leaf of each walk that ends with a bonus (the algorithmic figure also counts "
                                 "the q rows of leaves no walk samples from)"),
        "bytes_read_per_step": int(step_bytes),
        "block_ms_per_step": [round(t / K, 5) for t in blocks_ms],
        "alpha_measured": round(acc_sum / max(acc_n, 1), 4),
        "tokens_per_round": round(tok_sum / max(tok_n, 1), 4),
        "roofline": {
            "kernel": ("k_chain_tab (the whole step in one launch: every logit row once, then the row(s) each "
                       "sequence samples from)" if one_launch(w) else
                       "k_rows (row statistics of every logit row the step reads, then the accept tests; the dominant kernel)"),
            "bound": "hbm",
            "achieved": round(k_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(k_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel_ms": round(k_mean, 5),
            "algorithmic_bytes_per_launch": int(row_bytes),
        },
        "call_ms_with_kernel_events": round(call_mean, 5),
        "wall_s_timed": round(sum(walls), 3),
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_budget:.0f} s of oracle work)")
        result["cpu_baseline"] = cpu_baseline(w, sets, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
