"""fp64 CPU oracle of the speculative-decoding verify-and-accept step.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``rejection_sampling_verify_14_amd``) never imports this package and never
falls back to it.

The arithmetic lives in ``sv_oracle.c`` (plain C, IEEE double, sequential
loops, its own Philox4x32-10).  This module only marshals numpy arrays.
Logit arrays are numpy ``float32``, ``float64`` or ``uint16`` (raw bf16 bit
patterns).  Every function cites, in ``sv_oracle.c``, the passage of the pages
it follows.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` except Philox beyond its known-answer vectors,
which is additionally checked only for agreement with the device generator.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import analytic  # noqa: F401  (closed forms of the pages' speed-up model)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsv_oracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2
KIND_RESIDUAL, KIND_BONUS, KIND_RESIDUAL_WAS_ZERO, KIND_ERROR = 0, 1, 2, -1

_OUT_FIELDS = [
    "tokens", "num_accepted", "path_nodes", "accept", "q_tok", "p_tok", "ratio", "u_acc", "u_samp",
    "resid_mass", "weight_total", "target", "edge_lo", "edge_hi", "query", "qedge_lo", "qedge_hi",
    "stop_node", "sample_kind", "lse_q", "lse_p",
]


class _Out(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _OUT_FIELDS]


def lib():
    """Load the compiled oracle, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.orc_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.orc_philox4x32_10.restype = None
        L.orc_u53.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.orc_u53.restype = ctypes.c_double
        L.orc_philox_block.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, u32p]
        L.orc_philox_block.restype = None
        dp = ctypes.POINTER(ctypes.c_double)
        L.orc_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, dp, dp]
        L.orc_uniforms.restype = None
        L.orc_uniform_grid.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
        L.orc_uniform_grid.restype = None
        L.orc_row_lse.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp]
        L.orc_row_lse.restype = ctypes.c_int
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_verify_chain.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, i32, i32, i32, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_double, vp, i32, i32, i32, ctypes.POINTER(_Out)]
        L.orc_verify_chain.restype = ctypes.c_int
        L.orc_verify_tree.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                      ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, vp, i32, i32, i32,
                                      ctypes.POINTER(_Out)]
        L.orc_verify_tree.restype = ctypes.c_int
        L.orc_kv_compact.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, i64, i64, i32, i32, i64]
        L.orc_kv_compact.restype = ctypes.c_int
        L.orc_sample_draft.argtypes = [vp, i64, i64, i32, i32, i32, i32, ctypes.c_double, ctypes.c_uint64,
                                       ctypes.c_uint64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        L.orc_sample_draft.restype = ctypes.c_int
        L.orc_tree_build.argtypes = [vp, i64, i64, i32, i32, i32, i32, i32, i32, ctypes.c_double, vp, vp, vp, vp, vp]
        L.orc_tree_build.restype = ctypes.c_int
        L.orc_tree_mask.argtypes = [vp, i32, vp, i32, i32, vp, vp]
        L.orc_tree_mask.restype = ctypes.c_int
        L.orc_accept_prob.argtypes = [vp, vp, i32, i32, ctypes.c_double, i32]
        L.orc_accept_prob.restype = ctypes.c_double
        L.orc_residual_probs.argtypes = [vp, vp, i32, i32, ctypes.c_double, vp]
        L.orc_residual_probs.restype = ctypes.c_int
        L.orc_inverse_cdf.argtypes = [vp, i32, ctypes.c_double]
        L.orc_inverse_cdf.restype = ctypes.c_int
        L.orc_num_threads_available.argtypes = []
        L.orc_num_threads_available.restype = ctypes.c_int
        _lib = L
    return _lib


def _swap_library(path):
    """Point this module at another build of the oracle (used only by the
    mutation test, which plants mistakes in a copy of the source).  Returns
    the previous library handle; pass it back to restore."""
    global _lib
    prev = _lib
    if isinstance(path, ctypes.CDLL) or path is None:
        _lib = path
    else:
        _lib = None
        global _LIB_PATH
        saved, _LIB_PATH = _LIB_PATH, path
        try:
            lib()
        finally:
            _LIB_PATH = saved
    return prev


def _temperature(T) -> float:
    """The temperature as the device library receives it: a 32-bit float
    (the C ABI's `float temperature`), widened exactly to double."""
    return float(np.float32(T))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"logits must be float32, float64 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _strides3(a: np.ndarray):
    if a.ndim != 3 or a.strides[2] != a.itemsize:
        raise ValueError("logits must be [B, rows, V] with a unit last-axis stride")
    return a.strides[0] // a.itemsize, a.strides[1] // a.itemsize


def threads_available() -> int:
    return int(lib().orc_num_threads_available())


# --------------------------------------------------------------------------- #
# Philox and uniforms
# --------------------------------------------------------------------------- #
def philox4x32_10(ctr, key):
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def u53(a: int, b: int) -> float:
    return float(lib().orc_u53(a & 0xFFFFFFFF, b & 0xFFFFFFFF))


def philox_block(seed: int, rnd: int, seq: int, pos: int, stream: int = 0):
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox_block(seed, rnd, seq, pos, stream, o)
    return [int(x) for x in o]


def uniforms(seed: int, rnd: int, seq: int, pos: int):
    """(accept uniform of position pos, sampling uniform of slot pos)."""
    ua, us = ctypes.c_double(), ctypes.c_double()
    lib().orc_uniforms(seed, rnd, seq, pos, ctypes.byref(ua), ctypes.byref(us))
    return ua.value, us.value


def uniform_grid(seed: int, rnd: int, nseq: int, npos: int):
    """(u_acc, u_samp), each [nseq, npos], for positions 1..npos."""
    a = np.empty((nseq, npos), np.float64)
    s = np.empty((nseq, npos), np.float64)
    lib().orc_uniform_grid(seed, rnd, nseq, npos, _ptr(a), _ptr(s))
    return a, s


# --------------------------------------------------------------------------- #
# Primitives
# --------------------------------------------------------------------------- #
def row_lse(row: np.ndarray, T: float = 1.0):
    """(max of z/T, log-sum-exp of z/T) of one row, or None on a data error."""
    row = np.ascontiguousarray(row)
    m, l = ctypes.c_double(), ctypes.c_double()
    err = lib().orc_row_lse(_ptr(row), _dtype_code(row), row.shape[0], float(T), ctypes.byref(m), ctypes.byref(l))
    return None if err else (m.value, l.value)


def accept_prob(qrow, prow, d: int, T: float = 1.0) -> float:
    qrow, prow = np.ascontiguousarray(qrow), np.ascontiguousarray(prow)
    return float(lib().orc_accept_prob(_ptr(qrow), _ptr(prow), _dtype_code(qrow), qrow.shape[0], float(T), int(d)))


def residual_probs(qrow, prow, T: float = 1.0):
    """(normalised residual distribution, kind)."""
    qrow, prow = np.ascontiguousarray(qrow), np.ascontiguousarray(prow)
    out = np.empty(qrow.shape[0], np.float64)
    kind = lib().orc_residual_probs(_ptr(qrow), _ptr(prow), _dtype_code(qrow), qrow.shape[0], float(T), _ptr(out))
    return out, int(kind)


def inverse_cdf(w, u: float) -> int:
    w = np.ascontiguousarray(w, dtype=np.float64)
    return int(lib().orc_inverse_cdf(_ptr(w), w.shape[0], float(u)))


# --------------------------------------------------------------------------- #
# Full chain / tree / KV
# --------------------------------------------------------------------------- #
def _alloc_out(B: int, width: int, nslots: int, rows: int, tree: bool, query):
    o = {
        "tokens": np.full((B, width), -7, np.int32),
        "num_accepted": np.full(B, -7, np.int32),
        "accept": np.full((B, nslots), -7, np.int32),
        "q_tok": np.full((B, nslots), np.nan),
        "p_tok": np.full((B, nslots), np.nan),
        "ratio": np.full((B, nslots), np.nan),
        "u_acc": np.full((B, nslots), np.nan),
        "u_samp": np.full(B, np.nan),
        "resid_mass": np.full(B, np.nan),
        "weight_total": np.full(B, np.nan),
        "target": np.full(B, np.nan),
        "edge_lo": np.full(B, np.nan),
        "edge_hi": np.full(B, np.nan),
        "stop_node": np.full(B, -7, np.int32),
        "sample_kind": np.full(B, -7, np.int32),
        "lse_q": np.full((B, rows), np.nan),
        "lse_p": np.full((B, rows), np.nan),
    }
    if tree:
        o["path_nodes"] = np.full((B, width), -7, np.int32)
    if query is not None:
        o["query"] = np.ascontiguousarray(query, dtype=np.int32)
        o["qedge_lo"] = np.full(B, np.nan)
        o["qedge_hi"] = np.full(B, np.nan)
    s = _Out()
    for f in _OUT_FIELDS:
        setattr(s, f, o[f].ctypes.data if f in o else None)
    return o, s


def verify_chain(zq, zp, d, seed: int, rnd: int, T: float = 1.0, *, u=None, b_range=None, nthreads=None,
                 query=None):
    """Chain verify of B sequences.  zq [B, N+1, V], zp [B, N, V], d [B, N].
    T is rounded to float32 first, as the device library receives it.

    u (optional) [B, 2N+1] overrides Philox: accept uniforms of positions
    1..N, then sampling uniforms of slots 1..N+1.  b_range = (lo, hi)
    computes only those sequences (the other outputs keep their fill
    values).  Returns a dict of numpy arrays.
    """
    B, N1, V = zq.shape
    N = N1 - 1
    d = np.ascontiguousarray(d, dtype=np.int32).reshape(B, N)
    qs, qr = _strides3(zq)
    if N > 0:
        ps, pr = _strides3(zp)
        if zp.dtype != zq.dtype or zp.shape != (B, N, V):
            raise ValueError("zp must be [B, N, V] with the dtype of zq")
    else:
        ps = pr = 0
        zp = zq
    if u is not None:
        u = np.ascontiguousarray(u, dtype=np.float64).reshape(B, 2 * N + 1)
    lo, hi = b_range if b_range is not None else (0, B)
    o, s = _alloc_out(B, N + 1, max(N, 1), N + 1, False, query)
    rc = lib().orc_verify_chain(_ptr(zq), qs, qr, _ptr(zp), ps, pr, _dtype_code(zq), _ptr(d), B, N, V, seed, rnd,
                                _temperature(T), _ptr(u), lo, hi, nthreads or threads_available(), ctypes.byref(s))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o


def verify_tree(zq, zp, node_tokens, parents, seed: int, rnd: int, T: float = 1.0, *, max_depth: int, u=None,
                b_range=None, nthreads=None, query=None, walk: int = 0):
    """Tree verify.  zq, zp [B, T+1, V]; node_tokens [B, T+1]; parents [T+1]
    (shared) or [B, T+1].  u (optional) [B, T + max_depth + 1].  walk 0:
    descend into the first accepted child; walk 1: the pages' literal walk,
    only the best (lowest-index) child is followed and its rejection ends
    the walk."""
    B, nn, V = zq.shape
    Tn = nn - 1
    qs, qr = _strides3(zq)
    ps, pr = _strides3(zp)
    node_tokens = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, nn)
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    shared = 1 if parents.ndim == 1 else 0
    if u is not None:
        u = np.ascontiguousarray(u, dtype=np.float64).reshape(B, Tn + max_depth + 1)
    lo, hi = b_range if b_range is not None else (0, B)
    o, s = _alloc_out(B, max_depth + 1, nn, nn, True, query)
    rc = lib().orc_verify_tree(_ptr(zq), qs, qr, _ptr(zp), ps, pr, _dtype_code(zq), _ptr(node_tokens), _ptr(parents),
                               shared, B, Tn, V, max_depth, int(walk), seed, rnd, _temperature(T), _ptr(u), lo, hi,
                               nthreads or threads_available(), ctypes.byref(s))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o


def sample_draft(zp, seed: int, rnd: int, T: float = 1.0, *, pos0: int = 0, u=None, query=None, nthreads=None):
    """Draft tokens d ~ softmax(z / T), one per row of zp [B, R, V] (float32,
    float64 or bf16 bits as uint16), by the inverse CDF in token order with
    the uniform of Philox stream 1 at (sequence b, position pos0 + r).  u
    [B, R] replaces the uniforms; query [B, R] int32 asks for the CDF edges
    of given tokens.  Returns tokens, logprob, u, target, W, edge_lo, edge_hi
    (and qedge_lo, qedge_hi with query), each [B, R]."""
    zp = np.asarray(zp)
    B, R, V = zp.shape
    ss, rs = _strides3(zp)
    o = {"tokens": np.empty((B, R), np.int32)}
    for k in ("logprob", "u", "target", "W", "edge_lo", "edge_hi"):
        o[k] = np.full((B, R), np.nan)
    if u is not None:
        u = np.ascontiguousarray(u, dtype=np.float64).reshape(B, R)
    if query is not None:
        query = np.ascontiguousarray(query, dtype=np.int32).reshape(B, R)
        o["qedge_lo"] = np.full((B, R), np.nan)
        o["qedge_hi"] = np.full((B, R), np.nan)
    rc = lib().orc_sample_draft(_ptr(zp), ss, rs, _dtype_code(zp), B, R, V, _temperature(T), seed, rnd, pos0, _ptr(u),
                                _ptr(o["tokens"]), _ptr(o["logprob"]), _ptr(o["u"]), _ptr(o["target"]), _ptr(o["W"]),
                                _ptr(o["edge_lo"]), _ptr(o["edge_hi"]), _ptr(query), _ptr(o.get("qedge_lo")),
                                _ptr(o.get("qedge_hi")), nthreads or threads_available())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o


def tree_build(rows, depth: int, topk: int, budget: int, T: float = 1.0):
    """EAGLE-2 dynamic draft tree ("投机解码与 EAGLE", section 4, eagle_round
    step 2; section 5, the dynamic tree).  rows [B, 1 + topk*(depth-1), V]
    (float32, float64 or bf16 bits as uint16): the draft logits of the root
    (row 0) and of each level's frontier in rank order.  Returns parents,
    tokens, depth (int32 [B, budget+1]), log-scores (float64 [B, budget+1])
    and the frontiers' candidate ids (int32 [B, depth-1, topk])."""
    rows = np.ascontiguousarray(rows)
    B, n_exp, V = rows.shape
    if n_exp != 1 + topk * (depth - 1):
        raise ValueError("rows must hold 1 + topk*(depth-1) expanded rows")
    ss, rs = _strides3(rows)
    nn = budget + 1
    par = np.empty((B, nn), np.int32)
    tok = np.empty((B, nn), np.int32)
    dep = np.empty((B, nn), np.int32)
    score = np.empty((B, nn), np.float64)
    front = np.full((B, max(depth - 1, 0), topk), -1, np.int32)
    rc = lib().orc_tree_build(_ptr(rows), ss, rs, _dtype_code(rows), B, V, depth, topk, budget, _temperature(T),
                              _ptr(par), _ptr(tok), _ptr(dep), _ptr(score), _ptr(front))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return {"parents": par, "tokens": tok, "depth": dep, "score": score, "frontier": front}


def tree_mask(parents, kv_len_in=None, B: int = None):
    """Tree attention mask and position ids ("投机解码与 EAGLE", section 3):
    parents [T+1] (shared; B required) or [B, T+1].  Returns mask uint64
    [B, T+1, ceil((T+1)/64)] (bit j of row n: j is n or an ancestor of n) and
    positions int32 [B, T+1] = kv_len_in[b] + depth(n)."""
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    shared = parents.ndim == 1
    if shared:
        if B is None:
            raise ValueError("B is required with shared parents")
    else:
        B = parents.shape[0]
    nn = parents.shape[-1]
    W = (nn + 63) // 64
    if kv_len_in is not None:
        kv_len_in = np.ascontiguousarray(kv_len_in, dtype=np.int32)
    mask = np.zeros((B, nn, W), np.uint64)
    pos = np.zeros((B, nn), np.int32)
    if lib().orc_tree_mask(_ptr(parents), int(shared), _ptr(kv_len_in), B, nn - 1, _ptr(mask), _ptr(pos)) != 0:
        raise ValueError("oracle rejected the arguments")
    return mask, pos


def kv_compact(path_nodes, num_accepted, kv_len_in, max_depth: int, kv=None):
    """KV compaction indices, and (kv given: uint8 array [planes, B, L, row_bytes]
    modified in place) the gather.  path_nodes None = chain (identity)."""
    num_accepted = np.ascontiguousarray(num_accepted, dtype=np.int32)
    kv_len_in = np.ascontiguousarray(kv_len_in, dtype=np.int32)
    B = num_accepted.shape[0]
    if path_nodes is not None:
        path_nodes = np.ascontiguousarray(path_nodes, dtype=np.int32).reshape(B, max_depth + 1)
    src = np.empty((B, max_depth + 1), np.int32)
    kvl = np.empty(B, np.int32)
    if kv is not None:
        assert kv.dtype == np.uint8 and kv.ndim == 4 and kv.flags.c_contiguous
        P, _, _, rb = kv.shape
        rc = lib().orc_kv_compact(_ptr(path_nodes), _ptr(num_accepted), _ptr(kv_len_in), B, max_depth, _ptr(src),
                                  _ptr(kvl), _ptr(kv), kv.strides[1], kv.strides[2], rb, P, kv.strides[0])
    else:
        rc = lib().orc_kv_compact(_ptr(path_nodes), _ptr(num_accepted), _ptr(kv_len_in), B, max_depth, _ptr(src),
                                  _ptr(kvl), None, 0, 0, 0, 0, 0)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return src, kvl
