"""MI355X (gfx950) speculative-decoding verify-and-accept step.

Thin Python binding of ``libspecverify.so`` (C ABI declared in
``include/specverify.h``).  This module only marshals arguments: it checks
tensor shapes, allocates outputs and the workspace with torch on the logits'
device, and passes raw device pointers plus torch's current HIP stream.  All
of the step runs in the library's HIP kernels; there is no CPU or PyTorch
fallback, and importing this module raises if the library is not built.

Functions (same names as the C ABI):
  spec_verify_chain  -- chain verify ([PT] "Decodificacao Especulativa e
                        EAGLE-3", O Conceito and Implementando, Passo 1-3)
  spec_verify_tree   -- flattened-tree verify ([ZH] "投机解码与 EAGLE",
                        sections 3 and 4)
  kv_compact_indices -- KV rollback / compaction ([PT] Passo 4; [ZH]
                        section 3)
  tree_attention_mask -- ancestor mask and position ids of flattened draft
                        trees, the verifier-side inputs of a tree verify
                        pass ([ZH] section 3)
  tree_expand, tree_select, tree_finalize -- EAGLE-2 dynamic draft tree,
                        level by level ([ZH] sections 4 and 5); tree_build
                        chains them over draft rows given up front
  sample_draft       -- draft tokens d ~ p from draft logits ([PT] O Conceito;
                        [ZH] section 2)
  sv_philox_uniforms -- the step's uniforms (for tests)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_WALK_FIRST_ACCEPTED, SV_WALK_BEST_CHILD = 0, 1
STATUS = {0: "SV_OK", 1: "SV_EINVAL", 2: "SV_EDTYPE", 3: "SV_ESHAPE", 4: "SV_EALIGN", 5: "SV_EWORKSPACE",
          6: "SV_EHIP", 7: "SV_ESCRATCH"}


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({_lib().sv_status_string(code).decode()})")


class SvTiming(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_void_p), ("rows_done", ctypes.c_void_p), ("end", ctypes.c_void_p)]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t
        L.sv_abi_version.restype = i32
        L.sv_abi_version.argtypes = []
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_status_string.argtypes = [i32]
        L.sv_chain_workspace_bytes.restype = sz
        L.sv_chain_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_tree_workspace_bytes.restype = sz
        L.sv_tree_workspace_bytes.argtypes = [i32, i32, i32]
        L.spec_verify_chain.restype = i32
        L.spec_verify_chain.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, i32, i32, i32, u64, u64,
                                        ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                        ctypes.POINTER(SvTiming), vp]
        L.spec_verify_chain_noalloc.restype = i32
        L.spec_verify_chain_noalloc.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, i32, i32, i32, u64, u64,
                                                ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.POINTER(SvTiming), vp]
        L.spec_verify_tree.restype = i32
        L.spec_verify_tree.argtypes = [vp, i64, i64, vp, i64, i64, i32, vp, vp, i32, i32, i32, i32, i32, i32, u64, u64,
                                       ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                       ctypes.POINTER(SvTiming), vp]
        L.kv_compact_indices.restype = i32
        L.kv_compact_indices.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, i32, i64, i64, i32, i32, i64, vp]
        L.tree_expand.restype = i32
        L.tree_expand.argtypes = [vp, i64, i64, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp, i32, i32, i32, vp, vp,
                                  vp, vp, vp]
        L.tree_select.restype = i32
        L.tree_select.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
        L.tree_finalize.restype = i32
        L.tree_finalize.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.tree_attention_mask.restype = i32
        L.tree_attention_mask.argtypes = [vp, i32, vp, i32, i32, vp, vp, vp]
        L.sv_philox_uniforms.restype = i32
        L.sv_sample_draft.restype = i32
        L.sv_sample_draft.argtypes = [vp, i64, i64, i32, i32, i32, i32, ctypes.c_float, u64, u64, i32, vp, vp, vp]
        L.sv_philox_uniforms.argtypes = [u64, u64, i32, i32, vp, vp, vp]
        if L.sv_abi_version() != 6:
            raise ImportError("libspecverify.so ABI version mismatch")
        _L = L
    return _L


def library():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check_logits(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be [B, rows, V] with a unit stride on V")


def _timing(timing):
    """(begin, end) or (begin, rows_done, end) hipEvent_t handles (None for
    any not wanted) stamped by the call's kernels, or None."""
    if timing is None:
        return None
    if len(timing) == 2:
        return ctypes.byref(SvTiming(timing[0], None, timing[1]))
    return ctypes.byref(SvTiming(timing[0], timing[1], timing[2]))


def chain_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(_lib().sv_chain_workspace_bytes(B, N, V))


def tree_workspace_bytes(B: int, T: int, V: int) -> int:
    return int(_lib().sv_tree_workspace_bytes(B, T, V))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace.  Zero-filled once: each call tags its records
    and counters with its own number (the low word of the library's 64-bit
    call counter, which starts at a value drawn when the library is loaded),
    so a record an earlier call left reads as stale and one workspace serves
    any number of later calls without being cleared again."""
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return alloc_workspace(nbytes, device)


def alloc_chain_outputs(B: int, N: int, device, kv: bool = False):
    o = {
        "tokens": torch.empty((B, N + 1), dtype=torch.int32, device=device),
        "num_accepted": torch.empty(B, dtype=torch.int32, device=device),
        "accept": torch.empty((B, N), dtype=torch.int8, device=device),
        "probs": torch.empty((B, N, 2), dtype=torch.float32, device=device),
        "residual_mass": torch.empty(B, dtype=torch.float64, device=device),
    }
    if kv:
        o["src_rows"] = torch.empty((B, N + 1), dtype=torch.int32, device=device)
        o["kv_len"] = torch.empty(B, dtype=torch.int32, device=device)
    return o


def spec_verify_chain(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor], draft_tokens: torch.Tensor,
                      seed: int, round: int, temperature: float = 1.0, *, kv_len_in: Optional[torch.Tensor] = None,
                      out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, timing=None,
                      stream=None) -> dict:
    """Verify B chains: target_logits [B, N+1, V], draft_logits [B, N, V]
    (float32 or bfloat16), draft_tokens [B, N] int32.  Returns (or fills)
    a dict with tokens [B, N+1], num_accepted [B], accept [B, N] (int8),
    probs [B, N, 2] (q(d), p(d)) and residual_mass [B]; with kv_len_in
    (int32 [B], the KV row of the pending token) also src_rows [B, N+1] and
    kv_len [B], the KV rows kept."""
    _check_logits(target_logits, "target_logits")
    B, N1, V = target_logits.shape
    N = N1 - 1
    if N > 0:
        _check_logits(draft_logits, "draft_logits")
        if draft_logits.shape != (B, N, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [B, N, V] with the dtype of target_logits")
        if draft_tokens.shape != (B, N) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
            raise ValueError("draft_tokens must be a contiguous int32 [B, N] tensor")
    dev = target_logits.device
    o = out if out is not None else alloc_chain_outputs(B, N, dev, kv=kv_len_in is not None)
    _check_kv(kv_len_in, o, B)
    nbytes = chain_workspace_bytes(B, N, V)
    ws = _workspace(nbytes, dev, workspace)
    dl = draft_logits if N > 0 else None
    rc = _lib().spec_verify_chain(
        _p(target_logits), target_logits.stride(0), target_logits.stride(1),
        _p(dl), dl.stride(0) if dl is not None else 0, dl.stride(1) if dl is not None else 0,
        _dtype_code(target_logits), _p(draft_tokens) if N > 0 else None, B, N, V, seed & (2 ** 64 - 1),
        round & (2 ** 64 - 1), float(temperature), _p(o["tokens"]), _p(o["num_accepted"]), _p(o.get("accept")),
        _p(o.get("probs")), _p(o.get("residual_mass")), *_kv_args(kv_len_in, o), _p(ws),
        ws.numel() * ws.element_size(), _timing(timing), _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_chain")
    return o


def spec_verify_chain_noalloc(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                              draft_tokens: torch.Tensor, seed: int, round: int, temperature: float = 1.0, *,
                              kv_len_in: Optional[torch.Tensor] = None, out: dict, timing=None, stream=None) -> dict:
    """spec_verify_chain through the entry point that allocates nothing: the
    library's static per-GPU scratch replaces the workspace, and `out`
    (preallocated outputs, alloc_chain_outputs) is required, so the call
    itself allocates no device memory."""
    _check_logits(target_logits, "target_logits")
    B, N1, V = target_logits.shape
    N = N1 - 1
    if N > 0:
        _check_logits(draft_logits, "draft_logits")
        if draft_logits.shape != (B, N, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [B, N, V] with the dtype of target_logits")
        if draft_tokens.shape != (B, N) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
            raise ValueError("draft_tokens must be a contiguous int32 [B, N] tensor")
    _check_kv(kv_len_in, out, B)
    dl = draft_logits if N > 0 else None
    rc = _lib().spec_verify_chain_noalloc(
        _p(target_logits), target_logits.stride(0), target_logits.stride(1),
        _p(dl), dl.stride(0) if dl is not None else 0, dl.stride(1) if dl is not None else 0,
        _dtype_code(target_logits), _p(draft_tokens) if N > 0 else None, B, N, V, seed & (2 ** 64 - 1),
        round & (2 ** 64 - 1), float(temperature), _p(out["tokens"]), _p(out["num_accepted"]), _p(out.get("accept")),
        _p(out.get("probs")), _p(out.get("residual_mass")), *_kv_args(kv_len_in, out), _timing(timing),
        _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_chain_noalloc")
    return out


def alloc_tree_outputs(B: int, T: int, max_depth: int, device, kv: bool = False):
    o = {
        "tokens": torch.empty((B, max_depth + 1), dtype=torch.int32, device=device),
        "path_nodes": torch.empty((B, max_depth + 1), dtype=torch.int32, device=device),
        "num_accepted": torch.empty(B, dtype=torch.int32, device=device),
        "accept": torch.empty((B, T + 1), dtype=torch.int8, device=device),
        "probs": torch.empty((B, T + 1, 2), dtype=torch.float32, device=device),
        "residual_mass": torch.empty(B, dtype=torch.float64, device=device),
    }
    if kv:
        o["src_rows"] = torch.empty((B, max_depth + 1), dtype=torch.int32, device=device)
        o["kv_len"] = torch.empty(B, dtype=torch.int32, device=device)
    return o


def _check_kv(kv_len_in, o, B):
    if kv_len_in is None:
        return
    if kv_len_in.shape != (B,) or kv_len_in.dtype != torch.int32 or not kv_len_in.is_contiguous():
        raise ValueError("kv_len_in must be a contiguous int32 [B] tensor")
    if "src_rows" not in o or "kv_len" not in o:
        raise ValueError("out must hold src_rows and kv_len when kv_len_in is given")


def _kv_args(kv_len_in, o):
    if kv_len_in is None:
        return None, None, None
    return _p(kv_len_in), _p(o["src_rows"]), _p(o["kv_len"])


def spec_verify_tree(target_logits: torch.Tensor, draft_logits: torch.Tensor, node_tokens: torch.Tensor,
                     parents: torch.Tensor, seed: int, round: int, temperature: float = 1.0, *, max_depth: int,
                     walk: int = 0, kv_len_in: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                     workspace: Optional[torch.Tensor] = None, timing=None, stream=None) -> dict:
    """Verify B flattened trees: logits [B, T+1, V] per node, node_tokens
    [B, T+1] int32, parents [T+1] (shared) or [B, T+1] int32.  walk 0
    (SV_WALK_FIRST_ACCEPTED) descends into the first accepted child; walk 1
    (SV_WALK_BEST_CHILD) is the pages' literal best-child walk."""
    _check_logits(target_logits, "target_logits")
    _check_logits(draft_logits, "draft_logits")
    B, nn, V = target_logits.shape
    T = nn - 1
    if draft_logits.shape != (B, nn, V) or draft_logits.dtype != target_logits.dtype:
        raise ValueError("draft_logits must be [B, T+1, V] with the dtype of target_logits")
    if node_tokens.shape != (B, nn) or node_tokens.dtype != torch.int32 or not node_tokens.is_contiguous():
        raise ValueError("node_tokens must be a contiguous int32 [B, T+1] tensor")
    if parents.dtype != torch.int32 or not parents.is_contiguous() or parents.shape not in ((nn,), (B, nn)):
        raise ValueError("parents must be a contiguous int32 [T+1] or [B, T+1] tensor")
    dev = target_logits.device
    o = out if out is not None else alloc_tree_outputs(B, T, max_depth, dev, kv=kv_len_in is not None)
    _check_kv(kv_len_in, o, B)
    nbytes = tree_workspace_bytes(B, T, V)
    ws = _workspace(nbytes, dev, workspace)
    rc = _lib().spec_verify_tree(
        _p(target_logits), target_logits.stride(0), target_logits.stride(1), _p(draft_logits),
        draft_logits.stride(0), draft_logits.stride(1), _dtype_code(target_logits), _p(node_tokens), _p(parents),
        1 if parents.dim() == 1 else 0, B, T, V, max_depth, int(walk), seed & (2 ** 64 - 1), round & (2 ** 64 - 1),
        float(temperature), _p(o["tokens"]), _p(o["path_nodes"]), _p(o["num_accepted"]), _p(o.get("accept")),
        _p(o.get("probs")), _p(o.get("residual_mass")), *_kv_args(kv_len_in, o), _p(ws),
        ws.numel() * ws.element_size(), _timing(timing), _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "spec_verify_tree")
    return o


def kv_compact_indices(path_nodes: Optional[torch.Tensor], num_accepted: torch.Tensor, kv_len_in: torch.Tensor,
                       max_depth: int, kv: Optional[torch.Tensor] = None, *, stacked_planes: bool = False,
                       out: Optional[dict] = None, stream=None) -> dict:
    """KV rollback/compaction.  path_nodes [B, max_depth+1] int32 (None for
    a chain); kv (optional) is compacted in place: [B, L, ...] or, with
    stacked_planes=True, [P, B, L, ...] (P planes, e.g. K and V of every
    layer).  Returns src_rows [B, max_depth+1] and kv_len [B]."""
    B = num_accepted.shape[0]
    dev = num_accepted.device
    o = out if out is not None else {
        "src_rows": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
        "kv_len": torch.empty(B, dtype=torch.int32, device=dev),
    }
    kv_args = (None, 0, 0, 0, 0, 0, 0)
    if kv is not None:
        planes = kv if stacked_planes else kv.unsqueeze(0)
        if planes.dim() < 3 or planes.shape[1] != B:
            raise ValueError("kv must be [B, L, ...] (or [P, B, L, ...] with stacked_planes=True)")
        es = planes.element_size()
        row = planes[0, 0, 0]
        if not row.is_contiguous():
            raise ValueError("a KV row must be contiguous")
        kv_args = (_p(planes), planes.shape[2], planes.stride(1) * es, planes.stride(2) * es, row.numel() * es,
                   planes.shape[0], planes.stride(0) * es)
    rc = _lib().kv_compact_indices(_p(path_nodes), _p(num_accepted), _p(kv_len_in), B, max_depth, _p(o["src_rows"]),
                                   _p(o["kv_len"]), *kv_args, _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "kv_compact_indices")
    return o


def tree_attention_mask(parents: torch.Tensor, kv_len_in: Optional[torch.Tensor] = None, B: Optional[int] = None,
                        out: Optional[dict] = None, stream=None) -> dict:
    """Tree attention mask and position ids of flattened draft trees.
    parents int32 [T+1] (shared; B required) or [B, T+1]; kv_len_in int32 [B]
    (the KV row of node 0) or None (0).  Returns mask int64 [B, T+1, W]
    (W = ceil((T+1)/64) 64-bit words; bit j of row n: node j is n or an
    ancestor of n) and positions int32 [B, T+1] (kv_len_in + depth)."""
    shared = parents.dim() == 1
    if shared and B is None:
        raise ValueError("B is required with shared parents")
    B = B if shared else parents.shape[0]
    nn = parents.shape[-1]
    W = (nn + 63) // 64
    dev = parents.device
    o = out if out is not None else {
        "mask": torch.empty((B, nn, W), dtype=torch.int64, device=dev),
        "positions": torch.empty((B, nn), dtype=torch.int32, device=dev),
    }
    rc = _lib().tree_attention_mask(_p(parents), int(shared), _p(kv_len_in), B, nn - 1, _p(o["mask"]),
                                    _p(o["positions"]), _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "tree_attention_mask")
    return o


def alloc_tree_table(B: int, n_max: int, device) -> dict:
    """A candidate table for tree_expand / tree_select / tree_finalize."""
    return {"token": torch.empty((B, n_max), dtype=torch.int32, device=device),
            "parent": torch.empty((B, n_max), dtype=torch.int32, device=device),
            "level": torch.empty((B, n_max), dtype=torch.int32, device=device),
            "score": torch.empty((B, n_max), dtype=torch.float64, device=device)}


def tree_expand(frontier_logits: torch.Tensor, table: dict, *, topk: int, level: int, offset: int,
                temperature: float = 1.0, frontier_ids: Optional[torch.Tensor] = None,
                frontier_score: Optional[torch.Tensor] = None, stream=None) -> None:
    """One level of a dynamic draft tree: frontier_logits [B, F, V] (rows
    with a unit last stride) add topk candidates per row at offset +
    f*topk of the table."""
    if frontier_logits.dim() != 3 or frontier_logits.stride(2) != 1:
        raise ValueError("frontier_logits must be [B, F, V] with a unit last stride")
    B, F, V = frontier_logits.shape
    n_max = table["score"].shape[1]
    rc = _lib().tree_expand(_p(frontier_logits), frontier_logits.stride(0), frontier_logits.stride(1),
                            _dtype_code(frontier_logits), B, F, V, topk, float(temperature), _p(frontier_ids),
                            _p(frontier_score), level, n_max, offset, _p(table["token"]), _p(table["parent"]),
                            _p(table["level"]), _p(table["score"]), _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "tree_expand")


def tree_select(table: dict, *, offset: int, count: int, k: int, stream=None):
    """The next frontier: ids and scores [B, k] of the k best candidates in
    [offset, offset + count)."""
    B, n_max = table["score"].shape
    dev = table["score"].device
    ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    sc = torch.empty((B, k), dtype=torch.float64, device=dev)
    rc = _lib().tree_select(_p(table["score"]), B, n_max, offset, count, k, _p(ids), _p(sc), _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "tree_select")
    return ids, sc


def tree_finalize(table: dict, *, n: int, budget: int, stream=None) -> dict:
    """The kept set of candidates [0, n), flattened: parents, tokens, depth
    [B, budget+1] int32 and score [B, budget+1] float64."""
    B, n_max = table["score"].shape
    dev = table["score"].device
    o = {"parents": torch.empty((B, budget + 1), dtype=torch.int32, device=dev),
         "tokens": torch.empty((B, budget + 1), dtype=torch.int32, device=dev),
         "depth": torch.empty((B, budget + 1), dtype=torch.int32, device=dev),
         "score": torch.empty((B, budget + 1), dtype=torch.float64, device=dev)}
    rc = _lib().tree_finalize(_p(table["token"]), _p(table["parent"]), _p(table["level"]), _p(table["score"]), B,
                              n_max, n, budget, _p(o["parents"]), _p(o["tokens"]), _p(o["depth"]), _p(o["score"]),
                              _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "tree_finalize")
    return o


def tree_build(rows: torch.Tensor, *, depth: int, topk: int, budget: int, temperature: float = 1.0,
               stream=None) -> dict:
    """A whole dynamic tree from draft rows that exist up front (synthetic
    runs): rows [B, 1 + topk*(depth-1), V] hold the root's row, then each
    level's frontier rows in rank order.  Chains tree_expand (per level),
    tree_select (between levels) and tree_finalize; adds the frontiers'
    candidate ids [B, depth-1, topk] to the result."""
    B, n_exp, V = rows.shape
    if n_exp != 1 + topk * (depth - 1):
        raise ValueError("rows must hold 1 + topk*(depth-1) expanded rows")
    n = topk + (depth - 1) * topk * topk
    table = alloc_tree_table(B, n, rows.device)
    ids = sc = None
    frontiers = []
    offset, F = 0, 1
    for level in range(1, depth + 1):
        slot = 0 if level == 1 else 1 + (level - 2) * topk
        tree_expand(rows[:, slot:slot + F], table, topk=topk, level=level, offset=offset, temperature=temperature,
                    frontier_ids=ids, frontier_score=sc, stream=stream)
        if level < depth:
            ids, sc = tree_select(table, offset=offset, count=F * topk, k=topk, stream=stream)
            frontiers.append(ids)
        offset += F * topk
        F = topk
    out = tree_finalize(table, n=n, budget=budget, stream=stream)
    out["frontier"] = torch.stack(frontiers, 1) if frontiers else torch.empty((B, 0, topk), dtype=torch.int32,
                                                                               device=rows.device)
    return out


def sample_draft(logits: torch.Tensor, seed: int, round: int, temperature: float = 1.0, *, pos0: int = 0,
                 logprob: bool = True, stream=None):
    """Draft tokens d ~ softmax(logits / T), one per row of logits [B, R, V]
    (unit last stride): int32 tokens [B, R] and, with logprob, float64
    ln p(token) [B, R]; uniforms from Philox stream 1 at positions pos0 + r."""
    if logits.dim() != 3 or logits.stride(2) != 1:
        raise ValueError("logits must be [B, R, V] with a unit last stride")
    B, R, V = logits.shape
    tok = torch.empty((B, R), dtype=torch.int32, device=logits.device)
    lp = torch.empty((B, R), dtype=torch.float64, device=logits.device) if logprob else None
    rc = _lib().sv_sample_draft(_p(logits), logits.stride(0), logits.stride(1), _dtype_code(logits), B, R, V,
                                float(temperature), seed & (2 ** 64 - 1), round & (2 ** 64 - 1), pos0, _p(tok),
                                _p(lp), _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "sv_sample_draft")
    return tok, lp


def sv_philox_uniforms(seed: int, round: int, nseq: int, npos: int, device="cuda", stream=None):
    """(u_acc, u_samp) [nseq, npos] float64 for positions 1..npos."""
    a = torch.empty((nseq, npos), dtype=torch.float64, device=device)
    s = torch.empty((nseq, npos), dtype=torch.float64, device=device)
    rc = _lib().sv_philox_uniforms(seed & (2 ** 64 - 1), round & (2 ** 64 - 1), nseq, npos, _p(a), _p(s),
                                   _stream(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "sv_philox_uniforms")
    return a, s


__all__ = ["spec_verify_chain", "spec_verify_chain_noalloc", "spec_verify_tree", "kv_compact_indices", "tree_attention_mask", "sample_draft",
           "tree_expand",
           "tree_select", "tree_finalize", "tree_build", "alloc_tree_table", "sv_philox_uniforms",
           "chain_workspace_bytes", "tree_workspace_bytes", "alloc_workspace", "alloc_chain_outputs", "alloc_tree_outputs",
           "SpecVerifyError", "library", "LIB_PATH", "SV_F32", "SV_BF16", "SV_WALK_FIRST_ACCEPTED",
           "SV_WALK_BEST_CHILD"]
