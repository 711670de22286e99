"""ctypes binding of ``libmisa.so`` (the C ABI declared in include/misa.h).

Argument marshalling only: torch tensors in, device pointers and the current
HIP stream out. Every step of the indexer runs in the library's kernels; there
is no fallback of any kind, and a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmisa.so")

MISA_OK = 0
MISA_ERR_ARG = -1
MISA_ERR_ALIGN = -2
MISA_ERR_WORKSPACE = -3
MISA_ERR_HIP = -4

OP_ROUTE = 1
OP_SCORE_TOPK = 2
OP_HIER_RERANK = 3
OP_DSA_DENSE = 4
OP_INDEXER = 5
OP_HIER_INDEXER = 6
OP_BLOCK_FILTER = 7
OP_BLOCK_INDEXER = 8
OP_PIVOT_INDEXER = 9

KERNEL_SCORE = 1
KERNEL_TOPK = 2
KERNEL_ROUTE = 3
KERNEL_POOL = 4
KERNEL_GATHER_SCORE = 5

_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "misa_version": (_I32, []),
    "misa_status_string": (ctypes.c_char_p, [_I32]),
    "misa_last_error": (ctypes.c_char_p, []),
    "misa_workspace_bytes": (_SZ, [_I32, _I64, _I32, _I64, _I32, _I32, _I32]),
    "misa_pool_keys": (_I32, [_P, _I64, _I64, _I32, _I32, _P, _P]),
    "misa_pool_update": (_I32, [_P, _I64, _I64, _I32, _I32, _P, _P, _I32, _P, _P]),
    "misa_route": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "misa_score_topk": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _P, _P, _P, _SZ,
                               _P]),
    "misa_hier_rerank": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _P, _P, _P, _SZ,
                                _P]),
    "dsa_index_dense": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _P, _P, _P, _SZ, _P]),
    "misa_debug_scores": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I64, _I32, _I32, _I64, _I64, _P, _P]),
    "misa_indexer": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P,
                            _SZ, _P]),
    "misa_hier_indexer": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P,
                                 _P, _P, _P, _SZ, _P]),
    "misa_block_filter": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _P, _P,
                                 _P, _SZ, _P]),
    "misa_block_indexer": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _I32, _I32, _P,
                                  _P, _P, _P, _P, _SZ, _P]),
    "misa_pivot_indexer": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _I32, _P, _P, _P,
                                  _P, _SZ, _P]),
    "misa_hier_indexer_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I64, _I64, _I32, _I32, _I32,
                                         _I32, _P, _P, _P, _P, _P]),
    "misa_timing_begin": (_I32, [_I32, _I32, _P]),
    "misa_timing_end": (_I32, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]),
}


class MisaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {code}: {msg}")
        self.code = code


def lib():
    """Load ``libmisa.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m routed_token_indexer_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(fn: str, rc: int):
    if rc != MISA_OK:
        raise MisaError(fn, rc, lib().misa_last_error().decode())


def _ptr(x: Optional[torch.Tensor]):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _req(x: torch.Tensor, dtype, name: str, ndim: int):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {x.dtype}")
    if x.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(x.shape)}")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def workspace_bytes(op: int, T: int, H: int, Lmax: int, B: int = 0, topk: int = 0, kc: int = 0) -> int:
    return int(lib().misa_workspace_bytes(op, T, H, Lmax, B, topk, kc))


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is not None and ws.numel() >= need:
        return ws
    return torch.empty(max(need, 256), dtype=torch.uint8, device=device)


def pool_keys(k: torch.Tensor, B: int, kbar: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Mean of each complete block of B keys: kbar [nseq, Lmax // B, d] fp32."""
    _req(k, torch.bfloat16, "k", 3)
    nseq, L, d = k.shape
    if kbar is None:
        kbar = torch.empty((nseq, L // B, d), dtype=torch.float32, device=k.device)
    _check("misa_pool_keys", lib().misa_pool_keys(_ptr(k), nseq, L, d, B, _ptr(kbar), _stream(stream)))
    return kbar


def pool_update(k: torch.Tensor, B: int, prev_len: torch.Tensor, new_len: torch.Tensor, max_new: int,
                kbar: torch.Tensor, stream=None) -> torch.Tensor:
    """Pools, in place in ``kbar``, the blocks that growing each sequence from
    ``prev_len`` to ``new_len`` tokens completed (at most ``max_new`` new tokens)."""
    _req(k, torch.bfloat16, "k", 3)
    nseq, L, d = k.shape
    _check("misa_pool_update", lib().misa_pool_update(_ptr(k), nseq, L, d, B, _ptr(prev_len), _ptr(new_len), max_new,
                                                      _ptr(kbar), _stream(stream)))
    return kbar


def route(q, w, k, kbar, q_seq, q_len, B: int, h: int, heads=None, router_key=None, ws=None, stream=None):
    """Routed heads [T, h] (ascending) and, if ``router_key`` is given, the importance r [T, H]."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    if heads is None:
        heads = torch.empty((T, h), dtype=torch.int32, device=q.device)
    ws = _workspace(ws, workspace_bytes(OP_ROUTE, T, H, L, B), q.device)
    _check("misa_route", lib().misa_route(_ptr(q), _ptr(w), _ptr(k), _ptr(kbar), _ptr(q_seq), _ptr(q_len), T, H, d,
                                          nseq, L, B, h, _ptr(heads), _ptr(router_key), _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return heads


def _outs(T, topk, device, idx, score, want_score):
    if idx is None:
        idx = torch.empty((T, topk), dtype=torch.int32, device=device)
    if score is None and want_score:
        score = torch.empty((T, topk), dtype=torch.float32, device=device)
    return idx, score


def score_topk(q, w, k, heads, q_seq, q_len, topk: int, idx=None, score=None, want_score=True, ws=None,
               stream=None):
    """Routed scoring + per-query top-k: idx [T, topk] (ascending, -1 padded), score [T, topk]."""
    _req(q, torch.bfloat16, "q", 3)
    _req(heads, torch.int32, "heads", 2)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_SCORE_TOPK, T, H, L, 0, topk), q.device)
    _check("misa_score_topk", lib().misa_score_topk(_ptr(q), _ptr(w), _ptr(k), _ptr(heads), heads.shape[1],
                                                    _ptr(q_seq), _ptr(q_len), T, H, d, nseq, L, topk, _ptr(idx),
                                                    _ptr(score), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, score


def hier_rerank(q, w, k, cand, q_seq, q_len, topk: int, idx=None, score=None, want_score=True, ws=None,
                stream=None):
    """MISA† fine stage: dense re-rank of the candidate rows cand [T, kc] to idx [T, topk]."""
    _req(q, torch.bfloat16, "q", 3)
    _req(cand, torch.int32, "cand", 2)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    kc = cand.shape[1]
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_HIER_RERANK, T, H, L, 0, topk, kc), q.device)
    _check("misa_hier_rerank", lib().misa_hier_rerank(_ptr(q), _ptr(w), _ptr(k), _ptr(cand), kc, _ptr(q_seq),
                                                      _ptr(q_len), T, H, d, nseq, L, topk, _ptr(idx), _ptr(score),
                                                      _ptr(ws), ws.numel(), _stream(stream)))
    return idx, score


def dsa_index_dense(q, w, k, q_seq, q_len, topk: int, idx=None, score=None, want_score=True, ws=None,
                    stream=None):
    """Dense DSA indexer (all H heads) + top-k."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_DSA_DENSE, T, H, L, 0, topk), q.device)
    _check("dsa_index_dense", lib().dsa_index_dense(_ptr(q), _ptr(w), _ptr(k), _ptr(q_seq), _ptr(q_len), T, H, d,
                                                    nseq, L, topk, _ptr(idx), _ptr(score), _ptr(ws), ws.numel(),
                                                    _stream(stream)))
    return idx, score


def indexer(q, w, k, kbar, q_seq, q_len, B: int, h: int, topk: int, heads=None, idx=None, score=None,
            want_score=True, ws=None, stream=None):
    """Whole MISA indexer (route + routed scoring + top-k) in one call."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_INDEXER, T, H, L, B, topk), q.device)
    _check("misa_indexer", lib().misa_indexer(_ptr(q), _ptr(w), _ptr(k), _ptr(kbar), _ptr(q_seq), _ptr(q_len), T, H,
                                              d, nseq, L, B, h, topk, _ptr(heads), _ptr(idx), _ptr(score), _ptr(ws),
                                              ws.numel(), _stream(stream)))
    return idx, score


def hier_indexer(q, w, k, kbar, q_seq, q_len, B: int, h: int, kc: int, topk: int, heads=None, cand=None, idx=None,
                 score=None, want_score=True, ws=None, stream=None):
    """Whole MISA† indexer (route + routed top-k' + dense re-rank to top-k) in one call."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_HIER_INDEXER, T, H, L, B, topk, kc), q.device)
    _check("misa_hier_indexer", lib().misa_hier_indexer(_ptr(q), _ptr(w), _ptr(k), _ptr(kbar), _ptr(q_seq),
                                                        _ptr(q_len), T, H, d, nseq, L, B, h, kc, topk, _ptr(heads),
                                                        _ptr(cand), _ptr(idx), _ptr(score), _ptr(ws), ws.numel(),
                                                        _stream(stream)))
    return idx, score


def block_filter(q, w, kbar, heads, q_seq, q_len, Lmax: int, B: int, m: int, blocks=None, cand=None,
                 want_cand=True, ws=None, stream=None):
    """Coarse stage: the m best complete blocks of each query by the routed
    formula on the pooled keys (blocks [T, m], ascending, -1 padded) and the
    candidate token list cand [T, (m + 1) * B] (kept blocks, then the partial one)."""
    _req(q, torch.bfloat16, "q", 3)
    _req(heads, torch.int32, "heads", 2)
    _req(kbar, torch.float32, "kbar", 3)
    T, H, d = q.shape
    nseq = kbar.shape[0]
    if blocks is None:
        blocks = torch.empty((T, m), dtype=torch.int32, device=q.device)
    if cand is None and want_cand:
        cand = torch.empty((T, (m + 1) * B), dtype=torch.int32, device=q.device)
    ws = _workspace(ws, workspace_bytes(OP_BLOCK_FILTER, T, H, Lmax, B, 0, m), q.device)
    _check("misa_block_filter", lib().misa_block_filter(_ptr(q), _ptr(w), _ptr(kbar), _ptr(heads), heads.shape[1],
                                                        _ptr(q_seq), _ptr(q_len), T, H, d, nseq, Lmax, B, m,
                                                        _ptr(blocks), _ptr(cand), _ptr(ws), ws.numel(),
                                                        _stream(stream)))
    return blocks, cand


def block_indexer(q, w, k, kbar, q_seq, q_len, B: int, h: int, m: int, topk: int, heads=None, blocks=None, idx=None,
                  score=None, want_score=True, ws=None, stream=None):
    """Route, keep the m best complete blocks (+ the partial one), routed top-k among their tokens."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_BLOCK_INDEXER, T, H, L, B, topk, m), q.device)
    _check("misa_block_indexer", lib().misa_block_indexer(_ptr(q), _ptr(w), _ptr(k), _ptr(kbar), _ptr(q_seq),
                                                          _ptr(q_len), T, H, d, nseq, L, B, h, m, topk, _ptr(heads),
                                                          _ptr(blocks), _ptr(idx), _ptr(score), _ptr(ws), ws.numel(),
                                                          _stream(stream)))
    return idx, score


def pivot_indexer(q, w, k, q_seq, q_len, G: int, kc: int, topk: int, cand=None, idx=None, score=None,
                  want_score=True, ws=None, stream=None):
    """PIVOT-Refine over groups of G consecutive queries: the group proxy's dense
    scan keeps kc candidates, each query re-ranks them densely to its top-k."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    ws = _workspace(ws, workspace_bytes(OP_PIVOT_INDEXER, T, H, L, G, topk, kc), q.device)
    _check("misa_pivot_indexer", lib().misa_pivot_indexer(_ptr(q), _ptr(w), _ptr(k), _ptr(q_seq), _ptr(q_len), T, H,
                                                          d, nseq, L, G, kc, topk, _ptr(cand), _ptr(idx), _ptr(score),
                                                          _ptr(ws), ws.numel(), _stream(stream)))
    return idx, score


def debug_scores(q, w, k, heads, q_seq, q_len, out=None, stream=None):
    """Full routed score rows [T, Lmax] (row t valid for s < q_len[t]); heads=None: dense."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    if out is None:
        out = torch.zeros((T, L), dtype=torch.float32, device=q.device)
    h = H if heads is None else heads.shape[1]
    _check("misa_debug_scores", lib().misa_debug_scores(_ptr(q), _ptr(w), _ptr(k), _ptr(heads), h, _ptr(q_seq),
                                                        _ptr(q_len), T, H, d, nseq, L, _ptr(out), _stream(stream)))
    return out


def hier_indexer_noalloc(q, w, k, kbar, q_seq, q_len, B: int, h: int, kc: int, topk: int, heads=None, cand=None,
                         idx=None, score=None, want_score=True, stream=None):
    """misa_hier_indexer with the library's own per-GPU scratch: no workspace,
    nothing allocated by the library (outputs passed in are used as they are)."""
    _req(q, torch.bfloat16, "q", 3)
    T, H, d = q.shape
    nseq, L, _ = k.shape
    idx, score = _outs(T, topk, q.device, idx, score, want_score)
    _check("misa_hier_indexer_noalloc",
           lib().misa_hier_indexer_noalloc(_ptr(q), _ptr(w), _ptr(k), _ptr(kbar), _ptr(q_seq), _ptr(q_len), T, H, d,
                                           nseq, L, B, h, kc, topk, _ptr(heads), _ptr(cand), _ptr(idx), _ptr(score),
                                           _stream(stream)))
    return idx, score


def timing_begin(kernel: int, capacity: int = 4096, stream=None):
    """Time the launches of one kernel class on ``stream`` (default: the current stream)."""
    _check("misa_timing_begin", lib().misa_timing_begin(kernel, capacity, _stream(stream)))


def timing_end(stream=None):
    ms = ctypes.c_float(0.0)
    n = ctypes.c_int32(0)
    _check("misa_timing_end", lib().misa_timing_end(_stream(stream), ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)
