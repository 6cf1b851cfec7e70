"""Thin Python binding of libfocus.so (the C ABI in include/focus.h).

Argument marshalling only: shapes are read from torch tensors, outputs and workspaces are
allocated with torch on the tensors' device, and every call goes straight to the library on the
current HIP stream.  No step of the computation runs here.  If the library has not been built,
importing this module raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# FOCUS_LIBRARY may name another build of the same library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("FOCUS_LIBRARY") or os.path.join(_PKG, "libfocus.so")

FOCUS_OK = 0
FOCUS_ERR_INVALID_ARG = -1
FOCUS_ERR_UNSUPPORTED = -2
FOCUS_ERR_WORKSPACE = -3
FOCUS_ERR_HIP = -4
FOCUS_F32 = 0
FOCUS_BF16 = 1
FOCUS_KV_HEAD_MAJOR = 0
FOCUS_KV_TOKEN_MAJOR = 1

_c_void_p, _c_int, _c_float, _c_size_t = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_c_int64 = ctypes.c_int64

# name -> (restype, argtypes), mirroring include/focus.h
SIGNATURES = {
    "focus_status_string": (ctypes.c_char_p, [_c_int]),
    "focus_version": (_c_int, []),
    "focus_score_l01_workspace_size": (_c_size_t, [_c_int] * 5),
    "focus_score_l01": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 + [_c_float, _c_void_p, _c_void_p,
                                                                  _c_size_t, _c_void_p]),
    "focus_score_l01_lse": (_c_int, [_c_void_p] * 6 + [_c_int] * 6 + [_c_float, _c_void_p,
                                                                      _c_void_p, _c_size_t,
                                                                      _c_void_p]),
    "focus_select_budget": (_c_int, [_c_void_p] * 3 + [_c_int, _c_float, _c_int, _c_int, _c_int,
                                                       _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "focus_compact": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_int64, _c_int, _c_void_p,
                               _c_void_p, _c_void_p, _c_void_p]),
    "focus_ragged_paged_attn_workspace_size": (_c_size_t, [_c_int] * 8),
    "focus_ragged_paged_attn": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                         _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                         _c_void_p] + [_c_int] * 7 + [_c_float, _c_void_p,
                                                                      _c_void_p, _c_void_p,
                                                                      _c_size_t, _c_void_p]),
    "focus_ragged_paged_attn_pos": (_c_int, [_c_void_p] * 3 + [_c_int, _c_void_p, _c_void_p,
                                             _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                             _c_void_p] + [_c_int] * 7 + [_c_float, _c_void_p,
                                                                          _c_void_p, _c_void_p,
                                                                          _c_size_t, _c_void_p]),
    "focus_score_select": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 + [_c_float, _c_void_p,
                                                                  _c_void_p, _c_int, _c_float,
                                                                  _c_int, _c_int, _c_void_p,
                                                                  _c_void_p, _c_void_p,
                                                                  _c_void_p, _c_size_t,
                                                                  _c_void_p]),
    "focus_compact_multi": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                     _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "focus_score_select_compact": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 +
                                   [_c_float] + [_c_void_p] * 5 + [_c_int] +
                                   [_c_void_p] * 3 + [_c_int] + [_c_void_p] * 2 + [_c_int] +
                                   [_c_void_p, _c_size_t, _c_void_p]),
    "focus_noalloc_scratch_bytes": (_c_size_t, []),
    "focus_score_select_compact_noalloc": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 +
                                           [_c_float] + [_c_void_p] * 5 + [_c_int] +
                                           [_c_void_p] * 3 + [_c_int] + [_c_void_p] * 2 +
                                           [_c_int, _c_void_p]),
    "focus_kv_writeback": (_c_int, [_c_void_p] * 4 + [_c_int] * 5 + [_c_void_p] * 3),
    "focus_block_commit": (_c_int, [_c_void_p] * 3 + [_c_int] * 5 + [_c_void_p] * 2 +
                           [_c_int, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_int,
                            _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "focus_kv_pack": (_c_int, [_c_void_p] * 2 + [_c_int] * 5 + [_c_void_p] * 3),
}


class FocusError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or `python -m decodability_aware_token_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_string(code: int) -> str:
    return lib().focus_status_string(int(code)).decode()


def _check(fn: str, code: int):
    if code != FOCUS_OK:
        raise FocusError(fn, code)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors handed to libfocus must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Tuple[Optional[torch.Tensor], int]:
    """A caller's workspace, or a new zero-filled one (the attention needs zeros on first use)."""
    if nbytes == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ------------------------------------------------------------------------------------------
def score_l01(q0, k0, q1, k1, sm_scale: float, delta=None, workspace=None) -> torch.Tensor:
    """delta [B, blk] f32 = layer-1 minus layer-0 importance (see focus_score_l01)."""
    B, blk, Hq, d = q0.shape
    Hkv = k0.shape[2]
    dt = {torch.float32: FOCUS_F32, torch.bfloat16: FOCUS_BF16}[q0.dtype]
    if delta is None:
        delta = torch.empty((B, blk), dtype=torch.float32, device=q0.device)
    need = lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d)
    workspace, wsb = _workspace(need, q0.device, workspace)
    rc = lib().focus_score_l01(_ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), dt, B, blk, Hq, Hkv, d,
                               float(sm_scale), _ptr(delta), _ptr(workspace), wsb,
                               _stream(q0.device))
    _check("focus_score_l01", rc)
    return delta


def score_l01_lse(q0, k0, q1, k1, lse0, lse1, sm_scale: float, delta=None,
                  workspace=None) -> torch.Tensor:
    """delta [B, blk] f32 over the full attention domain, given each block query's log-sum-exp
    over prefix + block keys per layer, lse_l [B, blk, Hq] f32 (see focus_score_l01_lse)."""
    B, blk, Hq, d = q0.shape
    Hkv = k0.shape[2]
    dt = {torch.float32: FOCUS_F32, torch.bfloat16: FOCUS_BF16}[q0.dtype]
    if delta is None:
        delta = torch.empty((B, blk), dtype=torch.float32, device=q0.device)
    need = lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d)
    workspace, wsb = _workspace(need, q0.device, workspace)
    rc = lib().focus_score_l01_lse(_ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), _ptr(lse0),
                                   _ptr(lse1), dt, B, blk, Hq, Hkv, d, float(sm_scale),
                                   _ptr(delta), _ptr(workspace), wsb, _stream(q0.device))
    _check("focus_score_l01_lse", rc)
    return delta


def select_budget(delta, masked, budget=None, adaptive=None, keep=None, kept_count=None):
    """keep [B, blk] u8, kept_count [B] i32 (see focus_select_budget).

    ``adaptive`` is None (use ``budget``) or a tuple (beta, lo, hi)."""
    B, blk = delta.shape
    if keep is None:
        keep = torch.empty((B, blk), dtype=torch.uint8, device=delta.device)
    if kept_count is None:
        kept_count = torch.empty(B, dtype=torch.int32, device=delta.device)
    beta, lo, hi = adaptive if adaptive is not None else (0.0, 0, 0)
    rc = lib().focus_select_budget(_ptr(delta), _ptr(masked), _ptr(budget),
                                   1 if adaptive is not None else 0, float(beta), int(lo), int(hi),
                                   B, blk, _ptr(keep), _ptr(kept_count), _stream(delta.device))
    _check("focus_select_budget", rc)
    return keep, kept_count


def compact(keep, rows=None, cap: Optional[int] = None, offsets=None, kept_pos=None,
            gathered=None, with_pos: bool = True):
    """offsets [B+1], kept_pos [cap], gathered [cap, *row] (see focus_compact)."""
    B, blk = keep.shape
    dev = keep.device
    if cap is None:
        cap = B * blk
    if offsets is None:
        offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if kept_pos is None and with_pos:
        kept_pos = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    row_bytes = 0
    if rows is not None:
        row_shape = rows.shape[2:]
        row_bytes = rows[0, 0].numel() * rows.element_size()
        if gathered is None:
            gathered = torch.empty((max(cap, 1),) + tuple(row_shape), dtype=rows.dtype, device=dev)
    rc = lib().focus_compact(_ptr(keep), B, blk, _ptr(rows), row_bytes, int(cap), _ptr(offsets),
                             _ptr(kept_pos), _ptr(gathered), _stream(dev))
    _check("focus_compact", rc)
    return offsets, kept_pos, gathered


def attn_workspace_bytes(B, blk, Hq, Hkv, d, S, max_pages, max_kept) -> int:
    return int(lib().focus_ragged_paged_attn_workspace_size(B, blk, Hq, Hkv, d, S, max_pages,
                                                            max_kept))


def ragged_paged_attn(q, offsets, k_cache, v_cache, page_table, prefix_len, k_blk, v_blk,
                      max_kept: int, sm_scale: float, out=None, lse=None, want_lse=True,
                      workspace=None, want_out=True):
    """out [cap, Hq, d] bf16, lse [cap, Hq] f32 (see focus_ragged_paged_attn); want_out=False:
    log-sum-exp only (out is None; v_cache and v_blk may be None).

    q [cap, Hq, d]; k_cache [pages, Hkv, d/8, S, 8]; v_cache [pages, Hkv, S/8, d, 8];
    k_blk [B, Hkv, d/8, blk, 8]; v_blk [B, Hkv, blk/8, d, 8]; page_table [B, max_pages]."""
    cap, Hq, d = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    S = k_cache.shape[3]
    B, max_pages = page_table.shape
    blk = k_blk.shape[3]
    dev = q.device
    if not want_out:
        out, want_lse = None, True
    elif out is None:
        out = torch.empty((cap, Hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((cap, Hq), dtype=torch.float32, device=dev)
    need = attn_workspace_bytes(B, blk, Hq, Hkv, d, S, max_pages, max_kept)
    workspace, wsb = _workspace(need, dev, workspace)
    rc = lib().focus_ragged_paged_attn(_ptr(q), _ptr(offsets), cap, _ptr(k_cache), _ptr(v_cache),
                                       num_pages, _ptr(page_table), max_pages, _ptr(prefix_len),
                                       _ptr(k_blk), _ptr(v_blk), B, blk, Hq, Hkv, d, S,
                                       int(max_kept), float(sm_scale), _ptr(out), _ptr(lse),
                                       _ptr(workspace), wsb, _stream(dev))
    _check("focus_ragged_paged_attn", rc)
    return out, lse


def ragged_paged_attn_pos(q_block, kept_pos, offsets, k_cache, v_cache, page_table, prefix_len,
                          k_blk, v_blk, max_kept: int, sm_scale: float, out=None, lse=None,
                          want_lse=True, workspace=None):
    """ragged_paged_attn with the queries read in place (see focus_ragged_paged_attn_pos):
    q_block [B, blk, Hq, d] bf16 and kept_pos [cap] i32; out [cap, Hq, d], lse [cap, Hq]."""
    B, blk, Hq, d = q_block.shape
    cap = kept_pos.shape[0]
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    S = k_cache.shape[3]
    max_pages = page_table.shape[1]
    if page_table.shape[0] != B or prefix_len.shape[0] != B or k_blk.shape[0] != B or \
            k_blk.shape[3] != blk:
        raise ValueError("q_block, page_table, prefix_len and k_blk disagree on B or blk")
    dev = q_block.device
    if out is None:
        out = torch.empty((cap, Hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((cap, Hq), dtype=torch.float32, device=dev)
    need = attn_workspace_bytes(B, blk, Hq, Hkv, d, S, max_pages, max_kept)
    workspace, wsb = _workspace(need, dev, workspace)
    rc = lib().focus_ragged_paged_attn_pos(
        _ptr(q_block), _ptr(kept_pos), _ptr(offsets), cap, _ptr(k_cache), _ptr(v_cache),
        num_pages, _ptr(page_table), max_pages, _ptr(prefix_len), _ptr(k_blk), _ptr(v_blk), B, blk,
        Hq, Hkv, d, S, int(max_kept), float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
        _stream(dev))
    _check("focus_ragged_paged_attn_pos", rc)
    return out, lse


def kv_writeback(k_rows, v_rows, offsets, kept_pos, k_blk, v_blk):
    """Scatter the kept rows' K/V [cap, Hkv, d] into k_blk/v_blk in place (see
    focus_kv_writeback)."""
    cap, Hkv, d = k_rows.shape
    B, blk = k_blk.shape[0], k_blk.shape[3]
    rc = lib().focus_kv_writeback(_ptr(k_rows), _ptr(v_rows), _ptr(offsets), _ptr(kept_pos),
                                  cap, B, blk, Hkv, d, _ptr(k_blk), _ptr(v_blk),
                                  _stream(k_rows.device))
    _check("focus_kv_writeback", rc)


def kv_pack(k_src=None, v_src=None, token_major: bool = False, k_out=None, v_out=None):
    """K/V stored as plain token rows -> the library's layouts (see focus_kv_pack).

    k_src, v_src: bf16 [n, Hkv, S, d] (token_major=False) or [n, S, Hkv, d] (token_major=True);
    either may be None.  Returns (k_out [n, Hkv, d/8, S, 8], v_out [n, Hkv, S/8, d, 8]), the
    missing one as None; outputs are allocated unless given."""
    src = k_src if k_src is not None else v_src
    if src is None:
        raise ValueError("kv_pack needs k_src or v_src")
    n = src.shape[0]
    S, Hkv = (src.shape[1], src.shape[2]) if token_major else (src.shape[2], src.shape[1])
    d = src.shape[3]
    dev = src.device
    for x in (k_src, v_src):
        if x is not None and tuple(x.shape) != tuple(src.shape):
            raise ValueError("k_src and v_src must have the same shape")
    if k_src is not None and k_out is None:
        k_out = torch.empty((n, Hkv, d // 8, S, 8), dtype=torch.bfloat16, device=dev)
    if v_src is not None and v_out is None:
        v_out = torch.empty((n, Hkv, S // 8, d, 8), dtype=torch.bfloat16, device=dev)
    if k_src is not None and k_out.numel() != src.numel():
        raise ValueError("k_out must hold n * Hkv * S * d elements")
    if v_src is not None and v_out.numel() != src.numel():
        raise ValueError("v_out must hold n * Hkv * S * d elements")
    layout = FOCUS_KV_TOKEN_MAJOR if token_major else FOCUS_KV_HEAD_MAJOR
    rc = lib().focus_kv_pack(_ptr(k_src) if k_src is not None else None,
                             _ptr(v_src) if v_src is not None else None, layout, n, Hkv, S, d,
                             _ptr(k_out) if k_src is not None else None,
                             _ptr(v_out) if v_src is not None else None, _stream(dev))
    _check("focus_kv_pack", rc)
    return (k_out if k_src is not None else None), (v_out if v_src is not None else None)


def block_commit(commit, k_blk, v_blk, k_cache, v_cache, page_table, prefix_len_in,
                 prefix_len_out, free_pages, free_count_in, free_count_out, status):
    """Append committed requests' blocks to their paged prefix (see focus_block_commit); the
    cache, page table and the *_out / status tensors are updated in place."""
    B, Hkv = k_blk.shape[0], k_blk.shape[1]
    d, blk = k_blk.shape[2] * 8, k_blk.shape[3]
    num_pages, S = k_cache.shape[0], k_cache.shape[3]
    max_pages = page_table.shape[1]
    rc = lib().focus_block_commit(_ptr(commit), _ptr(k_blk), _ptr(v_blk), B, blk, Hkv, d, S,
                                  _ptr(k_cache), _ptr(v_cache), num_pages, _ptr(page_table),
                                  max_pages, _ptr(prefix_len_in), _ptr(prefix_len_out),
                                  _ptr(free_pages), free_pages.numel(), _ptr(free_count_in),
                                  _ptr(free_count_out), _ptr(status), _stream(k_blk.device))
    _check("focus_block_commit", rc)


def score_select(q0, k0, q1, k1, sm_scale: float, masked, budget=None, adaptive=None, delta=None,
                 keep=None, kept_count=None, workspace=None):
    """delta, keep, kept_count of focus_score_l01 followed by focus_select_budget, in one launch
    (see focus_score_select)."""
    B, blk, Hq, d = q0.shape
    Hkv = k0.shape[2]
    dev = q0.device
    dt = {torch.float32: FOCUS_F32, torch.bfloat16: FOCUS_BF16}[q0.dtype]
    if delta is None:
        delta = torch.empty((B, blk), dtype=torch.float32, device=dev)
    if keep is None:
        keep = torch.empty((B, blk), dtype=torch.uint8, device=dev)
    if kept_count is None:
        kept_count = torch.empty(B, dtype=torch.int32, device=dev)
    ad, beta, lo, hi = (0, 0.0, 0, 0) if adaptive is None else (1,) + tuple(adaptive)
    need = lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d)
    workspace, wsb = _workspace(need, dev, workspace)
    rc = lib().focus_score_select(_ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), dt, B, blk, Hq, Hkv, d,
                                  float(sm_scale), _ptr(masked), _ptr(budget), ad, float(beta),
                                  int(lo), int(hi), _ptr(delta), _ptr(keep), _ptr(kept_count),
                                  _ptr(workspace), wsb, _stream(dev))
    _check("focus_score_select", rc)
    return delta, keep, kept_count


def _row_set_arrays(row_sets, gathered):
    if not all(t.is_contiguous() for t in list(row_sets) + list(gathered)):
        raise ValueError("tensors handed to libfocus must be contiguous")
    n = len(row_sets)
    rows_arr = (_c_void_p * max(n, 1))(*[r.data_ptr() for r in row_sets])
    bytes_arr = (_c_int64 * max(n, 1))(*[r[0, 0].numel() * r.element_size() for r in row_sets])
    out_arr = (_c_void_p * max(n, 1))(*[g.data_ptr() for g in gathered])
    return rows_arr, bytes_arr, out_arr


def score_select_compact(q0, k0, q1, k1, sm_scale: float, masked, budget, row_sets, cap: int,
                         max_kept=None, delta=None, keep=None, kept_count=None, offsets=None,
                         kept_pos=None, gathered=None, workspace=None, noalloc=False):
    """delta, keep, kept_count, offsets, kept_pos and the gathered row sets of
    focus_score_select with per-request budgets followed by focus_compact_multi, in two launches
    (see focus_score_select_compact).  noalloc=True calls focus_score_select_compact_noalloc,
    which keeps its partials in the library's own device array (no workspace); the output
    tensors are then best passed in, so that nothing is allocated here either."""
    B, blk, Hq, d = q0.shape
    Hkv = k0.shape[2]
    dev = q0.device
    dt = {torch.float32: FOCUS_F32, torch.bfloat16: FOCUS_BF16}[q0.dtype]
    if delta is None:
        delta = torch.empty((B, blk), dtype=torch.float32, device=dev)
    if keep is None:
        keep = torch.empty((B, blk), dtype=torch.uint8, device=dev)
    if kept_count is None:
        kept_count = torch.empty(B, dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if kept_pos is None:
        kept_pos = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if gathered is None:
        gathered = [torch.empty((max(cap, 1),) + tuple(r.shape[2:]), dtype=r.dtype, device=dev)
                    for r in row_sets]
    rows_arr, bytes_arr, out_arr = _row_set_arrays(row_sets, gathered)
    if noalloc:
        rc = lib().focus_score_select_compact_noalloc(
            _ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), dt, B, blk, Hq, Hkv, d, float(sm_scale),
            _ptr(masked), _ptr(budget), _ptr(delta), _ptr(keep), _ptr(kept_count),
            len(row_sets), rows_arr, bytes_arr, out_arr, int(cap), _ptr(offsets),
            _ptr(kept_pos), int(blk if max_kept is None else max_kept), _stream(dev))
        _check("focus_score_select_compact_noalloc", rc)
        return delta, keep, kept_count, offsets, kept_pos, gathered
    need = lib().focus_score_l01_workspace_size(B, blk, Hq, Hkv, d)
    workspace, wsb = _workspace(need, dev, workspace)
    rc = lib().focus_score_select_compact(
        _ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), dt, B, blk, Hq, Hkv, d, float(sm_scale),
        _ptr(masked), _ptr(budget), _ptr(delta), _ptr(keep), _ptr(kept_count), len(row_sets),
        rows_arr, bytes_arr, out_arr, int(cap), _ptr(offsets), _ptr(kept_pos),
        int(blk if max_kept is None else max_kept), _ptr(workspace), wsb, _stream(dev))
    _check("focus_score_select_compact", rc)
    return delta, keep, kept_count, offsets, kept_pos, gathered


def compact_multi(keep, row_sets, cap: int, offsets=None, kept_pos=None, gathered=None):
    """offsets, kept_pos and one gathered tensor per row set [B, blk, ...] (see
    focus_compact_multi); ``gathered`` optionally gives the output tensors."""
    B, blk = keep.shape
    dev = keep.device
    n = len(row_sets)
    if offsets is None:
        offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if kept_pos is None:
        kept_pos = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if gathered is None:
        gathered = [torch.empty((max(cap, 1),) + tuple(r.shape[2:]), dtype=r.dtype, device=dev)
                    for r in row_sets]
    rows_arr, bytes_arr, out_arr = _row_set_arrays(row_sets, gathered)
    rc = lib().focus_compact_multi(_ptr(keep), B, blk, n, rows_arr, bytes_arr, out_arr, int(cap),
                                   _ptr(offsets), _ptr(kept_pos), _stream(dev))
    _check("focus_compact_multi", rc)
    return offsets, kept_pos, gathered
