"""MI355X-native exact ring attention (gfx950 HIP kernels behind a C ABI).

This package is a thin binding over ``libra.so`` (see ``include/ra.h``):
the functions below only check tensor shapes and dtypes, take raw device
pointers and the current HIP stream from PyTorch, and call the C entry point
of the same name.  All arithmetic runs in the library's kernels; there is no
fallback.  If the library is missing the first call raises.

Tensors are [B, S, H, d] with d contiguous; sequence dimensions are in the
rank-sharded order described in ``include/ra.h``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP = 0, -1, -2, -3
LAYOUTS = {"contiguous": 0, "zigzag": 1, "striped": 2}
MAX_CHUNKS_PER_RANK = 64


def layout_zigzag_k(k: int) -> int:
    """Code of the zig-zag split with k chunks per rank (RA_LAYOUT_ZIGZAG_K)."""
    return 0x100 | int(k)
DTYPE_F32, DTYPE_BF16 = 0, 1

EXPORTS = ("ra_fwd_rank", "ra_fwd_all", "ra_fwd_rank_ws", "ra_fwd_all_ws", "ra_fwd_workspace_bytes",
           "ra_fwd_rank_noalloc",
           "ra_ring_step", "ra_ring_step_ws", "ra_kv_append_rr", "ra_attn_partial_rr", "ra_head_a2a",
           "ra_merge_partials", "ra_attn_partial",
           "ra_layout_gather", "ra_last_error", "ra_version")

_lib = None


class RaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libra status {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libra.so (built in-tree by ``long_context_exact_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m long_context_exact_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.ra_fwd_rank.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i64, i32, i32, i32, i32, i32,
                                  i32, i32, vp]
        L.ra_fwd_all.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i64, i32, i32, i32, i32, i32, i32,
                                 vp]
        L.ra_fwd_rank_ws.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i64, i32, i32, i32, i32,
                                     i32, i32, i32, i32, vp, i64, vp]
        L.ra_fwd_all_ws.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i64, i32, i32, i32, i32,
                                    i32, i32, i32, vp, i64, vp]
        L.ra_fwd_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32, i32, i32, i32, i32, i32]
        L.ra_fwd_rank_noalloc.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i64, i32, i32, i32, i32,
                                          i32, i32, i32, i32, vp]
        L.ra_ring_step.argtypes = [vp, vp, vp, fp, fp, i32, i32, i32, i64, i32, i32, i32, i32, i32,
                                   i32, i32, vp]
        L.ra_ring_step_ws.argtypes = [vp, vp, vp, fp, fp, i32, i32, i32, i64, i32, i32, i32, i32, i32,
                                      i32, i32, i32, vp, i64, vp]
        L.ra_head_a2a.argtypes = [vp, vp, i64, i64, i32, i64, i32, vp]
        L.ra_kv_append_rr.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, i64, i64, i32, vp]
        L.ra_attn_partial_rr.argtypes = [vp, vp, vp, fp, fp, i32, i32, i32, i64, i64, i64, i64, i32,
                                         i32, i32, i32, vp]
        L.ra_fwd_workspace_bytes.restype = ctypes.c_int64
        L.ra_merge_partials.argtypes = [fp, fp, vp, fp, i32, i64, i32, i32, vp]
        L.ra_attn_partial.argtypes = [vp, vp, vp, fp, fp, i32, i32, i32, i64, i64, i32, i32, i32, vp]
        L.ra_layout_gather.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, vp]
        for f in ("ra_fwd_rank", "ra_fwd_all", "ra_fwd_rank_ws", "ra_fwd_all_ws", "ra_fwd_rank_noalloc",
                  "ra_ring_step", "ra_ring_step_ws",
                  "ra_kv_append_rr", "ra_attn_partial_rr", "ra_head_a2a",
                  "ra_merge_partials", "ra_attn_partial", "ra_layout_gather"):
            getattr(L, f).restype = ctypes.c_int
        L.ra_last_error.restype = ctypes.c_char_p
        L.ra_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().ra_last_error().decode()


def _check(rc: int) -> None:
    if rc != RA_OK:
        raise RaError(rc, last_error())


def _torch():
    import torch
    return torch


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _layout(layout) -> int:
    """"contiguous", "zigzag", "striped", "zigzag<k>" (e.g. "zigzag4") or an
    integer code; unknown names raise, unknown codes are left to the library."""
    if not isinstance(layout, str):
        return int(layout)
    if layout in LAYOUTS:
        return LAYOUTS[layout]
    if layout.startswith("zigzag") and layout[6:].isdigit():
        return layout_zigzag_k(int(layout[6:]))
    raise ValueError(f"unknown layout {layout!r}")


def ra_fwd_rank(Q_r, K, V, O_r, LSE_r, P: int, rank: int, causal: bool, layout, stream=None):
    """One simulated rank: Q_r/O_r [B, S/P, Hq, d], K/V [B, S, Hkv, d] (all P
    shards, sharded order), LSE_r [B, Hq, S/P] float32.  O_r may be float32
    or, for bf16 inputs, bfloat16."""
    B, S, Hkv, d = K.shape
    Hq = Q_r.shape[2]
    if tuple(Q_r.shape) != (B, S // P, Hq, d) or O_r.shape != Q_r.shape or V.shape != K.shape:
        raise ValueError("shape mismatch")
    if tuple(LSE_r.shape) != (B, Hq, S // P) or LSE_r.dtype != _torch().float32:
        raise ValueError("LSE_r must be float32 [B, Hq, S/P]")
    dt = _dtype_code(Q_r)
    if not (K.dtype == V.dtype == Q_r.dtype):
        raise TypeError("Q, K, V must share a dtype")
    _check(lib().ra_fwd_rank(_dev(Q_r, "Q_r"), _dev(K, "K"), _dev(V, "V"), _dev(O_r, "O_r"),
                             _dev(LSE_r, "LSE_r"), B, Hq, Hkv, S, d, P, rank, int(bool(causal)),
                             _layout(layout), dt, _dtype_code(O_r), _stream(stream)))


def ra_fwd_all(Q, K, V, O, LSE, P: int, causal: bool, layout, stream=None):
    """All P simulated ranks: Q/O [B, S, Hq, d], K/V [B, S, Hkv, d],
    LSE [B, Hq, S] float32, sharded order.  O may be float32 or, for bf16
    inputs, bfloat16."""
    B, S, Hkv, d = K.shape
    Hq = Q.shape[2]
    if tuple(Q.shape) != (B, S, Hq, d) or O.shape != Q.shape or V.shape != K.shape:
        raise ValueError("shape mismatch")
    if tuple(LSE.shape) != (B, Hq, S) or LSE.dtype != _torch().float32:
        raise ValueError("LSE must be float32 [B, Hq, S]")
    dt = _dtype_code(Q)
    if not (K.dtype == V.dtype == Q.dtype):
        raise TypeError("Q, K, V must share a dtype")
    _check(lib().ra_fwd_all(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(O, "O"),
                            _dev(LSE, "LSE"), B, Hq, Hkv, S, d, P, int(bool(causal)),
                            _layout(layout), dt, _dtype_code(O), _stream(stream)))


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def ra_fwd_workspace_bytes(B: int, Hq: int, Hkv: int, S: int, d: int, P: int, all_ranks: bool,
                           causal: bool, layout, dtype: int, kv_splits: int = 0) -> int:
    """Workspace bytes ra_fwd_rank_ws (all_ranks False) or ra_fwd_all_ws
    (True) needs for kv_splits key ranges (0: the automatic choice)."""
    n = lib().ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, int(bool(all_ranks)), int(bool(causal)),
                                     _layout(layout), int(dtype), int(kv_splits))
    if n < 0:
        raise RaError(int(n), last_error())
    return int(n)


def ra_fwd_rank_ws(Q_r, K, V, O_r, LSE_r, P: int, rank: int, causal: bool, layout,
                   kv_splits: int = 0, workspace=None, stream=None):
    """ra_fwd_rank with key-range splits merged through ``workspace`` (a
    device tensor of at least ra_fwd_workspace_bytes bytes, or None)."""
    B, S, Hkv, d = K.shape
    Hq = Q_r.shape[2]
    if tuple(Q_r.shape) != (B, S // P, Hq, d) or O_r.shape != Q_r.shape or V.shape != K.shape:
        raise ValueError("shape mismatch")
    if tuple(LSE_r.shape) != (B, Hq, S // P) or LSE_r.dtype != _torch().float32:
        raise ValueError("LSE_r must be float32 [B, Hq, S/P]")
    dt = _dtype_code(Q_r)
    if not (K.dtype == V.dtype == Q_r.dtype):
        raise TypeError("Q, K, V must share a dtype")
    wp, wb = _ws(workspace)
    _check(lib().ra_fwd_rank_ws(_dev(Q_r, "Q_r"), _dev(K, "K"), _dev(V, "V"), _dev(O_r, "O_r"),
                                _dev(LSE_r, "LSE_r"), B, Hq, Hkv, S, d, P, rank, int(bool(causal)),
                                _layout(layout), dt, _dtype_code(O_r), int(kv_splits), wp, wb,
                                _stream(stream)))


SCRATCH_BYTES = 128 << 20  # RA_SCRATCH_BYTES: the library's scratch per GPU (ra_fwd_rank_noalloc)


def ra_fwd_rank_noalloc(Q_r, K, V, O_r, LSE_r, P: int, rank: int, causal: bool, layout,
                        kv_splits: int = 0, stream=None):
    """ra_fwd_rank_ws whose key-range partials go to the library's own device
    scratch (SCRATCH_BYTES per GPU): the call allocates nothing.  Calls that
    overlap in time on one GPU share that scratch and must be ordered."""
    B, S, Hkv, d = K.shape
    Hq = Q_r.shape[2]
    if tuple(Q_r.shape) != (B, S // P, Hq, d) or O_r.shape != Q_r.shape or V.shape != K.shape:
        raise ValueError("shape mismatch")
    if tuple(LSE_r.shape) != (B, Hq, S // P) or LSE_r.dtype != _torch().float32:
        raise ValueError("LSE_r must be float32 [B, Hq, S/P]")
    dt = _dtype_code(Q_r)
    if not (K.dtype == V.dtype == Q_r.dtype):
        raise TypeError("Q, K, V must share a dtype")
    _check(lib().ra_fwd_rank_noalloc(_dev(Q_r, "Q_r"), _dev(K, "K"), _dev(V, "V"), _dev(O_r, "O_r"),
                                     _dev(LSE_r, "LSE_r"), B, Hq, Hkv, S, d, P, rank,
                                     int(bool(causal)), _layout(layout), dt, _dtype_code(O_r),
                                     int(kv_splits), _stream(stream)))


def ra_fwd_all_ws(Q, K, V, O, LSE, P: int, causal: bool, layout, kv_splits: int = 0,
                  workspace=None, stream=None):
    """ra_fwd_all with key-range splits merged through ``workspace``."""
    B, S, Hkv, d = K.shape
    Hq = Q.shape[2]
    if tuple(Q.shape) != (B, S, Hq, d) or O.shape != Q.shape or V.shape != K.shape:
        raise ValueError("shape mismatch")
    if tuple(LSE.shape) != (B, Hq, S) or LSE.dtype != _torch().float32:
        raise ValueError("LSE must be float32 [B, Hq, S]")
    dt = _dtype_code(Q)
    if not (K.dtype == V.dtype == Q.dtype):
        raise TypeError("Q, K, V must share a dtype")
    wp, wb = _ws(workspace)
    _check(lib().ra_fwd_all_ws(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(O, "O"),
                               _dev(LSE, "LSE"), B, Hq, Hkv, S, d, P, int(bool(causal)),
                               _layout(layout), dt, _dtype_code(O), int(kv_splits), wp, wb,
                               _stream(stream)))


def _ring_step_args(Q_r, K_blk, V_blk, O_acc, LSE_acc, S, P, rank, t, causal, layout):
    B, n, Hkv, d = K_blk.shape
    Hq = Q_r.shape[2]
    torch = _torch()
    if n * P != S or tuple(Q_r.shape) != (B, n, Hq, d) or V_blk.shape != K_blk.shape:
        raise ValueError("shape mismatch")
    if O_acc.shape != Q_r.shape or O_acc.dtype != torch.float32:
        raise ValueError("O_acc must be float32 [B, S/P, Hq, d]")
    if tuple(LSE_acc.shape) != (B, Hq, n) or LSE_acc.dtype != torch.float32:
        raise ValueError("LSE_acc must be float32 [B, Hq, S/P]")
    if not (K_blk.dtype == V_blk.dtype == Q_r.dtype):
        raise TypeError("Q, K, V must share a dtype")
    return (_dev(Q_r, "Q_r"), _dev(K_blk, "K_blk"), _dev(V_blk, "V_blk"), _dev(O_acc, "O_acc"),
            _dev(LSE_acc, "LSE_acc"), B, Hq, Hkv, S, d, P, rank, t, int(bool(causal)), _layout(layout),
            _dtype_code(Q_r))


def ra_ring_step(Q_r, K_blk, V_blk, O_acc, LSE_acc, S: int, P: int, rank: int, t: int,
                 causal: bool, layout, stream=None):
    """One ring step: fold the block of shard (rank - t) mod P (K_blk, V_blk
    [B, S/P, Hkv, d]) into the running fp32 state O_acc [B, S/P, Hq, d],
    LSE_acc [B, Hq, S/P] of the rank's queries Q_r [B, S/P, Hq, d]."""
    args = _ring_step_args(Q_r, K_blk, V_blk, O_acc, LSE_acc, S, P, rank, t, causal, layout)
    _check(lib().ra_ring_step(*args, _stream(stream)))


def ra_ring_step_ws(Q_r, K_blk, V_blk, O_acc, LSE_acc, S: int, P: int, rank: int, t: int,
                    causal: bool, layout, kv_splits: int = 0, workspace=None, stream=None):
    """ra_ring_step with key-range splits merged, with the running state,
    through ``workspace`` (a device tensor of at least
    ra_fwd_workspace_bytes(..., all_ranks=False, ...) bytes, or None)."""
    args = _ring_step_args(Q_r, K_blk, V_blk, O_acc, LSE_acc, S, P, rank, t, causal, layout)
    wp, wb = _ws(workspace)
    _check(lib().ra_ring_step_ws(*args, int(kv_splits), wp, wb, _stream(stream)))


def ra_kv_append_rr(K_cache, V_cache, K_new, V_new, length: int, block: int, stream=None):
    """Append new tokens' K/V ([B, n_new, Hkv, d]) at positions length ..
    length+n_new-1 to the round-robin shard caches K_cache, V_cache
    [P, B, cap, Hkv, d]."""
    P, B, cap, Hkv, d = K_cache.shape
    if V_cache.shape != K_cache.shape or K_new.shape != V_new.shape:
        raise ValueError("shape mismatch")
    if K_new.shape[0] != B or tuple(K_new.shape[2:]) != (Hkv, d):
        raise ValueError("new K/V must be [B, n_new, Hkv, d]")
    if not (K_cache.dtype == V_cache.dtype == K_new.dtype == V_new.dtype):
        raise TypeError("caches and new rows must share a dtype")
    _check(lib().ra_kv_append_rr(_dev(K_cache, "K_cache"), _dev(V_cache, "V_cache"),
                                 _dev(K_new, "K_new"), _dev(V_new, "V_new"), B, Hkv, d, P, cap,
                                 int(length), K_new.shape[1], int(block), _dtype_code(K_new),
                                 _stream(stream)))


def ra_attn_partial_rr(Q, K_cache, V_cache, O_parts, lse_parts, length: int, block: int,
                       parts_per_shard: int, stream=None):
    """Per-part partials of Q [B, Sq, Hq, d] over the round-robin shard caches
    [P, B, cap, Hkv, d] holding `length` keys: O_parts [P*parts_per_shard,
    B*Sq*Hq, d], lse_parts [P*parts_per_shard, B*Sq*Hq], both float32."""
    P, B, cap, Hkv, d = K_cache.shape
    Sq, Hq = Q.shape[1], Q.shape[2]
    n_parts = P * parts_per_shard
    rows = B * Sq * Hq
    torch = _torch()
    if tuple(Q.shape) != (B, Sq, Hq, d) or V_cache.shape != K_cache.shape:
        raise ValueError("shape mismatch")
    if tuple(O_parts.shape) != (n_parts, rows, d) or tuple(lse_parts.shape) != (n_parts, rows):
        raise ValueError("partials must be [P*parts_per_shard, B*Sq*Hq, (d)]")
    if O_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if not (K_cache.dtype == V_cache.dtype == Q.dtype):
        raise TypeError("Q, K, V must share a dtype")
    _check(lib().ra_attn_partial_rr(_dev(Q, "Q"), _dev(K_cache, "K_cache"), _dev(V_cache, "V_cache"),
                                    _dev(O_parts, "O_parts"), _dev(lse_parts, "lse_parts"), B, Hq,
                                    Hkv, Sq, cap, int(length), int(block), P, int(parts_per_shard),
                                    d, _dtype_code(Q), _stream(stream)))


def ra_head_a2a(src, dst, B: int, S: int, P: int, run_bytes: int, inverse: bool, stream=None):
    """Ulysses all-to-all: src [B, S, P, run] -> dst [P, B, S, run] (inverse:
    back), run = one head group of one token in bytes."""
    nbytes = int(B) * int(S) * int(P) * int(run_bytes)
    for t, name in ((src, "src"), (dst, "dst")):
        if t.numel() * t.element_size() != nbytes:
            raise ValueError(f"{name} must hold B*S*P*run_bytes bytes")
    _check(lib().ra_head_a2a(_dev(src, "src"), _dev(dst, "dst"), int(B), int(S), int(P),
                             int(run_bytes), int(bool(inverse)), _stream(stream)))


def ra_merge_partials(O_parts, lse_parts, O, lse=None, stream=None):
    """O_parts [n_parts, rows, d] fp32, lse_parts [n_parts, rows] fp32 ->
    O [rows, d] (bf16 or fp32), lse [rows] fp32 (optional)."""
    n_parts, rows, d = O_parts.shape
    torch = _torch()
    if O_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if tuple(lse_parts.shape) != (n_parts, rows) or O.numel() != rows * d:
        raise ValueError("shape mismatch")
    lse_ptr = ctypes.c_void_p(0)
    if lse is not None:
        if lse.numel() != rows or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [rows]")
        lse_ptr = _dev(lse, "lse")
    _check(lib().ra_merge_partials(_dev(O_parts, "O_parts"), _dev(lse_parts, "lse_parts"),
                                   _dev(O, "O"), lse_ptr, n_parts, rows, d, _dtype_code(O),
                                   _stream(stream)))


def ra_attn_partial(Q, K, V, O_parts, lse_parts, n_parts: int, stream=None):
    """Q [B, Sq, Hq, d], K/V [B, Skv, Hkv, d] -> O_parts [n_parts, B*Sq*Hq, d]
    and lse_parts [n_parts, B*Sq*Hq] (fp32), keys cut into n_parts parts."""
    B, Sq, Hq, d = Q.shape
    _, Skv, Hkv, _ = K.shape
    rows = B * Sq * Hq
    if tuple(O_parts.shape) != (n_parts, rows, d) or tuple(lse_parts.shape) != (n_parts, rows):
        raise ValueError("partials shape mismatch")
    if not (K.dtype == V.dtype == Q.dtype):
        raise TypeError("Q, K, V must share a dtype")
    _check(lib().ra_attn_partial(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"),
                                 _dev(O_parts, "O_parts"), _dev(lse_parts, "lse_parts"), B, Hq, Hkv,
                                 Sq, Skv, d, n_parts, _dtype_code(Q), _stream(stream)))


def ra_layout_gather(src, dst, S: int, P: int, layout, inverse: bool, outer: int | None = None,
                     stream=None):
    """Natural <-> sharded order of a tensor viewed as [outer, S, inner]."""
    if src.shape != dst.shape or src.dtype != dst.dtype:
        raise ValueError("src and dst must match")
    nbytes = src.numel() * src.element_size()
    if outer is None:
        outer = src.shape[0]
    inner = nbytes // (outer * S)
    if outer * S * inner != nbytes:
        raise ValueError("tensor does not view as [outer, S, inner]")
    _check(lib().ra_layout_gather(_dev(src, "src"), _dev(dst, "dst"), outer, S, inner, P,
                                  _layout(layout), int(bool(inverse)), _stream(stream)))


def version() -> str:
    return lib().ra_version().decode()
