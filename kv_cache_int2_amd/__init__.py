"""Python binding of the MI355X OSCAR INT2 KV-cache library (include/oscar.h).

Argument marshalling only: every step of the hot path runs in the HIP library
(``libkv_cache_int2_amd.so``).  Device buffers are torch tensors (torch is used
for device memory and streams); host buffers of ``oscar_calibrate`` are numpy
arrays.  Functions keep the C names; a non-zero status raises ``OscarError``.
bf16 / fp16 buffers may be ``torch.bfloat16``, ``torch.int16`` or ``torch.uint16``
tensors holding the bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from ._lib import OscarShape, lib

__all__ = [
    "OscarError", "OscarShape", "make_shape", "oscar_calibrate", "oscar_quantize_append",
    "oscar_decode_workspace_bytes", "oscar_decode_attn", "oscar_bf16_append",
    "oscar_bf16_decode_attn", "oscar_hbm_copy", "oscar_hbm_read", "oscar_gpu_wait", "Event",
    "oscar_quantize_append_timed", "oscar_decode_attn_timed", "oscar_bf16_decode_attn_timed",
    "oscar_decode_step", "oscar_decode_step_timed",
    "oscar_strerror", "BLOCK_BYTES", "BF16_BLOCK_ELEMS", "PAGE_SIZE", "HEAD_DIM", "block_bytes",
    "oscar_calibrate_layers", "oscar_rotation_file_bytes", "oscar_rotation_write", "oscar_rotation_read_info",
    "oscar_rotation_read", "oscar_quantize_append_layers", "oscar_decode_layers_workspace_bytes",
    "oscar_decode_attn_layers", "oscar_decode_attn_noalloc", "oscar_decode_noalloc_scratch_bytes",
    "NOALLOC_SCRATCH_BYTES",
]

BLOCK_BYTES = 1152  # bytes per (page, KV head) block at group size 128
BF16_BLOCK_ELEMS = 4096  # bf16 comparator pool: K [16][128] then V^T [128][16] per (page, KV head)
PAGE_SIZE = 16
HEAD_DIM = 128
NOALLOC_SCRATCH_BYTES = 32 << 20  # the library's static decode scratch per device


class OscarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {lib.oscar_strerror(status).decode()} (status {status})")
        self.status = status


def make_shape(n_q_heads: int, n_kv_heads: int, window: int = 128, head_dim: int = 128,
               group_size: int = 128, page_size: int = 16, n_sink: int = 0) -> OscarShape:
    return OscarShape(n_q_heads, n_kv_heads, head_dim, group_size, page_size, window, n_sink)


def block_bytes(group_size: int = 128) -> int:
    """Bytes per (page, KV head) block of the INT2 pool: 1024 of codes plus one
    8-byte record per token and quantisation group (1152, 1280, 1536 for
    groups of 128, 64, 32 channels)."""
    return 1024 + 8 * PAGE_SIZE * (HEAD_DIM // group_size)


_SHAPES_SEEN: set = set()


def _want(t, dims, name):
    """t must be a tensor/array of len(dims) dimensions; an int entry of dims
    fixes that dimension, a (">=", n) entry bounds it from below, None leaves it
    free.  Raises ValueError otherwise.  (Shapes already accepted against the
    same dims are remembered, so a serving loop pays one set look-up.)"""
    if t is None:
        raise ValueError(f"{name}: missing")
    key = (tuple(t.shape), dims)
    if key in _SHAPES_SEEN:
        return
    shape = key[0]
    ok = len(shape) == len(dims)
    if ok:
        for have, want in zip(shape, dims):
            if want is None:
                continue
            if isinstance(want, tuple):
                if have < want[1]:
                    ok = False
            elif have != want:
                ok = False
    if not ok:
        txt = ", ".join("*" if w is None else (f">={w[1]}" if isinstance(w, tuple) else str(w)) for w in dims)
        raise ValueError(f"{name}: shape {list(shape)}, expected [{txt}]")
    if len(_SHAPES_SEEN) < 4096:
        _SHAPES_SEEN.add(key)


def _ring_rows(shape) -> int:
    return int(shape.window) + int(shape.n_sink)


def _check_rings(shape, win_k, win_v, batch, lead=()):
    """bf16 rings [*lead][>= batch][W + n_sink][Hkv][128], required when W + n_sink > 0."""
    if _ring_rows(shape) == 0:
        return
    for name, w in (("win_k", win_k), ("win_v", win_v)):
        _want(w, (*lead, (">=", batch), _ring_rows(shape), shape.n_kv_heads, HEAD_DIM), name)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise OscarError(fn, status)


def _dev(t, dtypes, name):
    """Device pointer of a contiguous torch tensor (None -> NULL)."""
    if t is None:
        return None
    try:
        if t.is_cuda and t.dtype in dtypes and t.is_contiguous():
            return t.data_ptr()
    except AttributeError:
        raise TypeError(f"{name}: expected a torch tensor") from None
    if not t.is_cuda:
        raise ValueError(f"{name}: must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {sorted(str(d) for d in dtypes)}")
    raise ValueError(f"{name}: must be contiguous")


_DTYPES = None


def _dt():
    """(bf16-like, int32, uint8, float32) dtype sets accepted for the buffers."""
    global _DTYPES
    if _DTYPES is None:
        import torch

        _DTYPES = (frozenset((torch.bfloat16, torch.int16, torch.uint16, torch.float16)),
                   frozenset((torch.int32,)), frozenset((torch.uint8,)), frozenset((torch.float32,)))
    return _DTYPES


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def oscar_calibrate(shape: OscarShape, q_cal: np.ndarray, k_cal: np.ndarray, v_cal: np.ndarray):
    """Host calibration.  q_cal float32 [Hkv][n_q][128]; k_cal, v_cal float32
    [Hkv][n_kv][128].  Returns (r_k, r_v) uint16 [Hkv][128][128] bf16 bits and
    (eig_k, eig_v) float64 [Hkv][128]."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    k = np.ascontiguousarray(k_cal, dtype=np.float32)
    v = np.ascontiguousarray(v_cal, dtype=np.float32)
    hkv = shape.n_kv_heads
    if (q.ndim != 3 or k.shape != v.shape or k.ndim != 3 or q.shape[0] != hkv or k.shape[0] != hkv
            or q.shape[2] != HEAD_DIM or k.shape[2] != HEAD_DIM):
        raise ValueError("calibration arrays must be [Hkv][n][128]")
    rk = np.empty((hkv, 128, 128), np.uint16)
    rv = np.empty_like(rk)
    ek = np.empty((hkv, 128), np.float64)
    ev = np.empty_like(ek)
    _check("oscar_calibrate", lib.oscar_calibrate(
        C.byref(shape), q.ctypes.data, q.shape[1], k.ctypes.data, v.ctypes.data, k.shape[1],
        rk.ctypes.data, rv.ctypes.data, ek.ctypes.data, ev.ctypes.data))
    return rk, rv, ek, ev


def oscar_calibrate_layers(shape: OscarShape, q_cal: np.ndarray, k_cal: np.ndarray, v_cal: np.ndarray):
    """Host calibration of every layer at once.  q_cal float32 [L][Hkv][n_q][128];
    k_cal, v_cal float32 [L][Hkv][n_kv][128].  Returns (r_k, r_v) uint16
    [L][Hkv][128][128] and (eig_k, eig_v) float64 [L][Hkv][128]."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    k = np.ascontiguousarray(k_cal, dtype=np.float32)
    v = np.ascontiguousarray(v_cal, dtype=np.float32)
    hkv = shape.n_kv_heads
    if (q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[:2] != k.shape[:2] or q.shape[1] != hkv
            or q.shape[3] != HEAD_DIM or k.shape[3] != HEAD_DIM):
        raise ValueError("calibration arrays must be [L][Hkv][n][128]")
    n_layers = q.shape[0]
    rk = np.empty((n_layers, hkv, 128, 128), np.uint16)
    rv = np.empty_like(rk)
    ek = np.empty((n_layers, hkv, 128), np.float64)
    ev = np.empty_like(ek)
    _check("oscar_calibrate_layers", lib.oscar_calibrate_layers(
        C.byref(shape), n_layers, q.ctypes.data, q.shape[2], k.ctypes.data, v.ctypes.data, k.shape[2],
        rk.ctypes.data, rv.ctypes.data, ek.ctypes.data, ev.ctypes.data))
    return rk, rv, ek, ev


def oscar_rotation_file_bytes(n_layers: int, n_kv_heads: int, with_eigenvalues: bool = True) -> int:
    return int(lib.oscar_rotation_file_bytes(int(n_layers), int(n_kv_heads), int(bool(with_eigenvalues))))


def oscar_rotation_write(path: str, shape: OscarShape, r_k: np.ndarray, r_v: np.ndarray,
                         eig_k: np.ndarray | None = None, eig_v: np.ndarray | None = None) -> None:
    """Write rotations uint16 [L][Hkv][128][128] (and eigenvalues float64
    [L][Hkv][128], optional) to a rotation file."""
    rk = np.ascontiguousarray(r_k, dtype=np.uint16)
    rv = np.ascontiguousarray(r_v, dtype=np.uint16)
    if rk.ndim != 4 or rk.shape != rv.shape or rk.shape[1:] != (shape.n_kv_heads, 128, 128):
        raise ValueError("rotations must be [L][Hkv][128][128]")
    ek = None if eig_k is None else np.ascontiguousarray(eig_k, dtype=np.float64)
    ev = None if eig_v is None else np.ascontiguousarray(eig_v, dtype=np.float64)
    for e in (ek, ev):
        if e is not None and e.shape != rk.shape[:3]:
            raise ValueError("eigenvalues must be [L][Hkv][128]")
    _check("oscar_rotation_write", lib.oscar_rotation_write(
        os.fsencode(path), C.byref(shape), rk.shape[0], rk.ctypes.data, rv.ctypes.data,
        None if ek is None else ek.ctypes.data, None if ev is None else ev.ctypes.data))


def oscar_rotation_read_info(path: str) -> dict:
    """Header of a rotation file: n_layers, n_kv_heads, group_size, has_eigenvalues."""
    vals = [C.c_int32() for _ in range(4)]
    _check("oscar_rotation_read_info", lib.oscar_rotation_read_info(os.fsencode(path), *[C.byref(x) for x in vals]))
    return dict(zip(("n_layers", "n_kv_heads", "group_size", "has_eigenvalues"), (int(x.value) for x in vals)))


def oscar_rotation_read(path: str, shape: OscarShape, n_layers: int, eigenvalues: bool = False):
    """Rotations (r_k, r_v) uint16 [L][Hkv][128][128] of a rotation file whose
    header matches shape and n_layers; with ``eigenvalues`` also (eig_k, eig_v)."""
    hkv = shape.n_kv_heads
    rk = np.empty((n_layers, hkv, 128, 128), np.uint16)
    rv = np.empty_like(rk)
    ek = np.empty((n_layers, hkv, 128), np.float64) if eigenvalues else None
    ev = np.empty_like(ek) if eigenvalues else None
    _check("oscar_rotation_read", lib.oscar_rotation_read(
        os.fsencode(path), C.byref(shape), int(n_layers), rk.ctypes.data, rv.ctypes.data,
        None if ek is None else ek.ctypes.data, None if ev is None else ev.ctypes.data))
    return (rk, rv, ek, ev) if eigenvalues else (rk, rv)


def _append_checks(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after, pool, win_k, win_v,
                   lead=()):
    hkv = shape.n_kv_heads
    _want(r_k, (*lead, hkv, HEAD_DIM, HEAD_DIM), "r_k")
    _want(r_v, (*lead, hkv, HEAD_DIM, HEAD_DIM), "r_v")
    _want(k_new, (*lead, None, hkv, HEAD_DIM), "k_new")
    n_tokens = int(k_new.shape[len(lead)])
    _want(v_new, (*lead, n_tokens, hkv, HEAD_DIM), "v_new")
    _want(seq_idx, (n_tokens,), "seq_idx")
    _want(pos, (n_tokens,), "pos")
    _want(block_table, (None, None), "block_table")
    batch = int(block_table.shape[0])
    _want(seq_len_after, (batch,), "seq_len_after")
    _want(pool, (*lead, None, hkv, block_bytes(shape.group_size)), "pool")
    if n_tokens > 0:  # an empty append touches nothing
        _check_rings(shape, win_k, win_v, batch, lead)
    return n_tokens, batch


def _append_args(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after, pool, win_k, win_v,
                 stream):
    b16, i32, u8, _ = _dt()
    n_tokens, batch = _append_checks(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
                                     pool, win_k, win_v)
    return (C.byref(shape), _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(k_new, b16, "k_new"),
            _dev(v_new, b16, "v_new"), n_tokens, _dev(seq_idx, i32, "seq_idx"), _dev(pos, i32, "pos"), batch,
            _dev(block_table, i32, "block_table"), int(block_table.shape[1]),
            _dev(seq_len_after, i32, "seq_len_after"), _dev(pool, u8, "pool"), int(pool.shape[0]),
            _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"), _stream(stream))


def oscar_quantize_append(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
                          pool, win_k=None, win_v=None, stream=None) -> None:
    _check("oscar_quantize_append", lib.oscar_quantize_append(
        *_append_args(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after, pool, win_k, win_v,
                      stream)))


def oscar_quantize_append_timed(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
                                pool, win_k, win_v, start, stop, stream=None) -> None:
    """oscar_quantize_append with the Event pair (start, stop) attached to the
    append kernel's dispatch."""
    _check("oscar_quantize_append_timed", lib.oscar_quantize_append_timed(
        *_append_args(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after, pool, win_k, win_v,
                      stream), start.handle, stop.handle))


def oscar_decode_workspace_bytes(shape, batch: int, max_seq_len: int) -> int:
    n = lib.oscar_decode_workspace_bytes(C.byref(shape), int(batch), int(max_seq_len))
    if n == 0:
        raise OscarError("oscar_decode_workspace_bytes", -1)
    return int(n)


def _decode_checks(shape, r_k, r_v, q, seq_lens, block_table, pool, win_k, win_v, out, lead=()):
    hkv, hq = shape.n_kv_heads, shape.n_q_heads
    _want(q, (*lead, None, hq, HEAD_DIM), "q")
    batch = int(q.shape[len(lead)])
    _want(r_k, (*lead, hkv, HEAD_DIM, HEAD_DIM), "r_k")
    _want(r_v, (*lead, hkv, HEAD_DIM, HEAD_DIM), "r_v")
    _want(seq_lens, (batch,), "seq_lens")
    _want(block_table, ((">=", batch), None), "block_table")
    _want(pool, (*lead, None, hkv, block_bytes(shape.group_size)), "pool")
    _check_rings(shape, win_k, win_v, batch, lead)
    _want(out, (*lead, batch, hq, HEAD_DIM), "out")
    return batch


def _decode_args(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out, workspace,
                 stream):
    b16, i32, u8, f32 = _dt()
    batch = _decode_checks(shape, r_k, r_v, q, seq_lens, block_table, pool, win_k, win_v, out)
    return (C.byref(shape), _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(q, b16, "q"), batch,
            _dev(seq_lens, i32, "seq_lens"), int(max_seq_len), _dev(block_table, i32, "block_table"),
            int(block_table.shape[1]), _dev(pool, u8, "pool"), int(pool.shape[0]), _dev(win_k, b16, "win_k"),
            _dev(win_v, b16, "win_v"), _dev(out, f32, "out"), _dev(workspace, u8, "workspace"),
            int(workspace.numel()), _stream(stream))


def oscar_decode_attn(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v,
                      out, workspace, stream=None) -> None:
    _check("oscar_decode_attn", lib.oscar_decode_attn(
        *_decode_args(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out, workspace,
                      stream)))


def _step_checks(shape, r_k, r_v, k_new, v_new, q, seq_lens, block_table, pool, win_k, win_v, out):
    batch = _decode_checks(shape, r_k, r_v, q, seq_lens, block_table, pool, win_k, win_v, out)
    _want(k_new, (batch, shape.n_kv_heads, HEAD_DIM), "k_new")
    _want(v_new, (batch, shape.n_kv_heads, HEAD_DIM), "v_new")
    return batch


def _step_args(shape, r_k, r_v, k_new, v_new, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out,
               workspace, stream):
    b16, i32, u8, f32 = _dt()
    batch = _step_checks(shape, r_k, r_v, k_new, v_new, q, seq_lens, block_table, pool, win_k, win_v, out)
    return (C.byref(shape), _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(k_new, b16, "k_new"),
            _dev(v_new, b16, "v_new"), _dev(q, b16, "q"), batch, _dev(seq_lens, i32, "seq_lens"), int(max_seq_len),
            _dev(block_table, i32, "block_table"), int(block_table.shape[1]), _dev(pool, u8, "pool"),
            int(pool.shape[0]), _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"), _dev(out, f32, "out"),
            _dev(workspace, u8, "workspace"), int(workspace.numel()), _stream(stream))


def oscar_decode_step(shape, r_k, r_v, k_new, v_new, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v,
                      out, workspace, stream=None) -> None:
    """One decode step: the new token (k_new[b], v_new[b]) [B][Hkv][128] of
    every sequence b appended at position seq_lens[b] - 1 (seq_lens: the
    lengths after it), then decode attention over the whole sequence; the
    same pool, rings and output as oscar_quantize_append followed by
    oscar_decode_attn, one launch fewer."""
    _check("oscar_decode_step", lib.oscar_decode_step(
        *_step_args(shape, r_k, r_v, k_new, v_new, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out,
                    workspace, stream)))


def oscar_decode_step_timed(shape, r_k, r_v, k_new, v_new, q, seq_lens, max_seq_len, block_table, pool, win_k,
                            win_v, out, workspace, start, stop, stream=None) -> None:
    """oscar_decode_step with the Event pair (start, stop) attached to the
    split kernel's launch."""
    _check("oscar_decode_step_timed", lib.oscar_decode_step_timed(
        *_step_args(shape, r_k, r_v, k_new, v_new, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out,
                    workspace, stream), start.handle, stop.handle))


def oscar_decode_attn_timed(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v,
                            out, workspace, start, stop, stream=None) -> None:
    """oscar_decode_attn with the Event pair (start, stop) attached to the INT2
    split kernel's dispatch."""
    _check("oscar_decode_attn_timed", lib.oscar_decode_attn_timed(
        *_decode_args(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out, workspace,
                      stream), start.handle, stop.handle))


def oscar_decode_noalloc_scratch_bytes(shape, batch: int, max_seq_len: int) -> int:
    n = lib.oscar_decode_noalloc_scratch_bytes(C.byref(shape), int(batch), int(max_seq_len))
    if n == 0:
        raise OscarError("oscar_decode_noalloc_scratch_bytes", -1)
    return int(n)


def oscar_decode_attn_noalloc(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v, out,
                              stream=None) -> None:
    """oscar_decode_attn with the library's static scratch instead of a
    workspace: no device allocation (calls overlapping on one GPU race)."""
    b16, i32, u8, f32 = _dt()
    batch = _decode_checks(shape, r_k, r_v, q, seq_lens, block_table, pool, win_k, win_v, out)
    _check("oscar_decode_attn_noalloc", lib.oscar_decode_attn_noalloc(
        C.byref(shape), _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(q, b16, "q"), batch,
        _dev(seq_lens, i32, "seq_lens"), int(max_seq_len), _dev(block_table, i32, "block_table"),
        int(block_table.shape[1]), _dev(pool, u8, "pool"), int(pool.shape[0]), _dev(win_k, b16, "win_k"),
        _dev(win_v, b16, "win_v"), _dev(out, f32, "out"), _stream(stream)))


def oscar_quantize_append_layers(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
                                 pool, win_k=None, win_v=None, stream=None) -> None:
    """Layer-batched append: r_k, r_v [L][Hkv][128][128]; k_new, v_new
    [L][T][Hkv][128]; pool [L][n_pages][Hkv][block]; rings [L][B][W + S][Hkv][128]."""
    b16, i32, u8, _ = _dt()
    _want(pool, (None, None, shape.n_kv_heads, block_bytes(shape.group_size)), "pool")
    n_layers = int(pool.shape[0])
    _append_checks(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after, pool, win_k, win_v,
                   lead=(n_layers,))
    _check("oscar_quantize_append_layers", lib.oscar_quantize_append_layers(
        C.byref(shape), n_layers, _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(k_new, b16, "k_new"),
        _dev(v_new, b16, "v_new"), int(k_new.shape[1]), _dev(seq_idx, i32, "seq_idx"),
        _dev(pos, i32, "pos"), int(block_table.shape[0]), _dev(block_table, i32, "block_table"),
        int(block_table.shape[1]), _dev(seq_len_after, i32, "seq_len_after"), _dev(pool, u8, "pool"),
        int(pool.shape[1]), _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"), _stream(stream)))


def oscar_decode_layers_workspace_bytes(shape, n_layers: int, batch: int, max_seq_len: int) -> int:
    n = lib.oscar_decode_layers_workspace_bytes(C.byref(shape), int(n_layers), int(batch), int(max_seq_len))
    if n == 0:
        raise OscarError("oscar_decode_layers_workspace_bytes", -1)
    return int(n)


def oscar_decode_attn_layers(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v,
                             out, workspace, stream=None) -> None:
    """Layer-batched decode: q [L][B][Hq][128], out [L][B][Hq][128] float32,
    other per-layer buffers stacked as for oscar_quantize_append_layers."""
    b16, i32, u8, f32 = _dt()
    _want(pool, (None, None, shape.n_kv_heads, block_bytes(shape.group_size)), "pool")
    n_layers = int(pool.shape[0])
    _decode_checks(shape, r_k, r_v, q, seq_lens, block_table, pool, win_k, win_v, out, lead=(n_layers,))
    _check("oscar_decode_attn_layers", lib.oscar_decode_attn_layers(
        C.byref(shape), n_layers, _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(q, b16, "q"),
        int(q.shape[1]), _dev(seq_lens, i32, "seq_lens"), int(max_seq_len),
        _dev(block_table, i32, "block_table"), int(block_table.shape[1]), _dev(pool, u8, "pool"),
        int(pool.shape[1]), _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"),
        _dev(out, f32, "out"), _dev(workspace, u8, "workspace"), int(workspace.numel()),
        _stream(stream)))


def oscar_bf16_append(shape, k_new, v_new, seq_idx, pos, block_table, kv_pool, stream=None) -> None:
    b16, i32, _, _ = _dt()
    hkv = shape.n_kv_heads
    _want(k_new, (None, hkv, HEAD_DIM), "k_new")
    n_tokens = int(k_new.shape[0])
    _want(v_new, (n_tokens, hkv, HEAD_DIM), "v_new")
    _want(seq_idx, (n_tokens,), "seq_idx")
    _want(pos, (n_tokens,), "pos")
    _want(block_table, (None, None), "block_table")
    _want(kv_pool, (None, hkv, BF16_BLOCK_ELEMS), "kv_pool")
    _check("oscar_bf16_append", lib.oscar_bf16_append(
        C.byref(shape), _dev(k_new, b16, "k_new"), _dev(v_new, b16, "v_new"), n_tokens,
        _dev(seq_idx, i32, "seq_idx"), _dev(pos, i32, "pos"), int(block_table.shape[0]),
        _dev(block_table, i32, "block_table"), int(block_table.shape[1]),
        _dev(kv_pool, b16, "kv_pool"), int(kv_pool.shape[0]), _stream(stream)))


def _bf16_decode_args(shape, q, seq_lens, max_seq_len, block_table, kv_pool, out, workspace, stream):
    b16, i32, u8, f32 = _dt()
    hq = shape.n_q_heads
    _want(q, (None, hq, HEAD_DIM), "q")
    batch = int(q.shape[0])
    _want(seq_lens, (batch,), "seq_lens")
    _want(block_table, ((">=", batch), None), "block_table")
    _want(kv_pool, (None, shape.n_kv_heads, BF16_BLOCK_ELEMS), "kv_pool")
    _want(out, (batch, hq, HEAD_DIM), "out")
    return (C.byref(shape), _dev(q, b16, "q"), batch, _dev(seq_lens, i32, "seq_lens"), int(max_seq_len),
            _dev(block_table, i32, "block_table"), int(block_table.shape[1]), _dev(kv_pool, b16, "kv_pool"),
            int(kv_pool.shape[0]), _dev(out, f32, "out"), _dev(workspace, u8, "workspace"), int(workspace.numel()),
            _stream(stream))


def oscar_bf16_decode_attn(shape, q, seq_lens, max_seq_len, block_table, kv_pool, out, workspace,
                           stream=None) -> None:
    _check("oscar_bf16_decode_attn", lib.oscar_bf16_decode_attn(
        *_bf16_decode_args(shape, q, seq_lens, max_seq_len, block_table, kv_pool, out, workspace, stream)))


def oscar_bf16_decode_attn_timed(shape, q, seq_lens, max_seq_len, block_table, kv_pool, out, workspace, start,
                                 stop, stream=None) -> None:
    _check("oscar_bf16_decode_attn_timed", lib.oscar_bf16_decode_attn_timed(
        *_bf16_decode_args(shape, q, seq_lens, max_seq_len, block_table, kv_pool, out, workspace, stream),
        start.handle, stop.handle))


def oscar_hbm_copy(src, dst, nbytes: int | None = None, stream=None) -> None:
    n = int(src.numel() * src.element_size()) if nbytes is None else int(nbytes)
    if src.device.type != "cuda" or dst.device.type != "cuda":
        raise ValueError("oscar_hbm_copy: tensors must be on the GPU")
    if n > src.numel() * src.element_size() or n > dst.numel() * dst.element_size():
        raise ValueError("oscar_hbm_copy: nbytes exceeds a buffer")
    _check("oscar_hbm_copy", lib.oscar_hbm_copy(src.data_ptr(), dst.data_ptr(), n, _stream(stream)))


def oscar_hbm_read(src, block_bytes_: int, blocks, n_blocks: int, sink, n_workgroups: int = 0, stream=None,
                   nt: bool = False) -> None:
    """Read probe: n_blocks blocks of block_bytes_ from the device buffer src,
    block i at blocks[i] (int32 device tensor) or, with blocks None, at i;
    sink: int32/uint32 device tensor of at least n_workgroups (0: 8 per CU) words.
    nt: the loads carry the non-temporal hint (oscar_hbm_read_nt)."""
    _, i32, _, _ = _dt()
    import torch

    nbytes = src.numel() * src.element_size()
    if blocks is None:
        if n_blocks * block_bytes_ > nbytes:
            raise ValueError("oscar_hbm_read: the blocks exceed src")
    else:
        _want(blocks, ((">=", n_blocks),), "blocks")
    if sink.dtype not in (torch.int32, torch.uint32) or sink.device.type != "cuda":
        raise TypeError("sink: int32 device tensor")
    fn = "oscar_hbm_read_nt" if nt else "oscar_hbm_read"
    _check(fn, getattr(lib, fn)(
        src.data_ptr(), int(block_bytes_), _dev(blocks, i32, "blocks"), int(n_blocks), sink.data_ptr(),
        int(n_workgroups), _stream(stream)))


def oscar_gpu_wait(microseconds: int, stream=None) -> None:
    """Hold the stream for `microseconds` of device time without touching memory."""
    _check("oscar_gpu_wait", lib.oscar_gpu_wait(int(microseconds), _stream(stream)))


class Event:
    """A HIP event owned by the caller (oscar_event_create).  Pass a pair to the
    *_timed entry points; ``elapsed_ms(start, stop)`` waits for stop."""

    def __init__(self):
        h = C.c_void_p()
        _check("oscar_event_create", lib.oscar_event_create(C.byref(h)))
        self.handle = h.value

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            lib.oscar_event_destroy(h)

    @staticmethod
    def elapsed_ms(start: "Event", stop: "Event") -> float:
        ms = C.c_float()
        _check("oscar_event_elapsed_ms", lib.oscar_event_elapsed_ms(start.handle, stop.handle, C.byref(ms)))
        return float(ms.value)


def oscar_strerror(status: int) -> str:
    return lib.oscar_strerror(int(status)).decode()
