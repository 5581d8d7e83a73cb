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
    "oscar_bf16_decode_attn", "oscar_hbm_copy", "oscar_gpu_wait", "oscar_timing_begin", "oscar_timing_end",
    "oscar_strerror", "BLOCK_BYTES", "BF16_BLOCK_ELEMS", "PAGE_SIZE", "HEAD_DIM", "block_bytes",
    "oscar_calibrate_layers", "oscar_rotation_file_bytes", "oscar_rotation_write", "oscar_rotation_read_info",
    "oscar_rotation_read", "oscar_quantize_append_layers", "oscar_decode_layers_workspace_bytes",
    "oscar_decode_attn_layers",
]

BLOCK_BYTES = 1152  # bytes per (page, KV head) block at group size 128
BF16_BLOCK_ELEMS = 4096  # bf16 comparator pool: K [16][128] then V^T [128][16] per (page, KV head)
PAGE_SIZE = 16
HEAD_DIM = 128


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


def _check_pool(shape, pool) -> None:
    if pool is None:
        return
    want = shape.n_kv_heads * block_bytes(shape.group_size) if shape.group_size in (32, 64, 128) else None
    if want is not None and pool.numel() != pool.shape[0] * want:
        raise ValueError(f"pool: expected [n_pages][{shape.n_kv_heads}][{block_bytes(shape.group_size)}] bytes")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise OscarError(fn, status)


def _dev(t, dtypes, name):
    """Device pointer of a contiguous torch tensor (None -> NULL)."""
    if t is None:
        return None
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _dt():
    import torch

    b16 = (torch.bfloat16, torch.int16, torch.uint16, torch.float16)
    return b16, (torch.int32,), (torch.uint8,), (torch.float32,)


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
    if q.ndim != 3 or k.shape != v.shape or k.ndim != 3 or q.shape[0] != hkv or k.shape[0] != hkv:
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
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[:2] != k.shape[:2] or q.shape[1] != hkv:
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


def oscar_quantize_append(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
                          pool, win_k=None, win_v=None, stream=None) -> None:
    b16, i32, u8, _ = _dt()
    _check_pool(shape, pool)
    _check("oscar_quantize_append", lib.oscar_quantize_append(
        C.byref(shape), _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(k_new, b16, "k_new"),
        _dev(v_new, b16, "v_new"), int(k_new.shape[0]), _dev(seq_idx, i32, "seq_idx"),
        _dev(pos, i32, "pos"), int(block_table.shape[0]), _dev(block_table, i32, "block_table"),
        int(block_table.shape[1]), _dev(seq_len_after, i32, "seq_len_after"), _dev(pool, u8, "pool"),
        int(pool.shape[0]), _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"), _stream(stream)))


def oscar_decode_workspace_bytes(shape, batch: int, max_seq_len: int) -> int:
    n = lib.oscar_decode_workspace_bytes(C.byref(shape), int(batch), int(max_seq_len))
    if n == 0:
        raise OscarError("oscar_decode_workspace_bytes", -1)
    return int(n)


def oscar_decode_attn(shape, r_k, r_v, q, seq_lens, max_seq_len, block_table, pool, win_k, win_v,
                      out, workspace, stream=None) -> None:
    b16, i32, u8, f32 = _dt()
    _check_pool(shape, pool)
    _check("oscar_decode_attn", lib.oscar_decode_attn(
        C.byref(shape), _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(q, b16, "q"),
        int(q.shape[0]), _dev(seq_lens, i32, "seq_lens"), int(max_seq_len),
        _dev(block_table, i32, "block_table"), int(block_table.shape[1]), _dev(pool, u8, "pool"),
        int(pool.shape[0]), _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"),
        _dev(out, f32, "out"), _dev(workspace, u8, "workspace"), int(workspace.numel()),
        _stream(stream)))


def oscar_quantize_append_layers(shape, r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
                                 pool, win_k=None, win_v=None, stream=None) -> None:
    """Layer-batched append: r_k, r_v [L][Hkv][128][128]; k_new, v_new
    [L][T][Hkv][128]; pool [L][n_pages][Hkv][block]; rings [L][B][W + S][Hkv][128]."""
    b16, i32, u8, _ = _dt()
    n_layers = int(pool.shape[0])
    for name, t in (("r_k", r_k), ("r_v", r_v), ("k_new", k_new), ("v_new", v_new)):
        if t.shape[0] != n_layers:
            raise ValueError(f"{name}: leading (layer) dimension must be {n_layers}")
    if pool.dim() != 4 or pool.shape[2] != shape.n_kv_heads or pool.shape[3] != block_bytes(shape.group_size):
        raise ValueError("pool must be [L][n_pages][Hkv][block bytes]")
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
    n_layers = int(pool.shape[0])
    for name, t in (("r_k", r_k), ("r_v", r_v), ("q", q), ("out", out)):
        if t.shape[0] != n_layers:
            raise ValueError(f"{name}: leading (layer) dimension must be {n_layers}")
    if pool.dim() != 4 or pool.shape[2] != shape.n_kv_heads or pool.shape[3] != block_bytes(shape.group_size):
        raise ValueError("pool must be [L][n_pages][Hkv][block bytes]")
    _check("oscar_decode_attn_layers", lib.oscar_decode_attn_layers(
        C.byref(shape), n_layers, _dev(r_k, b16, "r_k"), _dev(r_v, b16, "r_v"), _dev(q, b16, "q"),
        int(q.shape[1]), _dev(seq_lens, i32, "seq_lens"), int(max_seq_len),
        _dev(block_table, i32, "block_table"), int(block_table.shape[1]), _dev(pool, u8, "pool"),
        int(pool.shape[1]), _dev(win_k, b16, "win_k"), _dev(win_v, b16, "win_v"),
        _dev(out, f32, "out"), _dev(workspace, u8, "workspace"), int(workspace.numel()),
        _stream(stream)))


def oscar_bf16_append(shape, k_new, v_new, seq_idx, pos, block_table, kv_pool, stream=None) -> None:
    b16, i32, _, _ = _dt()
    _check("oscar_bf16_append", lib.oscar_bf16_append(
        C.byref(shape), _dev(k_new, b16, "k_new"), _dev(v_new, b16, "v_new"), int(k_new.shape[0]),
        _dev(seq_idx, i32, "seq_idx"), _dev(pos, i32, "pos"), int(block_table.shape[0]),
        _dev(block_table, i32, "block_table"), int(block_table.shape[1]),
        _dev(kv_pool, b16, "kv_pool"), int(kv_pool.shape[0]), _stream(stream)))


def oscar_bf16_decode_attn(shape, q, seq_lens, max_seq_len, block_table, kv_pool, out, workspace,
                           stream=None) -> None:
    b16, i32, u8, f32 = _dt()
    _check("oscar_bf16_decode_attn", lib.oscar_bf16_decode_attn(
        C.byref(shape), _dev(q, b16, "q"), int(q.shape[0]), _dev(seq_lens, i32, "seq_lens"),
        int(max_seq_len), _dev(block_table, i32, "block_table"), int(block_table.shape[1]),
        _dev(kv_pool, b16, "kv_pool"), int(kv_pool.shape[0]), _dev(out, f32, "out"),
        _dev(workspace, u8, "workspace"), int(workspace.numel()), _stream(stream)))


def oscar_hbm_copy(src, dst, nbytes: int | None = None, stream=None) -> None:
    n = int(src.numel() * src.element_size()) if nbytes is None else int(nbytes)
    if src.device.type != "cuda" or dst.device.type != "cuda":
        raise ValueError("oscar_hbm_copy: tensors must be on the GPU")
    _check("oscar_hbm_copy", lib.oscar_hbm_copy(src.data_ptr(), dst.data_ptr(), n, _stream(stream)))


def oscar_gpu_wait(microseconds: int, stream=None) -> None:
    """Hold the stream for `microseconds` of device time without touching memory."""
    _check("oscar_gpu_wait", lib.oscar_gpu_wait(int(microseconds), _stream(stream)))


def oscar_timing_begin(capacity: int) -> None:
    _check("oscar_timing_begin", lib.oscar_timing_begin(int(capacity)))


def oscar_timing_end(capacity: int):
    """Returns (ms, kinds) lists for the recorded main-kernel launches."""
    ms = (C.c_float * capacity)()
    kinds = (C.c_int32 * capacity)()
    n = C.c_int32(0)
    _check("oscar_timing_end", lib.oscar_timing_end(ms, kinds, int(capacity), C.byref(n)))
    return list(ms[:n.value]), list(kinds[:n.value])


def oscar_strerror(status: int) -> str:
    return lib.oscar_strerror(int(status)).decode()
