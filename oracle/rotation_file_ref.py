"""Plain reference of the rotation file format (numpy, struct, zlib).

TEST INFRASTRUCTURE ONLY: nothing on the library's path imports this module;
tests use it to check the library's writer and reader byte for byte.

The pages describe calibration as an offline, once-per-model step whose results
ship for supported models (P1 gen-hub.ru «Открытый код — это серьёзно»; P2
encorp.ai «OSCAR има значение…»; P4 aiforradalom.hu «OSCAR: figyelem-tudatos és
bevetésre kész») but fix no file layout; this is the layout's definition,
written out field by field (little endian):

  offset  field
   0      8 bytes   magic b"OSCARROT"
   8      u32       version 1
  12      u32       header bytes 64
  16      u32       head_dim 128
  20      u32       n_layers
  24      u32       n_kv_heads
  28      u32       group_size the rotations were calibrated for
  32      u32       flags (bit 0: eigenvalues present)
  36      u32       0
  40      u64       payload bytes
  48      u32       CRC-32 of the payload
  52      u32       CRC-32 of bytes [0, 52)
  56      8 bytes   0
  payload, per layer: R_K bf16 [Hkv][128][128], R_V bf16 [Hkv][128][128], and
  with flag bit 0 eig_K, eig_V float64 [Hkv][128].

CRC-32 is zlib's (reflected polynomial 0xEDB88320, init and final xor
0xFFFFFFFF), used here as a library routine.
"""
from __future__ import annotations

import struct
import zlib

import numpy as np

MAGIC = b"OSCARROT"
VERSION = 1
HEADER = 64
D = 128


def encode(r_k, r_v, group_size: int = 128, eig_k=None, eig_v=None) -> bytes:
    """File bytes of rotations uint16 [L][Hkv][128][128] (+ eigenvalues [L][Hkv][128])."""
    rk = np.asarray(r_k, dtype="<u2")
    rv = np.asarray(r_v, dtype="<u2")
    n_layers, hkv = rk.shape[:2]
    eig = eig_k is not None
    parts = []
    for l in range(n_layers):
        parts += [rk[l].tobytes(), rv[l].tobytes()]
        if eig:
            parts += [np.asarray(eig_k[l], "<f8").tobytes(), np.asarray(eig_v[l], "<f8").tobytes()]
    body = b"".join(parts)
    head = struct.pack("<8sIIIIIIII", MAGIC, VERSION, HEADER, D, n_layers, hkv, group_size, int(eig), 0)
    head += struct.pack("<QI", len(body), zlib.crc32(body))
    head += struct.pack("<I", zlib.crc32(head))
    head += bytes(8)
    assert len(head) == HEADER
    return head + body


def decode(data: bytes):
    """(info dict, r_k, r_v, eig_k, eig_v) of a file; raises ValueError on any
    inconsistency (magic, version, sizes, checksums)."""
    if len(data) < HEADER:
        raise ValueError("short header")
    magic, version, header, d, n_layers, hkv, group, flags, zero = struct.unpack_from("<8sIIIIIIII", data, 0)
    payload, crc_body = struct.unpack_from("<QI", data, 40)
    (crc_head,) = struct.unpack_from("<I", data, 52)
    if magic != MAGIC or zlib.crc32(data[:52]) != crc_head:
        raise ValueError("not a rotation file, or damaged header")
    if version != VERSION or header != HEADER or d != D or flags & ~1 or group not in (32, 64, 128):
        raise ValueError("unsupported header")
    if zero != 0 or data[56:HEADER] != bytes(HEADER - 56):
        raise ValueError("reserved header bytes not zero")
    eig = bool(flags & 1)
    per_layer = hkv * D * D * 2 * 2 + (hkv * D * 8 * 2 if eig else 0)
    body = data[HEADER:]
    if payload != n_layers * per_layer or len(body) != payload or zlib.crc32(body) != crc_body:
        raise ValueError("payload size or checksum")
    rk = np.empty((n_layers, hkv, D, D), np.uint16)
    rv = np.empty_like(rk)
    ek = np.empty((n_layers, hkv, D)) if eig else None
    ev = np.empty((n_layers, hkv, D)) if eig else None
    o = 0
    for l in range(n_layers):
        rk[l] = np.frombuffer(body, "<u2", hkv * D * D, o).reshape(hkv, D, D)
        o += hkv * D * D * 2
        rv[l] = np.frombuffer(body, "<u2", hkv * D * D, o).reshape(hkv, D, D)
        o += hkv * D * D * 2
        if eig:
            ek[l] = np.frombuffer(body, "<f8", hkv * D, o).reshape(hkv, D)
            o += hkv * D * 8
            ev[l] = np.frombuffer(body, "<f8", hkv * D, o).reshape(hkv, D)
            o += hkv * D * 8
    info = dict(n_layers=n_layers, n_kv_heads=hkv, group_size=group, has_eigenvalues=int(eig))
    return info, rk, rv, ek, ev
