"""Rotation files (CPU only): the format's plain definition is pinned by hand
(header fields at their offsets, zlib's CRC-32 over the stated ranges, exact
file size), and the library's writer and reader agree with it byte for byte;
damaged, truncated or mismatched files are refused.  Multi-layer calibration
equals calibrating each layer on its own."""
import struct
import zlib

import numpy as np
import pytest

import workloads as wl
from oracle import rotation_file_ref as rf

K = pytest.importorskip("kv_cache_int2_amd", reason="library not built")

EIO, EFORMAT = -5, -6


def random_rotations(rng, n_layers, hkv):
    rk = rng.integers(0, 65536, (n_layers, hkv, 128, 128), dtype=np.uint16)
    rv = rng.integers(0, 65536, (n_layers, hkv, 128, 128), dtype=np.uint16)
    ek = rng.standard_normal((n_layers, hkv, 128))
    ev = rng.standard_normal((n_layers, hkv, 128))
    return rk, rv, ek, ev


def test_reference_layout_by_hand(rng):
    rk, rv, ek, ev = random_rotations(rng, 2, 1)
    data = rf.encode(rk, rv, 64, ek, ev)
    per_layer = 2 * 128 * 128 * 2 + 2 * 128 * 8
    assert len(data) == 64 + 2 * per_layer
    assert data[:8] == b"OSCARROT"
    assert struct.unpack_from("<7I", data, 8) == (1, 64, 128, 2, 1, 64, 1)
    assert struct.unpack_from("<Q", data, 40)[0] == 2 * per_layer
    assert struct.unpack_from("<I", data, 48)[0] == zlib.crc32(data[64:])
    assert struct.unpack_from("<I", data, 52)[0] == zlib.crc32(data[:52])
    assert data[36:40] == bytes(4) and data[56:64] == bytes(8)
    # layer 1's R_V starts after layer 0's record and layer 1's R_K
    o = 64 + per_layer + 128 * 128 * 2
    assert np.array_equal(np.frombuffer(data, "<u2", 128 * 128, o).reshape(128, 128), rv[1, 0])
    o = 64 + per_layer - 128 * 8
    assert np.array_equal(np.frombuffer(data, "<f8", 128, o), ev[0, 0])
    info, rk2, rv2, ek2, ev2 = rf.decode(data)
    assert info == dict(n_layers=2, n_kv_heads=1, group_size=64, has_eigenvalues=1)
    assert np.array_equal(rk2, rk) and np.array_equal(rv2, rv) and np.array_equal(ek2, ek) and np.array_equal(ev2, ev)


@pytest.mark.parametrize("eig,group", [(True, 128), (False, 64), (True, 32)])
def test_library_writer_matches_reference(rng, tmp_path, eig, group):
    rk, rv, ek, ev = random_rotations(rng, 3, 2)
    shape = K.make_shape(8, 2, group_size=group)
    path = tmp_path / "r.oscarrot"
    K.oscar_rotation_write(str(path), shape, rk, rv, ek if eig else None, ev if eig else None)
    want = rf.encode(rk, rv, group, ek if eig else None, ev if eig else None)
    got = path.read_bytes()
    assert got == want
    assert K.oscar_rotation_file_bytes(3, 2, eig) == len(want)


def test_library_reader_reads_reference_file(rng, tmp_path):
    rk, rv, ek, ev = random_rotations(rng, 4, 3)
    path = tmp_path / "r.oscarrot"
    path.write_bytes(rf.encode(rk, rv, 128, ek, ev))
    assert K.oscar_rotation_read_info(str(path)) == dict(n_layers=4, n_kv_heads=3, group_size=128,
                                                         has_eigenvalues=1)
    shape = K.make_shape(12, 3)
    rk2, rv2, ek2, ev2 = K.oscar_rotation_read(str(path), shape, 4, eigenvalues=True)
    assert np.array_equal(rk2, rk) and np.array_equal(rv2, rv) and np.array_equal(ek2, ek) and np.array_equal(ev2, ev)
    rk3, rv3 = K.oscar_rotation_read(str(path), shape, 4)
    assert np.array_equal(rk3, rk) and np.array_equal(rv3, rv)


def status_of(fn, *args, **kw):
    with pytest.raises(K.OscarError) as e:
        fn(*args, **kw)
    return e.value.status


def test_damaged_and_mismatched_files_are_refused(rng, tmp_path):
    rk, rv, ek, ev = random_rotations(rng, 2, 2)
    good = rf.encode(rk, rv, 64, ek, ev)
    shape = K.make_shape(8, 2, group_size=64)
    p = tmp_path / "f"
    cases = {
        "payload byte": good[:5000] + bytes([good[5000] ^ 1]) + good[5001:],
        "header field": good[:20] + bytes([good[20] ^ 4]) + good[21:],
        "magic": b"X" + good[1:],
        "truncated": good[:-1],
        "trailing byte": good + b"\0",
        "short header": good[:40],
        "reserved bytes after the header checksum": good[:60] + bytes([good[60] ^ 1]) + good[61:],
    }
    for name, data in cases.items():
        p.write_bytes(data)
        assert status_of(K.oscar_rotation_read, str(p), shape, 2) == EFORMAT, name
        with pytest.raises(ValueError):
            rf.decode(data)
    p.write_bytes(good)
    assert status_of(K.oscar_rotation_read, str(p), K.make_shape(12, 3, group_size=64), 2) == EFORMAT  # heads
    assert status_of(K.oscar_rotation_read, str(p), shape, 3) == EFORMAT                                # layers
    assert status_of(K.oscar_rotation_read, str(p), K.make_shape(8, 2), 2) == EFORMAT                    # group
    p.write_bytes(rf.encode(rk, rv, 64))
    assert status_of(K.oscar_rotation_read, str(p), shape, 2, eigenvalues=True) == EFORMAT  # none stored
    assert status_of(K.oscar_rotation_read, str(tmp_path / "missing"), shape, 2) == EIO
    assert status_of(K.oscar_rotation_read_info, str(tmp_path / "missing")) == EIO
    assert status_of(K.oscar_rotation_write, str(tmp_path / "no_dir" / "f"), shape, rk, rv) == EIO


def test_calibrate_layers_equals_per_layer(tmp_path):
    """Two layers (the config-1 calibration set and a rescaled copy) in one call
    give the rotations and eigenvalues of two separate calls, bit for bit; they
    round-trip through a file."""
    s = wl.spec(1)
    qc, kc, vc = wl.calibration_set(s)
    qc, kc, vc = qc[:2], kc[:2, :256], vc[:2, :256]
    q2 = np.stack([qc, 0.5 * qc[::-1]])
    k2 = np.stack([kc, 2.0 * kc[::-1]])
    v2 = np.stack([vc, vc[::-1] + 0.25])
    shape = K.make_shape(8, 2)
    rk, rv, ek, ev = K.oscar_calibrate_layers(shape, q2, k2, v2)
    for l in range(2):
        a = K.oscar_calibrate(shape, q2[l], k2[l], v2[l])
        assert np.array_equal(rk[l], a[0]) and np.array_equal(rv[l], a[1])
        assert np.array_equal(ek[l], a[2]) and np.array_equal(ev[l], a[3])
    path = str(tmp_path / "model.oscarrot")
    K.oscar_rotation_write(path, shape, rk, rv, ek, ev)
    back = K.oscar_rotation_read(path, shape, 2, eigenvalues=True)
    for x, y in zip(back, (rk, rv, ek, ev)):
        assert np.array_equal(x, y)
