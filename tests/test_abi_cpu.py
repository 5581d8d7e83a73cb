"""C ABI checks that need no GPU: the library loads, exports every function
include/oscar.h declares, rejects bad arguments on the host before any launch,
and its host-side calibration matches the oracle."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import workloads as wl
from oracle import oscar_ref as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")

K = pytest.importorskip("kv_cache_int2_amd", reason="library not built")
from kv_cache_int2_amd import _lib  # noqa: E402

EINVAL, EUNSUP, ENOSPACE = -1, -2, -4


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared()
    assert len(names) >= 10
    lib = C.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_strerror():
    assert K.oscar_strerror(0) == "ok"
    assert "invalid" in K.oscar_strerror(EINVAL)
    assert "unsupported" in K.oscar_strerror(EUNSUP)


def bad_shapes():
    return [K.make_shape(32, 8, head_dim=64), K.make_shape(32, 8, group_size=16),
            K.make_shape(32, 8, group_size=48), K.make_shape(32, 8, group_size=0),
            K.make_shape(32, 8, page_size=32), K.make_shape(24, 8), K.make_shape(32, 8, window=4096),
            K.make_shape(32, 8, n_sink=-1), K.make_shape(32, 8, n_sink=2048)]


def test_host_validation_before_launch():
    lib = _lib.lib
    good = K.make_shape(32, 8)
    for s in bad_shapes():
        st = lib.oscar_quantize_append(C.byref(s), *([None] * 4), 1, None, None, 1, None, 1, None, None, 1,
                                       None, None, None)
        assert st in (EINVAL, EUNSUP)
        assert lib.oscar_decode_workspace_bytes(C.byref(s), 1, 100) == 0
    assert lib.oscar_quantize_append(C.byref(K.make_shape(32, 8, head_dim=64)), *([None] * 4), 1, None, None,
                                     1, None, 1, None, None, 1, None, None, None) == EUNSUP
    # null pointers
    assert lib.oscar_quantize_append(C.byref(good), *([None] * 4), 5, None, None, 1, None, 1, None, None, 1,
                                     None, None, None) == EINVAL
    # zero tokens is a no-op
    assert lib.oscar_quantize_append(C.byref(good), *([None] * 4), 0, None, None, 1, None, 1, None, None, 1,
                                     None, None, None) == 0
    ws = lib.oscar_decode_workspace_bytes(C.byref(good), 8, 100000)
    assert ws > 8 * 32 * 128 * 4
    # workspace too small / sequence longer than the block table
    fake = C.c_void_p(256)
    args = [C.byref(good), fake, fake, fake, 8, fake, 100000, fake, 100000 // 16 + 1, fake, 1, fake, fake, fake,
            fake]
    assert lib.oscar_decode_attn(*args, ws - 1, None) == ENOSPACE
    args[8] = 100
    assert lib.oscar_decode_attn(*args, ws, None) == ENOSPACE
    # rows are read as 16-byte vectors: a misaligned query or rotation is refused
    args[8] = 100000 // 16 + 1
    for i in (1, 3):  # r_k, q
        bad = list(args)
        bad[i] = C.c_void_p(258)
        assert lib.oscar_decode_attn(*bad, ws, None) == EINVAL
    assert lib.oscar_decode_attn(C.byref(good), None, None, None, 8, None, 10, None, 1, None, 1, None, None,
                                 None, None, 0, None) == EINVAL
    # sinks without a window still need the ring
    sink_only = K.make_shape(32, 8, window=0, n_sink=4)
    assert lib.oscar_decode_attn(C.byref(sink_only), fake, fake, fake, 8, fake, 10, fake, 1, fake, 1, None, None,
                                 fake, fake, 1 << 30, None) == EINVAL
    assert lib.oscar_quantize_append(C.byref(sink_only), fake, fake, fake, fake, 1, fake, fake, 1, fake, 1, fake,
                                     fake, 1, None, None, None) == EINVAL
    # the sink chunks enlarge the workspace; so do finer groups (per-group query sums)
    assert lib.oscar_decode_workspace_bytes(C.byref(K.make_shape(32, 8, n_sink=64)), 8, 100000) > ws
    for g in (32, 64):
        assert lib.oscar_decode_workspace_bytes(C.byref(K.make_shape(32, 8, group_size=g)), 8, 100000) > 0
    assert lib.oscar_hbm_copy(fake, fake, 17, None) == EINVAL
    assert lib.oscar_gpu_wait(-1, None) == EINVAL
    assert lib.oscar_gpu_wait(10000001, None) == EINVAL
    assert lib.oscar_gpu_wait(0, None) == 0
    # read probe: sizes, alignment, workgroup count
    sink = C.c_void_p(1024)
    assert lib.oscar_hbm_read(fake, 1152, None, 0, sink, 0, None) == 0  # nothing to read
    assert lib.oscar_hbm_read(fake, 1000, None, 1, sink, 0, None) == EINVAL  # not a multiple of 16
    assert lib.oscar_hbm_read(fake, 0, None, 1, sink, 0, None) == EINVAL
    assert lib.oscar_hbm_read(fake, (1 << 20) + 16, None, 1, sink, 0, None) == EINVAL
    assert lib.oscar_hbm_read(C.c_void_p(264), 1152, None, 1, sink, 0, None) == EINVAL  # misaligned
    assert lib.oscar_hbm_read(fake, 1152, None, 1, None, 0, None) == EINVAL
    assert lib.oscar_hbm_read(fake, 1152, None, 1, sink, 65537, None) == EINVAL
    assert lib.oscar_hbm_read(fake, 1152, None, -1, sink, 0, None) == EINVAL
    # events: null arguments, and a timed call with only one of the two events
    assert lib.oscar_event_create(None) == EINVAL
    assert lib.oscar_event_destroy(None) == EINVAL
    assert lib.oscar_event_elapsed_ms(None, None, None) == EINVAL
    assert lib.oscar_decode_attn_timed(*args, ws, None, fake, None) == EINVAL
    assert lib.oscar_decode_attn_timed(*args, ws, None, None, fake) == EINVAL
    assert lib.oscar_quantize_append_timed(C.byref(good), fake, fake, fake, fake, 1, fake, fake, 1, fake, 1, fake,
                                           fake, 1, fake, fake, None, fake, None) == EINVAL
    assert lib.oscar_bf16_decode_attn_timed(C.byref(good), fake, 8, fake, 10, fake, 1, fake, 1, fake, fake,
                                            1 << 30, None, None, fake) == EINVAL
    # the fused decode step: both new-token row arrays, 16-byte aligned, then
    # the decode's own checks
    step = [C.byref(good), fake, fake, fake, fake, fake, 8, fake, 100000, fake, 100000 // 16 + 1, fake, 1, fake,
            fake, fake, fake]
    for i, v in ((3, None), (4, None), (3, C.c_void_p(258)), (4, C.c_void_p(258))):
        bad = list(step)
        bad[i] = v
        assert lib.oscar_decode_step(*bad, ws, None) == EINVAL
    assert lib.oscar_decode_step(*step, ws - 1, None) == ENOSPACE
    assert lib.oscar_decode_step_timed(*step, ws, None, fake, None) == EINVAL


def test_layered_entry_points_validate_on_host():
    lib = _lib.lib
    good = K.make_shape(32, 8)
    fake = C.c_void_p(256)
    one = lib.oscar_decode_layers_workspace_bytes(C.byref(good), 1, 8, 100000)
    assert one == lib.oscar_decode_workspace_bytes(C.byref(good), 8, 100000)
    four = lib.oscar_decode_layers_workspace_bytes(C.byref(good), 4, 8, 100000)
    assert four > one
    assert lib.oscar_decode_layers_workspace_bytes(C.byref(good), 0, 8, 100000) == 0
    for n_layers in (0, -1):
        assert lib.oscar_decode_attn_layers(C.byref(good), n_layers, fake, fake, fake, 8, fake, 100, fake, 16, fake,
                                            1, fake, fake, fake, fake, 1 << 30, None) == EINVAL
        assert lib.oscar_quantize_append_layers(C.byref(good), n_layers, fake, fake, fake, fake, 1, fake, fake, 1,
                                                fake, 1, fake, fake, 1, fake, fake, None) == EINVAL
    # n_layers * batch beyond one grid dimension
    assert lib.oscar_decode_attn_layers(C.byref(good), 4096, fake, fake, fake, 32, fake, 100, fake, 16, fake, 1,
                                        fake, fake, fake, fake, 1 << 40, None) == EINVAL
    # a workspace sized for fewer layers is refused
    assert lib.oscar_decode_attn_layers(C.byref(good), 4, fake, fake, fake, 8, fake, 100000, fake,
                                        100000 // 16 + 1, fake, 1, fake, fake, fake, fake, one, None) == ENOSPACE
    # zero tokens is a no-op for any layer count
    assert lib.oscar_quantize_append_layers(C.byref(good), 3, *([None] * 4), 0, None, None, 1, None, 1, None, None,
                                            1, None, None, None) == 0


def test_calibrate_rejects_bad_input():
    s = K.make_shape(32, 8)
    q = np.zeros((8, 4, 128), np.float32)
    k = np.zeros((8, 4, 128), np.float32)
    q[0, 0, 0] = np.nan
    with pytest.raises(K.OscarError):
        K.oscar_calibrate(s, q, k, k)
    with pytest.raises(K.OscarError):
        K.oscar_calibrate(K.make_shape(32, 8, head_dim=64), q * 0, k, k)


def near_bf16_midpoint(x, rel=1e-9):
    """True where x lies within rel*|x| of a bf16 rounding midpoint."""
    lo = ref.bf16_rne(x * (1 - rel))
    hi = ref.bf16_rne(x * (1 + rel))
    return lo != hi


def test_calibrate_matches_oracle():
    """Host Jacobi calibration vs the oracle (numpy eigh) on the config-1
    calibration set: eigenvalues to 1e-9 relative; R bf16 bits equal wherever the
    oracle's fp64 value is not within 1e-9 of a bf16 midpoint (eigenvectors of
    distinct eigenvalues are unique once the sign convention is fixed)."""
    s = wl.spec(1)
    qc, kc, vc = wl.calibration_set(s)
    shape = K.make_shape(32, 8)
    rk, rv, ek, ev = K.oscar_calibrate(shape, qc, kc, vc)
    rk_ref, rv_ref, ek_ref, ev_ref = ref.calibrate_ref(qc, kc, vc)
    assert np.allclose(ek, ek_ref, rtol=1e-9, atol=1e-12 * ek_ref.max())
    assert np.allclose(ev, ev_ref, rtol=1e-9, atol=1e-12 * ev_ref.max())
    for got, want in ((rk, rk_ref), (rv, rv_ref)):
        ok = ~near_bf16_midpoint(want)
        assert ok.mean() > 0.999
        assert np.array_equal(got[ok], ref.bf16_bits(want)[ok])
        # the bf16 R is orthogonal to bf16 precision
        r = ref.bf16_to_f64(got)
        assert np.abs(np.einsum("hij,hkj->hik", r, r) - np.eye(128)).max() < 2e-2


def test_calibrate_special_case_diagonal():
    """Queries along the coordinate axes with distinct energies: U_Q = I up to
    order, so R_K = P_br (H / sqrt d) P where P sorts the axes by energy."""
    d = 128
    shape = K.make_shape(1, 1)
    energy = np.linspace(2.0, 1.0, d)
    perm = np.random.default_rng(3).permutation(d)
    q = np.zeros((1, d, d), np.float32)
    q[0, np.arange(d), perm] = np.sqrt(d * energy).astype(np.float32)
    k = np.random.default_rng(4).standard_normal((1, 64, d)).astype(np.float32)
    rk, _, ek, _ = K.oscar_calibrate(shape, q, k, k)
    want_e = np.sort((q[0].astype(np.float64) ** 2).sum(0) / d)[::-1]
    assert np.allclose(ek[0], want_e, rtol=1e-12)
    u = np.zeros((d, d))
    u[perm, np.arange(d)] = 1.0  # eigenvector k is axis perm[k] (energies sorted descending)
    want = ref.apply_bitrev_rows(ref.hadamard(d) / np.sqrt(d) @ u.T)
    assert np.array_equal(rk[0], ref.bf16_bits(want))


class _Fake:
    """Stands in for a device tensor in the binding's shape checks (which run
    before any pointer is taken)."""

    def __init__(self, *shape):
        self.shape = tuple(shape)


def test_binding_checks_shapes_before_the_call():
    """The Python binding refuses buffers whose shapes do not fit the shape
    struct and the derived batch / token counts (an undersized ring or query
    would otherwise be read or written past its end on the device)."""
    F = _Fake
    shape = K.make_shape(32, 8, window=128, n_sink=4)
    rk = F(8, 128, 128)
    blk = K.block_bytes(128)
    good_append = dict(r_k=rk, r_v=rk, k_new=F(10, 8, 128), v_new=F(10, 8, 128), seq_idx=F(10), pos=F(10),
                       block_table=F(2, 7), seq_len_after=F(2), pool=F(14, 8, blk), win_k=F(2, 132, 8, 128),
                       win_v=F(2, 132, 8, 128))
    assert K._append_checks(shape, **good_append) == (10, 2)
    bad = [("v_new", F(9, 8, 128)), ("pos", F(11)), ("seq_idx", F(10, 1)), ("seq_len_after", F(1)),
           ("win_k", F(2, 128, 8, 128)),  # ring without the sink rows
           ("win_v", F(1, 132, 8, 128)),  # fewer sequences than the block table
           ("pool", F(14, 8, 1280)), ("r_k", F(8, 128, 64)), ("k_new", F(10, 4, 128))]
    for name, t in bad:
        kw = dict(good_append, **{name: t})
        with pytest.raises(ValueError, match=name):
            K._append_checks(shape, **kw)
    # an empty append needs no ring
    empty = dict(good_append, k_new=F(0, 8, 128), v_new=F(0, 8, 128), seq_idx=F(0), pos=F(0), win_k=None,
                 win_v=None)
    assert K._append_checks(shape, **empty) == (0, 2)

    good_dec = dict(r_k=rk, r_v=rk, q=F(3, 32, 128), seq_lens=F(3), block_table=F(3, 9), pool=F(20, 8, blk),
                    win_k=F(3, 132, 8, 128), win_v=F(3, 132, 8, 128), out=F(3, 32, 128))
    assert K._decode_checks(shape, **good_dec) == 3
    bad = [("q", F(3, 16, 128)), ("seq_lens", F(2)), ("block_table", F(2, 9)), ("out", F(2, 32, 128)),
           ("out", F(3, 32, 64)), ("win_k", F(2, 132, 8, 128)), ("win_v", None), ("r_v", F(4, 128, 128))]
    for name, t in bad:
        kw = dict(good_dec, **{name: t})
        with pytest.raises(ValueError, match=name):
            K._decode_checks(shape, **kw)
    # the decode step: one new K/V row per sequence and KV head
    good_step = dict(good_dec, k_new=F(3, 8, 128), v_new=F(3, 8, 128))
    assert K._step_checks(shape, **good_step) == 3
    for name, t in (("k_new", F(2, 8, 128)), ("v_new", F(3, 4, 128)), ("k_new", F(3, 8, 64)),
                    ("q", F(3, 16, 128))):
        with pytest.raises(ValueError, match=name):
            K._step_checks(shape, **dict(good_step, **{name: t}))
    # layer-batched: every per-layer buffer carries the layer count
    lay = dict(r_k=F(2, 8, 128, 128), r_v=F(2, 8, 128, 128), q=F(2, 3, 32, 128), seq_lens=F(3),
               block_table=F(3, 9), pool=F(2, 20, 8, blk), win_k=F(2, 3, 132, 8, 128), win_v=F(2, 3, 132, 8, 128),
               out=F(2, 3, 32, 128))
    assert K._decode_checks(shape, lead=(2,), **lay) == 3
    with pytest.raises(ValueError, match="out"):
        K._decode_checks(shape, lead=(2,), **dict(lay, out=F(1, 3, 32, 128)))
    # calibration arrays with a head dim other than 128
    with pytest.raises(ValueError):
        K.oscar_calibrate(K.make_shape(32, 8), np.zeros((8, 4, 64), np.float32), np.zeros((8, 4, 64), np.float32),
                          np.zeros((8, 4, 64), np.float32))


def test_noalloc_entry_point_refuses_oversized_calls_on_the_host():
    """The allocation-free decode checks its scratch need against the static
    array before anything touches the device."""
    lib = _lib.lib
    fake = C.c_void_p(256)
    small = K.make_shape(32, 8)
    need = lib.oscar_decode_noalloc_scratch_bytes(C.byref(small), 8, 100000)
    assert 0 < need <= K.NOALLOC_SCRATCH_BYTES
    # the workspace form's size includes the comparator's partials; the static
    # scratch holds only what the INT2 decode uses
    assert need <= lib.oscar_decode_workspace_bytes(C.byref(small), 8, 100000)
    big = K.make_shape(64, 8, window=1024, n_sink=1024, group_size=32)
    assert lib.oscar_decode_noalloc_scratch_bytes(C.byref(big), 64, 131073) > K.NOALLOC_SCRATCH_BYTES
    assert lib.oscar_decode_attn_noalloc(C.byref(big), fake, fake, fake, 64, fake, 131073, fake, 8193, fake, 1, fake,
                                         fake, fake, None) == ENOSPACE
    assert lib.oscar_decode_noalloc_scratch_bytes(C.byref(K.make_shape(32, 8, group_size=48)), 8, 10) == 0
    assert lib.oscar_decode_attn_noalloc(C.byref(K.make_shape(24, 8)), fake, fake, fake, 8, fake, 10, fake, 1, fake,
                                         1, fake, fake, fake, None) == EUNSUP
