"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Rotations come from the oracle's calibration (as data for both sides).  Small
cases compare every output; the full-size workloads (run in the same launch
configuration as bench.py) compare sampled outputs and size-independent
properties.
"""
import functools
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import oscar_ref as ref  # noqa: E402
import parity as P  # noqa: E402


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_int2_amd as K

    return K


DEV = "cuda:0"


def D(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def H(t, dtype=None):
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


@functools.lru_cache(maxsize=None)
def rotations(cfg, hkv=8):
    s = wl.spec(cfg)
    qc, kc, vc = wl.calibration_set(s)
    rk, rv, _, _ = ref.calibrate_ref(qc[:hkv], kc[:hkv], vc[:hkv])
    return ref.bf16_bits(rk), ref.bf16_bits(rv)


@functools.lru_cache(maxsize=None)
def arm_rotation(arm, hkv=8):
    """bf16 bits (r_k, r_v) [Hkv][128][128] of a comparison rotation of the
    quality harness, the same for keys and values: "hadamard" is the fixed
    transform alone, P_br (H / sqrt d) (the oracle's Sylvester matrix with
    bit-reversed rows); "identity" is plain per-token INT2."""
    if arm == "hadamard":
        r = ref.apply_bitrev_rows(ref.hadamard()) / np.sqrt(128)
    elif arm == "identity":
        r = np.eye(128)
    else:
        raise ValueError(arm)
    bits = np.ascontiguousarray(np.broadcast_to(ref.bf16_bits(r), (hkv, 128, 128)))
    return bits, bits.copy()


def make_spec(cfg, lens, window=128, hq=None, hkv=8, n_sink=0, group=128):
    s = wl.spec(cfg, batch=len(lens))
    s.seq_lens = np.asarray(lens, np.int32)
    s.window = window
    s.n_sink = n_sink
    s.group_size = group
    if hq is not None:
        s.n_q_heads = hq
    s.n_kv_heads = hkv
    return s


def token_list(s, order="inorder", rng=None):
    ks, vs, si, ps = [], [], [], []
    for b in range(s.batch):
        k, v, i, p = wl.prefill_tokens(s, b)
        ks.append(k[:, :s.n_kv_heads])
        vs.append(v[:, :s.n_kv_heads])
        si.append(i)
        ps.append(p)
    k, v, si, ps = (np.concatenate(x) for x in (ks, vs, si, ps))
    if order == "shuffled":
        o = rng.permutation(len(ps))
        k, v, si, ps = k[o], v[o], si[o], ps[o]
    return np.ascontiguousarray(k), np.ascontiguousarray(v), si, ps


def ring_rows(s):
    return max(s.window + s.n_sink, 1)


def run_append(K, s, rk, rv, k, v, si, ps, bt, pool0, wk0, wv0, lens_after):
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window, n_sink=s.n_sink, group_size=s.group_size)
    pool = D(pool0)
    wk = D(wk0) if s.window + s.n_sink > 0 else None
    wv = D(wv0) if s.window + s.n_sink > 0 else None
    K.oscar_quantize_append(shape, D(rk), D(rv), D(k), D(v), D(si), D(ps), D(bt), D(lens_after),
                            pool, wk, wv)
    torch.cuda.synchronize()
    return H(pool), (H(wk, np.uint16) if wk is not None else None), (H(wv, np.uint16) if wv is not None else None)


def append_case(K, s, order="inorder", split_at=None, seed=0, rot=None):
    rng = np.random.default_rng(seed)
    rk, rv = rotations(s.cfg, s.n_kv_heads) if rot is None else rot
    rkf, rvf = ref.bf16_to_f64(rk), ref.bf16_to_f64(rv)
    bt, n_pages = wl.page_table(s)
    pool0 = rng.integers(0, 256, (n_pages, s.n_kv_heads, ref.block_bytes(s.group_size)), dtype=np.uint8)
    wsh = (s.batch, ring_rows(s), s.n_kv_heads, 128)
    wk0 = rng.integers(0, 65536, wsh, dtype=np.uint16)
    wv0 = rng.integers(0, 65536, wsh, dtype=np.uint16)
    k, v, si, ps = token_list(s, order, rng)
    chunks = [(0, len(ps))] if split_at is None else [(0, split_at), (split_at, len(ps))]
    pool_ref, wk_ref, wv_ref = pool0.copy(), wk0.copy(), wv0.copy()
    pool_g, wk_g, wv_g = pool0, wk0, wv0
    for a, b in chunks:
        pool_g, wk_g2, wv_g2 = run_append(K, s, rk, rv, k[a:b], v[a:b], si[a:b], ps[a:b], bt, pool_g, wk_g, wv_g,
                                          s.seq_lens)
        if s.window + s.n_sink > 0:
            wk_g, wv_g = wk_g2, wv_g2
        ref.append_ref(rkf, rvf, k[a:b], v[a:b], si[a:b], ps[a:b], bt, s.seq_lens, pool_ref, wk_ref, wv_ref,
                       s.window, s.n_sink, s.group_size)
    mism, excl, stray = P.check_append(pool0, pool_g, rkf, rvf, k, v, si, ps, bt, group=s.group_size)
    log(f"append {s.cfg} lens={list(s.seq_lens)} W={s.window} sinks={s.n_sink} g={s.group_size} {order}: "
        f"mismatches={mism} excluded={excl} stray={stray}")
    assert mism == 0 and stray == 0
    if s.window + s.n_sink > 0:
        assert np.array_equal(wk_g, wk_ref) and np.array_equal(wv_g, wv_ref)
    return excl


def test_append_inorder_ragged(K):
    append_case(K, make_spec(1, [300]))


def test_append_shuffled_multi_sequence(K):
    append_case(K, make_spec(1, [300, 37, 129], window=100), order="shuffled", seed=1)


def test_append_continuation_mid_page(K):
    append_case(K, make_spec(1, [300, 70]), split_at=20, seed=2)


def test_append_no_window(K):
    append_case(K, make_spec(1, [77, 200], window=0), seed=3)


def test_append_with_sinks(K):
    append_case(K, make_spec(1, [300, 37, 129], window=100, n_sink=40), order="shuffled", seed=5)


def test_append_sinks_no_window(K):
    append_case(K, make_spec(1, [77, 20], window=0, n_sink=64), split_at=30, seed=6)


def test_append_inorder_many_iterations(K):
    # over 4096 tokens per launch (on 256 CUs): workgroups run more than one
    # 128-token iteration, the next tile's rows loaded while the current one is
    # encoded; the second sequence ends in a partial page
    append_case(K, make_spec(1, [4500, 337], window=100), seed=7)


def test_append_shuffled_many_iterations(K):
    # the same with the tokens shuffled: every tile takes the per-token path
    append_case(K, make_spec(1, [2500, 1700, 701], window=64, n_sink=16), order="shuffled", seed=8)


def test_append_single_tokens(K):
    s = make_spec(5, [40, 17, 1, 99, 64], hq=64)
    rng = np.random.default_rng(4)
    rk, rv = rotations(5)
    rkf, rvf = ref.bf16_to_f64(rk), ref.bf16_to_f64(rv)
    bt, n_pages = wl.page_table(s)
    pool0 = rng.integers(0, 256, (n_pages, 8, ref.BLOCK), dtype=np.uint8)
    wk0 = rng.integers(0, 65536, (5, 128, 8, 128), dtype=np.uint16)
    wv0 = wk0.copy()
    k, v = wl.step_tokens(s, 1)
    si = np.arange(5, dtype=np.int32)
    ps = (s.seq_lens - 1).astype(np.int32)
    pool_g, wk_g, wv_g = run_append(K, s, rk, rv, k, v, si, ps, bt, pool0, wk0, wv0, s.seq_lens)
    mism, excl, stray = P.check_append(pool0, pool_g, rkf, rvf, k, v, si, ps, bt)
    assert mism == 0 and stray == 0
    wk_ref, wv_ref = wk0.copy(), wv0.copy()
    pool_ref = pool0.copy()
    ref.append_ref(rkf, rvf, k, v, si, ps, bt, s.seq_lens, pool_ref, wk_ref, wv_ref, 128)
    assert np.array_equal(wk_g, wk_ref) and np.array_equal(wv_g, wv_ref)


def test_append_empty_is_noop(K):
    s = make_spec(1, [16])
    shape = K.make_shape(32, 8, 128)
    pool = torch.zeros((1, 8, K.BLOCK_BYTES), dtype=torch.uint8, device=DEV)
    e = torch.zeros((0, 8, 128), dtype=torch.int16, device=DEV)
    i = torch.zeros((0,), dtype=torch.int32, device=DEV)
    rk, rv = rotations(1)
    K.oscar_quantize_append(shape, D(rk), D(rv), e, e, i, i, D(np.zeros((1, 1), np.int32)),
                            D(np.array([16], np.int32)), pool, None, None)
    torch.cuda.synchronize()
    assert int(pool.sum()) == 0


# ---------------------------------------------------------------------------
# decode on oracle-built caches
# ---------------------------------------------------------------------------

def oracle_cache(s, seed=0, rot=None):
    rk, rv = rotations(s.cfg, s.n_kv_heads) if rot is None else rot
    rkf, rvf = ref.bf16_to_f64(rk), ref.bf16_to_f64(rv)
    bt, n_pages = wl.page_table(s)
    rng = np.random.default_rng(seed)
    # unused slots hold random bytes (the decode must never read them)
    pool = rng.integers(0, 256, (n_pages, s.n_kv_heads, ref.block_bytes(s.group_size)), dtype=np.uint8)
    wk = np.zeros((s.batch, ring_rows(s), s.n_kv_heads, 128), np.uint16)
    wv = np.zeros_like(wk)
    k, v, si, ps = token_list(s)
    ref.append_ref(rkf, rvf, k, v, si, ps, bt, s.seq_lens, pool, wk, wv, s.window, s.n_sink, s.group_size)
    q = wl.decode_queries(s)[:, :s.n_q_heads]
    return rk, rv, rkf, rvf, bt, pool, wk, wv, q


def run_decode(K, s, rk, rv, q, bt, pool, wk, wv, max_len=None):
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window, n_sink=s.n_sink, group_size=s.group_size)
    max_len = int(s.seq_lens.max()) if max_len is None else max_len
    ws = torch.empty(K.oscar_decode_workspace_bytes(shape, s.batch, max_len), dtype=torch.uint8, device=DEV)
    out = torch.full((s.batch, s.n_q_heads, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.oscar_decode_attn(shape, D(rk), D(rv), D(q), D(s.seq_lens), max_len, D(bt), D(pool),
                        D(wk) if s.window + s.n_sink > 0 else None, D(wv) if s.window + s.n_sink > 0 else None,
                        out, ws)
    torch.cuda.synchronize()
    return H(out)


@pytest.mark.parametrize("cfg,lens,window,hq", [
    (1, [1000, 777], 128, 32),        # several splits, ragged tails
    (5, [600, 129, 128], 128, 64),     # G = 8; n = W + 1; n = W
    (1, [1, 50], 128, 32),             # pure window
    (1, [300], 0, 32),                 # no window
    (1, [700, 333], 100, 8),           # G = 1, window not a multiple of 16
    (1, [515], 128, 16),               # G = 2
    (1, [260, 1030], 128, 128),        # G = 16
    (1, [4100, 2500, 16], 128, 32),    # longer, splits of 256+ tokens
    (1, [1500, 200, 333], 300, 32),    # window of 10 chunks, the last one partial; n < W
    (1, [0, 700], 128, 32),            # an empty sequence in the batch
    (1, [2000, 1030, 1024, 5], 1024, 32),  # the largest window
    (1, [1280], 128, 32),              # history of exactly 9 tiles
])
def test_decode_small(K, cfg, lens, window, hq):
    s = make_spec(cfg, lens, window, hq)
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, window)
    err = P.attn_rel_err(got, want)
    log(f"decode lens={lens} W={window} Hq={hq}: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


@pytest.mark.parametrize("lens,window,n_sink,hq", [
    ([700, 333], 128, 4, 32),          # a few sinks
    ([1500, 200], 256, 64, 32),        # W + sinks = 320 bf16 tokens (0.24 % of 128K)
    ([300, 90], 0, 100, 32),           # sinks and no window; n < n_sink
    ([5000, 129], 128, 300, 64),       # sinks over two tiles (masked in the INT2 tiles); G = 8
    ([2000, 1100], 1024, 1024, 32),    # the largest ring: sinks reach into the window
])
def test_decode_with_sinks(K, lens, window, n_sink, hq):
    s = make_spec(1, lens, window, hq, n_sink=n_sink)
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, window, n_sink=n_sink)
    err = P.attn_rel_err(got, want)
    log(f"decode sinks lens={lens} W={window} n_sink={n_sink} Hq={hq}: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


@pytest.mark.parametrize("hkv,hq", [(1, 4), (2, 8), (4, 16), (6, 24), (2, 2)])
def test_decode_kv_head_counts(K, hkv, hq):
    """KV head counts that give 1, 2 or 4 heads per split workgroup, and their groups."""
    s = make_spec(1, [1400, 531], 128, hq, hkv=hkv)
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, 128)
    err = P.attn_rel_err(got, want)
    log(f"decode Hkv={hkv} Hq={hq}: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


def test_decode_batch_above_64(K):
    """130 short ragged sequences (some empty, some shorter than the window):
    the per-sequence loops of the tile prefix run over several lane passes and
    the units outnumber the lanes of a wave."""
    lens = [int(x) for x in np.random.default_rng(7).integers(0, 700, 130)]
    lens[3] = 0
    lens[77] = 129
    s = make_spec(1, lens, 128, 32)
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, 128)
    err = P.attn_rel_err(got, want)
    log(f"decode B=130: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


def test_decode_every_sequence_empty(K):
    """seq_lens all 0 (and max_seq_len 0) over an existing cache: zeros."""
    s = make_spec(1, [40, 300])
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    s.seq_lens = np.zeros(2, np.int32)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv, max_len=0)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, 128)
    assert np.array_equal(want, np.zeros_like(want))
    assert np.array_equal(got, np.zeros_like(got))


def test_decode_max_len_above_actual(K):
    """The split plan follows the host max_seq_len; shorter sequences still work."""
    s = make_spec(1, [900, 20])
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    bt2 = np.full((2, 400), -1, np.int32)
    bt2[:, :bt.shape[1]] = bt
    got = run_decode(K, s, rk, rv, q, bt2, pool, wk, wv, max_len=6000)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, 128)
    assert P.attn_rel_err(got, want).max() <= P.ATTN_TOL


def test_bf16_comparator_small(K):
    s = make_spec(1, [1000, 77])
    bt, n_pages = wl.page_table(s)
    kv = np.zeros((n_pages, 8, ref.BF16_BLOCK), np.uint16)
    k, v, si, ps = token_list(s)
    ref.append_bf16_ref(k, v, si, ps, bt, kv)
    q = wl.decode_queries(s)
    shape = K.make_shape(32, 8, 128)
    kvd = torch.zeros((n_pages, 8, ref.BF16_BLOCK), dtype=torch.int16, device=DEV)
    K.oscar_bf16_append(shape, D(k), D(v), D(si), D(ps), D(bt), kvd)
    torch.cuda.synchronize()
    assert np.array_equal(H(kvd, np.uint16), kv)
    ws = torch.empty(K.oscar_decode_workspace_bytes(shape, 2, 1000), dtype=torch.uint8, device=DEV)
    out = torch.empty((2, 32, 128), dtype=torch.float32, device=DEV)
    K.oscar_bf16_decode_attn(shape, D(q), D(s.seq_lens), 1000, D(bt), kvd, out, ws)
    torch.cuda.synchronize()
    want = ref.decode_bf16_ref(q, s.seq_lens, bt, kv, 8)
    assert P.attn_rel_err(H(out), want).max() <= P.ATTN_TOL


def test_gpu_wait_holds_the_stream(K):
    """The measurement helper that holds a stream: the event pair around a 2 ms
    wait spans at least most of it, and the stream drains."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    K.oscar_gpu_wait(2000)
    e1.record()
    torch.cuda.synchronize()
    assert 1.5 <= e0.elapsed_time(e1) <= 200.0


# ---------------------------------------------------------------------------
# full-size workloads (sampled checks)
# ---------------------------------------------------------------------------

def full_cache(K, s, keep=(), rot=None, tokens=None):
    """Prefill every sequence of workload s through the HIP append (rotation
    ``rot``, default the oracle's calibration); returns the device state and the
    host token arrays of the sequences in ``keep``.  ``tokens(b)``, if given,
    returns sequence b's (k, v, seq_idx, pos) instead of drawing them."""
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window, group_size=s.group_size)
    rk, rv = rotations(s.cfg) if rot is None else rot
    rkd, rvd = D(rk), D(rv)
    bt, n_pages = wl.page_table(s)
    btd, lensd = D(bt), D(s.seq_lens)
    pool = torch.zeros((n_pages, 8, K.block_bytes(s.group_size)), dtype=torch.uint8, device=DEV)
    wk = torch.zeros((s.batch, s.window, 8, 128), dtype=torch.int16, device=DEV)
    wv = torch.zeros_like(wk)
    kept = {}
    for b in range(s.batch):
        k, v, si, ps = wl.prefill_tokens(s, b) if tokens is None else tokens(b)
        K.oscar_quantize_append(shape, rkd, rvd, D(k), D(v), D(si), D(ps), btd, lensd, pool, wk, wv)
        if b in keep:
            kept[b] = (k, v)
    torch.cuda.synchronize()
    return dict(shape=shape, rk=rk, rv=rv, rkd=rkd, rvd=rvd, bt=bt, btd=btd, pool=pool, wk=wk, wv=wv, kept=kept)


def decode_full(K, s, c, q, lens):
    ws = torch.empty(K.oscar_decode_workspace_bytes(c["shape"], s.batch, int(lens.max())), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty((s.batch, s.n_q_heads, 128), dtype=torch.float32, device=DEV)
    K.oscar_decode_attn(c["shape"], c["rkd"], c["rvd"], D(q), D(lens), int(lens.max()), c["btd"], c["pool"],
                        c["wk"], c["wv"], out, ws)
    torch.cuda.synchronize()
    return H(out)


def oracle_overwrite(s, c, b, extra=None, heads=None):
    """Encode sequence b with the oracle (its tokens plus ``extra``; the KV heads
    in ``heads``, default all) and upload those heads' blocks of its pages and
    their window rows into the device cache, so the device decode of (b, h) runs
    on exactly the oracle's cache.  Returns the oracle's local copy (pool rows of
    b's pages, window ring) for ``decode_ref``."""
    k, v = c["kept"][b]
    if extra is not None:
        k = np.concatenate([k, extra[0]])
        v = np.concatenate([v, extra[1]])
    hs = list(range(s.n_kv_heads)) if heads is None else list(heads)
    n = len(k)
    n_pg = -(-n // 16)
    pages = torch.from_numpy(c["bt"][b][:n_pg].astype(np.int64)).to(DEV)
    local = H(c["pool"].index_select(0, pages))
    wk = H(c["wk"][b], np.uint16).copy()
    wv = H(c["wv"][b], np.uint16).copy()
    sub = np.ascontiguousarray(local[:, hs])
    wks, wvs = np.ascontiguousarray(wk[:, hs]), np.ascontiguousarray(wv[:, hs])
    ref.append_sequence_ref(ref.bf16_to_f64(c["rk"][hs]), ref.bf16_to_f64(c["rv"][hs]),
                            np.ascontiguousarray(k[:, hs]), np.ascontiguousarray(v[:, hs]),
                            np.arange(n_pg, dtype=np.int32), sub, wks, wvs, s.window, group=s.group_size)
    local[:, hs] = sub
    wk[:, hs] = wks
    wv[:, hs] = wvs
    c["pool"].index_copy_(0, pages, D(local))
    c["wk"][b] = D(wk)
    c["wv"][b] = D(wv)
    torch.cuda.synchronize()
    return local, wk, wv, n


def check_sampled(s, c, q, got, pairs, oracle):
    """oracle: {b: (local pool, window k, window v, n)} from oracle_overwrite."""
    rkf, rvf = ref.bf16_to_f64(c["rk"]), ref.bf16_to_f64(c["rv"])
    g = s.gqa
    worst = 0.0
    for b, h in pairs:
        local, wk, wv, n = oracle[b]
        row = np.arange(local.shape[0], dtype=np.int32)[None]
        want = ref.decode_ref(rkf, rvf, q[b:b + 1], np.array([n]), row, local, wk[None], wv[None], s.window,
                              pairs=[(0, h)], group=s.group_size)[0, h * g:(h + 1) * g]
        err = P.attn_rel_err(got[b, h * g:(h + 1) * g], want)
        log(f"  pair ({b}, {h}): rel err per q head {np.array2string(err, precision=2)}")
        worst = max(worst, float(err.max()))
    log(f"config {s.cfg} g={s.group_size}: sampled pairs {pairs}: max rel err {worst:.3e}")
    assert worst <= P.ATTN_TOL


def sampled_append_check(s, c, b, n_sample=512, seed=0):
    rng = np.random.default_rng(seed)
    k, v = c["kept"][b]
    idx = rng.choice(len(k), size=min(n_sample, len(k)), replace=False)
    pool = H(c["pool"])
    pos = np.arange(len(k), dtype=np.int32)
    si = np.full(len(k), b, np.int32)
    mism, excl, _ = P.check_append(None, pool, ref.bf16_to_f64(c["rk"]), ref.bf16_to_f64(c["rv"]), k, v, si, pos,
                                   c["bt"], sample=idx, group=s.group_size)
    log(f"config {s.cfg} g={s.group_size} seq {b}: {len(idx)} sampled tokens, mismatches={mism} excluded={excl}")
    assert mism == 0
    return pool


def codes_span_levels(pool, bt, lens, hkv=8, group=128):
    """Every written group holds codes 0 and 3 (its min and max), any size."""
    for b in range(len(lens)):
        n = int(lens[b])
        pages = bt[b][:(n + 15) // 16]
        for c0 in range(0, len(pages), 256):
            pg = pages[c0:c0 + 256]
            blk = pool[pg]                                                   # [np][hkv][block bytes]
            kc = ref.unpack_k_rows(blk[..., :512].reshape(len(pg), hkv, 16, 32)).astype(np.int8)
            vc = ref.unpack_v_words(ref.v_words(blk)).astype(np.int8)       # [np][hkv][16][128]
            ntok = min(16 * len(pg), n - 16 * c0)
            for cc in (kc, vc):
                cc = cc.transpose(0, 2, 1, 3).reshape(-1, hkv, 128 // group, group)[:ntok]
                assert (cc.min(-1) == 0).all() and (cc.max(-1) == 3).all()


def test_full_config1(K):
    s = wl.spec(1)
    log("config 1 full: building cache")
    c = full_cache(K, s, keep=(0,))
    q = wl.decode_queries(s)
    pool = sampled_append_check(s, c, 0, n_sample=2048)
    codes_span_levels(pool, c["bt"], s.seq_lens)
    oracle = {0: oracle_overwrite(s, c, 0)}
    got = decode_full(K, s, c, q, s.seq_lens)
    check_sampled(s, c, q, got, [(0, h) for h in range(8)], oracle)


def test_full_config4_append(K):
    s = wl.spec(4)
    log("config 4 full: appending 65536 tokens")
    c = full_cache(K, s, keep=(0,))
    pool = sampled_append_check(s, c, 0, n_sample=1024, seed=4)
    codes_span_levels(pool, c["bt"], s.seq_lens)
    k, v = c["kept"][0]
    assert np.array_equal(H(c["wk"], np.uint16)[0][np.arange(65536 - 128, 65536) % 128], k[-128:])
    assert np.array_equal(H(c["wv"], np.uint16)[0][np.arange(65536 - 128, 65536) % 128], v[-128:])


def test_full_config2(K):
    s = wl.spec(2)
    log("config 2 full: building cache")
    c = full_cache(K, s, keep=(3, 11))
    q = wl.decode_queries(s)
    sampled_append_check(s, c, 11, n_sample=512, seed=2)
    oracle = {b: oracle_overwrite(s, c, b) for b in (3, 11)}
    got = decode_full(K, s, c, q, s.seq_lens)
    assert np.isfinite(got).all()
    check_sampled(s, c, q, got, [(3, 0), (3, 5), (11, 7)], oracle)


@functools.lru_cache(maxsize=1)
def config3_tokens():
    """Every sequence's prefill tokens of the long-context workload, drawn once
    for the tests that build its cache (about 3.3 GB of bf16 on the host)."""
    s = wl.spec(3)
    return s, {b: wl.prefill_tokens(s, b) for b in range(s.batch)}


@pytest.mark.timeout(900)
def test_full_config3(K):
    """Long-context workload at full size, in the bench's launch configuration:
    two KV heads of every sequence (one in each group of 4 heads a split
    workgroup reads side by side, so every merge unit, and with it the share
    boundaries of every one of its workgroups, is covered) decoded from
    oracle-encoded blocks and compared with the oracle."""
    s, toks = config3_tokens()
    log("config 3 full: building cache")
    c = full_cache(K, s, keep=tuple(range(s.batch)), tokens=toks.__getitem__)
    q = wl.decode_queries(s)
    sampled_append_check(s, c, 7, n_sample=512, seed=3)
    pairs = [(b, h) for b in range(s.batch) for h in (b % 4, 4 + (3 * b + 1) % 4)]
    oracle = {b: oracle_overwrite(s, c, b, heads=[h for bb, h in pairs if bb == b]) for b in range(s.batch)}
    got = decode_full(K, s, c, q, s.seq_lens)
    assert np.isfinite(got).all()
    check_sampled(s, c, q, got, pairs, oracle)


@pytest.mark.parametrize("arm", ["hadamard", "identity"])
def test_arm_append(K, arm):
    """The quality harness's comparison rotations through the append kernel:
    codes, scales and zeros under the encoder rule, bf16 ring byte-exact."""
    append_case(K, make_spec(1, [300, 37, 129], window=100), order="shuffled", seed=11, rot=arm_rotation(arm))
    append_case(K, make_spec(1, [77, 200], window=0), seed=12, rot=arm_rotation(arm))


@pytest.mark.parametrize("arm", ["hadamard", "identity"])
@pytest.mark.parametrize("cfg,lens,window,hq", [
    (1, [1000, 777], 128, 32),
    (5, [600, 129, 128], 128, 64),
    (1, [4100, 2500, 16], 128, 32),
    (1, [0, 700], 128, 8),
])
def test_arm_decode_small(K, arm, cfg, lens, window, hq):
    """Decode under the comparison rotations on oracle-built caches, every
    output compared with the oracle."""
    s = make_spec(cfg, lens, window, hq)
    rot = arm_rotation(arm)
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s, rot=rot)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, window)
    err = P.attn_rel_err(got, want)
    log(f"decode {arm} lens={lens} W={window} Hq={hq}: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("arm", ["hadamard", "identity"])
def test_full_config3_arm(K, arm):
    """Long-context workload at full size under a comparison rotation: sampled
    append records and sampled (sequence, KV head) outputs against the oracle."""
    s, toks = config3_tokens()
    log(f"config 3 full, {arm}: building cache")
    c = full_cache(K, s, keep=(1, 6), rot=arm_rotation(arm), tokens=toks.__getitem__)
    q = wl.decode_queries(s)
    sampled_append_check(s, c, 6, n_sample=256, seed=13)
    pairs = [(1, 2), (1, 5), (6, 0), (6, 7)]
    oracle = {b: oracle_overwrite(s, c, b, heads=[h for bb, h in pairs if bb == b]) for b in (1, 6)}
    got = decode_full(K, s, c, q, s.seq_lens)
    assert np.isfinite(got).all()
    check_sampled(s, c, q, got, pairs, oracle)


def test_full_config5_two_steps(K):
    s = wl.spec(5)
    log(f"config 5 full: lens sum {int(s.seq_lens.sum())} max {int(s.seq_lens.max())}")
    longest = int(np.argmax(s.seq_lens))
    keep = (0, longest)
    c = full_cache(K, s, keep=keep)
    q0 = wl.decode_queries(s, 0)
    sampled_append_check(s, c, longest, n_sample=256, seed=5)
    oracle = {b: oracle_overwrite(s, c, b) for b in keep}
    got0 = decode_full(K, s, c, q0, s.seq_lens)
    check_sampled(s, c, q0, got0, [(0, 3), (longest, 5)], oracle)
    # append one token per sequence through the device, then decode again
    lens1 = (s.seq_lens + 1).astype(np.int32)
    k1, v1 = wl.step_tokens(s, 1)
    pool_before = H(c["pool"])
    K.oscar_quantize_append(c["shape"], c["rkd"], c["rvd"], D(k1), D(v1), D(np.arange(s.batch, dtype=np.int32)),
                            D(s.seq_lens), c["btd"], D(lens1), c["pool"], c["wk"], c["wv"])
    torch.cuda.synchronize()
    mism, excl, stray = P.check_append(pool_before, H(c["pool"]), ref.bf16_to_f64(c["rk"]), ref.bf16_to_f64(c["rv"]),
                                       k1, v1, np.arange(s.batch), s.seq_lens, c["bt"])
    assert mism == 0 and stray == 0
    q1 = wl.decode_queries(s, 1)
    oracle = {b: oracle_overwrite(s, c, b, extra=(k1[b:b + 1], v1[b:b + 1])) for b in keep}
    got1 = decode_full(K, s, c, q1, lens1)
    check_sampled(s, c, q1, got1, [(0, 0), (longest, 7)], oracle)


def test_full_config3_bf16_comparator(K):
    s = wl.spec(3)
    shape = K.make_shape(32, 8, 128)
    bt, n_pages = wl.page_table(s)
    btd = D(bt)
    kv = torch.zeros((n_pages, 8, K.BF16_BLOCK_ELEMS), dtype=torch.int16, device=DEV)
    kept = {}
    for b in range(s.batch):
        k, v, si, ps = wl.prefill_tokens(s, b)
        K.oscar_bf16_append(shape, D(k), D(v), D(si), D(ps), btd, kv)
        if b in (5,):
            kept[b] = (k, v)
    q = wl.decode_queries(s)
    ws = torch.empty(K.oscar_decode_workspace_bytes(shape, 8, 100000), dtype=torch.uint8, device=DEV)
    out = torch.empty((8, 32, 128), dtype=torch.float32, device=DEV)
    K.oscar_bf16_decode_attn(shape, D(q), D(s.seq_lens), 100000, btd, kv, out, ws)
    torch.cuda.synchronize()
    k, v = kept[5]
    got = H(out)
    worst = 0.0
    for h in (0, 4):
        kk = ref.bf16_to_f64(k[:, h])
        vv = ref.bf16_to_f64(v[:, h])
        for j in range(4):
            qq = ref.bf16_to_f64(q[5, 4 * h + j])
            sc = kk @ qq / np.sqrt(128)
            p = np.exp(sc - sc.max())
            want = (p @ vv) / p.sum()
            worst = max(worst, np.abs(got[5, 4 * h + j] - want).max() / np.abs(want).max())
    log(f"bf16 comparator config 3 sampled: max rel err {worst:.3e}")
    assert worst <= P.ATTN_TOL
