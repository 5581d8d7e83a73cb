"""GPU parity of the fused decode step (oscar_decode_step, through the C ABI).

The step appends the newest token of every sequence inside the decode's
query-preparation launch.  Its pool, rings and output must equal, byte for
byte, those of oscar_quantize_append of the same tokens followed by
oscar_decode_attn on the same cache state (both paths are checked against the
oracle elsewhere); one case is also compared with the oracle directly.
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

DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_int2_amd as K

    return K


def D(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def H(t, dtype=None):
    a = t.cpu().numpy()
    return a.view(dtype) if dtype is not None else a


@functools.lru_cache(maxsize=None)
def rotations(cfg, hkv=8):
    s = wl.spec(cfg)
    qc, kc, vc = wl.calibration_set(s)
    rk, rv, _, _ = ref.calibrate_ref(qc[:hkv], kc[:hkv], vc[:hkv])
    return ref.bf16_bits(rk), ref.bf16_bits(rv)


def make_spec(cfg, lens, window=128, hq=None, n_sink=0, group=128):
    s = wl.spec(cfg, batch=len(lens))
    s.seq_lens = np.asarray(lens, np.int32)
    s.window = window
    s.n_sink = n_sink
    s.group_size = group
    if hq is not None:
        s.n_q_heads = hq
    return s


def step_case(K, s, max_len=None, seed=0, oracle=False):
    """Cache of every sequence's tokens but its newest (appended on the GPU
    into a pool of random bytes), then the newest tokens (a) appended and
    decoded by the two plain calls, (b) by one oscar_decode_step; returns the
    host copies of (b)'s pool, rings and output."""
    hkv = s.n_kv_heads
    rk, rv = rotations(s.cfg, hkv)
    shape = K.make_shape(s.n_q_heads, hkv, s.window, n_sink=s.n_sink, group_size=s.group_size)
    max_len = int(s.seq_lens.max()) if max_len is None else max_len
    bt, n_pages = wl.page_table(s)
    rng = np.random.default_rng(seed)
    ring = max(s.window + s.n_sink, 1)
    pool = D(rng.integers(0, 256, (n_pages, hkv, ref.block_bytes(s.group_size)), dtype=np.uint8))
    wk = D(rng.integers(0, 65536, (s.batch, ring, hkv, 128), dtype=np.uint16))
    wv = D(rng.integers(0, 65536, (s.batch, ring, hkv, 128), dtype=np.uint16))
    rkd, rvd, btd, lens = D(rk), D(rv), D(bt), D(s.seq_lens)
    k_new = np.zeros((s.batch, hkv, 128), np.uint16)
    v_new = np.zeros_like(k_new)
    newest = []  # sequences that get a new token: 1 <= n <= max_len
    for b in range(s.batch):
        n = int(s.seq_lens[b])
        if n < 1:
            continue
        k, v, si, ps = wl.prefill_tokens(s, b)
        k, v = k[:, :hkv], v[:, :hkv]
        if n <= max_len:
            k_new[b], v_new[b] = k[n - 1], v[n - 1]
            newest.append(b)
            k, v, si, ps = k[:-1], v[:-1], si[:-1], ps[:-1]
        if len(ps):
            K.oscar_quantize_append(shape, rkd, rvd, D(k), D(v), D(si), D(ps), btd, lens, pool,
                                    wk if s.window + s.n_sink > 0 else None, wv if s.window + s.n_sink > 0 else None)
    torch.cuda.synchronize()
    q = D(wl.decode_queries(s)[:, :s.n_q_heads])
    use_ring = s.window + s.n_sink > 0
    ws = torch.empty(K.oscar_decode_workspace_bytes(shape, s.batch, max_len), dtype=torch.uint8, device=DEV)

    # (a) the two plain calls
    pa, wka, wva = pool.clone(), wk.clone(), wv.clone()
    nb = np.asarray(newest, np.int32)
    if len(nb):
        K.oscar_quantize_append(shape, rkd, rvd, D(k_new[nb]), D(v_new[nb]), D(nb), D(s.seq_lens[nb] - 1), btd, lens,
                                pa, wka if use_ring else None, wva if use_ring else None)
    out_a = torch.full((s.batch, s.n_q_heads, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.oscar_decode_attn(shape, rkd, rvd, q, lens, max_len, btd, pa, wka if use_ring else None,
                        wva if use_ring else None, out_a, ws)
    # (b) the fused step on the same state
    pb, wkb, wvb = pool.clone(), wk.clone(), wv.clone()
    out_b = torch.full_like(out_a, float("nan"))
    K.oscar_decode_step(shape, rkd, rvd, D(k_new), D(v_new), q, lens, max_len, btd, pb, wkb if use_ring else None,
                        wvb if use_ring else None, out_b, ws)
    torch.cuda.synchronize()
    log(f"step lens={list(s.seq_lens)} max_len={max_len} W={s.window} sinks={s.n_sink} g={s.group_size} "
        f"Hq={s.n_q_heads}: newest appended for {len(newest)} sequences")
    assert torch.equal(pa, pb), "pool differs from append + decode"
    assert torch.equal(wka, wkb) and torch.equal(wva, wvb), "rings differ from append + decode"
    assert np.array_equal(H(out_a).view(np.uint32), H(out_b).view(np.uint32)), "output differs from append + decode"
    assert np.isfinite(H(out_b)).all()
    if oracle:
        rkf, rvf = ref.bf16_to_f64(rk), ref.bf16_to_f64(rv)
        want = ref.decode_ref(rkf, rvf, H(q, np.uint16), np.minimum(s.seq_lens, max_len), bt, H(pb),
                              H(wkb, np.uint16), H(wvb, np.uint16), s.window, n_sink=s.n_sink, group=s.group_size)
        err = P.attn_rel_err(H(out_b), want)
        log(f"  against the oracle: max rel err {err.max():.3e}")
        assert err.max() <= P.ATTN_TOL
    return H(pb), H(wkb, np.uint16), H(wvb, np.uint16), H(out_b)


def test_step_matches_append_then_decode(K):
    # a one-token and an empty sequence among ragged ones; checked against the oracle too
    step_case(K, make_spec(1, [300, 37, 129, 1, 0]), oracle=True)


def test_step_no_window(K):
    # the newest token is INT2 history, read by the split kernel after the append
    step_case(K, make_spec(1, [700, 333, 16, 17], window=0))


def test_step_sinks(K):
    # the newest token of the shortest sequence also enters its sink row
    step_case(K, make_spec(1, [300, 90, 30], window=100, n_sink=40), oracle=True)


def test_step_sinks_no_window(K):
    # without a window the second sequence's newest token is read as a sink
    step_case(K, make_spec(1, [150, 90], window=0, n_sink=100), oracle=True)


@pytest.mark.parametrize("group", [64, 32])
def test_step_finer_groups(K, group):
    step_case(K, make_spec(1, [500, 129, 64], group=group))


@pytest.mark.parametrize("cfg,hq", [(1, 8), (5, 64), (1, 128)])
def test_step_query_head_counts(K, cfg, hq):
    step_case(K, make_spec(cfg, [400, 131], hq=hq))


def test_step_many_sequences(K):
    # more than 64 sequences: several append workgroups per (KV head, K|V)
    lens = np.random.default_rng(11).integers(1, 300, 70)
    step_case(K, make_spec(1, list(lens)))


def test_step_length_above_max_len(K):
    # a sequence longer than max_seq_len gets no new token and is decoded clamped
    step_case(K, make_spec(1, [300, 500, 120]), max_len=400)


def test_step_timed_equals_plain(K):
    s = make_spec(1, [260, 77])
    pool1, wk1, wv1, out1 = step_case(K, s)
    # the same step through the timed entry point
    hkv = s.n_kv_heads
    rk, rv = rotations(s.cfg, hkv)
    shape = K.make_shape(s.n_q_heads, hkv, s.window)
    bt, n_pages = wl.page_table(s)
    rng = np.random.default_rng(0)
    pool = D(rng.integers(0, 256, (n_pages, hkv, ref.BLOCK), dtype=np.uint8))
    wk = D(rng.integers(0, 65536, (s.batch, s.window, hkv, 128), dtype=np.uint16))
    wv = D(rng.integers(0, 65536, (s.batch, s.window, hkv, 128), dtype=np.uint16))
    rkd, rvd, btd, lens = D(rk), D(rv), D(bt), D(s.seq_lens)
    k_new = np.zeros((s.batch, hkv, 128), np.uint16)
    v_new = np.zeros_like(k_new)
    for b in range(s.batch):
        k, v, si, ps = wl.prefill_tokens(s, b)
        k_new[b], v_new[b] = k[-1, :hkv], v[-1, :hkv]
        K.oscar_quantize_append(shape, rkd, rvd, D(k[:-1, :hkv]), D(v[:-1, :hkv]), D(si[:-1]), D(ps[:-1]), btd, lens,
                                pool, wk, wv)
    q = D(wl.decode_queries(s)[:, :s.n_q_heads])
    ws = torch.empty(K.oscar_decode_workspace_bytes(shape, s.batch, int(s.seq_lens.max())), dtype=torch.uint8,
                     device=DEV)
    out = torch.full((s.batch, s.n_q_heads, 128), float("nan"), dtype=torch.float32, device=DEV)
    e0, e1 = K.Event(), K.Event()
    K.oscar_decode_step_timed(shape, rkd, rvd, D(k_new), D(v_new), q, lens, int(s.seq_lens.max()), btd, pool, wk, wv,
                              out, ws, e0, e1)
    torch.cuda.synchronize()
    assert K.Event.elapsed_ms(e0, e1) > 0
    assert np.array_equal(H(pool), pool1)
    assert np.array_equal(H(wk, np.uint16), wk1) and np.array_equal(H(wv, np.uint16), wv1)
    assert np.array_equal(H(out).view(np.uint32), out1.view(np.uint32))
