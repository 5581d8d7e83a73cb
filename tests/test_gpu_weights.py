"""GPU parity of the INT2 decode on caches built to stress the softmax weights.

The split kernel carries each softmax weight w = p s_v of a 128-token tile as
fixed-point digits relative to the largest weight of its head in that tile.
These cases push that representation to its edges, each on an oracle-built
cache compared with the oracle's decode at the usual tolerance:

- one token per tile whose score stands far above the rest of the tile (the
  tile's other weights are then tiny next to its largest);
- value groups with zero scale (all-zero V tokens: s_v = 0, so w = 0), up to
  whole tiles of them;
- a few tokens whose scores exceed the bulk of the history by ~40-80 in the
  natural-log domain, so that whole tiles carry weights of 2^-60 .. 2^-115,
  partly under the kernel's 2^-100 exponent floor, next to tiles with
  moderate gaps.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from oracle import oscar_ref as ref  # noqa: E402
import parity as P  # noqa: E402
from test_gpu_parity import K, log, make_spec, oracle_cache, rotations, run_decode, token_list  # noqa: E402,F401


def f32(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def key_toward_queries(q_heads, gap):
    """A key whose score, averaged over the query heads q_heads [G][128], is
    ``gap`` (natural-log units, scale 1/sqrt(d)): a multiple of their mean."""
    qm = q_heads.mean(axis=0)
    c = gap * np.sqrt(128.0) / max(float(np.mean(q_heads @ qm)), 1e-12)
    return c * qm


def cache_from_tokens(s, k, v, seed=0):
    """Oracle-encoded cache of the given in-order tokens of every sequence."""
    rk, rv = rotations(s.cfg, s.n_kv_heads)
    rkf, rvf = ref.bf16_to_f64(rk), ref.bf16_to_f64(rv)
    bt, n_pages = wl.page_table(s)
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 256, (n_pages, s.n_kv_heads, ref.block_bytes(s.group_size)), dtype=np.uint8)
    wk = np.zeros((s.batch, max(s.window + s.n_sink, 1), s.n_kv_heads, 128), np.uint16)
    wv = np.zeros_like(wk)
    si = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(s.seq_lens)])
    ps = np.concatenate([np.arange(n, dtype=np.int32) for n in s.seq_lens])
    ref.append_ref(rkf, rvf, k, v, si, ps, bt, s.seq_lens, pool, wk, wv, s.window, s.n_sink, s.group_size)
    return rk, rv, rkf, rvf, bt, pool, wk, wv


def check(K, s, k, v, q, label):
    rk, rv, rkf, rvf, bt, pool, wk, wv = cache_from_tokens(s, k, v)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, s.window)
    err = P.attn_rel_err(got, want)
    log(f"{label} lens={list(s.seq_lens)} Hq={s.n_q_heads}: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


def seq_offsets(s):
    return np.concatenate([[0], np.cumsum(s.seq_lens)])


@pytest.mark.parametrize("hq,gap", [(32, 12.0), (64, 12.0), (32, 30.0)])
def test_decode_one_dominant_token_per_tile(K, hq, gap):
    s = make_spec(1, [3000, 1290], 128, hq)
    k, v, _, _ = token_list(s)
    q = wl.decode_queries(s)[:, :hq]
    qf = f32(q)
    kf = f32(k)
    rng = np.random.default_rng(11)
    off = seq_offsets(s)
    G = s.gqa
    for b in range(s.batch):
        hist = int(s.seq_lens[b]) - s.window
        for t0 in range(0, hist, 128):
            t = off[b] + t0 + int(rng.integers(0, min(128, hist - t0)))
            for h in range(s.n_kv_heads):
                # the tile's standout: well above the rest, by a different
                # margin per tile (some tiles stand above the running maximum)
                kf[t, h] = key_toward_queries(qf[b, h * G:(h + 1) * G], gap * (0.5 + rng.random()))
    check(K, s, ref.bf16_bits(kf), v, q, f"dominant token per tile (gap {gap})")


def test_decode_zero_value_groups(K):
    s = make_spec(1, [2000, 700, 900], 128, 32)
    k, v, _, _ = token_list(s)
    q = wl.decode_queries(s)[:, :32]
    vf = f32(v)
    rng = np.random.default_rng(12)
    off = seq_offsets(s)
    # sequence 0: a random 30 % of the tokens (per KV head) and two whole tiles
    n0 = int(s.seq_lens[0])
    mask = rng.random((n0, s.n_kv_heads)) < 0.3
    vf[off[0]:off[0] + n0][mask] = 0.0
    vf[off[0] + 256:off[0] + 512] = 0.0
    # sequence 1: every history token (the window keeps its values)
    vf[off[1]:off[1] + int(s.seq_lens[1]) - s.window] = 0.0
    # sequence 2: one KV head entirely
    vf[off[2]:off[2] + int(s.seq_lens[2]), 3] = 0.0
    check(K, s, k, ref.bf16_bits(vf), q, "zero value groups")


@pytest.mark.parametrize("hq", [32, 64])
def test_decode_vanishing_weights(K, hq):
    s = make_spec(1, [2600, 1500], 128, hq)
    k, v, _, _ = token_list(s)
    q = wl.decode_queries(s)[:, :hq]
    qf, kf = f32(q), f32(k)
    rng = np.random.default_rng(13)
    off = seq_offsets(s)
    G = s.gqa
    for b in range(s.batch):
        hist = int(s.seq_lens[b]) - s.window
        for h in range(s.n_kv_heads):
            qh = qf[b, h * G:(h + 1) * G]
            # the bulk of the history below zero and three tokens above it, ~20
            # each way on the group's average (single heads see up to about
            # twice that): gaps of ~40-80 (natural log), so in most heads the
            # bulk's weights are ~2^-60 .. 2^-115 of the largest, nonzero in
            # fp32 and partly under the 2^-100 exponent floor
            kf[off[b]:off[b] + hist, h] += key_toward_queries(qh, -20.0)
            for t in rng.choice(hist, 3, replace=False):
                kf[off[b] + t, h] = key_toward_queries(qh, 20.0)
            # tiles with standouts anywhere in between
            for t in rng.choice(hist, 12, replace=False):
                kf[off[b] + t, h] = key_toward_queries(qh, -18.0 + 36.0 * rng.random())
    check(K, s, ref.bf16_bits(kf), v, q, "vanishing weights")
