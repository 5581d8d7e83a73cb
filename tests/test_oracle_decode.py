"""Pins of the oracle's decode attention (CPU only).

(i)   brute force on tiny inputs: un-rotate the dequantised history with an exactly
      orthogonal R and run textbook softmax attention in pure Python loops over
      the original token order (no pool, no ring) -- this also pins the page /
      slot / window-ring addressing of append_ref and decode_ref;
(ii)  n <= W: equals torch's scaled_dot_product_attention in fp64 on the bf16 K/V;
(iii) n = 1, W = 0: o = R_V^T v';
(iv)  identical keys, W = 0: o = mean of the un-rotated dequantised values;
(v)   the bf16 comparator equals torch SDPA.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import oscar_ref as ref


def orthogonal(rng, hkv):
    return np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(hkv)])


def build(rng, lens, window, hq=8, hkv=2, cfg=1, rot=None, n_sink=0, group=128):
    s = wl.spec(cfg, batch=len(lens))
    s.seq_lens = np.asarray(lens, dtype=np.int32)
    s.window = window
    s.n_q_heads, s.n_kv_heads = hq, hkv
    bt, n_pages = wl.page_table(s)
    pool = np.zeros((n_pages, hkv, ref.block_bytes(group)), dtype=np.uint8)
    win_k = np.zeros((len(lens), max(window + n_sink, 1), hkv, 128), dtype=np.uint16)
    win_v = np.zeros_like(win_k)
    rk, rv = rot if rot is not None else (orthogonal(rng, hkv), orthogonal(rng, hkv))
    kv = {}
    for b in range(len(lens)):
        k, v = wl.context_kv(s, b)
        k, v = k[:, :hkv], v[:, :hkv]
        n = k.shape[0]
        ref.append_ref(rk, rv, k, v, np.full(n, b, np.int32), np.arange(n, dtype=np.int32),
                       bt, s.seq_lens, pool, win_k, win_v, window, n_sink, group)
        kv[b] = (k, v)
    q = wl.decode_queries(s)[:, :hq]
    return s, bt, pool, win_k, win_v, rk, rv, kv, q


def brute_force(q_bits, kv, lens, window, rk, rv, hkv, n_sink=0, group=128):
    """Pure-Python textbook attention over the dequantised, un-rotated cache
    (positions below min(n_sink, n - w) and the last w = min(n, W) are the raw
    bf16 tokens).  Each run of ``group`` rotated channels is encoded on its own
    with the single-group encoder."""
    bsz, hq, d = q_bits.shape
    g = hq // hkv
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        k_bits, v_bits = kv[b]
        n = int(lens[b])
        hist = n - min(n, window)
        ns = min(n_sink, hist)
        for j in range(hq):
            h = j // g
            kx = ref.bf16_to_f64(k_bits[:, h])
            vx = ref.bf16_to_f64(v_bits[:, h])
            kx_r, vx_r = ref.rotate(rk[h], kx), ref.rotate(rv[h], vx)
            k_hat, v_hat = np.empty_like(kx_r), np.empty_like(vx_r)
            for c0 in range(0, d, group):
                ck, sk, zk, _ = ref.quantize(kx_r[:, c0:c0 + group])
                cv, sv, zv, _ = ref.quantize(vx_r[:, c0:c0 + group])
                k_hat[:, c0:c0 + group] = zk[:, None] + ck * sk[:, None]
                v_hat[:, c0:c0 + group] = zv[:, None] + cv * sv[:, None]
            keys, vals = [], []
            for t in range(n):
                if ns <= t < hist:
                    kr = k_hat[t]
                    vr = v_hat[t]
                    keys.append(rk[h].T @ kr)
                    vals.append(rv[h].T @ vr)
                else:
                    keys.append(kx[t])
                    vals.append(vx[t])
            qq = ref.bf16_to_f64(q_bits[b, j])
            logits = [sum(float(qq[c]) * float(kk[c]) for c in range(d)) / math.sqrt(d) for kk in keys]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            den = sum(w)
            for c in range(d):
                out[b, j, c] = sum(w[t] * vals[t][c] for t in range(n)) / den
    return out


def test_decode_matches_brute_force(rng):
    lens, window = (37, 5, 20), 16          # several pages, ragged tail, n < W case
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window)
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window)
    want = brute_force(q, kv, lens, window, rk, rv, 2)
    assert np.abs(got - want).max() <= 1e-11 * np.abs(want).max()


def test_decode_with_sinks_matches_brute_force(rng):
    lens, window, n_sink = (37, 5, 20, 30), 8, 6   # sinks inside the history, n < W, sinks past the history
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window, n_sink=n_sink)
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window, n_sink=n_sink)
    want = brute_force(q, kv, lens, window, rk, rv, 2, n_sink=n_sink)
    assert np.abs(got - want).max() <= 1e-11 * np.abs(want).max()


def test_decode_sinks_covering_the_history_is_sdpa(rng):
    """n_sink >= n - w: every position is a raw bf16 token, so decode is plain
    softmax attention (torch SDPA in fp64)."""
    lens, window, n_sink = (40, 25), 16, 24
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window, n_sink=n_sink)
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window, n_sink=n_sink)
    for b in range(2):
        k, v = kv[b]
        kk = torch.from_numpy(ref.bf16_to_f64(k)).permute(1, 0, 2)
        vv = torch.from_numpy(ref.bf16_to_f64(v)).permute(1, 0, 2)
        qq = torch.from_numpy(ref.bf16_to_f64(q[b])).view(2, 4, 1, 128)
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk[:, None], vv[:, None])
        assert np.allclose(got[b], o.reshape(8, 128).numpy(), rtol=1e-12, atol=1e-13)


def test_append_ref_sink_rows(rng):
    """Position p < n_sink is also stored raw in ring row W + p; other rows of
    that block of the ring stay untouched."""
    lens, window, n_sink = (50,), 8, 5
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window, n_sink=n_sink)
    k, v = kv[0]
    assert np.array_equal(wk[0, window:window + n_sink], k[:n_sink])
    assert np.array_equal(wv[0, window:window + n_sink], v[:n_sink])
    assert np.array_equal(wk[0, :window], k[np.arange(42, 50)][np.argsort(np.arange(42, 50) % window)])


def test_decode_pure_window_is_sdpa(rng):
    lens, window = (9, 16), 16
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window)
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window)
    for b in range(2):
        k, v = kv[b]
        kk = torch.from_numpy(ref.bf16_to_f64(k)).permute(1, 0, 2)      # [Hkv][n][d]
        vv = torch.from_numpy(ref.bf16_to_f64(v)).permute(1, 0, 2)
        qq = torch.from_numpy(ref.bf16_to_f64(q[b])).view(2, 4, 1, 128)  # [Hkv][G][1][d]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk[:, None], vv[:, None])
        assert np.allclose(got[b], o.reshape(8, 128).numpy(), rtol=1e-12, atol=1e-13)


def test_decode_single_int2_token(rng):
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, (1,), 0)
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, 0)
    for h in range(2):
        _, vh = ref.read_history(pool, bt[0], 1, h)
        for j in range(4):
            assert np.allclose(got[0, h * 4 + j], rv[h].T @ vh[0], atol=1e-13)


def test_decode_empty_sequence_is_zero_and_leaves_others_alone(rng):
    """A sequence of length 0 has no position to attend: its output is zero
    (reading S19), and the other sequences of the batch are unaffected."""
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, (30, 1), 8)
    full = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, 8)
    lens0 = np.array([30, 0], np.int32)
    got = ref.decode_ref(rk, rv, q, lens0, bt, pool, wk, wv, 8)
    assert np.array_equal(got[1], np.zeros_like(got[1]))
    assert np.array_equal(got[0], full[0])


def test_decode_identical_keys_average_values(rng):
    s = wl.spec(1, batch=1)
    s.seq_lens = np.array([50], np.int32)
    s.n_kv_heads = 1
    bt, n_pages = wl.page_table(s)
    pool = np.zeros((n_pages, 1, ref.BLOCK), np.uint8)
    wk = np.zeros((1, 1, 1, 128), np.uint16)
    rk, rv = orthogonal(rng, 1), orthogonal(rng, 1)
    k, v = wl.context_kv(s, 0)
    k = np.repeat(k[:1, :1], 50, axis=0)
    v = v[:, :1]
    ref.append_ref(rk, rv, k, v, np.zeros(50, np.int32), np.arange(50, dtype=np.int32), bt,
                   s.seq_lens, pool, wk, wk.copy(), 0)
    q = wl.decode_queries(s)[:, :3]
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wk, 0)
    _, vh = ref.read_history(pool, bt[0], 50, 0)
    want = rv[0].T @ vh.mean(axis=0)
    assert np.allclose(got[0], want[None, :], atol=1e-12)


def test_decode_sampled_pairs_match_full(rng):
    lens, window = (40, 33), 8
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window)
    full = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window)
    part = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window, pairs=[(1, 0)])
    assert np.array_equal(part[1, :4], full[1, :4])
    assert np.isnan(part[0]).all() and np.isnan(part[1, 4:]).all()


def test_bf16_comparator_is_sdpa(rng):
    s = wl.spec(1, batch=2)
    s.seq_lens = np.array([45, 17], np.int32)
    bt, n_pages = wl.page_table(s)
    pool = np.zeros((n_pages, 8, ref.BF16_BLOCK), np.uint16)
    q = wl.decode_queries(s)
    for b in range(2):
        k, v, si, pos = wl.prefill_tokens(s, b)
        ref.append_bf16_ref(k, v, si, pos, bt, pool)
        got = ref.decode_bf16_ref(q, s.seq_lens, bt, pool, 8)
        kk = torch.from_numpy(ref.bf16_to_f64(k)).permute(1, 0, 2)[:, None]
        vv = torch.from_numpy(ref.bf16_to_f64(v)).permute(1, 0, 2)[:, None]
        qq = torch.from_numpy(ref.bf16_to_f64(q[b])).view(8, 4, 1, 128)
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).reshape(32, 128).numpy()
        assert np.allclose(got[b], o, rtol=1e-12, atol=1e-13)


def test_bf16_comparator_layout_by_hand():
    """K row j of a page at elements [128 j, 128 j + 128); V of slot j, channel c at
    element 2048 + 16 c + j; round trip through bf16_pages_kv."""
    bt = np.array([[1, 0]], np.int32)
    pool = np.zeros((2, 1, ref.BF16_BLOCK), np.uint16)
    k = np.zeros((1, 1, 128), np.uint16)
    v = np.zeros((1, 1, 128), np.uint16)
    k[0, 0, 5] = 0x3F80                     # 1.0 at channel 5
    v[0, 0, 9] = 0x4000                     # 2.0 at channel 9
    ref.append_bf16_ref(k, v, np.array([0]), np.array([3]), bt, pool)   # position 3: page 1, slot 3
    assert pool[1, 0, 3 * 128 + 5] == 0x3F80 and pool[1, 0, 2048 + 16 * 9 + 3] == 0x4000
    assert np.count_nonzero(pool) == 2
    kk, vv = ref.bf16_pages_kv(pool, np.array([1]), 0)
    assert kk[3, 5] == 0x3F80 and vv[3, 9] == 0x4000 and np.count_nonzero(kk) == 1 and np.count_nonzero(vv) == 1


@pytest.mark.parametrize("n_sink", [0, 4, 200])
def test_direct_decode_equals_paged_decode(rng, n_sink):
    lens, window = (300, 20, 129), 128
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window, n_sink=n_sink)
    full = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window, n_sink=n_sink)
    for b in range(3):
        k, v = kv[b]
        for h in range(2):
            got = ref.decode_direct_ref(rk, rv, q[b, 4 * h:4 * h + 4], k[:, h], v[:, h], lens[b], window, h,
                                        n_sink=n_sink)
            assert np.array_equal(got, full[b, 4 * h:4 * h + 4]) or np.allclose(got, full[b, 4 * h:4 * h + 4],
                                                                              rtol=1e-13, atol=1e-15)
