"""Pins of the oracle's encoder and page layout (CPU only): hand-derived golden
encodings, exact-grid round trips, ties, clamping, degenerate groups, the
bit-reversal permutation acting as a pure code permutation at g = d, and the
pool/window writes of ``append_ref`` against a direct per-token encoding."""
import os

import numpy as np
import pytest

import workloads as wl
from oracle import oscar_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_examples.txt")


def golden_rows():
    rows = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, _, meta, row = [f.strip() for f in line.split("|")]
        sc, z = meta.split()
        rows[name] = (int(sc, 16), int(z, 16), bytes.fromhex(row))
    return rows


def golden_inputs():
    i = np.arange(128)
    ties = np.ones(128)
    ties[:5] = [0, 3, 0.5, 1.5, 2.5]
    return {"grid": -1.5 + 0.5 * (i % 4), "ties": ties, "flat": np.full(128, 0.75)}


@pytest.mark.parametrize("name", ["grid", "ties", "flat"])
def test_golden_encodings(name):
    sc, z, row = golden_rows()[name]
    x = golden_inputs()[name]
    xr = ref.rotate(np.eye(128), x)
    c, s16, z16, _ = ref.quantize(xr)
    assert int(ref.fp16_bits(s16)) == sc
    assert int(ref.fp16_bits(z16)) == z
    assert ref.pack_k_row(c).tobytes() == row
    assert np.array_equal(ref.unpack_k_rows(np.frombuffer(row, np.uint8)), c)


def test_exact_grid_round_trip(rng):
    """x on z + c s (fp16-exact z, s; codes 0 and 3 present) -> codes c, dequant x."""
    for z, s in [(-1.5, 0.5), (3.25, 0.125), (-40.0, 12.0), (0.0, 2.0 ** -10)]:
        c = rng.integers(0, 4, (50, 128))
        c[:, 0], c[:, 1] = 0, 3
        x = z + c * s
        cc, s16, z16, _ = ref.quantize(x)
        assert np.all(s16 == s) and np.all(z16 == z)
        assert np.array_equal(cc, c)
        assert np.array_equal(z16[:, None] + cc * s16[:, None], x)


def test_two_valued_group_uses_extreme_codes(rng):
    x = np.where(rng.random((20, 128)) < 0.5, -0.7, 1.9)
    x[:, 0], x[:, 1] = -0.7, 1.9
    c, _, _, _ = ref.quantize(x)
    assert set(np.unique(c)) == {0, 3}


def test_zero_rounding_up_clamps_to_code_zero():
    # min = 1 + 3*2^-12 rounds up to fp16 1 + 2^-10, so t(min) < 0: clamp, not -1
    x = np.full(128, 2.0)
    x[0] = 1.0 + 3 * 2.0 ** -12
    x[1] = 4.0
    c, s16, z16, diag = ref.quantize(x)
    assert z16 == 1.0 + 2.0 ** -10 and diag["t"][0] < 0
    assert c[0] == 0 and c.min() >= 0 and c.max() <= 3


def test_codes_follow_stored_scale_and_zero(rng):
    x = rng.standard_normal((200, 128)) * 3
    c, s16, z16, diag = ref.quantize(x)
    t = (x.astype(np.float32) - z16[:, None]) / s16[:, None]
    assert np.array_equal(c, np.clip(np.rint(t), 0, 3))
    assert np.all(np.abs(diag["sigma"] - (x.max(1) - x.min(1)) / 3) <= 1e-6 * np.abs(diag["sigma"]))
    # every dequantised value lies within half a step of x (z, s round to fp16)
    xh = z16[:, None] + c * s16[:, None]
    assert np.all(np.abs(xh - x) <= 0.5 * s16[:, None] * (1 + 2e-3))


def test_bitrev_only_permutes_codes_at_full_group(rng):
    """At group = d = 128 the bit-reversal permutation changes code order only."""
    u = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    a = ref.hadamard(128) / np.sqrt(128) @ u.T
    r = ref.apply_bitrev_rows(a)
    x = rng.standard_normal((30, 128))
    c1, s1, z1, _ = ref.quantize(ref.rotate(r, x))
    c2, s2, z2, _ = ref.quantize(ref.rotate(a, x))
    br = ref.bit_reverse_index(128)
    assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
    assert np.array_equal(c1, c2[:, br])


def test_pack_bit_positions_by_hand():
    c = np.zeros(128, dtype=np.int64)
    c[5] = 3                      # segment 1 (channels 4..7 of each 16), byte 0 -> row byte 8, bits 2-3
    c[127] = 2                    # segment 3, byte 7 -> row byte 31, bits 6-7
    c[16] = 1                     # segment 0, byte 1 -> row byte 1, bits 0-1
    row = ref.pack_k_row(c)
    assert row[8] == 0x0C and row[31] == 0x80 and row[1] == 0x01 and row.sum() == 0x0C + 0x80 + 0x01
    blk = np.zeros(1152, dtype=np.uint8)
    words = np.zeros(128, dtype="<u4")
    words[7] = 2 << 6             # channel 7, slot 3, code 2
    blk[ref.V_CODES:ref.V_CODES + 512] = words.view(np.uint8)
    codes = ref.unpack_v_words(ref.v_words(blk))
    assert codes[3, 7] == 2 and codes.sum() == 2
    assert blk[ref.V_CODES + 28] == 0x80  # little-endian word 7, low byte


def small_cache(cfg=1, batch=2, lens=(40, 23), window=16, seed=0, n_sink=0):
    s = wl.spec(cfg, seed=seed, batch=batch)
    s.seq_lens = np.asarray(lens, dtype=np.int32)
    s.window = window
    bt, n_pages = wl.page_table(s)
    pool = np.zeros((n_pages, s.n_kv_heads, ref.BLOCK), dtype=np.uint8)
    win_k = np.zeros((batch, max(window + n_sink, 1), s.n_kv_heads, 128), dtype=np.uint16)
    win_v = np.zeros_like(win_k)
    return s, bt, pool, win_k, win_v


def random_rotations(rng, hkv):
    rk = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(hkv)])
    rv = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(hkv)])
    return ref.bf16_to_f64(ref.bf16_bits(rk)), ref.bf16_to_f64(ref.bf16_bits(rv))


def test_append_ref_matches_direct_encoding(rng):
    s, bt, pool, win_k, win_v = small_cache()
    rk, rv = random_rotations(rng, s.n_kv_heads)
    toks = {}
    for b in range(s.batch):
        k, v, si, pos = wl.prefill_tokens(s, b)
        # shuffle the token order: the encoding must not depend on it
        o = rng.permutation(len(pos))
        ref.append_ref(rk, rv, k[o], v[o], si[o], pos[o], bt, s.seq_lens, pool, win_k, win_v, s.window)
        toks[b] = (k, v)
    for b in range(s.batch):
        k, v = toks[b]
        n = int(s.seq_lens[b])
        for h in range(s.n_kv_heads):
            kh, vh = ref.read_history(pool, bt[b], n, h)
            ck, sk, zk, _ = ref.quantize(ref.rotate(rk[h], ref.bf16_to_f64(k[:, h])))
            cv, sv, zv, _ = ref.quantize(ref.rotate(rv[h], ref.bf16_to_f64(v[:, h])))
            assert np.array_equal(kh, zk[:, None] + ck * sk[:, None])
            assert np.array_equal(vh, zv[:, None] + cv * sv[:, None])
        # window: the last W positions, at slot pos % W
        for p in range(max(0, n - s.window), n):
            assert np.array_equal(win_k[b, p % s.window], k[p])
            assert np.array_equal(win_v[b, p % s.window], v[p])


def test_append_ref_keeps_other_slots_and_skips_old_window_positions(rng):
    s, bt, pool, win_k, win_v = small_cache(lens=(40, 23))
    rk, rv = random_rotations(rng, s.n_kv_heads)
    k, v, si, pos = wl.prefill_tokens(s, 0)
    ref.append_ref(rk, rv, k[:20], v[:20], si[:20], pos[:20], bt, s.seq_lens, pool, win_k, win_v, s.window)
    before = pool.copy()
    wk_before = win_k.copy()
    ref.append_ref(rk, rv, k[20:], v[20:], si[20:], pos[20:], bt, s.seq_lens, pool, win_k, win_v, s.window)
    # positions 0..19 (pages 0 and the first 4 slots of page 1) are untouched
    pg0 = bt[0][0]
    assert np.array_equal(pool[pg0], before[pg0])
    kh, _ = ref.read_history(pool, bt[0], 40, 3)
    kh0, _ = ref.read_history(before, bt[0], 20, 3)
    assert np.array_equal(kh[:20], kh0)
    # only positions >= 40 - 16 reach the window; none of the first call did
    assert not wk_before[0].any()
    for p in range(24, 40):
        assert np.array_equal(win_k[0, p % 16], k[p])


def test_bulk_sequence_append_equals_per_token_append(rng):
    """append_sequence_ref is byte-identical to append_ref for an in-order prefill."""
    for n, window, n_sink in ((37, 16, 0), (64, 128, 0), (1, 4, 0), (37, 16, 5), (20, 0, 40)):
        s, bt, pool, win_k, win_v = small_cache(batch=1, lens=(n,), window=window, n_sink=n_sink)
        rk, rv = random_rotations(rng, s.n_kv_heads)
        k, v, si, pos = wl.prefill_tokens(s, 0)
        pool_a, wk_a, wv_a = pool.copy(), win_k.copy(), win_v.copy()
        ref.append_ref(rk, rv, k, v, si, pos, bt, s.seq_lens, pool_a, wk_a, wv_a, window, n_sink)
        pool_b = rng.integers(0, 256, pool.shape, dtype=np.uint8)
        used = np.zeros(pool.shape[0], bool)
        used[bt[0][bt[0] >= 0]] = True
        pool_b0 = pool_b.copy()
        wk_b, wv_b = win_k.copy(), win_v.copy()
        ref.append_sequence_ref(rk, rv, k, v, bt[0], pool_b, wk_b[0], wv_b[0], window, n_sink)
        # written slots equal; unwritten bytes of the last page keep their old values
        kh_a, vh_a = ref.read_history(pool_a, bt[0], n, 2)
        kh_b, vh_b = ref.read_history(pool_b, bt[0], n, 2)
        assert np.array_equal(kh_a, kh_b) and np.array_equal(vh_a, vh_b)
        pool_c = pool_b0.copy()
        ref.append_ref(rk, rv, k, v, si, pos, bt, s.seq_lens, pool_c, win_k.copy(), win_v.copy(), window, n_sink)
        assert np.array_equal(pool_b, pool_c)
        assert np.array_equal(wk_b, wk_a) and np.array_equal(wv_b, wv_a)
