"""Pins of the oracle's finer quantisation groups (g = 64, 32 rotated channels
per scale/zero pair; CPU only).

(i)   sizes: the page block is 1024 + 128 (d / g) bytes, which is 16 tokens of
      the per-token byte count of the cache (codes plus two fp16 per group);
(ii)  each group is encoded on its own: changing one group's values leaves every
      other group's codes, scale and zero as they were;
(iii) a token built on each group's exact grid z_j + c s_j comes back exactly;
(iv)  finer groups reconstruct Gaussian tokens better (g = 32 < 64 < 128);
(v)   the record of group j of slot t is read from 1024 + 8 (ng t + j), on a
      block written by hand;
(vi)  append + decode with groups equal pure-Python brute force over the
      per-group encoding, and the paged decode equals the direct one.
"""
import numpy as np
import pytest

from oracle import oscar_ref as ref
from test_oracle_decode import brute_force, build


@pytest.mark.parametrize("group", [32, 64, 128])
def test_block_bytes(group):
    ng = 128 // group
    assert ref.block_bytes(group) == 1024 + 128 * ng
    assert ref.block_bytes(group) == 16 * ref.int2_bytes_per_token_head(128, group)


@pytest.mark.parametrize("group", [32, 64])
def test_groups_are_encoded_independently(rng, group):
    x = rng.standard_normal((50, 128))
    c0, s0, z0 = ref.quantize_groups(x, group)
    j = 1
    y = x.copy()
    y[:, group * j:group * (j + 1)] = 7.0 * y[:, group * j:group * (j + 1)] + 3.0
    c1, s1, z1 = ref.quantize_groups(y, group)
    other = np.r_[0:group * j, group * (j + 1):128]
    assert np.array_equal(c0[:, other], c1[:, other])
    keep = [i for i in range(128 // group) if i != j]
    assert np.array_equal(s0[:, keep], s1[:, keep]) and np.array_equal(z0[:, keep], z1[:, keep])
    assert not np.array_equal(s0[:, j], s1[:, j])


@pytest.mark.parametrize("group", [32, 64])
def test_group_exact_grid_round_trip(rng, group):
    ng = 128 // group
    codes = rng.integers(0, 4, (20, 128))
    codes[:, ::group] = 0                   # every group reaches both ends of its grid
    codes[:, 1::group] = 3
    s = 2.0 ** rng.integers(-6, 2, (20, ng)) * rng.integers(1, 8, (20, ng))   # exact in fp16
    z = rng.integers(-64, 64, (20, ng)) / 8.0
    x = np.repeat(z, group, axis=1) + codes * np.repeat(s, group, axis=1)
    c, s_out, z_out = ref.quantize_groups(x, group)
    assert np.array_equal(c, codes) and np.array_equal(s_out, s) and np.array_equal(z_out, z)


def test_finer_groups_reconstruct_better(rng):
    x = rng.standard_normal((4000, 128))
    err = {}
    for g in (32, 64, 128):
        c, s, z = ref.quantize_groups(x, g)
        xh = np.repeat(z, g, axis=1) + c * np.repeat(s, g, axis=1)
        err[g] = float(np.mean((x - xh) ** 2))
        # every value within half a step of its group's grid, plus the fp16 rounding of s and z
        step = np.repeat(s, g, axis=1)
        rng_g = np.repeat(np.abs(z) + 3 * s, g, axis=1)
        assert np.all(np.abs(x - xh) <= 0.5 * step + 2.0 ** -9 * rng_g)
    assert err[32] < err[64] < err[128]


@pytest.mark.parametrize("group", [32, 64])
def test_group_records_read_by_hand(group):
    ng = 128 // group
    pool = np.zeros((2, 1, ref.block_bytes(group)), np.uint8)
    blk = pool[1, 0]
    blk[0:512] = 0x55                      # every K code 1
    blk[512:1024] = 0x55                   # every V code 1
    rec = np.zeros((16, ng, 4), np.uint16)
    for t in range(16):
        for j in range(ng):
            rec[t, j] = ref.fp16_bits(np.array([t + 1.0, 10.0 * j, 0.5 * (t + 1), -4.0 * j]))
    blk[1024:] = rec.view(np.uint8).reshape(-1)
    k, v = ref.read_history(pool, np.array([1]), 16, 0, group)
    t = np.arange(16)[:, None]
    jc = np.arange(128)[None, :] // group
    assert np.array_equal(k, 10.0 * jc + (t + 1.0))
    assert np.array_equal(v, -4.0 * jc + 0.5 * (t + 1.0))


@pytest.mark.parametrize("group", [32, 64])
def test_decode_with_groups_matches_brute_force(rng, group):
    lens, window, n_sink = (37, 5, 20), 8, 3
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window, n_sink=n_sink, group=group)
    got = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window, n_sink=n_sink, group=group)
    want = brute_force(q, kv, lens, window, rk, rv, 2, n_sink=n_sink, group=group)
    assert np.abs(got - want).max() <= 1e-11 * np.abs(want).max()


@pytest.mark.parametrize("group", [32, 64])
def test_direct_decode_equals_paged_decode_with_groups(rng, group):
    lens, window = (300, 20, 129), 64
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, lens, window, group=group)
    full = ref.decode_ref(rk, rv, q, s.seq_lens, bt, pool, wk, wv, window, group=group)
    for b in range(3):
        k, v = kv[b]
        for h in range(2):
            got = ref.decode_direct_ref(rk, rv, q[b, 4 * h:4 * h + 4], k[:, h], v[:, h], lens[b], window, h,
                                        group=group)
            assert np.allclose(got, full[b, 4 * h:4 * h + 4], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("group", [32, 64])
def test_bulk_append_equals_per_token_append_with_groups(rng, group):
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, (45, 16), 8, n_sink=2, group=group)
    pool2 = np.zeros_like(pool)
    wk2, wv2 = np.zeros_like(wk), np.zeros_like(wv)
    for b in range(2):
        k, v = kv[b]
        ref.append_sequence_ref(rk, rv, k, v, bt[b], pool2, wk2[b], wv2[b], 8, n_sink=2, group=group)
    assert np.array_equal(pool, pool2) and np.array_equal(wk, wk2) and np.array_equal(wv, wv2)
