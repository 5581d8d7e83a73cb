"""Pins of the rotation-quality harness's host parts (CPU only): its Hadamard
rotation is the oracle's P_br (H / sqrt d), and its decoder of the page blocks
reads exactly what the oracle's reader reads from a pool the oracle encoded."""
import numpy as np
import pytest

import workloads as wl
import quality
from oracle import oscar_ref as ref
from test_oracle_decode import build, orthogonal


def test_hadamard_rotation_is_the_oracles():
    want = ref.apply_bitrev_rows(ref.hadamard()) / np.sqrt(128)
    got = quality.hadamard_rotation()
    assert np.array_equal(got, want)
    assert np.allclose(got @ got.T, np.eye(128), atol=1e-12)


@pytest.mark.parametrize("group", [128, 64, 32])
def test_dequantize_history_matches_oracle_reader(rng, group):
    s, bt, pool, wk, wv, rk, rv, kv, q = build(rng, (70, 33, 16), 8, group=group)
    assert quality.block_bytes(group) == pool.shape[-1]
    for b, n in enumerate(s.seq_lens):
        hist = int(n) - min(int(n), 8)
        for h in range(s.n_kv_heads):
            k0, v0 = ref.read_history(pool, bt[b], hist, h, group) if hist else (np.zeros((0, 128)),) * 2
            k1, v1 = quality.dequantize_history(pool, bt[b], hist, h, group)
            assert np.array_equal(k0, k1) and np.array_equal(v0, v1)


def test_dequantize_history_every_code_and_slot(rng):
    """A page whose 16 tokens use every code level at known channels."""
    pool = np.zeros((3, 1, ref.BLOCK), np.uint8)
    codes_k = rng.integers(0, 4, (16, 128))
    codes_v = rng.integers(0, 4, (16, 128))
    blk = pool[2, 0]
    for t in range(16):
        blk[32 * t:32 * t + 32] = ref.pack_k_row(codes_k[t])
    words = np.zeros(128, np.uint32)
    for c in range(128):
        for t in range(16):
            words[c] |= np.uint32(codes_v[t, c]) << np.uint32(2 * t)
    blk[512:1024] = words.view(np.uint8)
    meta = np.zeros((16, 4), np.uint16)
    meta[:, 0] = ref.fp16_bits(np.full(16, 0.5))
    meta[:, 1] = ref.fp16_bits(np.full(16, -1.0))
    meta[:, 2] = ref.fp16_bits(np.full(16, 2.0))
    meta[:, 3] = ref.fp16_bits(np.full(16, 3.0))
    blk[1024:] = meta.view(np.uint8).reshape(-1)
    k, v = quality.dequantize_history(pool, np.array([2]), 16, 0)
    assert np.array_equal(k, -1.0 + 0.5 * codes_k)
    assert np.array_equal(v, 3.0 + 2.0 * codes_v)
