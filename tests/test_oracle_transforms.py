"""Pins of the oracle's fixed transforms and number formats (CPU only).

Hadamard and bit reversal are checked against independent constructions and
their algebraic identities; the rounding helpers against numpy's float16 and
torch's bfloat16 conversions (library routines) and hand-picked ties.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oscar_ref as ref


def sylvester_recursive(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [2, 8, 32, 128])
def test_hadamard_closed_form_matches_recursion(d):
    h = ref.hadamard(d)
    assert np.array_equal(h, sylvester_recursive(d))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, d * np.eye(d))


def test_bit_reversal_small_by_hand():
    assert list(ref.bit_reverse_index(8)) == [0, 4, 2, 6, 1, 5, 3, 7]
    assert list(ref.bit_reverse_index(2)) == [0, 1]


def test_bit_reversal_involution_and_fixed_points():
    br = ref.bit_reverse_index(128)
    assert sorted(br) == list(range(128))
    assert np.array_equal(br[br], np.arange(128))
    # 7-bit palindromes: 2^4 of them
    assert int(np.sum(br == np.arange(128))) == 16


def test_bitrev_commutes_with_sylvester_hadamard():
    h = ref.hadamard(128)
    p = np.eye(128)[ref.bit_reverse_index(128)]
    assert np.array_equal(ref.apply_bitrev_rows(np.eye(128)), p)
    assert np.array_equal(p @ h @ p, h)
    assert np.array_equal(p @ p, np.eye(128))


def test_fp16_rne_matches_numpy(rng):
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 4, 20000),
        # exact ties around 1 and in the subnormal range
        1.0 + (2 * np.arange(50) + 1) * 2.0 ** -11,
        (2 * np.arange(50) + 1) * 2.0 ** -25,
        [0.0, -0.0, 65504.0, 65519.99, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26],
    ])
    mine = ref.fp16_rne(x)
    lib = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(mine, lib)
    assert np.array_equal(ref.fp16_bits(x), x.astype(np.float16).view(np.uint16))


def test_fp16_rne_overflow_raises():
    with pytest.raises(OverflowError):
        ref.fp16_rne(65520.0)


def test_bf16_rne_matches_torch(rng):
    x32 = np.concatenate([
        (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32),
        (1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8).astype(np.float32),
    ])
    lib = torch.from_numpy(x32).to(torch.bfloat16)
    assert np.array_equal(ref.bf16_bits(x32.astype(np.float64)), lib.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(ref.bf16_rne(x32.astype(np.float64)), lib.to(torch.float64).numpy())


def test_bf16_ties_by_hand():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even -> 1
    assert ref.bf16_rne(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    assert ref.bf16_rne(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert ref.bf16_bits(1.0) == 0x3F80
    assert ref.bf16_bits(-2.0) == 0xC000


def test_bf16_roundtrip_bits(rng):
    bits = rng.integers(0, 0x7F80, 5000).astype(np.uint16)
    v = ref.bf16_to_f64(bits)
    assert np.array_equal(ref.bf16_bits(v), bits)
    assert math.isclose(float(ref.bf16_to_f64(np.uint16(0x3F80))), 1.0)
