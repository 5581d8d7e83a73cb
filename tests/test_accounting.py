"""The pages' printed byte-accounting figures (tests/golden/accounting.txt)
against the oracle's closed forms."""
import os

import numpy as np

from oracle import oscar_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accounting.txt")


def golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, value, tol = line.split("|")[0].split()
        vals[name] = (float(value), float(tol))
    return vals


def test_int2_layout_bytes():
    # 32 B of codes + fp16 scale + fp16 zero, for K and for V
    assert ref.int2_bytes_per_token_head() == 72
    assert ref.int2_bits_per_element() == 2.25
    assert 512 / 72 > 7.1


def test_effective_bits_with_bf16_share():
    g = golden()
    share = g["bf16_token_share_128k"][0]
    want, tol = g["effective_bits"]
    assert abs(ref.effective_bits(share) - want) <= tol


def test_llama70b_bf16_kv_sizes():
    # public Llama-3.1-70B shape (80 layers, 8 KV heads, head dim 128)
    g = golden()
    per_tok = ref.bf16_kv_bytes_per_token(80, 8, 128)
    assert abs(per_tok / 2 ** 20 - g["llama70b_mib_per_token"][0]) <= g["llama70b_mib_per_token"][1]
    assert abs(per_tok * 131072 / 2 ** 30 - g["llama70b_gib_at_128k"][0]) <= g["llama70b_gib_at_128k"][1]
    assert per_tok * 2 ** 20 / 2 ** 30 > g["llama70b_gib_at_1m_min"][0]


def test_nominal_ratios_and_levels():
    g = golden()
    assert 16 / 2 == g["nominal_ratio_vs_bf16"][0]
    assert 8 / 2 == g["nominal_ratio_vs_fp8"][0]
    assert 4 / 2 == g["nominal_ratio_vs_int4"][0]
    c, _, _, _ = ref.quantize(np.linspace(-3, 5, 128))
    assert len(np.unique(c)) == g["levels_int2"][0] == 2 ** 2
