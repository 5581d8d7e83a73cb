"""The GPU tests' matching rules, exercised on the CPU with the oracle standing
in for the device: a faithful encoding passes, planted mistakes are caught."""
import numpy as np

import workloads as wl
from oracle import oscar_ref as ref
import parity as P


def setup(seed=0):
    s = wl.spec(1, batch=2)
    s.seq_lens = np.array([70, 33], np.int32)
    rng = np.random.default_rng(seed)
    rk = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(8)])
    rv = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(8)])
    rk, rv = ref.bf16_to_f64(ref.bf16_bits(rk)), ref.bf16_to_f64(ref.bf16_bits(rv))
    bt, n_pages = wl.page_table(s)
    pool0 = rng.integers(0, 256, (n_pages, 8, ref.BLOCK), dtype=np.uint8)
    ks, vs, si, ps = [], [], [], []
    for b in range(2):
        k, v, i, p = wl.prefill_tokens(s, b)
        ks.append(k), vs.append(v), si.append(i), ps.append(p)
    k, v, si, ps = (np.concatenate(x) for x in (ks, vs, si, ps))
    pool = pool0.copy()
    w = np.zeros((2, 128, 8, 128), np.uint16)
    ref.append_ref(rk, rv, k, v, si, ps, bt, s.seq_lens, pool, w, w.copy(), 128)
    return pool0, pool, rk, rv, k, v, si, ps, bt


def test_faithful_encoding_passes():
    pool0, pool, rk, rv, k, v, si, ps, bt = setup()
    assert P.check_append(pool0, pool, rk, rv, k, v, si, ps, bt)[::2] == (0, 0)


def test_flipped_code_is_caught():
    pool0, pool, rk, rv, k, v, si, ps, bt = setup()
    page = bt[1][1]
    pool[page, 3, ref.K_CODES + 32 * 2 + 5] ^= 0x04     # one K code of seq 1, pos 18
    assert P.check_append(pool0, pool, rk, rv, k, v, si, ps, bt)[0] >= 1


def test_stray_write_is_caught():
    pool0, pool, rk, rv, k, v, si, ps, bt = setup()
    free = np.setdiff1d(np.arange(pool.shape[0]), bt[bt >= 0])
    last = bt[1][2]                                      # seq 1 holds 33 tokens: slot 1+ of page 2 unused
    pool[last, 0, ref.K_CODES + 32 * 9] ^= 0xFF
    assert P.check_append(pool0, pool, rk, rv, k, v, si, ps, bt)[2] >= 1
    assert free.size == 0


def test_wrong_scale_is_caught():
    pool0, pool, rk, rv, k, v, si, ps, bt = setup()
    page = bt[0][0]
    sc = pool[page, 1, ref.META + ref.V_SCALE:ref.META + ref.V_SCALE + 2].view(np.uint16)
    sc[0] ^= 0x0001
    assert P.check_append(pool0, pool, rk, rv, k, v, si, ps, bt)[0] >= 1


def test_attention_error_metric():
    want = np.array([[[1.0, -2.0, 0.5]]])
    got = want.copy()
    got[0, 0, 1] += 2e-3 * 2.0 * 1.01
    assert P.attn_rel_err(got, want).max() > P.ATTN_TOL
    got[0, 0, 1] = want[0, 0, 1] + 1e-3
    assert P.attn_rel_err(got, want).max() <= P.ATTN_TOL
