"""The allocation-free decode entry point (oscar_decode_attn_noalloc) against
oscar_decode_attn on the same inputs, through the C ABI: two calls in a row on
the library's static scratch, the second with a smaller batch and shorter
sequences, each bit-identical to the workspace form and within the attention
tolerance of the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import oscar_ref as ref  # noqa: E402
import parity as P  # noqa: E402
from test_gpu_parity import D, DEV, H, make_spec, oracle_cache, run_decode  # noqa: E402


def _noalloc(K, s, rk, rv, q, bt, pool, wk, wv):
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window, n_sink=s.n_sink, group_size=s.group_size)
    max_len = int(s.seq_lens.max())
    assert K.oscar_decode_noalloc_scratch_bytes(shape, s.batch, max_len) <= K.NOALLOC_SCRATCH_BYTES
    out = torch.full((s.batch, s.n_q_heads, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.oscar_decode_attn_noalloc(shape, D(rk), D(rv), D(q), D(s.seq_lens), max_len, D(bt), D(pool),
                                D(wk) if s.window + s.n_sink > 0 else None,
                                D(wv) if s.window + s.n_sink > 0 else None, out)
    torch.cuda.synchronize()
    return H(out)


@pytest.mark.parametrize("first,second", [
    ((1, [4100, 2500, 777], 128, 32), (1, [1000, 40], 128, 32)),
    ((5, [3000, 129, 1500, 700], 128, 64), (5, [600], 128, 64)),
])
def test_noalloc_matches_workspace_form(first, second):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_int2_amd as K

    for cfg, lens, window, hq in (first, second):
        s = make_spec(cfg, lens, window, hq)
        rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
        got = _noalloc(K, s, rk, rv, q, bt, pool, wk, wv)
        base = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
        want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, window)
        err = P.attn_rel_err(got, want)
        print(f"noalloc lens={lens} Hq={hq}: max rel err {err.max():.3e}", flush=True)
        assert np.isfinite(got).all()
        assert np.array_equal(got, base)
        assert err.max() <= P.ATTN_TOL


def test_noalloc_refuses_oversized_calls():
    """A call whose scratch exceeds the static array is refused on the host."""
    import kv_cache_int2_amd as K

    shape = K.make_shape(64, 8, window=1024, n_sink=1024, group_size=32)
    assert K.oscar_decode_noalloc_scratch_bytes(shape, 64, 131073) > K.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((64, 64, 128), dtype=torch.int16, device=DEV)
    lens = torch.full((64,), 131073, dtype=torch.int32, device=DEV)
    bt = torch.zeros((64, 8193), dtype=torch.int32, device=DEV)
    r = torch.zeros((8, 128, 128), dtype=torch.int16, device=DEV)
    pool = torch.zeros((1, 8, K.block_bytes(32)), dtype=torch.uint8, device=DEV)
    ring = torch.zeros((64, 2048, 8, 128), dtype=torch.int16, device=DEV)
    out = torch.zeros((64, 64, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(K.OscarError) as e:
        K.oscar_decode_attn_noalloc(shape, r, r, q, lens, 131073, bt, pool, ring, ring, out)
    assert e.value.status == -4
