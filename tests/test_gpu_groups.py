"""GPU parity of the finer quantisation groups (64 or 32 rotated channels per
scale/zero pair) against the oracle, through the C ABI: the append's per-group
records and codes under the encoder rule, and decode attention on
oracle-encoded caches within the attention tolerance."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import parity as P  # noqa: E402
from oracle import oscar_ref as ref  # noqa: E402
from test_gpu_parity import K, append_case, log, make_spec, oracle_cache, run_decode  # noqa: E402,F401


@pytest.mark.parametrize("group", [64, 32])
def test_append_groups_inorder_ragged(K, group):
    append_case(K, make_spec(1, [300, 45], group=group))


@pytest.mark.parametrize("group", [64, 32])
def test_append_groups_shuffled_partial_pages(K, group):
    # shuffled tokens: pages filled out of order take the per-token path
    append_case(K, make_spec(1, [300, 37, 129], window=100, group=group), order="shuffled", seed=11)


@pytest.mark.parametrize("group", [64, 32])
def test_append_groups_continuation_with_sinks(K, group):
    append_case(K, make_spec(1, [300, 70], n_sink=20, group=group), split_at=21, seed=12)


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("cfg,lens,window,hq,n_sink", [
    (1, [1000, 777], 128, 32, 0),        # G = 4, several tiles, ragged tails
    (5, [600, 129, 128], 128, 64, 0),     # G = 8 (two 4-head units per KV head)
    (1, [700, 333], 100, 8, 0),           # G = 1
    (1, [260, 1030], 128, 128, 0),        # G = 16
    (1, [1500, 200], 256, 32, 64),        # window and sinks
    (1, [0, 700, 5], 128, 32, 0),         # an empty sequence, a pure-window one
    (1, [2300], 0, 16, 0),                # no window, G = 2
])
def test_decode_groups(K, group, cfg, lens, window, hq, n_sink):
    s = make_spec(cfg, lens, window, hq, n_sink=n_sink, group=group)
    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    got = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    want = ref.decode_ref(rkf, rvf, q, s.seq_lens, bt, pool, wk, wv, window, n_sink=n_sink, group=group)
    err = P.attn_rel_err(got, want)
    log(f"decode g={group} lens={lens} W={window} Hq={hq} sinks={n_sink}: max rel err {err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.max() <= P.ATTN_TOL


@pytest.mark.parametrize("group", [64, 32])
def test_full_longctx_groups(K, group):
    """The long-context decode workload (B = 8, n = 100000, 32 q / 8 KV heads) at
    a finer group size: sampled append records and codes, every group spanning
    codes 0..3, and sampled decode outputs on oracle-encoded sequences."""
    import workloads as wl
    from test_gpu_parity import check_sampled, codes_span_levels, decode_full, full_cache, oracle_overwrite
    from test_gpu_parity import sampled_append_check

    s = wl.spec(3)
    s.group_size = group
    log(f"config 3 g={group} full: building cache")
    c = full_cache(K, s, keep=(2, 7))
    q = wl.decode_queries(s)
    pool = sampled_append_check(s, c, 7, n_sample=256, seed=31)
    codes_span_levels(pool, c["bt"], s.seq_lens[:1], group=group)
    oracle = {b: oracle_overwrite(s, c, b) for b in (2, 7)}
    got = decode_full(K, s, c, q, s.seq_lens)
    assert np.isfinite(got).all()
    check_sampled(s, c, q, got, [(2, 3), (7, 0)], oracle)
