"""GPU parity of the layer-batched entry points (several layers' caches in one
launch per kernel) through the C ABI: every layer's append equals the
single-layer append of that layer byte for byte (and the oracle under the
encoder rule); every layer's decode matches the oracle within the attention
tolerance and the single-layer decode of that layer closely."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import parity as P  # noqa: E402
import workloads as wl  # noqa: E402
from oracle import oscar_ref as ref  # noqa: E402
from test_gpu_parity import DEV, D, H, K, log, make_spec, ring_rows, rotations, token_list  # noqa: E402,F401

CFG_OF_LAYER = (1, 2, 3)  # each layer's rotations: the calibration of a different workload


def layer_specs(cfg, lens, window, hq, n_sink, group, n_layers):
    out = []
    for l in range(n_layers):
        s = make_spec(cfg, lens, window, hq, n_sink=n_sink, group=group)
        s.seed = l  # different K, V and queries per layer; the block table is layer 0's
        out.append(s)
    return out


def stack(arrs):
    return D(np.stack(arrs))


@pytest.mark.parametrize("cfg,lens,window,hq,n_sink,group", [
    (1, [1000, 777], 128, 32, 0, 128),
    (5, [600, 129, 128], 128, 64, 0, 128),
    (1, [1500, 200], 256, 32, 64, 64),
    (1, [0, 700, 5], 128, 32, 0, 32),
    (1, [900, 260], 0, 128, 40, 64),      # G = 16, no window but sinks, groups of 64
    (1, [1300], 64, 16, 0, 128),          # G = 2, a window of two chunks
])
def test_layers_append_and_decode(K, cfg, lens, window, hq, n_sink, group):
    n_layers = 3
    specs = layer_specs(cfg, lens, window, hq, n_sink, group, n_layers)
    s0 = specs[0]
    bt, n_pages = wl.page_table(s0)
    rng = np.random.default_rng(5)
    rots = [rotations(CFG_OF_LAYER[l]) for l in range(n_layers)]
    toks = [token_list(s) for s in specs]
    assert all(np.array_equal(t[2], toks[0][2]) and np.array_equal(t[3], toks[0][3]) for t in toks)
    si, ps = toks[0][2], toks[0][3]
    blk = ref.block_bytes(group)
    pool0 = rng.integers(0, 256, (n_layers, n_pages, 8, blk), dtype=np.uint8)
    wsh = (n_layers, s0.batch, ring_rows(s0), 8, 128)
    wk0 = rng.integers(0, 65536, wsh, dtype=np.uint16)
    wv0 = rng.integers(0, 65536, wsh, dtype=np.uint16)
    shape = K.make_shape(hq, 8, window, n_sink=n_sink, group_size=group)
    btd, lensd, sid, psd = D(bt), D(s0.seq_lens), D(si), D(ps)
    has_ring = window + n_sink > 0

    # ---- append: one layered call vs one call per layer ----
    pool = D(pool0)
    wk, wv = (D(wk0), D(wv0)) if has_ring else (None, None)
    K.oscar_quantize_append_layers(shape, stack([r[0] for r in rots]), stack([r[1] for r in rots]),
                                   stack([t[0] for t in toks]), stack([t[1] for t in toks]), sid, psd, btd, lensd,
                                   pool, wk, wv)
    torch.cuda.synchronize()
    for l in range(n_layers):
        pl = D(pool0[l])
        wkl, wvl = (D(wk0[l]), D(wv0[l])) if has_ring else (None, None)
        K.oscar_quantize_append(shape, D(rots[l][0]), D(rots[l][1]), D(toks[l][0]), D(toks[l][1]), sid, psd, btd,
                                lensd, pl, wkl, wvl)
        torch.cuda.synchronize()
        assert np.array_equal(H(pool[l]), H(pl)), f"layer {l} pool"
        if has_ring:
            assert np.array_equal(H(wk[l]), H(wkl)) and np.array_equal(H(wv[l]), H(wvl)), f"layer {l} ring"
    rkf, rvf = ref.bf16_to_f64(rots[1][0]), ref.bf16_to_f64(rots[1][1])
    mism, excl, stray = P.check_append(pool0[1], H(pool[1]), rkf, rvf, toks[1][0], toks[1][1], si, ps, bt,
                                       group=group)
    log(f"layers append g={group} lens={lens}: layer 1 vs oracle mismatches={mism} excluded={excl} stray={stray}")
    assert mism == 0 and stray == 0

    # ---- decode: one layered call vs the oracle and the single-layer call ----
    qs = [wl.decode_queries(s)[:, :hq] for s in specs]
    max_len = int(s0.seq_lens.max())
    ws = torch.empty(K.oscar_decode_layers_workspace_bytes(shape, n_layers, s0.batch, max_len), dtype=torch.uint8,
                     device=DEV)
    out = torch.full((n_layers, s0.batch, hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    K.oscar_decode_attn_layers(shape, stack([r[0] for r in rots]), stack([r[1] for r in rots]), stack(qs), lensd,
                               max_len, btd, pool, wk, wv, out, ws)
    torch.cuda.synchronize()
    got = H(out)
    ws1 = torch.empty(K.oscar_decode_workspace_bytes(shape, s0.batch, max_len), dtype=torch.uint8, device=DEV)
    for l in range(n_layers):
        pool_h = H(pool[l])
        wk_h = H(wk[l], np.uint16) if has_ring else np.zeros((s0.batch, 1, 8, 128), np.uint16)
        wv_h = H(wv[l], np.uint16) if has_ring else np.zeros((s0.batch, 1, 8, 128), np.uint16)
        want = ref.decode_ref(ref.bf16_to_f64(rots[l][0]), ref.bf16_to_f64(rots[l][1]), qs[l], s0.seq_lens, bt,
                              pool_h, wk_h, wv_h, window, n_sink=n_sink, group=group)
        err = P.attn_rel_err(got[l], want)
        one = torch.empty((s0.batch, hq, 128), dtype=torch.float32, device=DEV)
        K.oscar_decode_attn(shape, D(rots[l][0]), D(rots[l][1]), D(qs[l]), lensd, max_len, btd, pool[l],
                            wk[l] if has_ring else None, wv[l] if has_ring else None, one, ws1)
        torch.cuda.synchronize()
        err1 = P.attn_rel_err(got[l], H(one))
        log(f"layers decode g={group} lens={lens} Hq={hq} layer {l}: vs oracle {err.max():.3e}, "
            f"vs single-layer {err1.max():.3e}")
        assert np.isfinite(got[l]).all()
        assert err.max() <= P.ATTN_TOL
        assert err1.max() <= 1e-5


def test_one_layer_equals_plain_call(K):
    s = make_spec(1, [900, 20], 128, 32)
    from test_gpu_parity import oracle_cache, run_decode

    rk, rv, rkf, rvf, bt, pool, wk, wv, q = oracle_cache(s)
    plain = run_decode(K, s, rk, rv, q, bt, pool, wk, wv)
    shape = K.make_shape(32, 8, 128)
    ws = torch.empty(K.oscar_decode_layers_workspace_bytes(shape, 1, 2, 900), dtype=torch.uint8, device=DEV)
    out = torch.empty((1, 2, 32, 128), dtype=torch.float32, device=DEV)
    K.oscar_decode_attn_layers(shape, D(rk[None]), D(rv[None]), D(q[None]), D(s.seq_lens), 900, D(bt), D(pool[None]),
                               D(wk[None]), D(wv[None]), out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(H(out)[0], plain)
