"""The rotation-quality harness through the kernels (GPU): every metric is
finite, the identity rotation (plain per-token INT2, whose group range the x20
key outlier channels inflate) has the largest key logit error, and the
sampled logit error agrees with its Sigma_Q expectation."""
import math

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def test_quality_harness_small():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_int2_amd as K
    import quality

    s = wl.spec(1, batch=2, seq_len=700)
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window)
    q_cal, k_cal, v_cal = wl.calibration_set(s)
    rot = quality.rotations(shape, q_cal, k_cal, v_cal, K.oscar_calibrate)
    res = quality.measure(K, s, rot, wl, torch)
    print("quality", res)
    for name, r in res.items():
        assert all(math.isfinite(v) for v in r.values()), name
        assert r["kl"] >= 0.0
        assert 0.25 < r["logit_rms"] ** 2 / r["logit_sigma"] < 4.0, name
    assert res["identity"]["logit_sigma"] > res["oscar"]["logit_sigma"]
    assert res["identity"]["logit_sigma"] > res["hadamard"]["logit_sigma"]


def test_quality_finer_groups_reduce_error():
    """Smaller groups (more scale/zero metadata per token) quantise each channel
    against a narrower range: the Sigma_Q-weighted key error falls from 128 to 32
    channels per group for every rotation."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_int2_amd as K
    import quality

    s = wl.spec(1, batch=2, seq_len=700)
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window)
    q_cal, k_cal, v_cal = wl.calibration_set(s)
    rot = quality.rotations(shape, q_cal, k_cal, v_cal, K.oscar_calibrate)
    res = {g: quality.measure(K, s, rot, wl, torch, group=g) for g in (128, 32)}
    print("quality by group", res)
    for name in rot:
        assert all(math.isfinite(v) for v in res[32][name].values()), name
        assert res[32][name]["logit_sigma"] < res[128][name]["logit_sigma"], name
        assert res[32][name]["out_rel_l2"] < res[128][name]["out_rel_l2"], name
