"""Benchmark of the OSCAR INT2 KV-cache decode step on one MI355X.

Workload: long-context decode, batch 8, 100000 tokens per sequence, 32 q / 8 KV
heads, head_dim 128, INT2 history + 128-token bf16 window, 16-token pages
scattered in a shared pool (synthetic Gaussian K/V with 4 key outlier channels
x20, seeded).  One step = append the current token of every sequence + decode
attention over the whole context, as one oscar_decode_step (the appends run in
the decode's query-preparation launch); the same step as the two plain calls
(oscar_quantize_append, oscar_decode_attn) is timed beside it.  Calibration runs
once beforehand (it is an offline,
once-per-model step).  The same step on a bf16 paged cache (oscar_bf16_append +
oscar_bf16_decode_attn) on identical inputs is timed in the same session.

Every step reads a different one of ``--layers`` independent caches, as the
layers of a model would, so no step finds the previous step's cache in the
256 MB Infinity Cache.

Prints one JSON line (rank 0).  ``value`` = algorithmic HBM bytes of the INT2
step / step time (GB/s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
DECODE_SRC = os.path.join(ROOT, "kv_cache_int2_amd", "csrc", "decode.hip")
COUNTERS = os.path.join(ROOT, "profiles", "int2_split_counters_longctx_b8_n100000.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path=DECODE_SRC) -> str:
    """Hash of the decode source's code: line comments and blank lines are
    dropped, so a comment edit does not retire the committed counters."""
    import re

    code = []
    for line in open(path, encoding="utf-8"):
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def load_traffic(split_launch_bytes_alg: float):
    """HBM bytes per launch of the INT2 split kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    for line in open(COUNTERS):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("decode_source_sha") != source_sha():
        return None
    try:
        fetch = float(kv["fetch_bytes_per_launch"])
        write = float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # enough warm-up steps (~10 ms of decode) for the GPU to leave its idle
    # clocks: the first steps after an idle host gap run up to 15 % slower
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--window", type=int, default=None, help="bf16 recent-token window (default: the workload's)")
    ap.add_argument("--sinks", type=int, default=0, help="leading positions also kept in bf16 (attention sinks)")
    ap.add_argument("--group", type=int, default=128, choices=(128, 64, 32),
                    help="rotated channels per INT2 scale/zero pair (128 = one group per token)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the prefill-ingest (append) leg")
    ap.add_argument("--no-layers-leg", action="store_true", help="skip the layer-batched decode leg")
    ap.add_argument("--append-only", action="store_true",
                    help="only the prefill-ingest (append) leg, as one JSON line (for profiling it alone)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="decode time of each oracle baseline leg (one process; process pool)")
    ap.add_argument("--quality", action="store_true",
                    help="instead of the benchmark: cache quality of the OSCAR, Hadamard-only and identity "
                         "rotations through the same kernels (one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_int2_amd as K
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.quality:
        quality_leg(K, wl, torch)
        return
    if args.append_only:
        s1 = wl.spec(args.config)
        shape = K.make_shape(s1.n_q_heads, s1.n_kv_heads, s1.window, group_size=args.group)
        rk, rv, _, _ = K.oscar_calibrate(shape, *wl.calibration_set(s1))
        rkd, rvd = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev) for a in (rk, rv))
        res = append_leg(K, torch, dev, shape, rkd, rvd, args, 64 + 8 * (128 // args.group))
        # two launches of the copy probe (2 GiB each way): the known-size
        # dispatch that scales the traffic counters of a profiled run
        a = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        c = torch.empty_like(a)
        for _ in range(2):
            K.oscar_hbm_copy(a, c)
        torch.cuda.synchronize()
        del a, c
        print(json.dumps({"append": res, "data": "synthetic (seeded Gaussian K/V, 4 key outlier channels x20)"}),
              flush=True)
        return
    s = wl.spec(args.config)
    if args.window is not None:
        s.window = args.window
    s.n_sink = args.sinks
    B, HQ, HKV, W, S = s.batch, s.n_q_heads, s.n_kv_heads, s.window, s.n_sink
    lens = s.seq_lens.astype(np.int64)
    nmax = int(lens.max())
    G = args.group
    shape = K.make_shape(HQ, HKV, W, group_size=G, n_sink=S)
    tok_bytes = 64 + 8 * (128 // G)  # INT2 bytes per token and KV head: codes + one record per group

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # ---- offline calibration (host, once) ----
    t0 = time.time()
    qc, kc, vc = wl.calibration_set(s)
    rk, rv, _, _ = K.oscar_calibrate(shape, qc, kc, vc)
    rkd, rvd = T(rk), T(rv)
    log(f"calibration {time.time() - t0:.1f}s")

    # ---- caches: L independent layers, INT2 and bf16, identical K/V ----
    L = args.layers
    bt, n_pages = wl.page_table(s)
    btd, lensd = T(bt), T(lens.astype(np.int32))
    # stacked layer-major (each layer a contiguous view), so the layer-batched
    # decode can take all of them at once
    pool_all = torch.zeros((L, n_pages, HKV, K.block_bytes(G)), dtype=torch.uint8, device=dev)
    wk_all = torch.zeros((L, B, max(W + S, 1), HKV, 128), dtype=torch.int16, device=dev)
    wv_all = torch.zeros((L, B, max(W + S, 1), HKV, 128), dtype=torch.int16, device=dev)
    pools, wks, wvs = list(pool_all), list(wk_all), list(wv_all)
    kvp = [] if args.no_bf16 else [torch.zeros((n_pages, HKV, K.BF16_BLOCK_ELEMS), dtype=torch.int16, device=dev)
                                   for _ in range(L)]
    cur_k = np.empty((B, HKV, 128), np.uint16)
    cur_v = np.empty((B, HKV, 128), np.uint16)
    t0 = time.time()
    for b in range(B):
        k, v, si, ps = wl.prefill_tokens(s, b)
        cur_k[b], cur_v[b] = k[-1], v[-1]
        kd, vd, sid, psd = T(k), T(v), T(si), T(ps)
        for l in range(L):
            K.oscar_quantize_append(shape, rkd, rvd, kd, vd, sid, psd, btd, lensd, pools[l], wks[l], wvs[l])
            if kvp:
                K.oscar_bf16_append(shape, kd, vd, sid, psd, btd, kvp[l])
        del kd, vd
    torch.cuda.synchronize()
    log(f"caches built ({L} layers) {time.time() - t0:.1f}s")

    q = T(wl.decode_queries(s))
    cur_kd, cur_vd = T(cur_k), T(cur_v)
    cur_si = T(np.arange(B, dtype=np.int32))
    cur_pos = T((lens - 1).astype(np.int32))
    ws = torch.empty(K.oscar_decode_workspace_bytes(shape, B, nmax), dtype=torch.uint8, device=dev)
    out = torch.empty((B, HQ, 128), dtype=torch.float32, device=dev)

    def step_int2(i, ev=None):
        # the fused step: the newest token's append runs in the decode's
        # query-preparation launch
        l = i % L
        if ev is None:
            K.oscar_decode_step(shape, rkd, rvd, cur_kd, cur_vd, q, lensd, nmax, btd, pools[l], wks[l], wvs[l],
                                out, ws)
        else:
            K.oscar_decode_step_timed(shape, rkd, rvd, cur_kd, cur_vd, q, lensd, nmax, btd, pools[l], wks[l], wvs[l],
                                      out, ws, *ev)

    def step_int2_two_calls(i, ev=None):
        # the same step as two calls: oscar_quantize_append, oscar_decode_attn
        l = i % L
        K.oscar_quantize_append(shape, rkd, rvd, cur_kd, cur_vd, cur_si, cur_pos, btd, lensd, pools[l], wks[l], wvs[l])
        if ev is None:
            K.oscar_decode_attn(shape, rkd, rvd, q, lensd, nmax, btd, pools[l], wks[l], wvs[l], out, ws)
        else:
            K.oscar_decode_attn_timed(shape, rkd, rvd, q, lensd, nmax, btd, pools[l], wks[l], wvs[l], out, ws, *ev)

    def step_bf16(i, ev=None):
        l = i % L
        K.oscar_bf16_append(shape, cur_kd, cur_vd, cur_si, cur_pos, btd, kvp[l])
        if ev is None:
            K.oscar_bf16_decode_attn(shape, q, lensd, nmax, btd, kvp[l], out, ws)
        else:
            K.oscar_bf16_decode_attn_timed(shape, q, lensd, nmax, btd, kvp[l], out, ws, *ev)

    host_ms = {}

    def timed(step):
        """Wall time per step over the timed steps (no instrumentation), then the
        same steps again with a pair of events attached to each split kernel's
        dispatch for its duration.  Returns (s per step, mean split s, all split s)."""
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        t_enq = time.perf_counter()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t) / args.steps
        host_ms[step.__name__] = (t_enq - t) / args.steps * 1e3
        evs = [(K.Event(), K.Event()) for _ in range(args.steps)]
        # a 3 ms wait queued first: the host has enqueued every step before the
        # GPU reaches them, so no launch gap of the host falls between an event
        # and the kernel it brackets (the wait touches no memory, so it leaves
        # no dirty cache lines behind for the first step to write back)
        K.oscar_gpu_wait(3000)
        for i in range(args.steps):
            step(args.warmup + i, evs[i])
        torch.cuda.synchronize()
        kern = [K.Event.elapsed_ms(a, b) for a, b in evs]
        return dt, float(np.mean(kern)) / 1e3, kern

    # ---- in-session HBM probes ----
    probe = hbm_probes(K, torch, dev, pool_all, n_pages * L)

    # ---- algorithmic bytes ----
    win = np.minimum(lens, W)
    sink = np.minimum(S, lens - win)           # bf16 sink positions read by the decode
    hist = lens - win - sink                   # INT2 history positions
    b_hist = float(hist.sum() * HKV * tok_bytes)
    b_win = float((win + sink).sum() * HKV * 512)
    b_rot = 2 * HKV * 128 * 128 * 2
    b_q_out = B * HQ * 128 * (2 + 4)
    b_bt = float(sum(-(-int(n) // 16) for n in lens) * 4)
    b_append = B * HKV * (2 * 256 + tok_bytes + 2 * 256) + b_rot
    step_bytes_int2 = b_hist + b_win + b_rot + b_q_out + b_bt + b_append
    b_bf16_kv = float(lens.sum() * HKV * 512)
    step_bytes_bf16 = b_bf16_kv + b_q_out + b_bt + B * HKV * 2 * 2 * 256

    dt, split_s, split_all = timed(step_int2)
    if split_all:
        sa = np.asarray(split_all)
        log(f"split launches (ms): first {sa[0]:.4f} min {sa.min():.4f} median {np.median(sa):.4f} max {sa.max():.4f}")
    log(f"INT2 step {dt * 1e3:.3f} ms, split kernel {split_s * 1e3 if split_s else float('nan'):.3f} ms")
    # the same step as the two plain calls (append, then decode) against the
    # fused call: 3 alternating rounds of 60 warm-up + 50 timed steps each
    # (wall time), so that neither form gets the GPU's better or worse clocks
    def wall_per_step(step, n=50, warm=60):
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            step(warm + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / n

    rounds = {"fused": [], "two_calls": []}
    for _ in range(3):
        rounds["fused"].append(wall_per_step(step_int2))
        rounds["two_calls"].append(wall_per_step(step_int2_two_calls))
    res_two = {"fused_ms": [round(x * 1e3, 4) for x in rounds["fused"]],
               "two_calls_ms": [round(x * 1e3, 4) for x in rounds["two_calls"]],
               "two_calls_median_ms": float(np.median(rounds["two_calls"])) * 1e3,
               "fused_median_ms": float(np.median(rounds["fused"])) * 1e3,
               "workload": "the step as oscar_decode_step (fused) and as oscar_quantize_append + oscar_decode_attn "
                           "(two calls), alternating rounds"}
    log(f"step fused / two calls (ms, 3 alternating rounds): {res_two['fused_ms']} / {res_two['two_calls_ms']}")
    res_bf16 = None
    if kvp:
        dtb, split_b, _ = timed(step_bf16)
        log(f"bf16 step {dtb * 1e3:.3f} ms, split kernel {split_b * 1e3 if split_b else float('nan'):.3f} ms")
        res_bf16 = {
            "ms_per_step": dtb * 1e3,
            "decode_tokens_per_s": B / dtb,
            "hbm_gbs": step_bytes_bf16 / dtb / 1e9,
            "split_kernel_ms": split_b * 1e3 if split_b else None,
            "split_kernel_gbs": b_bf16_kv / split_b / 1e9 if split_b else None,
        }
    assert torch.isfinite(out).all()

    # ---- the decode call alone (prep, split, merge), back to back on layer 0 ----
    def call_time(reps=20):
        for _ in range(2):
            K.oscar_decode_attn(shape, rkd, rvd, q, lensd, nmax, btd, pools[0], wks[0], wvs[0], out, ws)
        K.oscar_gpu_wait(3000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            K.oscar_decode_attn(shape, rkd, rvd, q, lensd, nmax, btd, pools[0], wks[0], wvs[0], out, ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3
    b_call = b_hist + b_win + b_rot + b_q_out + b_bt
    t_call = call_time()
    res_call = {"ms": t_call * 1e3, "bytes": b_call, "gbs": b_call / t_call / 1e9,
                "frac_hbm": b_call / t_call / 1e9 / PEAK_HBM_GBS,
                "workload": "one oscar_decode_attn call (prep, split, merge kernels), calls back to back"}
    log(f"decode call {t_call * 1e6:.1f} us, {b_call / t_call / 1e9:.0f} GB/s")

    res_append = None if args.no_append else append_leg(K, torch, dev, shape, rkd, rvd, args, tok_bytes)

    # ---- layer batching: the L layers' decodes as L calls vs one call ----
    res_layers = None
    if not args.no_layers_leg and L > 1:
        q_all = q.unsqueeze(0).expand(L, -1, -1, -1).contiguous()
        rk_all = rkd.unsqueeze(0).expand(L, -1, -1, -1).contiguous()
        rv_all = rvd.unsqueeze(0).expand(L, -1, -1, -1).contiguous()
        out_all = torch.empty((L, B, HQ, 128), dtype=torch.float32, device=dev)
        ws_all = torch.empty(K.oscar_decode_layers_workspace_bytes(shape, L, B, nmax), dtype=torch.uint8, device=dev)

        def per_layer():
            for l in range(L):
                K.oscar_decode_attn(shape, rkd, rvd, q, lensd, nmax, btd, pools[l], wks[l], wvs[l], out_all[l], ws)

        def batched():
            K.oscar_decode_attn_layers(shape, rk_all, rv_all, q_all, lensd, nmax, btd, pool_all, wk_all, wv_all,
                                       out_all, ws_all)

        def time_it(fn, reps=10):
            for _ in range(2):
                fn()
            K.oscar_gpu_wait(3000)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        t_sep, t_one = time_it(per_layer), time_it(batched)
        b_dec = b_hist + b_win + b_rot + b_q_out + b_bt
        res_layers = {"n_layers": L, "per_layer_calls_ms": t_sep, "one_call_ms": t_one, "speedup": t_sep / t_one,
                      "one_call_gbs": L * b_dec / (t_one / 1e3) / 1e9,
                      "workload": f"decode of {L} layers' caches (B={B}, n={nmax}) without the append"}
        log(f"{L} layers: {t_sep:.3f} ms as {L} calls, {t_one:.3f} ms as one call ({t_sep / t_one:.2f}x)")

    # the split kernel's own bytes: the INT2 history (72 B per token and KV head
    # at group 128), the block-table entries of the history pages and the
    # rotated query operands (four e4m3 terms per channel and the group sums);
    # the window, the rotations and the output belong to the prep and merge
    b_bt_hist = float(sum(-(-int(n) // 16) for n in hist) * 4)
    b_qop = B * HQ * (4 * 128 + 4 * (128 // G))
    b_split = b_hist + b_bt_hist + b_qop
    achieved = b_split / split_s / 1e9 if split_s else None
    # the committed counters were taken on the long-context workload at its own
    # window, group 128 and no sinks: any other workload reports no traffic
    same_workload = args.config == 3 and G == 128 and S == 0 and args.window is None
    traffic = load_traffic(b_split) if same_workload else None
    line = {
        "metric": "INT2 decode-attn HBM GB/s (% of peak) + decode tokens/s at 100K ctx vs bf16 KV",
        "value": step_bytes_int2 / dt / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2 codes as fp4 x e4m3 terms (MFMA), f32 accumulate",
        "data": "synthetic (seeded Gaussian K/V, 4 key outlier channels x20; no dataset exists for this path)",
        "config": {"workload": f"long-context decode step (oscar_decode_step): append 1 token/seq + INT2 decode, "
                               f"B={B}, n={nmax}, "
                               f"{HQ}q/{HKV}kv heads, d=128, group {G}, 16-token scattered pages, bf16 window {W}"
                               + (f" + {S} sink tokens" if S else ""),
                   "layers_rotated": L, "pct_of_hbm_peak": 100 * step_bytes_int2 / dt / 1e9 / PEAK_HBM_GBS,
                   "decode_tokens_per_s": B / dt, "step_bytes": step_bytes_int2},
        "bf16_kv": res_bf16,
        "speedup_vs_bf16": (res_bf16["ms_per_step"] / (dt * 1e3)) if res_bf16 else None,
        "step_fused_vs_two_calls": res_two,
        "decode_call": res_call,
        "hbm_probe": probe,
        "host_enqueue_ms_per_step": host_ms.get("step_int2"),
        "append": res_append,
        "layers_batched": res_layers,
        "roofline": {
            "kernel": "int2_split_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS if achieved else None,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": b_split,
            "avg_launch_ms": split_s * 1e3 if split_s else None,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and G == 128 and S == 0:  # the oracle sample covers the default cache form
        line["cpu_baseline"] = cpu_baseline(s, rk, rv, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def hbm_probes(K, torch, dev, pool_all, n_pages_total):
    """In-session HBM ceilings: the copy kernel (2 GiB each way; also the scale of
    the traffic counters) and the read probe over the layer caches (n pages of
    9216 bytes, larger than the 256 MB Infinity Cache), sequentially and through
    random tables of whole pages (9216 B), half pages (the 4 KV heads a split
    workgroup reads side by side, 4608 B) and single KV-head blocks (1152 B)."""
    res = {}
    nb = 2 << 30
    a = torch.empty(nb, dtype=torch.uint8, device=dev)
    c = torch.empty(nb, dtype=torch.uint8, device=dev)
    K.oscar_hbm_copy(a, c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        K.oscar_hbm_copy(a, c)
    e1.record()
    torch.cuda.synchronize()
    res["copy_gbs"] = 2 * nb * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, c
    page = int(pool_all.shape[-1] * pool_all.shape[-2])
    total = n_pages_total * page
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    gen = np.random.default_rng(1234)
    for name, bb, table in (("seq_read_gbs", page, False), ("page_read_gbs", page, True),
                            ("half_page_read_gbs", page // 2, True), ("head_block_read_gbs", page // 8, True)):
        n = total // bb
        blocks = torch.from_numpy(gen.permutation(n).astype(np.int32)).to(dev) if table else None
        for nt in (False, True):  # plain loads, and the non-temporal hint the decode's loads carry
            K.oscar_hbm_read(pool_all, bb, blocks, n, sink, nt=nt)
            torch.cuda.synchronize()
            reps = 5
            e0.record()
            for _ in range(reps):
                K.oscar_hbm_read(pool_all, bb, blocks, n, sink, nt=nt)
            e1.record()
            torch.cuda.synchronize()
            res[name.replace("_gbs", "_nt_gbs") if nt else name] = total * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    res["bytes_per_read"] = total
    log("HBM probes (GB/s): " + ", ".join(f"{k} {v:.0f}" for k, v in res.items() if k.endswith("gbs")))
    return res


def append_leg(K, torch, dev, shape, rkd, rvd, args, tok_bytes=72):
    """Prefill ingest: oscar_quantize_append of 65536 new tokens x 8 KV heads into
    empty pages of one sequence (bf16 Gaussian K/V with outlier channels), timed
    on the append kernel's own events.  Algorithmic bytes per call: bf16 K and V
    read (512 B per token and KV head), codes + scale/zero records written
    (tok_bytes: 72 B at one group per token), the last 128 tokens written to the
    bf16 window (512 B), both rotations read."""
    import workloads as wl

    s4 = wl.spec(4)
    n, hkv, w = int(s4.seq_lens[0]), s4.n_kv_heads, s4.window
    k, v, si, ps = wl.prefill_tokens(s4, 0)
    bt, n_pages = wl.page_table(s4)

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    kd, vd, sid, psd, btd = T(k), T(v), T(si), T(ps), T(bt)
    lens = T(np.array([n], np.int32))
    pool = torch.zeros((n_pages, hkv, K.block_bytes(shape.group_size)), dtype=torch.uint8, device=dev)
    wk = torch.zeros((1, w, hkv, 128), dtype=torch.int16, device=dev)
    wv = torch.zeros_like(wk)
    for _ in range(2):
        K.oscar_quantize_append(shape, rkd, rvd, kd, vd, sid, psd, btd, lens, pool, wk, wv)
    torch.cuda.synchronize()
    reps = 20
    evs = [(K.Event(), K.Event()) for _ in range(reps)]
    # a 3 ms wait first, as for the split kernel: every timed launch is
    # dispatched from a full queue, with the GPU out of its idle clocks
    K.oscar_gpu_wait(3000)
    for i in range(reps):
        K.oscar_quantize_append_timed(shape, rkd, rvd, kd, vd, sid, psd, btd, lens, pool, wk, wv, *evs[i])
    torch.cuda.synchronize()
    t = float(np.mean([K.Event.elapsed_ms(a, b) for a, b in evs])) / 1e3
    byts = n * hkv * (512 + tok_bytes) + min(n, w) * hkv * 512 + 2 * hkv * 128 * 128 * 2
    flops = 2 * 2 * n * hkv * 128 * 128
    log(f"append 65536 tokens: {t * 1e6:.1f} us, {byts / t / 1e9:.0f} GB/s, rotation {flops / t / 1e12:.1f} TFLOP/s")
    return {"workload": "prefill ingest: 65536 bf16 K/V tokens x 8 KV heads into empty pages (one sequence)",
            "avg_launch_ms": t * 1e3, "algorithmic_bytes": byts, "achieved_gbs": byts / t / 1e9,
            "frac_hbm": byts / t / 1e9 / PEAK_HBM_GBS, "rotation_tflops": flops / t / 1e12,
            "mfma_frac_bf16": flops / t / 1e12 / 2500.0}


def quality_leg(K, wl, torch):
    """Quality of the three rotations on the 2048-token workload and on a
    shrunk copy of the 32K-context one (same distributions), at each group size
    (128, 64, 32 rotated channels per scale/zero pair)."""
    import quality

    res = {}
    for label, s in (("B1_n2048", wl.spec(1)), ("B2_n8192", wl.spec(2, batch=2, seq_len=8192))):
        shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window)
        q_cal, k_cal, v_cal = wl.calibration_set(s)
        rot = quality.rotations(shape, q_cal, k_cal, v_cal, K.oscar_calibrate)
        for g in (128, 64, 32):
            key = label if g == 128 else f"{label}_g{g}"
            t = time.perf_counter()
            res[key] = quality.measure(K, s, rot, wl, torch, group=g)
            log(f"quality {key}: {time.perf_counter() - t:.1f}s " +
                " | ".join(f"{k}: " + ", ".join(f"{m} {v:.3g}" for m, v in r.items()) for k, r in res[key].items()))
    print(json.dumps({"quality": res, "data": "synthetic (seeded Gaussian K/V, 4 key outlier channels x20)"}))


def _oracle_unit(s, rkf, rvf, b, h):
    """The oracle's cache of one (sequence, KV head) unit at full context
    (its own single-head pool and ring; building it is not timed)."""
    import workloads as wl
    from oracle import oscar_ref as ref

    n = int(s.seq_lens[b])
    k, v = wl.context_kv(s, b)
    s1 = wl.Spec(cfg=s.cfg, name=s.name, batch=1, n_q_heads=s.gqa, n_kv_heads=1,
                 seq_lens=np.array([n], np.int32), window=s.window)
    bt, n_pages = wl.page_table(s1)
    pool = np.zeros((n_pages, 1, ref.BLOCK), np.uint8)
    wk = np.zeros((1, s.window, 1, 128), np.uint16)
    wv = np.zeros_like(wk)
    ref.append_sequence_ref(rkf[h:h + 1], rvf[h:h + 1], np.ascontiguousarray(k[:, h:h + 1]),
                            np.ascontiguousarray(v[:, h:h + 1]), bt[0], pool, wk[0], wv[0], s.window)
    return n, bt, pool, wk, wv


def _oracle_decode(s, rkf, rvf, q, b, h, unit):
    """One oracle decode of a unit; returns its algorithmic cache bytes."""
    from oracle import oscar_ref as ref

    n, bt, pool, wk, wv = unit
    ref.decode_ref(rkf[h:h + 1], rvf[h:h + 1], q[b:b + 1, h * s.gqa:(h + 1) * s.gqa], np.array([n]), bt, pool, wk,
                   wv, s.window)
    w = min(n, s.window)
    return (n - w) * 72 + w * 512


_BARRIER = None


def _pool_init(barrier):
    global _BARRIER
    _BARRIER = barrier


def _pool_worker(task):
    """Worker of the process-pool leg: build one unit, wait for every worker,
    then decode it repeatedly for `seconds` of wall time (BLAS on one thread)."""
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle import oscar_ref as ref

    cfg, rk_bits, rv_bits, b, h, seconds = task
    s = wl.spec(cfg)
    rkf, rvf = ref.bf16_to_f64(rk_bits), ref.bf16_to_f64(rv_bits)
    q = wl.decode_queries(s)
    with threadpool_limits(limits=1):
        unit = _oracle_unit(s, rkf, rvf, b, h)
        _BARRIER.wait(timeout=600)  # a worker that failed to build breaks the barrier instead of hanging it
        t0 = time.perf_counter()
        nbytes, calls = 0, 0
        while time.perf_counter() - t0 < seconds:
            nbytes += _oracle_decode(s, rkf, rvf, q, b, h, unit)
            calls += 1
        return nbytes, calls, time.perf_counter() - t0


def cpu_baseline(s, rk_bits, rv_bits, target_s: float, max_units: int = 3):
    """The oracle (numpy fp64, untuned) decoding a bounded sample of the same
    workload on the host's cores, in the bench's unit (algorithmic cache bytes
    of the decoded (sequence, KV head) units per second):
      * one process, BLAS on one thread: up to ``max_units`` units at full
        context decoded round robin until ``target_s`` s of decode time;
      * a pool of P processes (P = the cores this process may run on, at most
        16), one unit each (P distinct units), all decoding their unit
        repeatedly for ``target_s`` s of wall time after a common barrier.
    ``value`` is the pool's aggregate rate; ``cores`` = P."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle import oscar_ref as ref

    rkf, rvf = ref.bf16_to_f64(rk_bits), ref.bf16_to_f64(rv_bits)
    q = wl.decode_queries(s)
    units_per_step = s.batch * s.n_kv_heads
    pairs = [(u % s.batch, (u // s.batch + 3 * u) % s.n_kv_heads) for u in range(units_per_step)]
    units = []
    with threadpool_limits(limits=1):
        for u in range(max_units):
            b, h = pairs[u]
            units.append((b, h, _oracle_unit(s, rkf, rvf, b, h)))
        total_t, total_bytes, calls = 0.0, 0.0, 0
        while total_t < target_s:
            b, h, unit = units[calls % len(units)]
            t = time.perf_counter()
            total_bytes += _oracle_decode(s, rkf, rvf, q, b, h, unit)
            total_t += time.perf_counter() - t
            calls += 1
    del units
    single = {"value": total_bytes / total_t / 1e9, "cores": 1,
              "sample": f"{calls} decode calls over {max_units} of the {units_per_step} (sequence, KV head) units, "
                        f"round robin, {total_t:.1f} s of decode time"}
    log(f"oracle, 1 process: {single['value']:.3f} GB/s")

    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    P = max(1, min(16, avail, units_per_step))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(P)
    tasks = [(s.cfg, rk_bits, rv_bits, *pairs[i], target_s) for i in range(P)]
    with ProcessPoolExecutor(max_workers=P, mp_context=ctx, initializer=_pool_init, initargs=(barrier,)) as ex:
        res = list(ex.map(_pool_worker, tasks))
    p_bytes = sum(r[0] for r in res)
    p_calls = sum(r[1] for r in res)
    p_wall = max(r[2] for r in res)
    value = p_bytes / p_wall / 1e9
    log(f"oracle, {P} processes: {value:.3f} GB/s")
    return {"value": value, "unit": "GB/s", "cores": P, "kind": "oracle",
            "sample": f"process pool of {P} (numpy fp64 oracle decode_ref, BLAS on one thread each): {P} distinct "
                      f"of the {units_per_step} (sequence, KV head) units at n={int(s.seq_lens.max())}, one per "
                      f"process, {p_calls} decode calls in {p_wall:.1f} s of wall time after a common barrier",
            "host_cpus": os.cpu_count(), "host_cpus_available": avail,
            "single_process": single,
            "decode_tokens_per_s_equiv": s.batch * value * 1e9 / (
                s.batch * s.n_kv_heads * ((int(s.seq_lens.max()) - s.window) * 72 + s.window * 512))}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (text under profiles/): kernel trace statistics and the
# HBM traffic counters of the INT2 split kernel, scaled by the copy probe.
# ---------------------------------------------------------------------------
def _short_kernel(name: str) -> str:
    n = name.replace("oscar::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0]


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_trace(directory: str, command: str) -> str:
    """Kernel statistics of a `rocprofv3 --kernel-trace --stats --output-format csv` run."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    out = ["# rocprofv3 kernel statistics", f"# command: {command}", "#",
           f"# {'kernel':44s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_%':>8s}"]
    for r in rows:
        k = _short_kernel(r["Name"])
        if k.startswith("at::"):
            continue
        out.append(f"  {k:44s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}")
    # the INT2 decode step kernel by kernel in launch order (prep, split,
    # merge; in the two-call form an append kernel before them), with the idle
    # gap before each (medians over the steps)
    trace = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    forms = {"fused step (oscar_decode_step)": ["prep_kernel", "int2_split_kernel", "merge_kernel"],
             "two calls (append kernel, then oscar_decode_attn)": ["append_kernel", "prep_kernel",
                                                                     "int2_split_kernel", "merge_kernel"]}
    for title, names in forms.items():
        k = len(names)
        dur, gap = {n: [] for n in names}, {n: [] for n in names}
        for i in range(k - 1, len(trace)):
            seq = trace[i - k + 1:i + 1]
            if not all(_short_kernel(r["Kernel_Name"]).startswith(n) for r, n in zip(seq, names)):
                continue
            if k == 3 and not re.fullmatch(r"prep_kernel<\d+,[124]>", _short_kernel(seq[0]["Kernel_Name"]).replace(" ", "")):
                continue  # a plain decode call (its prep kernel appends nothing)
            for j, (r, n) in enumerate(zip(seq, names)):
                dur[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                if j:
                    gap[n].append((int(r["Start_Timestamp"]) - int(seq[j - 1]["End_Timestamp"])) / 1e3)
        if dur["int2_split_kernel"]:
            out += ["#", f"# INT2 decode step, {title}, kernel by kernel ({len(dur['int2_split_kernel'])} steps; "
                    "the tracer itself lengthens the gaps)", f"# {'kernel':44s} {'median_us':>10s} {'gap_before_us':>14s}"]
            for n in names:
                g = f"{np.median(gap[n]):14.2f}" if gap[n] else f"{'-':>14s}"
                out.append(f"  {n:44s} {np.median(dur[n]):10.2f} {g}")
    return "\n".join(out) + "\n"


def summarize_pmc(fetch_dir: str, write_dir: str, command: str, bench_json: str = None) -> str:
    """HBM bytes per launch of the INT2 split kernel from FETCH_SIZE and WRITE_SIZE
    runs (KiB per dispatch), each scaled by what the same counter reads for the
    copy probe of known size (2 GiB read + 2 GiB written per launch)."""
    def per_kernel(directory, counter):
        acc = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(_short_kernel(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        out = {k: float(np.mean(v)) for k, v in acc.items()}
        # only the probe's dispatches (the largest copies) calibrate the scale
        cp = np.asarray(acc["copy_kernel"])
        out["copy_kernel"] = float(np.mean(cp[cp > 0.5 * cp.max()]))
        return out

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = float(2 << 30)
    f_copy = fetch["copy_kernel"] * 1024.0
    w_copy = write["copy_kernel"] * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    split = [k for k in fetch if k.startswith("int2_split_kernel")][0]
    fb = fetch[split] * 1024.0 * f_scale
    wb = write[split] * 1024.0 * w_scale
    lines = ["# HBM traffic of the INT2 split kernel (rocprofv3 --pmc), long-context decode B=8 n=100000",
             f"# command: {command}",
             "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by copy_bytes / (counter of the",
             "# copy probe), the probe moving 2 GiB each way per launch.",
             f"decode_source_sha: {source_sha()}",
             f"split_kernel: {split}",
             f"fetch_kib_raw: {fetch[split]:.1f}",
             f"write_kib_raw: {write[split]:.1f}",
             f"copy_fetch_kib_raw: {fetch['copy_kernel']:.1f}",
             f"copy_write_kib_raw: {write['copy_kernel']:.1f}",
             f"fetch_scale: {f_scale:.4f}",
             f"write_scale: {w_scale:.4f}",
             f"fetch_bytes_per_launch: {fb:.0f}",
             f"write_bytes_per_launch: {wb:.0f}"]
    for k in sorted(fetch):
        if k.startswith("at::"):
            continue
        lines.append(f"# {k:40s} FETCH_SIZE {fetch[k]:12.1f} KiB  WRITE_SIZE {write.get(k, float('nan')):12.1f} KiB (raw)")
    if bench_json:
        # second check of the fetch scale: the read probe's dispatches each read
        # bytes_per_read bytes (sequential and through random page tables)
        line = [json.loads(x) for x in open(bench_json) if x.startswith("{")][-1]
        nbytes = float(line["hbm_probe"]["bytes_per_read"])
        lines.append(f"read_probe_bytes_per_launch: {nbytes:.0f}")
        for variant, tag in (("read_kernel", ""), ("read_kernel<false>", ""), ("read_kernel<true>", "_nt")):
            reads = [float(r["Counter_Value"]) * 1024.0 for r in _csv_rows(fetch_dir, "counter_collection.csv")
                     if r["Counter_Name"] == "FETCH_SIZE" and _short_kernel(r["Kernel_Name"]) == variant]
            if reads:
                sc = nbytes / np.asarray(reads)
                lines.append(f"read_probe{tag}_fetch_scale: min {sc.min():.4f} median {np.median(sc):.4f} "
                             f"max {sc.max():.4f} ({len(sc)} dispatches)")
    return "\n".join(lines) + "\n"


def summarize_counters(command: str, dirs) -> str:
    """Per-kernel means per dispatch of every counter in one or more
    `rocprofv3 --pmc` runs (one pass each), for this library's kernels and the
    probes, with derived fractions.  GRBM_GUI_ACTIVE comes summed over the 8
    XCDs, so a dispatch lasts GRBM_GUI_ACTIVE / 8 cycles; SQ_ACTIVE_INST_* count
    quad-cycles (a wave64 VALU instruction issues over 4 cycles) summed over the
    1024 SIMDs, SQ_VALU_MFMA_BUSY_CYCLES cycles summed over the SIMDs."""
    acc = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            k = _short_kernel(r["Kernel_Name"])
            if k.startswith("at::") or "elementwise" in k or "rocclr" in k:
                continue
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = ["# rocprofv3 --pmc counters, mean per dispatch", f"# command: {command}", "#"]
    for k in sorted(acc):
        c = {n: float(np.mean(v)) for n, v in acc[k].items()}
        n = max(len(v) for v in acc[k].values())
        out.append(f"{k}  ({n} dispatches)")
        for name in sorted(c):
            out.append(f"  {name:34s} {c[name]:16.1f}")
        if c.get("GRBM_GUI_ACTIVE"):
            simd = 1024 * c["GRBM_GUI_ACTIVE"] / 8  # SIMD-cycles of the dispatch
            out.append(f"  {'=> dispatch cycles (per XCD)':34s} {c['GRBM_GUI_ACTIVE'] / 8:16.0f}")
            for cnt, label, mul in (("SQ_ACTIVE_INST_ANY", "issue busy", 4), ("SQ_ACTIVE_INST_VALU", "VALU busy", 4),
                                    ("SQ_ACTIVE_INST_LDS", "LDS issue busy", 4),
                                    ("SQ_VALU_MFMA_BUSY_CYCLES", "MFMA busy", 1)):
                if cnt in c:
                    out.append(f"  {'=> ' + label + ' (per SIMD)':34s} {mul * c[cnt] / simd:16.3f}")
        cp = acc.get("copy_kernel", {})
        for cnt in ("FETCH_SIZE", "WRITE_SIZE"):
            if cnt in c and cp.get(cnt):
                ref = np.asarray(cp[cnt])
                scale = float(2 << 30) / (1024.0 * float(np.mean(ref[ref > 0.5 * ref.max()])))
                out.append(f"  {'=> ' + cnt + ' bytes (x%.3f)' % scale:34s} {1024.0 * c[cnt] * scale:16.0f}")
        if c.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in c:
            out.append(f"  {'=> conflict cycles per LDS inst':34s} {c['SQ_LDS_BANK_CONFLICT'] / c['SQ_INSTS_LDS']:16.3f}")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # bench.py --summarize-trace DIR "COMMAND"
        sys.stdout.write(summarize_trace(sys.argv[2], sys.argv[3]))
    elif len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters "COMMAND" DIR [DIR ...]
        sys.stdout.write(summarize_counters(sys.argv[2], sys.argv[3:]))
    elif len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        # bench.py --summarize-pmc FETCH_DIR WRITE_DIR "COMMAND" [BENCH_JSON_OUTPUT]
        sys.stdout.write(summarize_pmc(sys.argv[2], sys.argv[3], sys.argv[4], *sys.argv[5:6]))
    else:
        main()
