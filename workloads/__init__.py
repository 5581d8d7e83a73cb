"""Seeded synthetic inputs for the OSCAR INT2 KV-cache hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no quantisation, no attention).  Both the
oracle-side tests and the HIP-side tests/bench take their inputs from here.

Every array comes from ``numpy.random.default_rng([seed, config, stream, ...])``
so any slice can be regenerated independently:

====== ==========================================================================
stream content
====== ==========================================================================
0      key outlier channels: 4 per KV head, fixed across tokens
1      per-KV-head Haar eigenbasis of the query covariance (QR with sign fix)
2      calibration queries, ``n_cal_q`` per KV head
3      calibration keys / values, ``n_cal_kv`` tokens per KV head
4      decode queries (one set per decode step)
5 / 6  context keys / values, one sub-stream per sequence (N(0,1), key outlier
       channels scaled x20 before bf16 rounding)
7      page placement: a random permutation of the shared pool
8      ragged sequence lengths (lognormal, median 8192, sigma 1, clipped)
9      tokens appended between decode steps
====== ==========================================================================

Shapes and sizes of the five workloads follow the configurations the method is
benchmarked on (one attention layer each; head_dim 128, INT2 group 128, fp16
scale/zero, 16-token pages, 128-token bf16 recent window).  The query spectrum
decays as i^-1.5.  None of this comes from a dataset: there is none for this
path, so everything is synthetic.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
GROUP = 128
PAGE = 16
WINDOW = 128
N_OUTLIERS = 4
OUTLIER_SCALE = 20.0
N_CAL_Q = 512
N_CAL_KV = 2048


def rng(seed: int, cfg: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg), int(stream), *[int(e) for e in extra]])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32/fp64 values to bf16 (round-to-nearest-even, via torch) -> uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Spec:
    cfg: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_lens: np.ndarray  # int32 [B]: context length at the first decode step
    head_dim: int = HEAD_DIM
    group_size: int = GROUP
    page_size: int = PAGE
    window: int = WINDOW
    n_sink: int = 0        # leading positions also kept in bf16 (attention sinks)
    decode_steps: int = 1  # >1: one appended token per sequence between steps
    seed: int = 0

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def capacity(self) -> np.ndarray:
        """Tokens each sequence must hold over all decode steps."""
        return self.seq_lens.astype(np.int64) + (self.decode_steps - 1)

    @property
    def max_pages(self) -> int:
        return int(max(1, -(-int(self.capacity.max()) // self.page_size)))

    @property
    def n_pages(self) -> int:
        return int(sum(-(-int(c) // self.page_size) for c in self.capacity))


NAMES = {
    1: "1L decode B1 n2048 32q/8kv",
    2: "Qwen3-8B-shaped decode B16 n32768 32q/8kv scattered pages",
    3: "long-context decode B8 n100000 32q/8kv",
    4: "prefill append T65536 x 8kv",
    5: "serving mix B64 64q/8kv lognormal n (median 8K, 1K-128K), 2 steps",
}


def ragged_lengths(seed: int, cfg: int, batch: int, median: int = 8192,
                   sigma: float = 1.0, lo: int = 1024, hi: int = 131072) -> np.ndarray:
    r = rng(seed, cfg, 8)
    n = r.lognormal(mean=math.log(median), sigma=sigma, size=batch)
    return np.clip(np.rint(n), lo, hi).astype(np.int32)


def spec(cfg: int, seed: int = 0, batch: int | None = None, seq_len: int | None = None) -> Spec:
    """Workload ``cfg`` (1..5).  ``batch``/``seq_len`` shrink it for parity runs
    (same distributions, fewer tokens)."""
    if cfg == 1:
        b, hq, lens = 1, 32, [2048]
    elif cfg == 2:
        b, hq, lens = 16, 32, [32768] * 16
    elif cfg == 3:
        b, hq, lens = 8, 32, [100000] * 8
    elif cfg == 4:
        b, hq, lens = 1, 32, [65536]
    elif cfg == 5:
        b, hq = 64, 64
        lens = list(ragged_lengths(seed, 5, 64))
    else:
        raise ValueError(f"unknown config {cfg}")
    if batch is not None:
        b = batch
        lens = (lens * ((b + len(lens) - 1) // len(lens)))[:b]
    if seq_len is not None:
        if cfg == 5:  # keep the ragged mix, rescaled so the longest is seq_len
            a = np.asarray(lens, dtype=np.float64)
            lens = list(np.maximum(1, np.rint(a * (seq_len / a.max()))).astype(int))
        else:
            lens = [seq_len] * b
    return Spec(cfg=cfg, name=NAMES[cfg], batch=b, n_q_heads=hq, n_kv_heads=8,
                seq_lens=np.asarray(lens, dtype=np.int32),
                decode_steps=2 if cfg == 5 else 1, seed=seed)


# ----------------------------------------------------------------------------
# model-side randomness (fixed per config)
# ----------------------------------------------------------------------------

def outlier_channels(s: Spec) -> np.ndarray:
    r = rng(s.seed, s.cfg, 0)
    return np.stack([r.choice(s.head_dim, N_OUTLIERS, replace=False)
                     for _ in range(s.n_kv_heads)]).astype(np.int64)


def query_spectrum(d: int = HEAD_DIM) -> np.ndarray:
    return np.arange(1, d + 1, dtype=np.float64) ** -1.5


def query_basis(s: Spec) -> np.ndarray:
    """[Hkv][d][d] Haar-orthogonal eigenbases (columns) of the true query covariance."""
    r = rng(s.seed, s.cfg, 1)
    out = np.empty((s.n_kv_heads, s.head_dim, s.head_dim))
    for h in range(s.n_kv_heads):
        g = r.standard_normal((s.head_dim, s.head_dim))
        q, rr = np.linalg.qr(g)
        out[h] = q * np.sign(np.diag(rr))[None, :]
    return out


def _draw_queries(r: np.random.Generator, basis: np.ndarray, n: int) -> np.ndarray:
    lam = query_spectrum(basis.shape[0])
    z = r.standard_normal((n, basis.shape[0]))
    return (z * np.sqrt(lam)[None, :]) @ basis.T


def _draw_kv(r: np.random.Generator, shape, outl: np.ndarray | None) -> np.ndarray:
    """N(0,1) fp32 of shape [..., Hkv, d]; if ``outl`` is given ([Hkv][4]) those
    channels of each KV head are scaled by 20."""
    x = r.standard_normal(shape, dtype=np.float32)
    if outl is not None:
        for h in range(shape[-2]):
            x[..., h, outl[h]] *= OUTLIER_SCALE
    return x


def calibration_set(s: Spec):
    """Host fp32 calibration data: q [Hkv][N_CAL_Q][d] (queries of the G heads that
    share each KV head, pooled), k, v [Hkv][N_CAL_KV][d]."""
    basis = query_basis(s)
    r = rng(s.seed, s.cfg, 2)
    q = np.stack([_draw_queries(r, basis[h], N_CAL_Q) for h in range(s.n_kv_heads)])
    r3 = rng(s.seed, s.cfg, 3)
    outl = outlier_channels(s)
    k = _draw_kv(r3, (N_CAL_KV, s.n_kv_heads, s.head_dim), outl).transpose(1, 0, 2)
    v = _draw_kv(r3, (N_CAL_KV, s.n_kv_heads, s.head_dim), None).transpose(1, 0, 2)
    return (q.astype(np.float32), np.ascontiguousarray(k, dtype=np.float32),
            np.ascontiguousarray(v, dtype=np.float32))


def decode_queries(s: Spec, step: int = 0) -> np.ndarray:
    """bf16 bits [B][Hq][d]; query head hq follows the spectrum of KV head hq // G."""
    basis = query_basis(s)
    r = rng(s.seed, s.cfg, 4, step)
    q = np.empty((s.batch, s.n_q_heads, s.head_dim), dtype=np.float32)
    for hq in range(s.n_q_heads):
        q[:, hq, :] = _draw_queries(r, basis[hq // s.gqa], s.batch)
    return to_bf16_bits(q)


def context_kv(s: Spec, b: int, n: int | None = None):
    """bf16 bits (k, v), each [n][Hkv][d], for positions 0..n-1 of sequence b."""
    n = int(s.seq_lens[b]) if n is None else int(n)
    outl = outlier_channels(s)
    k = _draw_kv(rng(s.seed, s.cfg, 5, b), (n, s.n_kv_heads, s.head_dim), outl)
    v = _draw_kv(rng(s.seed, s.cfg, 6, b), (n, s.n_kv_heads, s.head_dim), None)
    return to_bf16_bits(k), to_bf16_bits(v)


def step_tokens(s: Spec, step: int):
    """bf16 bits (k, v) [B][Hkv][d]: the token each sequence appends before decode
    step ``step`` >= 1."""
    outl = outlier_channels(s)
    r = rng(s.seed, s.cfg, 9, step)
    k = _draw_kv(r, (s.batch, s.n_kv_heads, s.head_dim), outl)
    v = _draw_kv(r, (s.batch, s.n_kv_heads, s.head_dim), None)
    return to_bf16_bits(k), to_bf16_bits(v)


def page_table(s: Spec, n_pages: int | None = None):
    """block_table int32 [B][max_pages] (unused entries -1) and the pool size.
    Pages are a random permutation of a shared pool of ``n_pages`` (default: just
    enough for every sequence's capacity)."""
    need = [-(-int(c) // s.page_size) for c in s.capacity]
    total = sum(need) if n_pages is None else int(n_pages)
    assert total >= sum(need)
    perm = rng(s.seed, s.cfg, 7).permutation(total).astype(np.int32)
    bt = np.full((s.batch, s.max_pages), -1, dtype=np.int32)
    o = 0
    for b, k in enumerate(need):
        bt[b, :k] = perm[o:o + k]
        o += k
    return bt, total


def prefill_tokens(s: Spec, b: int, n: int | None = None):
    """Token list for appending positions 0..n-1 of sequence b in one call:
    (k bits [n][Hkv][d], v bits, seq_idx int32 [n], pos int32 [n])."""
    k, v = context_kv(s, b, n)
    n = k.shape[0]
    return k, v, np.full(n, b, dtype=np.int32), np.arange(n, dtype=np.int32)
