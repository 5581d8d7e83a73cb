"""Plain CPU oracle for the OSCAR INT2 KV-cache hot path (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` use it.  It shares no code, table or constant generator with the
HIP library; the only thing both sides share is the seeded input generator
(``workloads``), which holds none of the method's arithmetic.

Sources (the text of five web pages about the method; cited below by key):

  P1  gen-hub.ru, "Together AI открывает OSCAR: сжатие KV-кэша до 2 бит без
      потери точности"
  P2  encorp.ai, "KV cache compression е инфраструктурно решение, не спор за модела"
  P3  bigsaas.top, "Revolução no Serviço de LLMs: Together AI Lança OSCAR para
      Contextos Extensos"
  P4  aiforradalom.hu, "Az Apple, a Google és a NYU új technikái felezik az
      LLM-ek memóriaigényét"
  P5  ru.arsentev.ai, "Гонка за сжатие памяти ИИ на длинном контексте"

The pages describe the method in prose only.  Where they leave a step open the
plainest reading is taken (each listed in the repository's design notes):
uncentred second moments; eigenvectors as columns, sorted by descending
eigenvalue, sign fixed so the largest-magnitude entry of each is positive;
value weights = total softmax mass each calibration token receives; Sylvester
Hadamard scaled by 1/sqrt(d); R = P_br . (H/sqrt d) . U^T acting on column
vectors; one quantisation group = g consecutive rotated channels of one token
(g = 128, the whole token, by default; 64 or 32 for the finer variant); float
zero point = group minimum; fp16 RNE for scale and zero; codes rounded half to
even from the stored fp16 scale/zero, clamped to [0, 3].

Precision.  Rotations, covariances, eigenproblems and attention are fp64.  The
integer decisions of the encoder (min/max, scale, zero, codes) are taken in
fp32 arithmetic on the fp32-rounded exact rotation, i.e. in the precision of
the device encoder, as no precision is fixed by the pages.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, library routines on special cases, invariants and brute force;
none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Page-block layout (per page, per KV head, 1152 bytes at group size 128)
#   [   0,  512)  K codes: 16 token rows x 32 B; channel c of a row in byte
#                 8 ((c >> 2) & 3) + (c >> 4), bits 2 (c & 3) (see k_row_byte)
#   [ 512, 1024)  V codes: 128 channel words x 4 B; token slot j at bit 2j
#   [1024, 1152)  16 token records of 8 bytes: fp16 K scale, K zero, V scale, V zero
# With groups of g < 128 channels (ng = 128 / g per token) the records grow to
# 16 x ng: the record of group j of slot t sits at 1024 + 8 (ng t + j), and the
# block is 1024 + 128 ng bytes (block_bytes).
# Pool = uint8 [n_pages][Hkv][block bytes].  Window ring = bf16 [B][W][Hkv][d], slot pos % W.
# bf16 comparator pool = bf16 [n_pages][Hkv][4096]: K rows [16 slots][d], then V
# transposed [d][16 slots] (see append_bf16_ref).
# ---------------------------------------------------------------------------
D = 128
PAGE = 16
K_CODES, V_CODES, META, BLOCK = 0, 512, 1024, 1152
# fields of a token's 8-byte record at META + 8 * slot (per group: META + 8 (ng slot + j))
K_SCALE, K_ZERO, V_SCALE, V_ZERO = 0, 2, 4, 6
GROUP_SIZES = (32, 64, 128)


def block_bytes(group: int = D) -> int:
    """Bytes of one (page, KV head) block: 1024 of K and V codes plus one 8-byte
    record per token and group."""
    assert group in GROUP_SIZES
    return META + 8 * PAGE * (D // group)


# ---------------------------------------------------------------------------
# floating-point formats
# ---------------------------------------------------------------------------

def _round_binary(x, p: int, emin: int) -> np.ndarray:
    """Round fp64 ``x`` to the nearest value of a binary format with ``p``
    significant bits and minimum normal exponent ``emin`` (ties to even),
    subnormals included.  Exact: only power-of-two scalings and np.rint."""
    x = np.asarray(x, dtype=np.float64)
    _, e2 = np.frexp(np.abs(x))          # |x| = m * 2**e2, m in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, emin)
    q = np.ldexp(1.0, (e - (p - 1)).astype(np.int64))
    return np.rint(x / q) * q


def fp16_rne(x) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of fp64 values (returned as fp64)."""
    r = _round_binary(x, 11, -14)
    if np.any(np.abs(r) > 65504.0):
        raise OverflowError("fp16 overflow")
    return r


def bf16_rne(x) -> np.ndarray:
    """bfloat16 round-to-nearest-even of fp64 values (returned as fp64)."""
    return _round_binary(x, 8, -126)


def fp16_bits(x) -> np.ndarray:
    return fp16_rne(x).astype(np.float16).view(np.uint16)


def bf16_bits(x) -> np.ndarray:
    return (bf16_rne(x).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# the fixed transforms: Hadamard and bit reversal  [P1 «Что придумали в
# Together AI»: after the eigenbasis, a Hadamard to even out channel importance,
# then a bit-reversal permutation so every quantisation group gets an even share
# of the importance order; P4 «OSCAR: figyelem-tudatos és bevetésre kész»]
# ---------------------------------------------------------------------------

def hadamard(d: int = D) -> np.ndarray:
    """Sylvester Hadamard matrix, closed form H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def bit_reverse_index(d: int = D) -> np.ndarray:
    """br(i): i with its log2(d) bits reversed."""
    nb = int(round(math.log2(d)))
    assert 1 << nb == d
    return np.array([int(format(i, f"0{nb}b")[::-1], 2) for i in range(d)], dtype=np.int64)


def apply_bitrev_rows(m: np.ndarray) -> np.ndarray:
    """P_br . m, where (P_br y)_i = y_{br(i)} (rows permuted)."""
    return m[bit_reverse_index(m.shape[0])]


# ---------------------------------------------------------------------------
# calibration  [P1 «Что придумали в Together AI»: keys are rotated into the
# eigenbasis of the empirical query covariance (it weights the error of the
# logits Q K^T); values into the eigenbasis of the value covariance weighted by
# attention scores (it weights the error of S V).  P1 «Открытый код — это
# серьёзно» and P3 «Como Funciona o OSCAR?»: offline, once per model.]
# ---------------------------------------------------------------------------

def eig_desc(s: np.ndarray):
    """Eigen-decomposition of a symmetric matrix: eigenvalues descending,
    eigenvectors as columns, each with its largest-|entry| positive (first index
    on ties).  numpy.linalg.eigh is the textbook routine."""
    s = 0.5 * (np.asarray(s, dtype=np.float64) + np.asarray(s, dtype=np.float64).T)
    w, u = np.linalg.eigh(s)
    order = np.argsort(-w, kind="stable")
    w, u = w[order], u[:, order]
    idx = np.argmax(np.abs(u), axis=0)
    sgn = np.sign(u[idx, np.arange(u.shape[1])])
    sgn[sgn == 0] = 1.0
    return w, u * sgn[None, :]


def query_covariance(q: np.ndarray) -> np.ndarray:
    """E[q q^T] over the calibration queries (uncentred)."""
    q = np.asarray(q, dtype=np.float64)
    return q.T @ q / q.shape[0]


def score_weights(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """a_j = sum_i softmax_j(q_i . k_j / sqrt(d)): attention mass token j gets."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    logits = q @ k.T / math.sqrt(q.shape[1])
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def value_covariance(v: np.ndarray, a: np.ndarray) -> np.ndarray:
    """sum_j a_j v_j v_j^T / sum_j a_j."""
    v = np.asarray(v, dtype=np.float64)
    return (v.T * a[None, :]) @ v / a.sum()


def rotation_from_basis(u: np.ndarray) -> np.ndarray:
    """R = P_br . (H / sqrt d) . U^T, acting on column vectors (x' = R x)."""
    d = u.shape[0]
    return apply_bitrev_rows(hadamard(d) / math.sqrt(d) @ u.T)


def calibrate_ref(q_cal, k_cal, v_cal):
    """Per KV head: (R_K, R_V) fp64 [Hkv][d][d], eigenvalues [Hkv][d] each.
    q_cal [Hkv][n_q][d]; k_cal, v_cal [Hkv][n_kv][d]."""
    hkv, _, d = np.shape(q_cal)
    rk, rv = np.empty((hkv, d, d)), np.empty((hkv, d, d))
    ek, ev = np.empty((hkv, d)), np.empty((hkv, d))
    for h in range(hkv):
        ek[h], uq = eig_desc(query_covariance(q_cal[h]))
        a = score_weights(q_cal[h], k_cal[h])
        ev[h], us = eig_desc(value_covariance(v_cal[h], a))
        rk[h] = rotation_from_basis(uq)
        rv[h] = rotation_from_basis(us)
    return rk, rv, ek, ev


# ---------------------------------------------------------------------------
# encoder: rotate -> asymmetric 2-bit quantise -> pack
# [P1 «Почему INT2 раньше не работал»: 2 bits = four levels; P1 «Что это даёт
#  на практике»: paged KV-cache systems; group size 128 and fp16 scale/zero are
#  the benchmark configuration's parameters]
# ---------------------------------------------------------------------------

def rotate(r: np.ndarray, x: np.ndarray) -> np.ndarray:
    """x' = R x for every vector in x [..., d] (fp64; exact for bf16 data)."""
    return np.einsum("ij,...j->...i", np.asarray(r, np.float64), np.asarray(x, np.float64))


def quantize(xr: np.ndarray):
    """Asymmetric INT2 codes of each group (last axis = the 128 rotated channels).

    Steps, all on the fp32 value of the rotation: m = min, M = max;
    s = fp16(fp32((M - m) / 3)); z = fp16(m); t = fp32((x' - z) / s);
    c = clamp(round_half_even(t), 0, 3); a zero scale gives all-zero codes.
    Returns codes int64, s and z as fp64 values, and the fp32 pre-rounding values
    (sigma, m, t) that the parity rule uses."""
    x32 = np.asarray(xr, dtype=np.float64).astype(np.float32)
    m = x32.min(axis=-1)
    mx = x32.max(axis=-1)
    sigma = ((mx - m).astype(np.float32) / np.float32(3.0)).astype(np.float32)
    s = fp16_rne(sigma.astype(np.float64))
    z = fp16_rne(m.astype(np.float64))
    s32 = s.astype(np.float32)
    z32 = z.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    t = ((x32 - z32[..., None]).astype(np.float32) / safe[..., None]).astype(np.float32)
    c = np.clip(np.rint(t), 0, 3).astype(np.int64)
    c = np.where((s32 == 0)[..., None], 0, c)
    return c, s, z, dict(sigma=sigma, m=m, t=t)


def quantize_groups(xr: np.ndarray, group: int = D):
    """``quantize`` applied to each run of ``group`` consecutive rotated channels
    [P1 «Что придумали в Together AI»: per-token asymmetric 2-bit groups; a group
    shorter than the token is the finer variant with more scale/zero metadata].
    Returns codes int64 [..., d] and s, z fp64 [..., d / group]."""
    xr = np.asarray(xr, dtype=np.float64)
    ng = D // group
    c, s, z, _ = quantize(xr.reshape(xr.shape[:-1] + (ng, group)))
    return c.reshape(xr.shape), s, z


def k_row_byte(c):
    """Byte of a K row holding channel c (its bits: 2 (c mod 4) .. +1).  The row is
    four 8-byte segments; segment s holds channels 16 m + 4 s + i (m = 0..7 is the
    byte within the segment, i = 0..3 the 2-bit field within the byte)."""
    c = np.asarray(c)
    return 8 * ((c >> 2) & 3) + (c >> 4)


def pack_k_row(codes: np.ndarray) -> np.ndarray:
    """[..., 128] codes -> [..., 32] bytes in the K-row layout of ``k_row_byte``."""
    c = np.asarray(codes, dtype=np.uint8)
    lead = c.shape[:-1]
    out = np.zeros(lead + (32,), dtype=np.uint8)
    for ch in range(128):
        out[..., k_row_byte(ch)] |= (c[..., ch] << (2 * (ch & 3))).astype(np.uint8)
    return out


def unpack_k_rows(rows: np.ndarray) -> np.ndarray:
    """[..., 32] bytes -> [..., 128] codes (inverse of ``pack_k_row``)."""
    r = np.asarray(rows, dtype=np.uint8)
    ch = np.arange(128)
    return ((r[..., k_row_byte(ch)] >> (2 * (ch & 3)).astype(np.uint8)) & 3).astype(np.int64)


def v_words(block: np.ndarray) -> np.ndarray:
    """uint32 view [..., 128] of the V-code region of page blocks [..., 1152]."""
    return np.ascontiguousarray(block[..., V_CODES:V_CODES + 512]).view("<u4")


def unpack_v_words(words: np.ndarray) -> np.ndarray:
    """[..., 128] channel words -> codes [..., 16 slots, 128 channels]."""
    w = np.asarray(words, dtype=np.uint32)[..., None, :]
    sh = (2 * np.arange(16, dtype=np.uint32))[:, None]
    return ((w >> sh) & 3).astype(np.int64)


def _put_fp16(block, field, slot, bits, grp: int = 0, ng: int = 1):
    a = META + 8 * (ng * slot + grp) + field
    block[a: a + 2] = np.array([bits], dtype=np.uint16).view(np.uint8)


def append_ref(r_k, r_v, k_new, v_new, seq_idx, pos, block_table, seq_len_after,
               pool, win_k, win_v, window: int, n_sink: int = 0, group: int = D):
    """Write each token into the paged INT2 cache and, if recent or a sink, the
    bf16 ring.

    r_k, r_v: fp64 [Hkv][d][d] (bf16 values as data); k_new, v_new: bf16 bits
    [T][Hkv][d]; pool uint8 [n_pages][Hkv][block_bytes(group)] and rings bf16 bits
    [B][W + n_sink][Hkv][d] are updated in place.  Token i lands in page
    block_table[b][pos // 16], slot pos % 16; its raw bf16 k/v also go to ring
    row pos % W when pos >= seq_len_after[b] - W, and to ring row W + pos when
    pos < n_sink  [P2 «OSCAR има значение…», P4 «OSCAR: figyelem-tudatos…»:
    sink and recent tokens stay bf16, history is INT2]."""
    k_new = np.asarray(k_new)
    hkv = k_new.shape[1]
    # x'[t, h] = R[h] x[t, h]
    kr = np.einsum("hij,thj->thi", np.asarray(r_k, np.float64), bf16_to_f64(k_new))
    vr = np.einsum("hij,thj->thi", np.asarray(r_v, np.float64), bf16_to_f64(v_new))
    ng = D // group
    kc, ks, kz = quantize_groups(kr, group)                 # s, z: [T][Hkv][ng]
    vc, vs, vz = quantize_groups(vr, group)
    ksb, kzb, vsb, vzb = fp16_bits(ks), fp16_bits(kz), fp16_bits(vs), fp16_bits(vz)
    krow = pack_k_row(kc)                                   # [T][Hkv][32]
    for i in range(k_new.shape[0]):
        b, p = int(seq_idx[i]), int(pos[i])
        page = int(block_table[b][p // PAGE])
        assert page >= 0, "position outside the block table"
        slot = p % PAGE
        for h in range(hkv):
            blk = pool[page, h]
            blk[K_CODES + 32 * slot: K_CODES + 32 * slot + 32] = krow[i, h]
            words = v_words(blk).copy()
            words &= ~np.uint32(3 << (2 * slot))
            words |= (vc[i, h].astype(np.uint32) << np.uint32(2 * slot))
            blk[V_CODES:V_CODES + 512] = words.astype("<u4").view(np.uint8)
            for j in range(ng):
                _put_fp16(blk, K_SCALE, slot, ksb[i, h, j], j, ng)
                _put_fp16(blk, K_ZERO, slot, kzb[i, h, j], j, ng)
                _put_fp16(blk, V_SCALE, slot, vsb[i, h, j], j, ng)
                _put_fp16(blk, V_ZERO, slot, vzb[i, h, j], j, ng)
        if window > 0 and p >= int(seq_len_after[b]) - window:
            win_k[b, p % window] = k_new[i]
            win_v[b, p % window] = v_new[i]
        if p < n_sink:
            win_k[b, window + p] = k_new[i]
            win_v[b, window + p] = v_new[i]


def read_history(pool, block_table_row, hist: int, h: int, group: int = D):
    """Dequantised rotated history of one (sequence, KV head): (k', v') fp64 [hist][d].
    x'_c = z + code_c s with the stored fp16 z, s of channel c's group."""
    n_pg = -(-hist // PAGE)
    ng = D // group
    pages = np.asarray(block_table_row[:n_pg], dtype=np.int64)
    assert np.all(pages >= 0)
    blk = pool[pages, h]                                    # [n_pg][block bytes]
    assert blk.shape[-1] == block_bytes(group)
    kc = unpack_k_rows(blk[:, K_CODES:K_CODES + 512].reshape(n_pg, PAGE, 32))
    vc = unpack_v_words(v_words(blk))                       # [n_pg][16][128]
    meta = np.ascontiguousarray(blk[:, META:]).view(np.uint16).reshape(n_pg, PAGE, ng, 4)
    # each group's value spread over its channels: [n_pg][16][128]
    ks, kz, vs, vz = (np.repeat(fp16_to_f64(meta[..., f // 2]), group, axis=-1)
                      for f in (K_SCALE, K_ZERO, V_SCALE, V_ZERO))
    with np.errstate(invalid="ignore", over="ignore"):  # unused slots of the last page
        k = kz + kc * ks
        v = vz + vc * vs
    return k.reshape(-1, D)[:hist], v.reshape(-1, D)[:hist]


# ---------------------------------------------------------------------------
# decode attention on the mixed-precision cache
# [P1 «Что придумали в Together AI»: keys in the query eigenbasis, so q is
#  rotated by the key transform; values are un-rotated by the value transform;
#  P2 «OSCAR има значение…», P4 «OSCAR: figyelem-tudatos…»: bf16 recent
#  tokens + INT2 history on paged storage]
# ---------------------------------------------------------------------------

def decode_ref(r_k, r_v, q_bits, seq_lens, block_table, pool, win_k, win_v,
               window: int, pairs=None, n_sink: int = 0, group: int = D):
    """Softmax attention of one query token per (sequence, q head) over the
    dequantised cache, fp64.  With w = min(n, W) and s = min(n_sink, n - w):
    positions [0, s) come from the bf16 sink rows W + pos of the ring, [s, n - w)
    from the INT2 pages (rotated domain: scores q'.k'/sqrt d with q' = R_K q;
    values un-rotated by R_V^T), [n - w, n) from the bf16 window rows pos % W
    (sink and window in the plain domain).  ``pairs``: iterable of (b, kv_head)
    to compute (default all); other outputs are NaN."""
    q = bf16_to_f64(q_bits)
    bsz, hq, d = q.shape
    hkv = np.shape(r_k)[0]
    g = hq // hkv
    out = np.full((bsz, hq, d), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(bsz) for h in range(hkv)]
    for b, h in pairs:
        n = int(seq_lens[b])
        if n == 0:  # no position to attend: the output is zero (a reading; softmax over nothing is undefined)
            out[b, h * g:(h + 1) * g] = 0.0
            continue
        w = min(n, window)
        hist = n - w
        ns = min(n_sink, hist)
        kh, vh = read_history(pool, block_table[b], hist, h, group) if hist > 0 else (np.zeros((0, d)), np.zeros((0, d)))
        kh, vh = kh[ns:], vh[ns:]
        # plain-domain rows: sinks (rows W + pos), then the window (rows pos % W)
        rows = np.concatenate([window + np.arange(ns), np.arange(hist, n) % max(window, 1)]).astype(np.int64)
        kw = bf16_to_f64(win_k[b, rows, h]) if rows.size else np.zeros((0, d))
        vw = bf16_to_f64(win_v[b, rows, h]) if rows.size else np.zeros((0, d))
        nh = hist - ns
        for j in range(g):
            qq = q[b, h * g + j]
            qr = np.asarray(r_k[h], np.float64) @ qq
            s = np.concatenate([kh @ qr, kw @ qq]) / math.sqrt(d)
            p = np.exp(s - s.max())
            o_rot = p[:nh] @ vh
            o = np.asarray(r_v[h], np.float64).T @ o_rot + p[nh:] @ vw
            out[b, h * g + j] = o / p.sum()
    return out


BF16_BLOCK = 2 * PAGE * D  # elements of one (page, KV head) block of the bf16 comparator pool


def append_bf16_ref(k_new, v_new, seq_idx, pos, block_table, kv_pool):
    """Scatter bf16 k/v [T][Hkv][d] into the comparator pool [n_pages][Hkv][4096]:
    K rows [16 slots][d], then V transposed [d][16 slots]."""
    ch = np.arange(D)
    for i in range(np.shape(k_new)[0]):
        b, p = int(seq_idx[i]), int(pos[i])
        page = int(block_table[b][p // PAGE])
        assert page >= 0
        slot = p % PAGE
        blk = kv_pool[page]                      # [Hkv][4096] view
        blk[:, slot * D:(slot + 1) * D] = k_new[i]
        blk[:, PAGE * D + ch * PAGE + slot] = v_new[i]


def bf16_pages_kv(kv_pool, pages, h):
    """K, V bits [len(pages) * 16][d] of KV head h from comparator pool blocks."""
    blk = np.asarray(kv_pool)[pages, h]                                  # [n_pg][4096]
    k = blk[:, :PAGE * D].reshape(-1, PAGE, D)
    v = blk[:, PAGE * D:].reshape(-1, D, PAGE).transpose(0, 2, 1)
    return k.reshape(-1, D), v.reshape(-1, D)


def decode_bf16_ref(q_bits, seq_lens, block_table, kv_pool, n_kv_heads: int, pairs=None):
    """Textbook softmax attention over a bf16 paged cache (the comparator), fp64."""
    q = bf16_to_f64(q_bits)
    bsz, hq, d = q.shape
    g = hq // n_kv_heads
    out = np.full((bsz, hq, d), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(bsz) for h in range(n_kv_heads)]
    for b, h in pairs:
        n = int(seq_lens[b])
        n_pg = -(-n // PAGE)
        pages = np.asarray(block_table[b][:n_pg], dtype=np.int64)
        assert np.all(pages >= 0)
        kb, vb = bf16_pages_kv(kv_pool, pages, h)
        k = bf16_to_f64(kb)[:n]
        v = bf16_to_f64(vb)[:n]
        for j in range(g):
            s = k @ q[b, h * g + j] / math.sqrt(d)
            p = np.exp(s - s.max())
            out[b, h * g + j] = (p @ v) / p.sum()
    return out


# ---------------------------------------------------------------------------
# byte accounting  [P3 «Resultados e Métricas de Desempenho»: about 2.28 bits per
# KV element; P2 «OSCAR има значение…»: about 0.24 % of tokens stay bf16 at 128K;
# P2 «KV cache compression става болезнен…»: Llama-3.1-70B bf16 KV about
# 0.31 MB per token, 40 GB at 128K, over 300 GB at 1M; P1 «Что это даёт на
# практике»: 2 bits is 4x below FP8 and 2x below INT4]
# ---------------------------------------------------------------------------

def int2_bytes_per_token_head(d: int = D, group: int = 128, meta_bytes: int = 2) -> int:
    """K + V bytes of one token of one KV head in the INT2 cache: codes plus an
    fp16 scale and zero per group."""
    return 2 * (d * 2 // 8 + 2 * meta_bytes * (d // group))


def int2_bits_per_element(d: int = D, group: int = 128) -> float:
    return int2_bytes_per_token_head(d, group) * 8 / (2 * d)


def effective_bits(bf16_share: float, d: int = D, group: int = 128) -> float:
    return int2_bits_per_element(d, group) * (1.0 - bf16_share) + 16.0 * bf16_share


def bf16_kv_bytes_per_token(n_layers: int, n_kv_heads: int, d: int) -> int:
    return 2 * n_layers * n_kv_heads * d * 2


def decode_direct_ref(r_k, r_v, q_bits, k_bits, v_bits, n: int, window: int, kv_head: int,
                      n_sink: int = 0, group: int = D):
    """Decode of one (sequence, KV head) straight from its token sequence, with
    no pool or ring: with w = min(n, W) and s = min(n_sink, n - w), positions
    [s, n - w) are encoded with ``quantize_groups`` (the cache's content by definition),
    positions [0, s) and the last w are the raw bf16 tokens.  Same attention as
    ``decode_ref``.  q_bits [G][d] (the G query heads of this KV head); k_bits,
    v_bits [>= n][d].  Returns fp64 [G][d]."""
    d = D
    w = min(n, window)
    hist = n - w
    ns = min(n_sink, hist)
    rk = np.asarray(r_k[kv_head], np.float64)
    rv = np.asarray(r_v[kv_head], np.float64)
    kx = bf16_to_f64(np.asarray(k_bits)[:n])
    vx = bf16_to_f64(np.asarray(v_bits)[:n])
    ck, sk, zk = quantize_groups(rotate(rk, kx[ns:hist]), group)
    cv, sv, zv = quantize_groups(rotate(rv, vx[ns:hist]), group)
    grp = np.arange(D) // group                     # group of each channel
    kh = zk[:, grp] + ck * sk[:, grp]
    vh = zv[:, grp] + cv * sv[:, grp]
    plain = np.r_[0:ns, hist:n]
    q = bf16_to_f64(q_bits)
    out = np.empty((q.shape[0], d))
    for j in range(q.shape[0]):
        s = np.concatenate([kh @ (rk @ q[j]), kx[plain] @ q[j]]) / math.sqrt(d)
        p = np.exp(s - s.max())
        nh = hist - ns
        out[j] = (rv.T @ (p[:nh] @ vh) + p[nh:] @ vx[plain]) / p.sum()
    return out


def append_sequence_ref(r_k, r_v, k_bits, v_bits, block_row, pool, win_k, win_v, window: int,
                        n_sink: int = 0, group: int = D):
    """Bulk form of ``append_ref`` for positions 0..n-1 of one sequence appended
    in order (seq_len_after = n): whole pages are packed at once.  Produces the
    same bytes as ``append_ref`` (pinned by a test).  k_bits, v_bits [n][Hkv][d];
    block_row int32 [max_pages]; pool [n_pages][Hkv][block_bytes(group)]; win_k, win_v
    [W + n_sink][Hkv][d] (this sequence's ring)."""
    k_bits = np.asarray(k_bits)
    n, hkv, _ = k_bits.shape
    kr = np.empty((n, hkv, D))
    vr = np.empty((n, hkv, D))
    for h in range(hkv):   # x' = R x for every token (library matmul per head)
        kr[:, h] = bf16_to_f64(k_bits[:, h]) @ np.asarray(r_k[h], np.float64).T
        vr[:, h] = bf16_to_f64(np.asarray(v_bits)[:, h]) @ np.asarray(r_v[h], np.float64).T
    ng = D // group
    kc, ks, kz = quantize_groups(kr, group)                        # s, z: [n][Hkv][ng]
    vc, vs, vz = quantize_groups(vr, group)
    del kr, vr
    n_pg = -(-n // PAGE)
    pad = n_pg * PAGE - n
    padt = lambda a: np.concatenate([a, np.zeros((pad,) + a.shape[1:], a.dtype)]) if pad else a
    kc, vc = padt(kc), padt(vc)
    bits = {o: padt(fp16_bits(x)) for o, x in ((K_SCALE, ks), (K_ZERO, kz), (V_SCALE, vs), (V_ZERO, vz))}
    pages = np.asarray(block_row[:n_pg], np.int64)
    assert np.all(pages >= 0)
    krow = pack_k_row(kc).reshape(n_pg, PAGE, hkv, 32)             # [pg][slot][h][32]
    vcode = vc.reshape(n_pg, PAGE, hkv, D).astype(np.uint32)       # [pg][slot][h][c]
    slots = np.arange(PAGE)
    nslot = np.full(n_pg, PAGE)
    nslot[-1] = PAGE - pad
    for j, pg in enumerate(pages):
        m = slots < nslot[j]
        blk = pool[pg]                                              # [Hkv][block bytes]
        kb = blk[:, K_CODES:K_CODES + 512].reshape(hkv, PAGE, 32)
        kb[:, m] = krow[j][m].transpose(1, 0, 2)
        words = np.ascontiguousarray(blk[:, V_CODES:V_CODES + 512]).view("<u4").copy()  # [Hkv][128]
        keep = ~np.uint32(sum(3 << (2 * int(t)) for t in slots[m]))
        words &= keep
        words |= np.bitwise_or.reduce((vcode[j][m] << (2 * slots[m])[:, None, None].astype(np.uint32)), axis=0)
        blk[:, V_CODES:V_CODES + 512] = words.astype("<u4").view(np.uint8).reshape(hkv, 512)
        rec = blk[:, META:].reshape(hkv, PAGE, ng, 4, 2)           # [h][slot][group][field][2 bytes]
        for f, b in bits.items():
            # b: [n][Hkv][ng] -> this page's live slots as [h][slot][group]
            src = np.ascontiguousarray(b[j * PAGE:(j + 1) * PAGE][m].transpose(1, 0, 2))
            field = rec[:, :, :, f // 2]                           # view [h][slot][group][2 bytes]
            field[:, m] = src.view(np.uint8).reshape(hkv, -1, ng, 2)
    if window > 0:
        for p in range(max(0, n - window), n):
            win_k[p % window] = k_bits[p]
            win_v[p % window] = v_bits[p]
    for p in range(min(n_sink, n)):
        win_k[window + p] = k_bits[p]
        win_v[window + p] = v_bits[p]
