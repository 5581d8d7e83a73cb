"""Quality of the INT2 cache under different rotations, through the same kernels.

The method's premise is that an attention-aware rotation makes per-token 2-bit
codes accurate where the attention needs them (P1 gen-hub.ru «Почему INT2 раньше
не работал», «Что придумали в Together AI»; P4 aiforradalom.hu «OSCAR:
figyelem-tudatos és bevetésre kész»).  This harness takes the rotation as data
and runs the product's append and decode kernels with each of:

  oscar     R = P_br (H / sqrt d) U^T from ``oscar_calibrate`` (the query
            eigenbasis for keys, the score-weighted value eigenbasis for values);
  hadamard  R = P_br (H / sqrt d): the fixed transform without the calibrated
            basis;
  identity  R = I: plain per-token INT2.

Against fp64 attention on the unquantised bf16 cache (the bf16 window is exact
in both), per rotation:

  logit_rms    sqrt of the mean over (q head, history token) of
               ((q . k - q . k_hat) / sqrt d)^2 on the decode queries;
  logit_sigma  the mean over history tokens and KV heads of
               dk^T Sigma_Q dk / d, Sigma_Q the KV head's uncentred calibration
               query covariance (the expectation the first one estimates);
  out_rel_l2   mean over (sequence, q head) of |o - o_exact|_2 / |o_exact|_2,
               o the decode kernel's output;
  out_rel_max  max over (sequence, q head) of |o - o_exact|_inf / |o_exact|_inf;
  kl           mean over (sequence, q head) of KL(p_exact || p_int2) of the
               softmax over all positions.

k_hat and v_hat are read back from the pool the append kernel wrote (decoded
here on the host from the page layout), so every number measures the kernels'
cache.  This is a measurement tool: nothing on the append or decode path calls it.
"""
from __future__ import annotations

import math

import numpy as np

D = 128
PAGE = 16


def block_bytes(group: int = D) -> int:
    """Bytes of one (page, KV head) block: codes plus one 8-byte record per token and group."""
    return 1024 + 8 * PAGE * (D // group)


def hadamard_rotation(d: int = D) -> np.ndarray:
    """P_br (H / sqrt d) as fp64 [d][d]: Sylvester H_ij = (-1)^popcount(i & j),
    rows permuted by the log2(d)-bit reversal of their index."""
    bits = d.bit_length() - 1
    idx = np.arange(d)
    h = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    rev = np.array([int(format(i, f"0{bits}b")[::-1], 2) for i in idx])
    return h[rev] / math.sqrt(d)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _fp16_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def rotations(shape, q_cal, k_cal, v_cal, lib_calibrate) -> dict:
    """bf16 bits (r_k, r_v) [Hkv][d][d] of the three rotations compared."""
    hkv = shape.n_kv_heads
    rk, rv, _, _ = lib_calibrate(shape, q_cal, k_cal, v_cal)
    had = np.broadcast_to(_bf16_bits(hadamard_rotation()), (hkv, D, D)).copy()
    eye = np.broadcast_to(_bf16_bits(np.eye(D)), (hkv, D, D)).copy()
    return {"oscar": (rk, rv), "hadamard": (had, had.copy()), "identity": (eye, eye.copy())}


def dequantize_history(pool: np.ndarray, bt_row: np.ndarray, n_hist: int, h: int, group: int = D):
    """Rotated-domain K and V (fp64 [n_hist][d]) of positions 0 .. n_hist - 1 of
    one sequence and KV head, decoded from the page blocks: K codes (token row
    of 32 bytes, channel c in byte 8 ((c >> 2) & 3) + (c >> 4) at bits 2 (c & 3)),
    V codes (channel word c, slot j at bits 2 j), then per token and group of
    ``group`` channels {K scale, K zero, V scale, V zero} fp16; value = zero +
    code * scale of the channel's group."""
    if n_hist == 0:
        return np.zeros((0, D)), np.zeros((0, D))
    n_pg = -(-n_hist // PAGE)
    ng = D // group
    blk = pool[np.asarray(bt_row[:n_pg], np.int64), h]            # [pages][block bytes]
    c = np.arange(D)
    kbyte = 8 * ((c >> 2) & 3) + (c >> 4)
    krows = blk[:, :512].reshape(n_pg, PAGE, 32)
    kc = (krows[:, :, kbyte] >> (2 * (c & 3))) & 3                # [pages][16][d]
    vw = np.ascontiguousarray(blk[:, 512:1024]).view(np.uint32).reshape(n_pg, D)
    slots = np.arange(PAGE)
    vc = (vw[:, None, :] >> (2 * slots[None, :, None]).astype(np.uint32)) & 3  # [pages][16][d]
    meta = np.ascontiguousarray(blk[:, 1024:]).view(np.uint16).reshape(n_pg, PAGE, ng, 4)
    ks, kz, vs, vz = (np.repeat(_fp16_f64(meta[..., i]), group, axis=-1) for i in range(4))
    k = (kz + kc * ks).reshape(-1, D)[:n_hist]
    v = (vz + vc * vs).reshape(-1, D)[:n_hist]
    return k, v


def measure(K, s, rot: dict, workloads, torch, group: int = D) -> dict:
    """Metrics of each rotation in ``rot`` on workload spec ``s`` (one full
    prefill through ``oscar_quantize_append``, one ``oscar_decode_attn``) with
    quantisation groups of ``group`` rotated channels."""
    dev = torch.device("cuda:0")
    shape = K.make_shape(s.n_q_heads, s.n_kv_heads, s.window, group_size=group)
    q_bits = workloads.decode_queries(s)
    q = _bf16_f64(q_bits)
    bt, n_pages = workloads.page_table(s)
    q_cal, _, _ = workloads.calibration_set(s)
    sig = np.einsum("hni,hnj->hij", q_cal.astype(np.float64), q_cal.astype(np.float64)) / q_cal.shape[1]
    kv = [workloads.context_kv(s, b) for b in range(s.batch)]
    g = s.n_q_heads // s.n_kv_heads
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    results = {}
    for name, (rk, rv) in rot.items():
        pool = torch.zeros((n_pages, s.n_kv_heads, block_bytes(group)), dtype=torch.uint8, device=dev)
        wsh = (s.batch, max(s.window, 1), s.n_kv_heads, D)
        wk = torch.zeros(wsh, dtype=torch.int16, device=dev)
        wv = torch.zeros(wsh, dtype=torch.int16, device=dev)
        for b in range(s.batch):
            k, v = kv[b]
            n = k.shape[0]
            K.oscar_quantize_append(shape, T(rk.view(np.int16)), T(rv.view(np.int16)), T(k.view(np.int16)),
                                    T(v.view(np.int16)), T(np.full(n, b, np.int32)), T(np.arange(n, dtype=np.int32)),
                                    T(bt), T(s.seq_lens), pool, wk, wv)
        max_len = int(s.seq_lens.max())
        ws = torch.empty(K.oscar_decode_workspace_bytes(shape, s.batch, max_len), dtype=torch.uint8, device=dev)
        out = torch.empty((s.batch, s.n_q_heads, D), dtype=torch.float32, device=dev)
        K.oscar_decode_attn(shape, T(rk.view(np.int16)), T(rv.view(np.int16)), T(q_bits.view(np.int16)),
                            T(s.seq_lens), max_len, T(bt), pool, wk, wv, out, ws)
        torch.cuda.synchronize()
        pool_h = pool.cpu().numpy()
        o_kernel = out.cpu().numpy().astype(np.float64)
        rkf = _bf16_f64(rk)
        sq_err, n_sq, sig_err, n_sig, kls, rel, rel2 = 0.0, 0, 0.0, 0, [], [], []
        for b in range(s.batch):
            n = int(s.seq_lens[b])
            w = min(n, s.window)
            hist = n - w
            kb, vb = _bf16_f64(kv[b][0]), _bf16_f64(kv[b][1])          # [n][Hkv][d]
            for h in range(s.n_kv_heads):
                kq, _ = dequantize_history(pool_h, bt[b], hist, h, group)  # rotated domain
                k_hat = kq @ rkf[h]                                      # R^T applied: x = R^T x'
                dk = kb[:hist, h] - k_hat
                sig_err += float(np.einsum("ti,ij,tj->", dk, sig[h], dk)) / D
                n_sig += hist
                k_all_hat = np.concatenate([k_hat, kb[hist:, h]])
                for j in range(g):
                    qq = q[b, h * g + j]
                    s_ex = kb[:, h] @ qq / math.sqrt(D)
                    s_q = k_all_hat @ qq / math.sqrt(D)
                    sq_err += float(np.sum((s_ex[:hist] - s_q[:hist]) ** 2))
                    n_sq += hist
                    p_ex = np.exp(s_ex - s_ex.max())
                    p_ex /= p_ex.sum()
                    lp_q = s_q - s_q.max() - math.log(np.exp(s_q - s_q.max()).sum())
                    kls.append(float(np.sum(p_ex * (np.log(p_ex) - lp_q))))
                    o_ex = p_ex @ vb[:, h]
                    do = o_kernel[b, h * g + j] - o_ex
                    rel.append(float(np.abs(do).max() / np.abs(o_ex).max()))
                    rel2.append(float(np.linalg.norm(do) / np.linalg.norm(o_ex)))
        results[name] = {
            "logit_rms": math.sqrt(sq_err / max(n_sq, 1)),
            "logit_sigma": sig_err / max(n_sig, 1),
            "out_rel_l2": float(np.mean(rel2)),
            "out_rel_max": max(rel),
            "kl": float(np.mean(kls)),
        }
    return results
