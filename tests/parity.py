"""Helpers of the GPU parity tests: the matching rules against the oracle and
the host <-> device plumbing.  Test-side code only.

Matching rules
  * encoder (per token, KV head, K|V group): fp16 scale and zero bit-exact unless
    the oracle's pre-rounding value (sigma = (M - m) / 3, resp. m) lies within
    1e-4 relative of an fp16 rounding midpoint; codes bit-exact unless the
    oracle's t = (x' - zero) / scale lies within 1e-4 (code units) of a decision
    boundary 0.5, 1.5, 2.5.  Where scale/zero legitimately differ, the codes are
    compared after recomputing t with the device's scale/zero.
  * everything else in the pool (other slots, other pages) byte-exact;
  * bf16 window byte-exact;
  * attention: max over (sequence, q head) of |o - o_ref|_inf / |o_ref|_inf <= 2e-3.
"""
from __future__ import annotations

import numpy as np

from oracle import oscar_ref as ref

REL = 1e-4
ATTN_TOL = 2e-3


def near_fp16_midpoint(x, rel=REL):
    x = np.asarray(x, dtype=np.float64)
    return ref.fp16_rne(x * (1 - rel)) != ref.fp16_rne(x * (1 + rel))


def rounding_neighbours(x, rel=REL):
    """fp16 bit patterns x may round to when perturbed by rel (one value unless
    x lies within rel of a rounding midpoint)."""
    x = float(x)
    return {int(ref.fp16_bits(x * (1 - rel))), int(ref.fp16_bits(x * (1 + rel)))}


def near_code_boundary(t, tol=REL):
    t = np.asarray(t, dtype=np.float64)
    return np.min(np.abs(t[..., None] - np.array([0.5, 1.5, 2.5])), axis=-1) <= tol


def gpu_group_fields(pool, page, h, slot, group=128):
    """(k_codes[128], v_codes[128], ks, kz, vs, vz) as stored in a pool block;
    the four fp16 fields are lists over the slot's d / group records."""
    blk = pool[page, h]
    ng = 128 // group
    kc = ref.unpack_k_rows(blk[ref.K_CODES + 32 * slot: ref.K_CODES + 32 * slot + 32])
    vc = ref.unpack_v_words(ref.v_words(blk))[slot]

    def f(fld):
        out = []
        for j in range(ng):
            a = ref.META + 8 * (ng * slot + j) + fld
            out.append(int(np.ascontiguousarray(blk[a:a + 2]).view(np.uint16)[0]))
        return out
    return kc, vc, f(ref.K_SCALE), f(ref.K_ZERO), f(ref.V_SCALE), f(ref.V_ZERO)


def clear_group(pool, page, h, slot, group=128):
    blk = pool[page, h]
    ng = 128 // group
    blk[ref.K_CODES + 32 * slot: ref.K_CODES + 32 * slot + 32] = 0
    w = ref.v_words(blk).copy() & ~np.uint32(3 << (2 * slot))
    blk[ref.V_CODES:ref.V_CODES + 512] = w.astype("<u4").view(np.uint8)
    blk[ref.META + 8 * ng * slot: ref.META + 8 * ng * (slot + 1)] = 0


def check_group(xr, codes_gpu, s_bits_gpu, z_bits_gpu):
    """Apply the encoder rule to one group.  xr: the oracle's exact rotation of
    the group's channels (fp64 [group]).  Returns (n_mismatch, n_excluded)."""
    c, s16, z16, diag = ref.quantize(xr[None, :])
    c, s16, z16 = c[0], float(s16[0]), float(z16[0])
    sig, m, t = float(diag["sigma"][0]), float(diag["m"][0]), diag["t"][0]
    s_ok = int(ref.fp16_bits(s16)) == s_bits_gpu
    z_ok = int(ref.fp16_bits(z16)) == z_bits_gpu
    bad = 0
    # a differing scale/zero must be the other neighbour of a nearby midpoint
    if not s_ok and s_bits_gpu not in rounding_neighbours(sig):
        bad += 1
    if not z_ok and z_bits_gpu not in rounding_neighbours(m):
        bad += 1
    if not (s_ok and z_ok):
        # recompute the codes with the device's scale/zero, in the same fp32 steps
        sg = np.float32(np.uint16(s_bits_gpu).view(np.float16))
        zg = np.float32(np.uint16(z_bits_gpu).view(np.float16))
        x32 = np.asarray(xr, np.float64).astype(np.float32)
        t = ((x32 - zg).astype(np.float32) / (sg if sg != 0 else np.float32(1))).astype(np.float32)
        c = np.zeros(len(xr), np.int64) if sg == 0 else np.clip(np.rint(t), 0, 3).astype(np.int64)
    amb = near_code_boundary(t)
    diff = c != codes_gpu
    bad += int(np.sum(diff & ~amb))
    return bad, int(np.sum(diff & amb)) + int(not (s_ok and z_ok))


def check_append(pool_before, pool_gpu, rk, rv, k_bits, v_bits, seq_idx, pos, block_table,
                 sample=None, group=128):
    """Compare a device-appended pool with the oracle's encoding of the same
    tokens, group by group.  ``sample``: indices of tokens to check (default
    all); with all tokens checked, every other byte of the pool must be
    untouched."""
    hkv = pool_gpu.shape[1]
    idx = np.arange(len(pos)) if sample is None else np.asarray(sample)
    kb = ref.bf16_to_f64(np.asarray(k_bits)[idx])
    vb = ref.bf16_to_f64(np.asarray(v_bits)[idx])
    kr = np.einsum("hij,thj->thi", rk, kb)
    vr = np.einsum("hij,thj->thi", rv, vb)
    mism = excl = 0
    rest_gpu = pool_gpu.copy() if sample is None else None
    rest_ref = pool_before.copy() if sample is None else None
    for n_i, i in enumerate(idx):
        b, p = int(seq_idx[i]), int(pos[i])
        page = int(block_table[b][p // 16])
        slot = p % 16
        for h in range(hkv):
            kc, vc, ks, kz, vs, vz = gpu_group_fields(pool_gpu, page, h, slot, group)
            m1 = e1 = m2 = e2 = 0
            for j in range(128 // group):
                c = slice(group * j, group * (j + 1))
                a, e = check_group(kr[n_i, h, c], kc[c], ks[j], kz[j])
                m1, e1 = m1 + a, e1 + e
                a, e = check_group(vr[n_i, h, c], vc[c], vs[j], vz[j])
                m2, e2 = m2 + a, e2 + e
            if (m1 or m2) and mism < 6:
                print(f"  mismatch: token {i} (seq {b}, pos {p}) head {h}: K {m1} V {m2}", flush=True)
            mism += m1 + m2
            excl += e1 + e2
            if rest_gpu is not None:
                clear_group(rest_gpu, page, h, slot, group)
                clear_group(rest_ref, page, h, slot, group)
    stray = 0 if rest_gpu is None else int(np.sum(rest_gpu != rest_ref))
    if stray:
        where = np.argwhere(rest_gpu != rest_ref)[:6]
        print(f"  stray bytes at [page, head, byte]: {where.tolist()}", flush=True)
    return mism, excl, stray


def attn_rel_err(got, want):
    """Per (sequence, q head): |o - o_ref|_inf / |o_ref|_inf; NaN rows of want skipped."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    ok = ~np.isnan(want).any(axis=-1)
    num = np.abs(got - want).max(axis=-1)
    den = np.abs(want).max(axis=-1)
    return np.where(ok, num / np.where(den == 0, 1, den), 0.0)
