"""Parity comparator between the HIP path and the fp64 oracle.

Contract (tolerances from the target statement; each check explained):
  scales   |s_gpu - s_ora| <= 1e-3 * s_ora, and s_ora == 0 <=> s_gpu == 0.
           1e-3 admits one fp16 ulp (2^-10): the GPU's fp32 abs-max and the
           oracle's fp64 abs-max can fall on either side of an fp16 midpoint.
  codes    compared with the oracle's codes RECOMPUTED WITH THE GPU'S STORED
           SCALE (so a legitimate scale flip does not cascade); equal, or off
           by exactly 1 where the exact pre-round value y/scale lies within
           1e-4 of a rounding boundary (a half-integer).
  dequant  the oracle dequantizes the GPU's own codes and scales;
           |xhat_gpu - xhat64| <= 2e-3 / lambda_c + 2^-11 * |xhat64|
           (2e-3 absolute in the lambda-normalised unit-variance domain, plus
           half an fp16 ulp for the final rounding).
  VQ       indices equal, or d64(idx_gpu) - d64(idx_ora) <=
           1e-4 * max(d64(idx_ora), 1e-6); exact-tie differences are counted
           separately (a tie must resolve to the lowest index).
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle

SCALE_REL = 1e-3
BOUNDARY = 1e-4
DEQ_ABS = 2e-3
DEQ_REL = 2.0 ** -11
VQ_REL = 1e-4


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


class ParityError(AssertionError):
    pass


def check_scales(sc_gpu, sc_ora):
    g, o = f16(sc_gpu), f16(sc_ora)
    zero_mismatch = (o == 0) != (g == 0)
    rel = np.where(o > 0, np.abs(g - o) / np.where(o > 0, o, 1), 0.0)
    bad = zero_mismatch | (rel > SCALE_REL) | ~np.isfinite(g)
    return {"n": int(g.size), "bad": int(bad.sum()), "flips": int((g != o).sum()),
            "max_rel": float(rel.max()) if rel.size else 0.0, "bad_mask": bad}


def check_codes(y64, sc_gpu, q_gpu, G, qmax=7):
    """y64 [n, D] exact rotated values; sc_gpu [n, D/G] fp16 bits; q_gpu [n, D]
    int8 codes of a quantizer with levels -qmax..qmax (7: int4, 127: int8)."""
    q_cond = (oracle.codes_given_scales if qmax == 7 else oracle.codes8_given_scales)(y64, sc_gpu, G)
    s = np.repeat(f16(sc_gpu), G, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, y64 / np.where(s > 0, s, 1), 0.0)
    dist = np.abs(r - (np.floor(r) + 0.5))          # distance to the nearest half-integer
    near = (dist < BOUNDARY) & (np.abs(r) < qmax + 0.5)
    diff = q_gpu.astype(np.int32) - q_cond.astype(np.int32)
    ok = (diff == 0) | ((np.abs(diff) == 1) & near)
    return {"n": int(diff.size), "exact": int((diff == 0).sum()), "boundary": int(((diff != 0) & ok).sum()),
            "bad": int((~ok).sum()), "bad_mask": ~ok, "q_cond": q_cond}


def check_dequant(x_gpu_bits, x64, lam):
    g = f16(x_gpu_bits)
    tol = DEQ_ABS / lam.astype(np.float64) + DEQ_REL * np.abs(x64)
    err = np.abs(g - x64)
    bad = ~(err <= tol)
    return {"n": int(g.size), "bad": int(bad.sum()), "max_err_over_tol": float((err / tol).max()),
            "max_abs_norm": float((err * lam).max()), "bad_mask": bad}


def check_vq(y64, codebooks, book, idx_gpu, idx_ora, sub):
    d_g = oracle.vq_distances(y64, codebooks, book, idx_gpu, sub)
    d_o = oracle.vq_distances(y64, codebooks, book, idx_ora, sub)
    same = idx_gpu == idx_ora
    tie = ~same & (d_g == d_o)
    close = (d_g - d_o) <= VQ_REL * np.maximum(d_o, 1e-6)
    bad = ~same & ~close
    return {"n": int(same.size), "exact": int(same.sum()), "near": int((~same & close & ~tie).sum()),
            "ties": int(tie.sum()), "bad": int(bad.sum()) + int(tie.sum()), "bad_mask": bad | tie}


def _raise(what, rep, extra=""):
    r = {k: v for k, v in rep.items() if not k.endswith("_mask") and k != "q_cond"}
    raise ParityError("%s parity failed: %s %s" % (what, r, extra))


def int4_parity(x_bits, lam_rows, signs, G, codes_gpu, scales_gpu, out_gpu=None, fourier=False):
    """Full int4 check of n vectors.  x_bits [n, D] fp16 bits, lam_rows [n, D]
    fp32, codes_gpu [n, D/2] u8, scales_gpu [n, D/G] fp16 bits, out_gpu
    (optional) [n, D] fp16 bits of the GPU dequantization of its own codes.
    fourier: the SRFT rotation instead of the Walsh-Hadamard one."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    lam_rows = np.ascontiguousarray(lam_rows, np.float32)
    quant = oracle.quantize_srft if fourier else oracle.quantize
    codes_o, scales_o, y64, nbad = quant(x_bits, lam_rows, signs, G)
    if nbad:
        raise ParityError("%d input vectors are outside the quantizer's domain" % nbad)
    rep = {}
    rs = check_scales(scales_gpu, scales_o)
    rep["scales"] = rs
    if rs["bad"]:
        i = np.argwhere(rs["bad_mask"])[:5]
        _raise("scale", rs, "first bad [row, group]: %s gpu=%s ora=%s" % (
            i.tolist(), f16(scales_gpu)[tuple(i.T)], f16(scales_o)[tuple(i.T)]))
    q_gpu = oracle.unpack_nibbles(np.ascontiguousarray(codes_gpu, np.uint8))
    rc = check_codes(y64, scales_gpu, q_gpu, G)
    rep["codes"] = rc
    if rc["bad"]:
        i = np.argwhere(rc["bad_mask"])[:5]
        _raise("code", rc, "first bad [row, coord]: %s gpu=%s ora=%s y/s=%s" % (
            i.tolist(), q_gpu[tuple(i.T)], rc["q_cond"][tuple(i.T)],
            (y64 / np.repeat(f16(scales_gpu), G, axis=1))[tuple(i.T)]))
    if out_gpu is not None:
        x64, _ = (oracle.dequantize_srft if fourier else oracle.dequantize)(codes_gpu, scales_gpu, lam_rows, signs, G)
        rd = check_dequant(out_gpu, x64, lam_rows)
        rep["dequant"] = rd
        if rd["bad"]:
            i = np.argwhere(rd["bad_mask"])[:5]
            _raise("dequant", rd, "first bad [row, coord]: %s gpu=%s ora=%s" % (
                i.tolist(), f16(out_gpu)[tuple(i.T)], x64[tuple(i.T)]))
    return rep


def summary(rep) -> str:
    parts = []
    for k, r in rep.items():
        parts.append("%s: %s" % (k, {a: b for a, b in r.items() if not a.endswith("_mask") and a != "q_cond"}))
    return "; ".join(parts)


def vq_parity(x_bits, lam_rows, signs, codebooks_bits, book, sub, idx_gpu, out_gpu=None):
    """Product-VQ check of n keys: indices against the oracle's (exact, or a
    distance within 1e-4 relative; an index that differs at an exactly equal
    distance breaks the lowest-index rule and fails), and, when given, the GPU
    decode of its own indices against the oracle's decode of the same ones."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    lam_rows = np.ascontiguousarray(lam_rows, np.float32)
    idx_gpu = np.ascontiguousarray(idx_gpu, np.uint16)
    idx_o, y64 = oracle.vq_encode(x_bits, lam_rows, signs, codebooks_bits, book, sub)
    K = codebooks_bits.shape[-2]
    if (idx_gpu >= K).any():
        raise ParityError("GPU index out of range: max %d >= %d" % (idx_gpu.max(), K))
    rep = {"vq": check_vq(y64, codebooks_bits, book, idx_gpu, idx_o, sub)}
    if rep["vq"]["bad"]:
        i = np.argwhere(rep["vq"]["bad_mask"])[:5]
        _raise("vq index", rep["vq"], "first bad [key, sub]: %s gpu=%s ora=%s" % (
            i.tolist(), idx_gpu[tuple(i.T)], idx_o[tuple(i.T)]))
    if out_gpu is not None:
        x64, _ = oracle.vq_decode(idx_gpu, codebooks_bits, book, lam_rows, signs, sub)
        rd = check_dequant(out_gpu, x64, lam_rows)
        rep["decode"] = rd
        if rd["bad"]:
            i = np.argwhere(rd["bad_mask"])[:5]
            _raise("vq decode", rd, "first bad [key, coord]: %s gpu=%s ora=%s" % (
                i.tolist(), f16(out_gpu)[tuple(i.T)], x64[tuple(i.T)]))
    return rep


def int8_parity(x_bits, lam_rows, signs, G, codes_gpu, scales_gpu, out_gpu=None):
    """int8 variant of int4_parity: codes_gpu [n, D] int8 (one byte per
    coordinate), same scale / code / dequant contract with 127 levels."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    lam_rows = np.ascontiguousarray(lam_rows, np.float32)
    codes_o, scales_o, y64, nbad = oracle.quantize8(x_bits, lam_rows, signs, G)
    if nbad:
        raise ParityError("%d input vectors are outside the quantizer's domain" % nbad)
    rep = {}
    rs = check_scales(scales_gpu, scales_o)
    rep["scales"] = rs
    if rs["bad"]:
        i = np.argwhere(rs["bad_mask"])[:5]
        _raise("int8 scale", rs, "first bad [row, group]: %s gpu=%s ora=%s" % (
            i.tolist(), f16(scales_gpu)[tuple(i.T)], f16(scales_o)[tuple(i.T)]))
    q_gpu = np.ascontiguousarray(codes_gpu).view(np.int8)
    rc = check_codes(y64, scales_gpu, q_gpu, G, qmax=127)
    rep["codes"] = rc
    if rc["bad"]:
        i = np.argwhere(rc["bad_mask"])[:5]
        _raise("int8 code", rc, "first bad [row, coord]: %s gpu=%s ora=%s" % (
            i.tolist(), q_gpu[tuple(i.T)], rc["q_cond"][tuple(i.T)]))
    if out_gpu is not None:
        x64, _ = oracle.dequantize8(q_gpu, scales_gpu, lam_rows, signs, G)
        rd = check_dequant(out_gpu, x64, lam_rows)
        rep["dequant"] = rd
        if rd["bad"]:
            i = np.argwhere(rd["bad_mask"])[:5]
            _raise("int8 dequant", rd, "first bad [row, coord]: %s gpu=%s ora=%s" % (
                i.tolist(), f16(out_gpu)[tuple(i.T)], x64[tuple(i.T)]))
    return rep


# ------------------------------------------------------------------ MXFP4
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_AMAX_REL = 2.0 ** -20      # fp32 vs fp64 abs-max straddling a power of two


def e2m1(codes):
    c = np.asarray(codes).astype(np.int64) & 0xF
    v = _E2M1[c & 7]
    return np.where(c & 8, -v, v)


def mxfp4_parity(x_bits, lam_rows, signs, codes_gpu, scales_gpu, out_gpu=None):
    """Block-scaled E2M1 contract.
    scales  equal E8M0 bytes, or one apart where the block's exact abs-max is
            within 2^-20 of a power of two (the GPU's fp32 abs-max may land on
            the other side);
    codes   compared with the oracle's codes recomputed under the GPU's
            scales: equal, or adjacent E2M1 values where the exact y / X lies
            within 1e-4 of the rounding midpoint between them (zero magnitude
            of either sign counts as equal);
    dequant the oracle decodes the GPU's own codes and scales, same bound as
            the int4 dequantizer."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    lam_rows = np.ascontiguousarray(lam_rows, np.float32)
    codes_o, scales_o, y64, nbad = oracle.quantize_mxfp4(x_bits, lam_rows, signs)
    if nbad:
        raise ParityError("%d input vectors are outside the quantizer's domain" % nbad)
    sg = np.ascontiguousarray(scales_gpu, np.uint8)
    n, D = y64.shape
    amax = np.abs(y64).reshape(n, D // 32, 32).max(axis=2)
    with np.errstate(divide="ignore"):
        l2 = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = np.abs(np.exp2(np.round(l2)) - amax) <= MX_AMAX_REL * amax
    ds = sg.astype(np.int64) - scales_o.astype(np.int64)
    sbad = ~((ds == 0) | ((np.abs(ds) == 1) & near_pow2))
    rep = {"scales": {"n": int(sg.size), "bad": int(sbad.sum()), "flips": int((ds != 0).sum())}}
    if sbad.any():
        i = np.argwhere(sbad)[:5]
        _raise("mxfp4 scale", rep["scales"], "first bad [row, block]: %s gpu=%s ora=%s" % (
            i.tolist(), sg[tuple(i.T)], scales_o[tuple(i.T)]))
    q_gpu = oracle.unpack_nibbles(np.ascontiguousarray(codes_gpu, np.uint8)).astype(np.int64) & 0xF
    q_cond = oracle.mxfp4_codes_given_scales(y64, sg).astype(np.int64)
    vg, vo = e2m1(q_gpu), e2m1(q_cond)
    X = np.repeat(np.exp2(sg.astype(np.float64) - 127), 32, axis=1)
    v = y64 / X
    same = (q_gpu == q_cond) | ((vg == 0) & (vo == 0))
    mid = (vg + vo) / 2
    adjacent = np.abs(np.searchsorted(_E2M1, np.abs(vg)) - np.searchsorted(_E2M1, np.abs(vo))) == 1
    boundary = ~same & adjacent & (np.sign(vg) * np.sign(vo) >= 0) & (np.abs(v - mid) <= 1e-4)
    cbad = ~(same | boundary)
    rep["codes"] = {"n": int(q_gpu.size), "exact": int(same.sum()), "boundary": int(boundary.sum()),
                    "bad": int(cbad.sum())}
    if cbad.any():
        i = np.argwhere(cbad)[:5]
        _raise("mxfp4 code", rep["codes"], "first bad [row, coord]: %s gpu=%s ora=%s y/X=%s" % (
            i.tolist(), q_gpu[tuple(i.T)], q_cond[tuple(i.T)], v[tuple(i.T)]))
    if out_gpu is not None:
        x64, _ = oracle.dequantize_mxfp4(np.ascontiguousarray(codes_gpu, np.uint8), sg, lam_rows, signs)
        rd = check_dequant(out_gpu, x64, lam_rows)
        rep["dequant"] = rd
        if rd["bad"]:
            i = np.argwhere(rd["bad_mask"])[:5]
            _raise("mxfp4 dequant", rd, "first bad [row, coord]: %s gpu=%s ora=%s" % (
                i.tolist(), f16(out_gpu)[tuple(i.T)], x64[tuple(i.T)]))
    return rep


# ------------------------------------------------------- k-means update step
KM_FIX = 2.0 ** -25
KM_ROT = 2.0 ** -19


def kmeans_parity(x_bits, lam_rows, signs, codebook_bits, idx_gpu, new_gpu, counts_gpu, sub=8):
    """One Lloyd step on n training vectors of one head against its codebook
    [K, sub] (fp16 bits).
    assignments  idx_gpu [n, D/sub] under the VQ index contract;
    counts       exactly the oracle's counts of the GPU's own assignments;
    centroids    the oracle's update from the GPU's own assignments: an empty
                 centroid keeps its exact old bits; otherwise the GPU's fp16
                 value must lie between fp16(m - delta) and fp16(m + delta),
                 m the fp64 mean, delta = 2^-25 (the sums are exact sums of
                 the coordinates rounded to multiples of 2^-24, so the mean
                 is off by at most half that) + 2^-19 * the largest
                 per-vector RMS of y (fp32 rotation error)."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    lam_rows = np.ascontiguousarray(lam_rows, np.float32)
    cb = np.ascontiguousarray(codebook_bits, np.uint16)
    K = cb.shape[0]
    idx_gpu = np.ascontiguousarray(idx_gpu, np.uint16)
    idx_o, y64 = oracle.vq_encode(x_bits, lam_rows, signs, cb[None], np.zeros(len(x_bits), np.int32), sub)
    if (idx_gpu >= K).any():
        raise ParityError("GPU assignment out of range: max %d >= %d" % (idx_gpu.max(), K))
    rep = {"assign": check_vq(y64, cb[None], np.zeros(len(x_bits), np.int32), idx_gpu, idx_o, sub)}
    if rep["assign"]["bad"]:
        i = np.argwhere(rep["assign"]["bad_mask"])[:5]
        _raise("k-means assignment", rep["assign"], "first bad [vector, sub]: %s gpu=%s ora=%s" % (
            i.tolist(), idx_gpu[tuple(i.T)], idx_o[tuple(i.T)]))
    ysub = y64.reshape(-1, sub)
    new_o, m64, cnt_o, am = oracle.kmeans_update(ysub, idx_gpu.reshape(-1), cb)
    cg = np.ascontiguousarray(counts_gpu).astype(np.int64).reshape(K)
    cbad = cg != cnt_o.astype(np.int64)
    rep["counts"] = {"n": K, "bad": int(cbad.sum()), "total": int(cg.sum())}
    if cbad.any():
        i = np.flatnonzero(cbad)[:5]
        _raise("k-means counts", rep["counts"], "first bad centroids %s gpu=%s ora=%s" % (
            i.tolist(), cg[i], cnt_o[i]))
    ng = np.ascontiguousarray(new_gpu, np.uint16).reshape(K, sub)
    ymax = float(np.sqrt((y64 ** 2).mean(axis=1)).max()) if len(y64) else 0.0
    delta = np.full(m64.shape, KM_FIX + KM_ROT * ymax)
    lo = f16(oracle.f64_to_f16(m64 - delta))
    hi = f16(oracle.f64_to_f16(m64 + delta))
    g = f16(ng)
    empty = cnt_o == 0
    ok = np.where(empty[:, None], ng == cb, (g >= lo) & (g <= hi))
    exact = np.where(empty[:, None], ng == cb, ng == new_o)
    rep["centroids"] = {"n": int(ng.size), "empty": int(empty.sum()), "exact": int(exact.sum()),
                        "bad": int((~ok).sum()), "bad_mask": ~ok}
    if (~ok).any():
        i = np.argwhere(~ok)[:5]
        _raise("k-means centroid", rep["centroids"], "first bad [k, t]: %s gpu=%s mean64=%s delta=%s" % (
            i.tolist(), g[tuple(i.T)], m64[tuple(i.T)], delta[tuple(i.T)]))
    return rep


# ------------------------------------------------------- sharded checks
def workers() -> int:
    """Threads for sharded checks: the host cores this process may use, at
    most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _merge(reps):
    """Sum the counts of shard reports, take the maxima of their float
    fields and concatenate their arrays."""
    out = {}
    for key in reps[0]:
        parts = [r[key] for r in reps]
        m = {}
        for f, v in parts[0].items():
            vals = [p[f] for p in parts]
            if isinstance(v, np.ndarray):
                m[f] = np.concatenate(vals)
            elif isinstance(v, (bool, np.bool_)):
                m[f] = any(vals)
            elif isinstance(v, (int, np.integer)):
                m[f] = int(sum(vals))
            else:
                m[f] = float(max(vals))
        out[key] = m
    return out


def sharded(check, n: int, n_workers: int | None = None):
    """Run check(row_slice) on disjoint row shards of n rows at once and
    merge the reports.  Each shard is an independent call of the
    single-threaded oracle (ctypes releases the GIL during the call), so
    the arithmetic for every row is exactly that of one unsharded call; a
    failing shard raises its own ParityError."""
    w = max(1, min(n_workers or workers(), n))
    bounds = np.linspace(0, n, w + 1).astype(int)
    slices = [slice(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    if len(slices) == 1:
        return check(slices[0])
    with cf.ThreadPoolExecutor(len(slices)) as ex:
        reps = list(ex.map(check, slices))
    return _merge(reps)
