"""fp64 CPU oracle for the fused KV-cache quantizer -- test infrastructure only.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does, and this package never
imports the product library: the two share no code.  The arithmetic lives in
``kvq_oracle.c`` (plain C, binary64, single-threaded); this module only
marshals numpy arrays into it.

Every function takes and returns numpy arrays; binary16 data travels as its
raw ``uint16`` bit patterns so that the oracle sees exactly the bytes a GPU
kernel saw.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libkvq_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    _lib = bind(_LIB)
    return _lib


def bind(path: str):
    """Load a compiled oracle library from `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64, I32 = ctypes.c_int64, ctypes.c_int
    sig = {
        "kvqo_f16_decode": (None, [I64, P, P]),
        "kvqo_f16_encode": (None, [I64, P, P]),
        "kvqo_hadamard_entry": (I32, [I32, I32]),
        "kvqo_rotate_rows": (I32, [I64, I32, P, P, P, P]),
        "kvqo_unrotate_rows": (I32, [I64, I32, P, P, P, P, P]),
        "kvqo_pack_nibbles": (None, [I64, P, P]),
        "kvqo_unpack_nibbles": (None, [I64, P, P]),
        "kvqo_codes_given_scales": (I32, [I64, I32, I32, P, P, P]),
        "kvqo_quantize_rows": (I64, [I64, I32, I32, P, P, P, P, P, P]),
        "kvqo_dequantize_rows": (I32, [I64, I32, I32, P, P, P, P, P, P]),
        "kvqo_srft_rows": (I32, [I64, I32, P, P, P, P]),
        "kvqo_isrft_rows": (I32, [I64, I32, P, P, P, P, P]),
        "kvqo_quantize_srft_rows": (I64, [I64, I32, I32, P, P, P, P, P, P]),
        "kvqo_dequantize_srft_rows": (I32, [I64, I32, I32, P, P, P, P, P, P]),
        "kvqo_vq_encode_rows": (I32, [I64, I32, I32, I32, P, P, P, P, P, P, P]),
        "kvqo_vq_distances": (I32, [I64, I32, I32, I32, P, P, P, P, P]),
        "kvqo_kmeans_update": (I32, [I64, I32, I32, P, P, P, P, P, P, P]),
        "kvqo_vq_decode_rows": (I32, [I64, I32, I32, I32, P, P, P, P, P, P, P]),
        "kvqo_codes8_given_scales": (I32, [I64, I32, I32, P, P, P]),
        "kvqo_quantize8_rows": (I64, [I64, I32, I32, P, P, P, P, P, P]),
        "kvqo_dequantize8_rows": (I32, [I64, I32, I32, P, P, P, P, P, P]),
        "kvqo_e2m1_value": (ctypes.c_double, [I32]),
        "kvqo_quantize_mxfp4_rows": (I64, [I64, I32, P, P, P, P, P, P]),
        "kvqo_mxfp4_codes_given_scales": (I32, [I64, I32, P, P, P]),
        "kvqo_dequantize_mxfp4_rows": (I32, [I64, I32, P, P, P, P, P, P]),
        "kvqo_attend_decode": (I32, [I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P,
                                     ctypes.c_double, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _out(shape, dtype):
    a = np.empty(shape, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _rows(x, D):
    x = np.asarray(x)
    return int(x.size // D)


# --------------------------------------------------------------------- fp16
def f16_to_f64(bits):
    bits, pb = _c(bits, np.uint16)
    out, po = _out(bits.shape, np.float64)
    _load().kvqo_f16_decode(bits.size, pb, po)
    return out


def f64_to_f16(v):
    v, pv = _c(v, np.float64)
    out, po = _out(v.shape, np.uint16)
    _load().kvqo_f16_encode(v.size, pv, po)
    return out


def hadamard_entry(i: int, j: int) -> int:
    return int(_load().kvqo_hadamard_entry(int(i), int(j)))


# ----------------------------------------------------------------- rotation
def rotate(x_bits, lam, signs):
    """y = D^-1/2 H diag(s) diag(lambda) x for every row; x as fp16 bits [n, D]."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    lam, pl = _c(np.broadcast_to(lam, x.shape), np.float32)
    s, ps = _c(signs, np.int8)
    y, py = _out(x.shape, np.float64)
    rc = _load().kvqo_rotate_rows(_rows(x, D), D, px, pl, ps, py)
    if rc:
        raise ValueError("oracle rotate rejected D=%d" % D)
    return y


def unrotate(yhat, lam, signs):
    """(x64, x16bits) = unscale(inverse rotation of yhat) for every row."""
    yh, py = _c(yhat, np.float64)
    D = yh.shape[-1]
    lam, pl = _c(np.broadcast_to(lam, yh.shape), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out(yh.shape, np.float64)
    x16, p16 = _out(yh.shape, np.uint16)
    rc = _load().kvqo_unrotate_rows(_rows(yh, D), D, py, pl, ps, p64, p16)
    if rc:
        raise ValueError("oracle unrotate rejected D=%d" % D)
    return x64, x16


def srft(x_bits, lam, signs):
    """SRFT rotation of every row: y = pack(unitary DFT of s * lambda * x),
    pack = [X_0, X_{D/2}, sqrt2 Re X_1, sqrt2 Im X_1, ...]; D even."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    lam, pl = _c(np.broadcast_to(lam, x.shape), np.float32)
    s, ps = _c(signs, np.int8)
    y, py = _out(x.shape, np.float64)
    rc = _load().kvqo_srft_rows(_rows(x, D), D, px, pl, ps, py)
    if rc:
        raise ValueError("oracle srft rejected D=%d" % D)
    return y


def isrft(yhat, lam, signs):
    """(x64, x16bits) = unscale(inverse SRFT of yhat) for every row."""
    yh, py = _c(yhat, np.float64)
    D = yh.shape[-1]
    lam, pl = _c(np.broadcast_to(lam, yh.shape), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out(yh.shape, np.float64)
    x16, p16 = _out(yh.shape, np.uint16)
    rc = _load().kvqo_isrft_rows(_rows(yh, D), D, py, pl, ps, p64, p16)
    if rc:
        raise ValueError("oracle isrft rejected D=%d" % D)
    return x64, x16


# ---------------------------------------------------------------- nibbles
def pack_nibbles(q):
    q, pq = _c(q, np.int8)
    out, po = _out(q.shape[:-1] + (q.shape[-1] // 2,), np.uint8)
    _load().kvqo_pack_nibbles(q.size, pq, po)
    return out


def unpack_nibbles(b):
    b, pb = _c(b, np.uint8)
    out, po = _out(b.shape[:-1] + (b.shape[-1] * 2,), np.int8)
    _load().kvqo_unpack_nibbles(b.size, pb, po)
    return out


# --------------------------------------------------------------- quantizer
def codes_given_scales(y, scales_bits, G):
    """Unpacked int8 codes of rotated rows y [n, D] under given fp16 scales."""
    y, py = _c(y, np.float64)
    D = y.shape[-1]
    sc, ps = _c(scales_bits, np.uint16)
    q, pq = _out(y.shape, np.int8)
    rc = _load().kvqo_codes_given_scales(_rows(y, D), D, int(G), py, ps, pq)
    if rc:
        raise ValueError("bad group size")
    return q


def quantize(x_bits, lam, signs, G):
    """Returns (codes u8 [.., D/2], scales fp16-bits [.., D/G], y fp64 [.., D], n_bad)."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    lam, pl = _c(np.broadcast_to(lam, x.shape), np.float32)
    s, ps = _c(signs, np.int8)
    codes, pc = _out(x.shape[:-1] + (D // 2,), np.uint8)
    scales, psc = _out(x.shape[:-1] + (D // G,), np.uint16)
    y, py = _out(x.shape, np.float64)
    bad = _load().kvqo_quantize_rows(_rows(x, D), D, int(G), px, pl, ps, pc, psc, py)
    if bad < 0:
        raise ValueError("oracle quantize rejected D=%d G=%d" % (D, G))
    return codes, scales, y, int(bad)


def dequantize(codes, scales_bits, lam, signs, G):
    """Returns (x64 fp64 [.., D], x16 fp16-bits [.., D])."""
    c, pc = _c(codes, np.uint8)
    D = c.shape[-1] * 2
    sc, psc = _c(scales_bits, np.uint16)
    shape = c.shape[:-1] + (D,)
    lam, pl = _c(np.broadcast_to(lam, shape), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out(shape, np.float64)
    x16, p16 = _out(shape, np.uint16)
    rc = _load().kvqo_dequantize_rows(_rows(x64, D), D, int(G), pc, psc, pl, ps, p64, p16)
    if rc:
        raise ValueError("oracle dequantize rejected D=%d G=%d" % (D, G))
    return x64, x16


def quantize_srft(x_bits, lam, signs, G):
    """quantize() on the SRFT rotation (D even)."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    lam, pl = _c(np.broadcast_to(lam, x.shape), np.float32)
    s, ps = _c(signs, np.int8)
    codes, pc = _out(x.shape[:-1] + (D // 2,), np.uint8)
    scales, psc = _out(x.shape[:-1] + (D // G,), np.uint16)
    y, py = _out(x.shape, np.float64)
    bad = _load().kvqo_quantize_srft_rows(_rows(x, D), D, int(G), px, pl, ps, pc, psc, py)
    if bad < 0:
        raise ValueError("oracle quantize_srft rejected D=%d G=%d" % (D, G))
    return codes, scales, y, int(bad)


def dequantize_srft(codes, scales_bits, lam, signs, G):
    """dequantize() with the inverse SRFT."""
    c, pc = _c(codes, np.uint8)
    D = c.shape[-1] * 2
    sc, psc = _c(scales_bits, np.uint16)
    shape = c.shape[:-1] + (D,)
    lam, pl = _c(np.broadcast_to(lam, shape), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out(shape, np.float64)
    x16, p16 = _out(shape, np.uint16)
    rc = _load().kvqo_dequantize_srft_rows(_rows(x64, D), D, int(G), pc, psc, pl, ps, p64, p16)
    if rc:
        raise ValueError("oracle dequantize_srft rejected D=%d G=%d" % (D, G))
    return x64, x16


# ---------------------------------------------------------------------- VQ
def vq_encode(x_bits, lam, signs, codebooks_bits, book, sub):
    """Returns (idx u16 [n, D/sub], y fp64 [n, D]).  codebooks [B, K, sub] fp16 bits."""
    x, px = _c(x_bits, np.uint16)
    n, D = x.shape
    cb, pcb = _c(codebooks_bits, np.uint16)
    K = cb.shape[-2]
    bk, pbk = _c(np.broadcast_to(book, (n,)), np.int32)
    lam, pl = _c(np.broadcast_to(lam, x.shape), np.float32)
    s, ps = _c(signs, np.int8)
    idx, pi = _out((n, D // sub), np.uint16)
    y, py = _out(x.shape, np.float64)
    rc = _load().kvqo_vq_encode_rows(n, D, int(sub), K, px, pl, ps, pcb, pbk, pi, py)
    if rc:
        raise ValueError("oracle vq_encode rejected")
    return idx, y


def vq_distances(y, codebooks_bits, book, idx, sub):
    y, py = _c(y, np.float64)
    n, D = y.shape
    cb, pcb = _c(codebooks_bits, np.uint16)
    K = cb.shape[-2]
    bk, pbk = _c(np.broadcast_to(book, (n,)), np.int32)
    ix, pix = _c(idx, np.uint16)
    d, pd = _out((n, D // sub), np.float64)
    rc = _load().kvqo_vq_distances(n, D, int(sub), K, py, pcb, pbk, pix, pd)
    if rc:
        raise ValueError("oracle vq_distances rejected (index out of range?)")
    return d


def vq_decode(idx, codebooks_bits, book, lam, signs, sub):
    ix, pix = _c(idx, np.uint16)
    n = ix.shape[0]
    D = ix.shape[1] * sub
    cb, pcb = _c(codebooks_bits, np.uint16)
    K = cb.shape[-2]
    bk, pbk = _c(np.broadcast_to(book, (n,)), np.int32)
    lam, pl = _c(np.broadcast_to(lam, (n, D)), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out((n, D), np.float64)
    x16, p16 = _out((n, D), np.uint16)
    rc = _load().kvqo_vq_decode_rows(n, D, int(sub), K, pix, pcb, pbk, pl, ps, p64, p16)
    if rc:
        raise ValueError("oracle vq_decode rejected (index out of range?)")
    return x64, x16


def kmeans_update(ysub, idx, codebook_bits):
    """Update half of one Lloyd step: ysub fp64 [n, sub] samples, idx [n]
    their assigned centroids, codebook fp16 bits [K, sub].  Returns
    (new codebook fp16 bits [K, sub], fp64 means [K, sub], counts u32 [K],
    mean |y| per centroid and coordinate [K, sub])."""
    y, py = _c(ysub, np.float64)
    n, sub = y.shape
    ix, pix = _c(np.asarray(idx).reshape(n), np.uint16)
    cb, pcb = _c(codebook_bits, np.uint16)
    K = cb.shape[0]
    m64, pm = _out((K, sub), np.float64)
    new, pn = _out((K, sub), np.uint16)
    cnt, pc = _out((K,), np.uint32)
    am, pa = _out((K, sub), np.float64)
    rc = _load().kvqo_kmeans_update(n, int(sub), K, py, pix, pcb, pm, pn, pc, pa)
    if rc:
        raise ValueError("oracle kmeans_update rejected (index out of range?)")
    return new, m64, cnt, am


def kmeans_step(x_bits, lam, signs, codebook_bits, sub):
    """One Lloyd step on the rotated sub-vectors of x [n, D] (all rows train
    the one codebook [K, sub]).  Returns (idx [n, D/sub] assignments to the
    input codebook, new codebook fp16 bits, fp64 means, counts, mean |y|,
    rotated sub-vectors fp64 [n * D/sub, sub])."""
    idx, y = vq_encode(x_bits, lam, signs, np.asarray(codebook_bits)[None], 0, sub)
    ysub = y.reshape(-1, sub)
    new, m64, cnt, am = kmeans_update(ysub, idx.reshape(-1), codebook_bits)
    return idx, new, m64, cnt, am, ysub


def attend_decode(q_bits, k_codes, k_scales, v_codes, v_scales, lam_k, lam_v, signs, G, scale,
                  lengths=None):
    """Decode attention in fp64 over an int4 cache.  q_bits [L, H*R, D]
    binary16 bits; k/v codes [L, T, H, D/2] u8; k/v scales [L, T, H, D/G]
    binary16 bits; lam_k/lam_v [L, H, D]; lengths [L] or None (all T).
    Returns out64 [L, H*R, D]."""
    kc, pkc = _c(k_codes, np.uint8)
    L, T, H, half = kc.shape
    D = 2 * half
    qb, pq = _c(q_bits, np.uint16)
    R = qb.shape[1] // H
    if qb.shape != (L, H * R, D):
        raise ValueError("q shape %s does not match [L, H*R, D]" % (qb.shape,))
    ks, pks = _c(k_scales, np.uint16)
    vc, pvc = _c(v_codes, np.uint8)
    vs, pvs = _c(v_scales, np.uint16)
    lk, plk = _c(lam_k, np.float32)
    lv, plv = _c(lam_v, np.float32)
    s, ps = _c(signs, np.int8)
    pl = None
    if lengths is not None:
        ln, pl = _c(lengths, np.int32)
    out, po = _out((L, H * R, D), np.float64)
    rc = _load().kvqo_attend_decode(L, T, H, R, D, int(G), pq, pkc, pks, pvc, pvs, plk, plv, ps, pl,
                                    float(scale), po)
    if rc:
        raise ValueError("oracle attend_decode rejected its arguments (%d)" % rc)
    return out


# ------------------------------------------------------------------ int8
def codes8_given_scales(y, scales_bits, G):
    """int8 codes of rotated values y [n, D] under given binary16 scales."""
    yy, py = _c(y, np.float64)
    D = yy.shape[-1]
    sc, ps = _c(scales_bits, np.uint16)
    q, pq = _out(yy.shape, np.int8)
    if _load().kvqo_codes8_given_scales(_rows(yy, D), D, int(G), py, ps, pq):
        raise ValueError("bad group size")
    return q


def quantize8(x_bits, lam, signs, G):
    """int8 group quantizer: x [n, D] binary16 bits, lam [n, D] fp32, signs
    [D] -> (codes int8 [n, D], scales binary16 bits [n, D/G], y fp64 [n, D],
    number of vectors outside the domain)."""
    x, px = _c(x_bits, np.uint16)
    n, D = x.shape
    lam, pl = _c(np.broadcast_to(lam, (n, D)), np.float32)
    s, ps = _c(signs, np.int8)
    codes, pc = _out((n, D), np.int8)
    scales, psc = _out((n, D // G), np.uint16)
    y, py = _out((n, D), np.float64)
    bad = _load().kvqo_quantize8_rows(n, D, int(G), px, pl, ps, pc, psc, py)
    if bad < 0:
        raise ValueError("oracle quantize8 rejected its arguments")
    return codes, scales, y, int(bad)


def dequantize8(codes, scales_bits, lam, signs, G):
    """Inverse of quantize8 -> (xhat fp64 [n, D], xhat binary16 bits [n, D])."""
    c, pc = _c(codes, np.int8)
    n, D = c.shape
    sc, psc = _c(scales_bits, np.uint16)
    lam, pl = _c(np.broadcast_to(lam, (n, D)), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out((n, D), np.float64)
    x16, p16 = _out((n, D), np.uint16)
    if _load().kvqo_dequantize8_rows(n, D, int(G), pc, psc, pl, ps, p64, p16):
        raise ValueError("oracle dequantize8 rejected its arguments")
    return x64, x16


# ----------------------------------------------------------------- MXFP4
def e2m1_value(code: int) -> float:
    return float(_load().kvqo_e2m1_value(int(code)))


def quantize_mxfp4(x_bits, lam, signs):
    """Block-scaled E2M1: x [n, D] binary16 bits -> (codes u8 [n, D/2] packed
    nibbles, E8M0 scales u8 [n, D/32], y fp64 [n, D], vectors out of domain)."""
    x, px = _c(x_bits, np.uint16)
    n, D = x.shape
    lam, pl = _c(np.broadcast_to(lam, (n, D)), np.float32)
    s, ps = _c(signs, np.int8)
    codes, pc = _out((n, D // 2), np.uint8)
    scales, psc = _out((n, D // 32), np.uint8)
    y, py = _out((n, D), np.float64)
    bad = _load().kvqo_quantize_mxfp4_rows(n, D, px, pl, ps, pc, psc, py)
    if bad < 0:
        raise ValueError("oracle quantize_mxfp4 rejected its arguments")
    return codes, scales, y, int(bad)


def mxfp4_codes_given_scales(y, scales):
    """E2M1 codes (one per byte) of rotated values y [n, D] under E8M0 scales."""
    yy, py = _c(y, np.float64)
    n, D = yy.shape
    sc, ps = _c(scales, np.uint8)
    q, pq = _out((n, D), np.uint8)
    if _load().kvqo_mxfp4_codes_given_scales(n, D, py, ps, pq):
        raise ValueError("head_dim must be a multiple of 32")
    return q


def dequantize_mxfp4(codes, scales, lam, signs):
    c, pc = _c(codes, np.uint8)
    n, half = c.shape
    D = 2 * half
    sc, psc = _c(scales, np.uint8)
    lam, pl = _c(np.broadcast_to(lam, (n, D)), np.float32)
    s, ps = _c(signs, np.int8)
    x64, p64 = _out((n, D), np.float64)
    x16, p16 = _out((n, D), np.uint16)
    if _load().kvqo_dequantize_mxfp4_rows(n, D, pc, psc, pl, ps, p64, p16):
        raise ValueError("oracle dequantize_mxfp4 rejected its arguments")
    return x64, x16
