"""Self-tests of the parity comparator (CPU): planted perturbations must be
classified as the contract says -- accepted where a legitimate fp32/fp64
difference can produce them, rejected otherwise."""
import numpy as np
import pytest

import oracle
from tests import parity

RNG = np.random.default_rng(7)


def _case(n=64, D=128, G=32):
    x = RNG.standard_normal((n, D)).astype(np.float16).view(np.uint16)
    lam = np.exp(RNG.standard_normal((n, D)) * 0.3).astype(np.float32)
    s = (RNG.integers(0, 2, D) * 2 - 1).astype(np.int8)
    codes, scales, y, _ = oracle.quantize(x, lam, s, G)
    return x, lam, s, G, codes, scales, y


def test_identical_outputs_pass():
    x, lam, s, G, codes, scales, y = _case()
    _, x16 = oracle.dequantize(codes, scales, lam, s, G)
    rep = parity.int4_parity(x, lam, s, G, codes, scales, x16)
    assert rep["codes"]["exact"] == rep["codes"]["n"]


def test_one_ulp_scale_flip_is_accepted_and_conditions_codes():
    x, lam, s, G, codes, scales, y = _case()
    sc = scales.copy()
    sc[3, 1] += 1                      # one fp16 ulp up
    q = oracle.codes_given_scales(y, sc, G)
    rep = parity.int4_parity(x, lam, s, G, oracle.pack_nibbles(q), sc)
    assert rep["scales"]["flips"] == 1 and rep["scales"]["bad"] == 0


def test_two_ulp_scale_change_is_rejected():
    x, lam, s, G, codes, scales, y = _case()
    sc = scales.copy()
    sc[0, 0] += 2
    rep = parity.check_scales(sc, scales)
    assert rep["bad"] == 1


def test_zero_scale_mismatch_is_rejected():
    z = np.zeros((1, 2), np.uint16)
    nz = np.array([[0x3c00, 0]], np.uint16)
    assert parity.check_scales(nz, z)["bad"] == 1
    assert parity.check_scales(z, nz)["bad"] == 1


def test_code_off_by_one_only_near_boundary():
    sc = np.array([[np.float16(0.5).view(np.uint16)]], np.uint16)
    G = 4
    # y/scale = 1.50004 (near boundary) and 1.2 (far from it)
    y = np.array([[0.75002, 0.6, -0.75001, 3.0]])
    q_ok = np.array([[2, 1, -1, 6]], np.int8)          # oracle gives [2, 1, -2, 6]
    rep = parity.check_codes(y, sc, q_ok, G)
    assert rep["bad"] == 0 and rep["boundary"] == 1
    q_bad = np.array([[2, 2, -2, 6]], np.int8)         # 1.2 -> 2 is wrong
    assert parity.check_codes(y, sc, q_bad, G)["bad"] == 1
    q_bad2 = np.array([[0, 1, -2, 6]], np.int8)        # off by 2 near a boundary
    assert parity.check_codes(y, sc, q_bad2, G)["bad"] == 1


def test_dequant_tolerance():
    lam = np.array([[1.0, 0.25]], np.float32)
    x64 = np.array([[1.0, 4.0]])
    ok = np.array([[1.0 + 1.9e-3, 4.0 + 7e-3]]).astype(np.float16).view(np.uint16)
    assert parity.check_dequant(ok, x64, lam)["bad"] == 0
    bad = np.array([[1.0 + 4e-3, 4.0]]).astype(np.float16).view(np.uint16)
    assert parity.check_dequant(bad, x64, lam)["bad"] == 1


def test_vq_classification():
    D, sub = 16, 8
    cb = np.zeros((1, 4, sub))
    cb[0, 0] = 1.0
    cb[0, 1] = 1.0 + 1e-3
    cb[0, 2] = 1.0            # exact duplicate of centroid 0
    cb[0, 3] = 5.0
    cbb = cb.astype(np.float16).view(np.uint16)
    y = np.ones((1, D)) * 1.0000001
    book = np.zeros(1, np.int32)
    ora = np.array([[0, 0]], np.uint16)
    assert parity.check_vq(y, cbb, book, ora, ora, sub)["bad"] == 0
    tie = np.array([[2, 0]], np.uint16)           # equal distance but not the lowest index
    assert parity.check_vq(y, cbb, book, tie, ora, sub)["bad"] == 1
    far = np.array([[3, 0]], np.uint16)
    assert parity.check_vq(y, cbb, book, far, ora, sub)["bad"] == 1


def _km_case(n=40, D=64, K=24):
    x = RNG.standard_normal((n, D)).astype(np.float16).view(np.uint16)
    lam = np.exp(RNG.standard_normal((n, D)) * 0.3).astype(np.float32)
    s = (RNG.integers(0, 2, D) * 2 - 1).astype(np.int8)
    cb = RNG.standard_normal((K, 8))
    cb[7] = 40.0                                   # never the nearest: stays empty
    cbb = cb.astype(np.float16).view(np.uint16)
    idx, new, m64, cnt, am, ysub = oracle.kmeans_step(x, lam, s, cbb, 8)
    return x, lam, s, cbb, idx, new, cnt


def test_kmeans_classification():
    x, lam, s, cbb, idx, new, cnt = _km_case()
    rep = parity.kmeans_parity(x, lam, s, cbb, idx, new, cnt)
    assert rep["centroids"]["bad"] == 0 and rep["centroids"]["empty"] >= 1
    assert rep["centroids"]["exact"] == rep["centroids"]["n"]
    # a count off by one is rejected
    c2 = cnt.copy()
    c2[int(np.argmax(cnt))] -= 1
    with pytest.raises(parity.ParityError):
        parity.kmeans_parity(x, lam, s, cbb, idx, new, c2)
    # a centroid two fp16 ulps away is rejected; so is a moved empty centroid
    k = int(np.argmax(cnt))
    for kk, t in ((k, 3), (7, 0)):
        n2 = new.copy()
        n2[kk, t] += 2
        with pytest.raises(parity.ParityError):
            parity.kmeans_parity(x, lam, s, cbb, idx, n2, cnt)
    # a non-nearest assignment is rejected
    i2 = idx.copy()
    i2[0, 0] = 7
    with pytest.raises(parity.ParityError):
        parity.kmeans_parity(x, lam, s, cbb, i2, new, cnt)


def test_sharded_check_matches_unsharded_and_still_fails():
    """The sharded runner gives the unsharded report's counts, and a planted
    wrong code in one shard still fails the whole check."""
    x, lam, s, G, codes, scales, y = _case(n=97)
    _, x16 = oracle.dequantize(codes, scales, lam, s, G)
    whole = parity.int4_parity(x, lam, s, G, codes, scales, x16)
    rep = parity.sharded(lambda k: parity.int4_parity(x[k], lam[k], s, G, codes[k], scales[k], x16[k]), 97,
                         n_workers=5)
    for part in ("scales", "codes", "dequant"):
        for f in ("n", "bad"):
            assert rep[part][f] == whole[part][f], (part, f)
    assert rep["codes"]["exact"] == 97 * 128
    bad = codes.copy()
    bad[80, 3] ^= 0x20                 # one nibble off by more than one step
    with pytest.raises(parity.ParityError):
        parity.sharded(lambda k: parity.int4_parity(x[k], lam[k], s, G, bad[k], scales[k]), 97, n_workers=5)
