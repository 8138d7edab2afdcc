"""Pins for the fp64 CPU oracle: each check ties it to something other than
itself -- numpy's binary16 conversion, scipy's Sylvester Hadamard matrix and
pairwise distances, closed forms, hand-derived worked examples and invariants
of the quantizer -- chosen so that a dropped term, a wrong sign, a wrong
index or a swapped order fails at least one of them."""
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.spatial.distance

import oracle

RNG = np.random.default_rng(20260507)


def f16bits(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def bits_to_f64(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def rand_x(n, D, scale=1.0):
    return f16bits(RNG.standard_normal((n, D)) * scale)


def rand_signs(D):
    return (RNG.integers(0, 2, D) * 2 - 1).astype(np.int8)


def rand_lambda(n, D):
    return np.exp(RNG.standard_normal((n, D)) * 0.5).astype(np.float32)


# ------------------------------------------------------------------ binary16
def test_f16_decode_all_patterns_match_numpy():
    b = np.arange(65536, dtype=np.uint16)
    got = oracle.f16_to_f64(b)
    ref = b.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_f16_encode_matches_numpy_rne():
    # numpy rounds binary64 -> binary16 directly with round-half-even.
    v = np.concatenate([
        RNG.standard_normal(200000),
        RNG.standard_normal(50000) * 1e-5,          # subnormal range
        RNG.standard_normal(50000) * 3e4,           # near overflow
        np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e9, -65520.0,
                  2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 0.0, -0.0]),
    ])
    got = oracle.f64_to_f16(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_encode_midpoints_go_to_even():
    # Every finite positive pair of neighbours: the exact midpoint (representable
    # in binary64) must round to the neighbour with an even fraction.
    lo = np.arange(0, 0x7bff, dtype=np.uint16)
    a = bits_to_f64(lo)
    b = bits_to_f64(lo + 1)
    mid = (a + b) / 2
    got = oracle.f64_to_f16(mid)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("D", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy_sylvester(D):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(D)] for i in range(D)])
    assert np.array_equal(H, scipy.linalg.hadamard(D))
    assert np.array_equal(H @ H.T, D * np.eye(D, dtype=H.dtype))   # H H^T = D I
    assert np.array_equal(H, H.T)
    if D >= 2:  # Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]]
        h = D // 2
        Hn = H[:h, :h]
        assert np.array_equal(H[:h, h:], Hn) and np.array_equal(H[h:, :h], Hn)
        assert np.array_equal(H[h:, h:], -Hn)


# ---------------------------------------------------------------- rotation
@pytest.mark.parametrize("D", [8, 64, 128, 256])
def test_rotate_matches_dense_scipy_product(D):
    n = 64
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    y = oracle.rotate(x, lam, s)
    H = scipy.linalg.hadamard(D).astype(np.float64)
    v = bits_to_f64(x) * lam.astype(np.float64) * s
    ref = (v @ H.T) / np.sqrt(D)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("D", [8, 128])
def test_rotate_basis_vectors_give_hadamard_columns(D):
    H = scipy.linalg.hadamard(D)
    ones = np.ones(D, np.float32)
    for k in (0, 1, D // 2 - 1, D - 1):
        x = np.zeros((1, D))
        x[0, k] = 1.0
        y = oracle.rotate(f16bits(x), ones, np.ones(D, np.int8))[0]
        assert np.allclose(y, H[:, k] / np.sqrt(D), atol=1e-15)


def test_lambda_multiplies_before_rotation():
    D = 16
    lam = np.ones(D, np.float32)
    lam[5] = 2.0
    x = np.zeros((1, D))
    x[0, 5] = 3.0
    y = oracle.rotate(f16bits(x), lam, np.ones(D, np.int8))[0]
    H = scipy.linalg.hadamard(D)
    assert np.allclose(y, 6.0 * H[:, 5] / 4.0, atol=1e-15)


def test_signs_apply_before_rotation():
    # s * x = all ones  =>  y = sqrt(D) e_0 exactly.
    D = 128
    s = rand_signs(D)
    y = oracle.rotate(f16bits(s.astype(np.float64)[None]), np.ones(D, np.float32), s)[0]
    want = np.zeros(D)
    want[0] = np.sqrt(D)
    assert np.allclose(y, want, atol=1e-12)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_parseval_and_roundtrip(D):
    n = 200
    x = rand_x(n, D, 3.0)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    y = oracle.rotate(x, lam, s)
    lx = bits_to_f64(x) * lam.astype(np.float64)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(lx, axis=1), rtol=1e-12)
    x64, _ = oracle.unrotate(y, lam, s)
    xr = bits_to_f64(x)
    assert np.abs(x64 - xr).max() <= 1e-12 * np.abs(xr).max()


def test_unrotate_closed_form():
    D = 32
    lam = rand_lambda(1, D)[0]
    s = rand_signs(D)
    H = scipy.linalg.hadamard(D)
    for k in (0, 7, 31):
        yh = np.zeros((1, D))
        yh[0, k] = 1.25
        x64, x16 = oracle.unrotate(yh, lam, s)
        want = (s / lam.astype(np.float64)) * 1.25 * H[k, :] / np.sqrt(D)
        assert np.allclose(x64[0], want, rtol=1e-15, atol=0)
        assert np.array_equal(x16[0], want.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------- nibbles
def test_nibbles_roundtrip_all_bytes():
    b = np.arange(256, dtype=np.uint8)[None]
    q = oracle.unpack_nibbles(b)
    assert q.min() == -8 and q.max() == 7
    assert np.array_equal(oracle.pack_nibbles(q), b)


def test_nibbles_golden(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "nibbles.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, b, h = line.split()
                rows.append((int(a), int(b), int(h, 16)))
    q = np.array([[a, b] for a, b, _ in rows], np.int8).reshape(1, -1)
    got = oracle.pack_nibbles(q)[0]
    assert list(got) == [h for _, _, h in rows]
    assert np.array_equal(oracle.unpack_nibbles(got[None])[0], q[0])


# ---------------------------------------------------------------- quantizer
def load_worked(golden_dir):
    cases, cur = [], {}
    with open(os.path.join(golden_dir, "worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line:
                if cur:
                    cases.append(cur)
                cur = {}
                continue
            if line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            cur[k.strip()] = v.split()
    if cur:
        cases.append(cur)
    return cases


def test_worked_examples(golden_dir):
    cases = load_worked(golden_dir)
    assert len(cases) == 4
    for c in cases:
        D, G = int(c["D"][0]), int(c["G"][0])
        lam = np.array([float(v) for v in c["lambda"]], np.float32)
        s = np.array([int(v) for v in c["signs"]], np.int8)
        x = np.array([int(v, 16) for v in c["x"]], np.uint16)[None]
        codes, scales, y, bad = oracle.quantize(x, lam, s, G)
        assert bad == 0
        assert [int(v) for v in scales[0]] == [int(v, 16) for v in c["scales"]], c["name"]
        assert [int(v) for v in codes[0]] == [int(v, 16) for v in c["codes"]], c["name"]
        _, x16 = oracle.dequantize(codes, scales, lam, s, G)
        assert [int(v) for v in x16[0]] == [int(v, 16) for v in c["xhat"]], c["name"]


@pytest.mark.parametrize("D", [64, 128, 256])
def test_case_single_spike(D):
    # x = a e_k, lambda = 1, s = 1: every |y_i| = |a|/sqrt(D); every scale is
    # fp16(|a|/(7 sqrt D)); every code is +-7 with the sign of a H[i][k].
    G = 32
    H = scipy.linalg.hadamard(D)
    for a, k in ((1.5, 3), (-2.0, D - 1), (0.75, 0)):
        x = np.zeros((1, D))
        x[0, k] = a
        codes, scales, _, bad = oracle.quantize(f16bits(x), np.ones(D, np.float32), np.ones(D, np.int8), G)
        assert bad == 0
        want_sc = np.float16(abs(a) / (7 * np.sqrt(D))).view(np.uint16)
        assert (scales == want_sc).all()
        q = oracle.unpack_nibbles(codes)[0]
        assert np.array_equal(q, 7 * np.sign(a) * H[:, k])


def test_case_all_ones_energy_in_group0():
    D, G = 128, 32
    s = rand_signs(D)
    x = f16bits(s.astype(np.float64)[None])
    codes, scales, _, bad = oracle.quantize(x, np.ones(D, np.float32), s, G)
    q = oracle.unpack_nibbles(codes)[0]
    assert scales[0, 0] == np.float16(np.sqrt(D) / 7).view(np.uint16)
    assert (scales[0, 1:] == 0).all()
    assert q[0] == 7 and (q[1:] == 0).all()


def test_group_equal_to_D_is_per_vector_absmax():
    D = 128
    x = rand_x(50, D)
    lam = rand_lambda(50, D)
    s = rand_signs(D)
    codes, scales, y, _ = oracle.quantize(x, lam, s, D)
    want = (np.abs(y).max(axis=1) / 7).astype(np.float16).view(np.uint16)
    assert np.array_equal(scales[:, 0], want)


def test_ties_round_half_to_even():
    # rotated values placed exactly on k + 1/2 steps of a stored scale
    sc = np.float16(0.375)
    sbar = float(sc)
    halves = np.array([-6.5, -5.5, -4.5, -3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5])
    y = np.zeros((1, 16))
    y[0, :14] = halves * sbar
    y[0, 14] = 7.4 * sbar    # clamps to 7
    y[0, 15] = -9.0 * sbar   # clamps to -7
    q = oracle.codes_given_scales(y, np.array([[sc.view(np.uint16)]]), 16)[0]
    want = list(np.round(halves).astype(int)) + [7, -7]     # numpy rounds half to even
    assert list(q) == want
    assert list(q[:14]) == [-6, -6, -4, -4, -2, -2, 0, 0, 2, 2, 4, 4, 6, 6]


@pytest.mark.parametrize("D,G", [(128, 32), (64, 8)])
def test_codes_given_scales_matches_quantizer(D, G):
    # Conditioning on a stored scale must reproduce the quantizer's own codes
    # when handed the quantizer's own scales (multi-group, so the group index
    # of every coordinate matters).
    x = rand_x(100, D)
    lam = rand_lambda(100, D)
    s = rand_signs(D)
    codes, scales, y, _ = oracle.quantize(x, lam, s, G)
    q = oracle.codes_given_scales(y, scales, G)
    assert np.array_equal(q, oracle.unpack_nibbles(codes))


def test_zero_scale_gives_zero_codes():
    y = np.ones((1, 8)) * 1e-30
    q = oracle.codes_given_scales(y, np.array([[0]], np.uint16), 8)
    assert (q == 0).all()
    codes, scales, _, bad = oracle.quantize(np.zeros((3, 64), np.uint16), np.ones(64, np.float32),
                                            np.ones(64, np.int8), 32)
    assert bad == 0 and (codes == 0).all() and (scales == 0).all()


@pytest.mark.parametrize("D,G", [(64, 16), (128, 32), (128, 8), (256, 64), (128, 128)])
def test_quantizer_invariants(D, G):
    n = 400
    x = rand_x(n, D, 2.0)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    codes, scales, y, bad = oracle.quantize(x, lam, s, G)
    assert bad == 0
    q = oracle.unpack_nibbles(codes).astype(np.float64)
    sb = bits_to_f64(scales)
    sbe = np.repeat(sb, G, axis=1)
    assert np.abs(q).max() <= 7
    # |y - q*scale| <= scale/2 for every element (uses the STORED scale)
    assert (np.abs(y - q * sbe) <= sbe / 2 * (1 + 1e-12)).all()
    # scale = fp16(amax/7) per group, and every non-zero group reaches |q| = 7
    amax = np.abs(y).reshape(n, D // G, G).max(axis=2)
    assert np.array_equal(scales, (amax / 7).astype(np.float16).view(np.uint16))
    qa = np.abs(q).reshape(n, D // G, G).max(axis=2)
    assert (qa[sb > 0] == 7).all()


def test_out_of_domain_is_rejected():
    D = 64
    x = np.zeros((3, D), np.uint16)
    x[1, 0] = 0x7c00                     # +inf
    x[2, :] = np.float16(60000).view(np.uint16)   # amax/7 above 65504 once lambda = 16
    lam = np.ones(D, np.float32) * 16
    codes, scales, y, bad = oracle.quantize(x, lam, np.ones(D, np.int8), 32)
    assert bad == 2


# ---------------------------------------------------------------- dequant
def test_dequant_single_code_closed_form():
    D, G = 64, 16
    lam = rand_lambda(1, D)[0]
    s = rand_signs(D)
    H = scipy.linalg.hadamard(D)
    for k, c in ((0, 7), (17, -3), (63, 1)):
        q = np.zeros((1, D), np.int8)
        q[0, k] = c
        scales = np.zeros((1, D // G), np.uint16)
        scales[0, k // G] = np.float16(0.3125).view(np.uint16)
        x64, x16 = oracle.dequantize(oracle.pack_nibbles(q), scales, lam, s, G)
        want = (s / lam.astype(np.float64)) * c * 0.3125 * H[k, :] / np.sqrt(D)
        assert np.allclose(x64[0], want, rtol=1e-14, atol=0)
        assert np.array_equal(x16[0], want.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("D,G", [(128, 32), (256, 64), (64, 16)])
def test_roundtrip_error_bound(D, G):
    # ||lambda*(xhat - x)|| = ||yhat - y|| <= 1/2 sqrt(G * sum scale^2)
    n = 300
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    codes, scales, y, _ = oracle.quantize(x, lam, s, G)
    x64, x16 = oracle.dequantize(codes, scales, lam, s, G)
    err = np.linalg.norm(lam * (x64 - bits_to_f64(x)), axis=1)
    bound = 0.5 * np.sqrt(G * (bits_to_f64(scales) ** 2).sum(axis=1))
    assert (err <= bound * (1 + 1e-9)).all()
    assert np.array_equal(x16, x64.astype(np.float16).view(np.uint16))


def test_byte_accounting_3_56x():
    # D=128, G=32: 64 code bytes + 4 fp16 scales = 72 B against 256 B of fp16,
    # the top of the 3.0-3.56x compression range the paper reports.
    D, G = 128, 32
    codes, scales, _, _ = oracle.quantize(rand_x(1, D), np.ones(D, np.float32), np.ones(D, np.int8), G)
    nbytes = codes.nbytes + scales.nbytes
    assert nbytes == 72 and abs(2 * D / nbytes - 3.56) < 0.005


# -------------------------------------------------------------------- SRFT
def srft_numpy(x_bits, lam, s):
    """numpy's orthonormal FFT of s * lambda * x, packed [X_0, X_{D/2},
    sqrt2 Re X_1, sqrt2 Im X_1, ...]."""
    v = s * lam.astype(np.float64) * bits_to_f64(x_bits)
    D = v.shape[-1]
    X = np.fft.fft(v, norm="ortho", axis=-1)
    y = np.empty_like(v)
    y[..., 0] = X[..., 0].real
    y[..., 1] = X[..., D // 2].real
    y[..., 2::2] = np.sqrt(2) * X[..., 1:D // 2].real
    y[..., 3::2] = np.sqrt(2) * X[..., 1:D // 2].imag
    return y


@pytest.mark.parametrize("D", [2, 6, 8, 64, 96, 128, 256])
def test_srft_matches_numpy_fft(D):
    n = 20
    x = rand_x(n, D, 3.0)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    y = oracle.srft(x, lam, s)
    want = srft_numpy(x, lam, s)
    assert np.allclose(y, want, rtol=0, atol=1e-12 * np.abs(want).max())
    # the real FFT of scipy gives the same half spectrum
    import scipy.fft
    R = scipy.fft.rfft(s * lam.astype(np.float64) * bits_to_f64(x), norm="ortho", axis=-1)
    assert np.allclose(y[:, 1], R[:, D // 2].real, atol=1e-12 * np.abs(want).max())
    assert np.allclose(y[:, 3::2], np.sqrt(2) * R[:, 1:D // 2].imag, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("D", [8, 96, 128])
def test_srft_orthonormal_parseval_and_roundtrip(D):
    # the packed map is an orthogonal matrix: rotate exact unit vectors
    eye = np.eye(D).astype(np.float16).view(np.uint16)
    Q = oracle.srft(eye, np.ones(D, np.float32), np.ones(D, np.int8)).T     # column j = image of e_j
    assert np.allclose(Q @ Q.T, np.eye(D), atol=1e-13)
    n = 50
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    y = oracle.srft(x, lam, s)
    v = lam * bits_to_f64(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(v, axis=1), rtol=1e-12)
    x64, x16 = oracle.isrft(y, lam, s)
    assert np.abs(x64 - bits_to_f64(x)).max() <= 1e-12 * np.abs(bits_to_f64(x)).max()
    assert np.array_equal(x16, x)


def test_srft_closed_forms():
    D = 16
    one, plus = np.ones(D, np.float32), np.ones(D, np.int8)
    j = np.arange(D)
    # impulse: flat spectrum X_k = D^-1/2
    imp = np.zeros((1, D))
    imp[0, 0] = 1
    y = oracle.srft(f16bits(imp), one, plus)[0]
    want = np.full(D, np.sqrt(2.0 / D))
    want[0] = want[1] = 1 / np.sqrt(D)
    want[3::2] = 0
    assert np.allclose(y, want, atol=1e-15)
    # alternating signs: everything in X_{D/2}
    y = oracle.srft(f16bits(((-1.0) ** j)[None]), one, plus)[0]
    want = np.zeros(D)
    want[1] = np.sqrt(D)
    assert np.allclose(y, want, atol=1e-14)
    # cos / sin at frequency D/4 (exact in fp16): sqrt(D/2) in Re / -sqrt(D/2) in Im of X_{D/4}
    k0 = D // 4
    c = np.round(np.cos(2 * np.pi * k0 * j / D))
    sn = np.round(np.sin(2 * np.pi * k0 * j / D))
    y = oracle.srft(f16bits(np.stack([c, sn])), one, plus)
    wc, ws = np.zeros(D), np.zeros(D)
    wc[2 * k0] = np.sqrt(D / 2)
    ws[2 * k0 + 1] = -np.sqrt(D / 2)
    assert np.allclose(y[0], wc, atol=1e-14) and np.allclose(y[1], ws, atol=1e-14)


@pytest.mark.parametrize("D,G", [(128, 32), (96, 32), (256, 64)])
def test_srft_quantizer_invariants_and_roundtrip(D, G):
    n = 300
    x = rand_x(n, D, 2.0)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    codes, scales, y, bad = oracle.quantize_srft(x, lam, s, G)
    assert bad == 0
    assert np.allclose(y, srft_numpy(x, lam, s), atol=1e-12 * np.abs(y).max())
    q = oracle.unpack_nibbles(codes).astype(np.float64)
    sb = bits_to_f64(scales)
    sbe = np.repeat(sb, G, axis=1)
    assert np.abs(q).max() <= 7
    assert (np.abs(y - q * sbe) <= sbe / 2 * (1 + 1e-12)).all()
    amax = np.abs(y).reshape(n, D // G, G).max(axis=2)
    assert np.array_equal(scales, (amax / 7).astype(np.float16).view(np.uint16))
    assert np.array_equal(oracle.codes_given_scales(y, scales, G), q.astype(np.int8))
    # round trip: ||lambda (xhat - x)|| = ||yhat - y|| <= 1/2 sqrt(G sum scale^2)
    x64, x16 = oracle.dequantize_srft(codes, scales, lam, s, G)
    err = np.linalg.norm(lam * (x64 - bits_to_f64(x)), axis=1)
    assert (err <= 0.5 * np.sqrt(G * (sb ** 2).sum(axis=1)) * (1 + 1e-9)).all()
    assert np.array_equal(x16, x64.astype(np.float16).view(np.uint16))


def test_srft_dequant_single_code_closed_form():
    """One code at packed position 2k (or 2k+1) decodes to sqrt(2/D) times a
    cosine (or minus a sine) at frequency k; positions 0 and 1 to a constant
    and an alternating vector."""
    D, G = 64, 16
    lam = rand_lambda(1, D)[0]
    s = rand_signs(D)
    j = np.arange(D)
    for pos, c in ((0, 7), (1, -2), (10, 3), (11, -5), (63, 1)):
        q = np.zeros((1, D), np.int8)
        q[0, pos] = c
        scales = np.zeros((1, D // G), np.uint16)
        scales[0, pos // G] = np.float16(0.3125).view(np.uint16)
        x64, _ = oracle.dequantize_srft(oracle.pack_nibbles(q), scales, lam, s, G)
        k = pos // 2
        if pos == 0:
            basis = np.ones(D) / np.sqrt(D)
        elif pos == 1:
            basis = (-1.0) ** j / np.sqrt(D)
        elif pos % 2 == 0:
            basis = np.sqrt(2.0 / D) * np.cos(2 * np.pi * j * k / D)
        else:
            basis = -np.sqrt(2.0 / D) * np.sin(2 * np.pi * j * k / D)
        want = (s / lam.astype(np.float64)) * c * 0.3125 * basis
        assert np.allclose(x64[0], want, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------- VQ
@pytest.mark.parametrize("sub", [1, 2, 4, 8])
@pytest.mark.parametrize("K", [1, 3, 16])
def test_vq_encode_bruteforce(sub, K):
    D, n = 16, 40
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    cb = f16bits(RNG.standard_normal((2, K, sub)))
    book = RNG.integers(0, 2, n).astype(np.int32)
    idx, y = oracle.vq_encode(x, lam, s, cb, book, sub)
    assert np.allclose(y, oracle.rotate(x, lam, s))
    for r in range(n):
        C = bits_to_f64(cb[book[r]])
        d = scipy.spatial.distance.cdist(y[r].reshape(-1, sub), C, "sqeuclidean")
        assert np.array_equal(idx[r], d.argmin(axis=1))      # first minimum = lowest index
        got = oracle.vq_distances(y[r:r + 1], cb, book[r:r + 1], idx[r:r + 1], sub)[0]
        assert np.allclose(got, d.min(axis=1), rtol=1e-13, atol=1e-15)


def test_vq_duplicate_centroids_lowest_index_and_exact_hits():
    # x = c * H[:, k]  =>  y = c * sqrt(D) * e_k exactly (D = 16, sqrt D = 4).
    D, sub = 16, 4
    H = scipy.linalg.hadamard(D)
    x = (0.5 * H[:, 6])[None]            # y = 2 e_6 : sub-vector 1 = (0, 0, 2, 0)
    cb = np.full((1, 8, sub), 3.0)
    cb[0, 0] = [1, 1, 1, 1]
    cb[0, 2] = [0, 0, 2, 0]               # exact hit for sub-vector 1
    cb[0, 5] = [0, 0, 2, 0]               # duplicate, higher index
    cb[0, 3] = [0, 0, 0, 0]               # exact hit for sub-vectors 0, 2, 3
    cb[0, 6] = [0, 0, 0, 0]
    cbb = f16bits(cb)
    idx, y = oracle.vq_encode(f16bits(x), np.ones(D, np.float32), np.ones(D, np.int8), cbb,
                              np.zeros(1, np.int32), sub)
    assert list(idx[0]) == [3, 2, 3, 3]
    d = oracle.vq_distances(y, cbb, np.zeros(1, np.int32), idx, sub)
    assert (d == 0).all()


def test_vq_decode_closed_form_and_roundtrip():
    D, sub, K = 32, 8, 5
    lam = rand_lambda(1, D)[0]
    s = rand_signs(D)
    cb = f16bits(RNG.standard_normal((1, K, sub)))
    idx = np.array([[4, 0, 2, 2]], np.uint16)
    x64, x16 = oracle.vq_decode(idx, cb, np.zeros(1, np.int32), lam, s, sub)
    yh = bits_to_f64(cb[0][idx[0]]).reshape(-1)
    H = scipy.linalg.hadamard(D)
    want = (s / lam.astype(np.float64)) * (H @ yh) / np.sqrt(D)
    assert np.allclose(x64[0], want, rtol=1e-13, atol=1e-15)
    # encoding the decoded vector's exact rotation recovers the same indices
    y = oracle.rotate(x16, lam, s)
    idx2 = oracle.vq_encode(x16, lam, s, cb, np.zeros(1, np.int32), sub)[0]
    assert np.array_equal(idx2, idx)


# ------------------------------------------------ codebook training (k-means)
def test_kmeans_step_matches_scipy_lloyd_iteration():
    """One step on rotated sub-vectors against scipy.cluster.vq.kmeans2 with the
    same initial codebook and iter=1 (assign with vq, move to the cluster
    means, keep empty clusters in place); one centroid is placed far away so
    that it gets no samples."""
    import warnings

    import scipy.cluster.vq
    D, sub, n, K = 64, 8, 40, 12
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    cb = RNG.standard_normal((K, sub))
    cb[5] = 50.0
    cbb = f16bits(cb)
    idx, new, m64, cnt, am, ysub = oracle.kmeans_step(x, lam, s, cbb, sub)
    assert np.allclose(ysub, oracle.rotate(x, lam, s).reshape(-1, sub))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        ref_cb, ref_lab = scipy.cluster.vq.kmeans2(ysub, bits_to_f64(cbb), iter=1, minit="matrix",
                                                   missing="warn")
    assert np.array_equal(idx.reshape(-1), ref_lab)
    assert np.allclose(m64, ref_cb, rtol=1e-13, atol=1e-15)
    assert cnt[5] == 0 and np.array_equal(new[5], cbb[5])
    assert np.array_equal(cnt, np.bincount(ref_lab, minlength=K))
    assert np.array_equal(new, f16bits(m64))


def test_kmeans_update_closed_form_clusters():
    """Samples built as mu_k +/- delta_t pairs around K centres: each centre's
    samples average to it exactly, and every sample is assigned to its own
    centre when the codebook is the centres themselves."""
    sub, K = 8, 6
    mu = np.round(RNG.standard_normal((K, sub)) * 8) / 4        # exact in fp16
    d = np.eye(sub) * 0.25
    ys, lab = [], []
    for k in range(K):
        for t in range(k + 1):                                  # k+1 pairs: counts 2, 4, ...
            ys += [mu[k] + d[t % sub], mu[k] - d[t % sub]]
            lab += [k, k]
    ys = np.array(ys)
    lab = np.array(lab)
    new, m64, cnt, am = oracle.kmeans_update(ys, lab, f16bits(mu))
    assert np.array_equal(m64, mu)
    assert np.array_equal(bits_to_f64(new), mu)
    assert np.array_equal(cnt, 2 * (np.arange(K) + 1))
    assert np.allclose(am, [np.abs(ys[lab == k]).mean(0) for k in range(K)], rtol=1e-15)


def test_kmeans_update_is_the_sse_minimiser_and_lloyd_descends():
    """For fixed assignments the update gives, per centroid, the point with the
    least summed squared distance (any perturbation costs more), and repeated
    steps never raise the within-cluster SSE by more than the fp16 storage
    rounding of the centroids."""
    D, sub, n, K = 32, 8, 60, 10
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    cbb = f16bits(RNG.standard_normal((K, sub)))
    idx, new, m64, cnt, am, ysub = oracle.kmeans_step(x, lam, s, cbb, sub)
    lab = idx.reshape(-1)
    for k in np.flatnonzero(cnt):
        yk = ysub[lab == k]
        best = ((yk - m64[k]) ** 2).sum()
        for _ in range(5):
            pert = m64[k] + RNG.standard_normal(sub) * 1e-3
            assert ((yk - pert) ** 2).sum() > best
    sse_prev, prev_idx = None, None
    for it in range(200):
        idx, new, m64, cnt, am, ysub = oracle.kmeans_step(x, lam, s, cbb, sub)
        C = bits_to_f64(cbb)
        sse = ((ysub - C[idx.reshape(-1)]) ** 2).sum()
        if sse_prev is not None:
            slack = 2.0 ** -10 * np.abs(ysub).sum() * 4
            assert sse <= sse_prev + slack
        if prev_idx is not None and np.array_equal(idx, prev_idx):
            break
        sse_prev, prev_idx = sse, idx
        cbb = new
    else:
        raise AssertionError("Lloyd steps did not settle")
    # settled: the same assignments give back the same (stored) centroids
    assert it > 1 and np.array_equal(new, cbb)


# ------------------------------------------------------- decode attention
def attn_case(L, T, H, R, D, G, seed, qscale=1.0):
    """Random int4 K/V caches produced by the oracle's own (pinned) quantizer,
    plus queries; returns everything attend_decode takes and the exact fp64
    dequantized K/V ([L, T, H, D]) for the library comparisons."""
    rng = np.random.default_rng(seed)
    s = (rng.integers(0, 2, D) * 2 - 1).astype(np.int8)
    out = {"s": s}
    for name in "kv":
        x = f16bits(rng.standard_normal((L, T, H, D)) * np.exp(0.5 * rng.standard_normal((L, 1, H, D))))
        lam = np.exp(0.3 * rng.standard_normal((L, H, D))).astype(np.float32)
        lam_rows = np.broadcast_to(lam[:, None], (L, T, H, D)).reshape(-1, D)
        codes, scales, _, _ = oracle.quantize(x.reshape(-1, D), lam_rows, s, G)
        x64, _ = oracle.dequantize(codes, scales, lam_rows, s, G)
        out[name] = (codes.reshape(L, T, H, D // 2), scales.reshape(L, T, H, D // G), lam,
                     x64.reshape(L, T, H, D))
    out["q"] = f16bits(rng.standard_normal((L, H * R, D)) * qscale)
    return out


def attend(c, G, scale, lengths=None):
    kc, ks, lk, _ = c["k"]
    vc, vs, lv, _ = c["v"]
    return oracle.attend_decode(c["q"], kc, ks, vc, vs, lk, lv, c["s"], G, scale, lengths)


def test_attend_single_token_returns_its_value():
    # softmax over one token is exactly 1, so the output is that token's vhat
    c = attn_case(2, 5, 3, 2, 64, 16, seed=1)
    out = attend(c, 16, 0.125, lengths=np.array([1, 1], np.int32))
    vhat = c["v"][3]
    for l in range(2):
        for j in range(6):
            assert np.array_equal(out[l, j], vhat[l, 0, j // 2])


def test_attend_zero_query_is_mean_of_values():
    c = attn_case(1, 37, 2, 3, 128, 32, seed=2)
    c["q"][:] = 0
    out = attend(c, 32, 0.1)
    want = c["v"][3].mean(axis=1)                       # [L, H, D]
    for j in range(6):
        assert np.allclose(out[0, j], want[0, j // 3], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D,G", [(128, 32), (256, 64)])
@pytest.mark.parametrize("R", [1, 2, 4])
def test_attend_matches_torch_sdpa(R, D, G):
    # the attention step against torch's scaled_dot_product_attention in
    # float64 on the (separately pinned) dequantized cache; GQA maps query
    # head j to KV head j // R; ragged lengths attend to a prefix
    import torch
    L, T, H = 3, 50, 3
    c = attn_case(L, T, H, R, D, G, seed=10 + R)
    lengths = np.array([50, 17, 1], np.int32)
    scale = 0.0883
    out = attend(c, G, scale, lengths)
    kh, vh = torch.from_numpy(c["k"][3]), torch.from_numpy(c["v"][3])
    q = torch.from_numpy(bits_to_f64(c["q"]))
    for l in range(L):
        n = int(lengths[l])
        k = kh[l, :n].permute(1, 0, 2).repeat_interleave(R, dim=0)     # [H*R, n, D]
        v = vh[l, :n].permute(1, 0, 2).repeat_interleave(R, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q[l][:, None, :], k, v, scale=scale)[:, 0]
        assert np.allclose(out[l], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attend_large_scores_stay_finite():
    # scores in the thousands: exp without the max shift would overflow
    import torch
    c = attn_case(1, 20, 1, 1, 64, 16, seed=4, qscale=30.0)
    out = attend(c, 16, 1.0)
    assert np.isfinite(out).all()
    k = torch.from_numpy(c["k"][3][0, :, 0])[None]
    v = torch.from_numpy(c["v"][3][0, :, 0])[None]
    q = torch.from_numpy(bits_to_f64(c["q"][0]))[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1.0)[:, 0]
    assert np.allclose(out[0], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attend_empty_context_gives_zeros():
    c = attn_case(2, 4, 1, 2, 64, 32, seed=5)
    out = attend(c, 32, 0.125, lengths=np.array([0, 4], np.int32))
    assert (out[0] == 0).all() and np.abs(out[1]).sum() > 0


# --------------------------------------------------------------------- int8
@pytest.mark.parametrize("D", [64, 128, 256])
def test_int8_single_spike(D):
    # x = a e_k, lambda = 1, s = 1: every |y_i| = |a|/sqrt(D); every scale is
    # fp16(|a|/(127 sqrt D)); every code is +-127 with the sign of a H[i][k]
    G = 32
    H = scipy.linalg.hadamard(D)
    for a, k in ((1.5, 3), (-2.0, D - 1), (0.75, 0)):
        x = np.zeros((1, D))
        x[0, k] = a
        codes, scales, _, bad = oracle.quantize8(f16bits(x), np.ones(D, np.float32), np.ones(D, np.int8), G)
        assert bad == 0
        assert (scales == np.float16(abs(a) / (127 * np.sqrt(D))).view(np.uint16)).all()
        assert np.array_equal(codes[0], 127 * np.sign(a) * H[:, k])


def test_int8_ties_round_half_to_even_and_clamp():
    sc = np.float16(0.0625)
    sbar = float(sc)
    halves = np.array([-126.5, -125.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 125.5, 126.5])
    y = np.zeros((1, 16))
    y[0, :10] = halves * sbar
    y[0, 10] = 127.4 * sbar      # rounds to 127
    y[0, 11] = 127.6 * sbar      # would round to 128: clamps to 127
    y[0, 12] = -300.0 * sbar     # clamps to -127
    q = oracle.codes8_given_scales(y, np.array([[sc.view(np.uint16)]]), 16)[0]
    assert list(q[:13]) == [-126, -126, -2, -2, 0, 0, 2, 2, 126, 126, 127, 127, -127]


@pytest.mark.parametrize("D,G", [(64, 16), (128, 32), (128, 8), (256, 64), (128, 128)])
def test_int8_quantizer_invariants(D, G):
    n = 300
    x = rand_x(n, D, 2.0)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    codes, scales, y, bad = oracle.quantize8(x, lam, s, G)
    assert bad == 0
    # the rotation is the (separately pinned) int4 quantizer's
    _, _, y4, _ = oracle.quantize(x, lam, s, G)
    assert np.array_equal(y, y4)
    q = codes.astype(np.float64)
    sb = bits_to_f64(scales)
    sbe = np.repeat(sb, G, axis=1)
    assert np.abs(q).max() <= 127
    assert (np.abs(y - q * sbe) <= sbe / 2 * (1 + 1e-12)).all()
    amax = np.abs(y).reshape(n, D // G, G).max(axis=2)
    assert np.array_equal(scales, (amax / 127).astype(np.float16).view(np.uint16))
    qa = np.abs(q).reshape(n, D // G, G).max(axis=2)
    assert (qa[sb > 0] == 127).all()
    assert np.array_equal(oracle.codes8_given_scales(y, scales, G), codes)


def test_int8_dequant_single_code_closed_form():
    D, G = 64, 16
    lam = rand_lambda(1, D)[0]
    s = rand_signs(D)
    H = scipy.linalg.hadamard(D)
    for k, c in ((0, 127), (17, -3), (63, -127)):
        q = np.zeros((1, D), np.int8)
        q[0, k] = c
        scales = np.zeros((1, D // G), np.uint16)
        scales[0, k // G] = np.float16(0.0078125).view(np.uint16)
        x64, x16 = oracle.dequantize8(q, scales, lam, s, G)
        want = (s / lam.astype(np.float64)) * c * 0.0078125 * H[k, :] / np.sqrt(D)
        assert np.allclose(x64[0], want, rtol=1e-14, atol=0)
        assert np.array_equal(x16[0], want.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("D,G", [(128, 32), (256, 64)])
def test_int8_roundtrip_error_bound_and_finer_than_int4(D, G):
    n = 300
    x = rand_x(n, D)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    codes, scales, _, _ = oracle.quantize8(x, lam, s, G)
    x64, _ = oracle.dequantize8(codes, scales, lam, s, G)
    err8 = np.linalg.norm(lam * (x64 - bits_to_f64(x)), axis=1)
    assert (err8 <= 0.5 * np.sqrt(G * (bits_to_f64(scales) ** 2).sum(axis=1)) * (1 + 1e-9)).all()
    c4, s4, _, _ = oracle.quantize(x, lam, s, G)
    x4, _ = oracle.dequantize(c4, s4, lam, s, G)
    err4 = np.linalg.norm(lam * (x4 - bits_to_f64(x)), axis=1)
    # 127 levels against 7: the error shrinks by about 127/7 on average
    assert err8.mean() * 10 < err4.mean()


# -------------------------------------------------------------------- MXFP4
def e2m1_golden(golden_dir):
    out = {}
    for line in open(os.path.join(golden_dir, "e2m1.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            out[int(c, 16)] = float(v)
    return out


def test_e2m1_table_golden(golden_dir):
    table = e2m1_golden(golden_dir)
    assert len(table) == 16
    for c, v in table.items():
        got = oracle.e2m1_value(c)
        assert got == v and np.signbit(got) == np.signbit(v), (c, got, v)


def test_e2m1_rounding_ties_even_and_saturation(golden_dir):
    # with scale byte 127 (X = 1) the codes are the E2M1 rounding of y itself
    table = e2m1_golden(golden_dir)
    mags = sorted(v for c, v in table.items() if c < 8)
    cases = []
    for lo, hi in zip(mags[:-1], mags[1:]):
        mid = (lo + hi) / 2
        even = min((c for c in range(8) if table[c] in (lo, hi)), key=lambda c: c & 1)   # mantissa bit 0
        cases += [(mid, table[even]), (np.nextafter(mid, 0), lo), (np.nextafter(mid, 10), hi), (lo, lo)]
    cases += [(6.0, 6.0), (6.5, 6.0), (7.0, 6.0), (1e30, 6.0), (0.0, 0.0)]
    y = np.array([[v for v, _ in cases] + [-v for v, _ in cases]])
    y = np.pad(y, ((0, 0), (0, (-y.shape[1]) % 32)))
    q = oracle.mxfp4_codes_given_scales(y, np.full((1, y.shape[1] // 32), 127, np.uint8))[0]
    got = [table[c] for c in q[:2 * len(cases)]]
    want = [w for _, w in cases] + [-w for _, w in cases]
    assert got == want
    # the sign bit follows the input's, -0 included
    assert all(np.signbit(g) == np.signbit(yv) for g, yv in zip(got, y[0]))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_mxfp4_block_scale_rule_and_invariants(D, golden_dir):
    table = e2m1_golden(golden_dir)
    n = 300
    x = rand_x(n, D, 2.0)
    lam = rand_lambda(n, D)
    s = rand_signs(D)
    codes, scales, y, bad = oracle.quantize_mxfp4(x, lam, s)
    assert bad == 0
    _, _, y4, _ = oracle.quantize(x, lam, s, 32)
    assert np.array_equal(y, y4)                                    # the int4 path's rotation
    e = scales.astype(np.int64) - 127
    amax = np.abs(y).reshape(n, D // 32, 32).max(axis=2)
    r = amax / np.exp2(e)
    assert ((r >= 4) & (r < 8)).all()                               # largest magnitude lands in [4, 8)
    q = oracle.unpack_nibbles(codes).astype(np.int64) & 0xF
    vals = np.vectorize(table.get)(q) * np.repeat(np.exp2(e), 32, axis=1)
    v = y / np.repeat(np.exp2(e), 32, axis=1)
    grid = np.array(sorted(set(abs(t) for t in table.values())))
    # nearest grid point (saturating at 6): |v - q| <= half the local spacing
    idx = np.clip(np.searchsorted(grid, np.abs(v)), 1, len(grid) - 1)
    half = (grid[idx] - grid[idx - 1]) / 2
    err = np.abs(np.abs(v) - np.abs(vals / np.repeat(np.exp2(e), 32, axis=1)))
    assert ((err <= half + 1e-12) | (np.abs(v) >= 6)).all()
    assert np.array_equal(np.sign(vals)[vals != 0], np.sign(y)[vals != 0])
    # conditioning on the quantizer's own scales reproduces its codes
    assert np.array_equal(oracle.mxfp4_codes_given_scales(y, scales) & 0xF, q)


def test_mxfp4_zero_block_and_single_spike(golden_dir):
    D = 128
    table = e2m1_golden(golden_dir)
    codes, scales, _, bad = oracle.quantize_mxfp4(np.zeros((2, D), np.uint16), np.ones(D, np.float32),
                                                  np.ones(D, np.int8))
    assert bad == 0 and (codes == 0).all() and (scales == 0).all()     # e = -127 for an all-zero block
    H = scipy.linalg.hadamard(D)
    for a, k in ((1.5, 3), (-2.0, D - 1)):
        x = np.zeros((1, D))
        x[0, k] = a
        codes, scales, _, _ = oracle.quantize_mxfp4(f16bits(x), np.ones(D, np.float32), np.ones(D, np.int8))
        m = abs(a) / np.sqrt(D)
        e = int(np.floor(np.log2(m))) - 2
        assert (scales == e + 127).all()
        v = m / 2.0 ** e                                              # in [4, 8)
        want_mag = 4.0 if v <= 5.0 else 6.0                           # ties at 5 go to 4 (even)
        q = oracle.unpack_nibbles(codes)[0].astype(np.int64) & 0xF
        got = np.array([table[c] for c in q])
        assert np.array_equal(got, want_mag * np.sign(a) * H[:, k])


def test_mxfp4_dequant_single_code_closed_form():
    D = 64
    lam = rand_lambda(1, D)[0]
    s = rand_signs(D)
    H = scipy.linalg.hadamard(D)
    for k, c, sb in ((0, 0x7, 120), (17, 0xB, 130), (63, 0x1, 127)):
        q = np.zeros((1, D), np.int8)
        q[0, k] = c if c < 8 else c - 16
        scales = np.full((1, D // 32), 127, np.uint8)
        scales[0, k // 32] = sb
        x64, x16 = oracle.dequantize_mxfp4(oracle.pack_nibbles(q), scales, lam, s)
        val = {0x7: 6.0, 0xB: -1.5, 0x1: 0.5}[c] * 2.0 ** (sb - 127)
        want = (s / lam.astype(np.float64)) * val * H[k, :] / np.sqrt(D)
        assert np.allclose(x64[0], want, rtol=1e-14, atol=0)
