"""GPU parity of the decode-attention kernels (rotated-domain attention
straight from the int4 cache) against the fp64 oracle, through the C ABI via
the binding.  The caches are written by the GPU quantizer; the oracle then
attends over the exact dequantization of those same codes and scales.

Tolerance, per output element c of query head j: |out - out64| <=
2e-3 / lambda_V[c] + 2^-11 |out64|.  The output is a convex combination of
dequantized value rows, so the dequantizer's bound carries over: 2e-3 in the
lambda-normalised unit-variance domain for fp32 arithmetic (scores, exp2,
accumulation over the context), plus half an fp16 ulp for the final
rounding."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import oracle
import synth
from tests.gpu_util import bits, device, log

pytestmark = pytest.mark.gpu

ATOL = 2e-3
RTOL = 2.0 ** -11


def make_cache(L, T, H, D, G, seed, dev, spread=0.5):
    g = torch.Generator(device="cpu").manual_seed(seed)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    out = {"s": s}
    for name in "kv":
        x = torch.randn((L, T, H, D), generator=g) * torch.exp(spread * torch.randn((L, 1, H, D), generator=g))
        lam = torch.exp(0.3 * torch.randn((L, H, D), generator=g)).to(torch.float32)
        x = x.to(torch.float16).to(dev)
        lam = lam.contiguous().to(dev)
        codes, scales = kvq.quantize(x, lam, s, G)
        out[name] = (codes, scales, lam)
    return out


def compare(out, out64, lam_v, H, R, what, unit=1.0):
    """out [L, H*R, D] fp16 (GPU), out64 [L, H*R, D], lam_v [L, H, D].  unit:
    the RMS of the lambda-scaled values when it is not about 1."""
    g = bits(out).view(np.float16).astype(np.float64)
    lam = np.repeat(lam_v.cpu().numpy().astype(np.float64), R, axis=1)       # [L, H*R, D]
    tol = ATOL * unit / lam + RTOL * np.abs(out64)
    err = np.abs(g - out64)
    bad = ~(err <= tol)
    rep = {"n": int(g.size), "bad": int(bad.sum()), "max_err_over_tol": float((err / tol).max()),
           "max_abs_norm": float((err * lam).max())}
    log(what, rep)
    if rep["bad"]:
        i = np.argwhere(bad)[:5]
        raise AssertionError("%s: %s; first bad %s gpu=%s ora=%s" % (
            what, rep, i.tolist(), g[tuple(i.T)], out64[tuple(i.T)]))
    return rep


def run_case(L, T, H, R, D, G, seed, lengths=None, qscale=1.0, scale=None):
    dev = device()
    c = make_cache(L, T, H, D, G, seed, dev)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    q = (torch.randn((L, H * R, D), generator=g) * qscale).to(torch.float16).to(dev)
    scale = (1.0 / D ** 0.5) if scale is None else scale
    kc, ks, lk = c["k"]
    vc, vs, lv = c["v"]
    ln = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device=dev)
    out = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, c["s"], G, softmax_scale=scale, lengths=ln)
    torch.cuda.synchronize()
    out64 = oracle.attend_decode(bits(q), kc.cpu().numpy(), bits(ks), vc.cpu().numpy(), bits(vs),
                                 lk.cpu().numpy(), lv.cpu().numpy(), c["s"].cpu().numpy(), G, scale,
                                 None if lengths is None else np.asarray(lengths, np.int32))
    return compare(out, out64, lv, H, R, "attend L=%d T=%d H=%d R=%d D=%d G=%d" % (L, T, H, R, D, G))


@pytest.mark.parametrize("D,G", [(64, 16), (128, 32), (128, 8), (256, 64), (128, 128)])
@pytest.mark.parametrize("R", [1, 2, 4])
def test_attend_small(D, G, R):
    run_case(2, 300, 2, R, D, G, seed=D + G + R)


@pytest.mark.parametrize("R", [3, 6, 8])
def test_attend_query_groups_over_passes(R):
    # R > 4 runs in passes of four query heads; R = 3 leaves one lane quad idle
    run_case(2, 257, 3, R, 128, 32, seed=40 + R)


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("H", [1, 4, 6, 8, 12, 16])
def test_attend_head_groups(H, D):
    # matrix-core blocks (head_dim 128 / group 32, head_dim 256 / group 64)
    # hold hb = 8, 4, 2 or 1 KV heads (the largest dividing H) times 8 / hb
    # token sub-ranges
    run_case(2, 333, H, 4, D, D // 4, seed=60 + H + D, lengths=[333, 97])


@pytest.mark.parametrize("R", [3, 8])
def test_attend_head_dim_256_query_passes(R):
    run_case(2, 257, 2, R, 256, 64, seed=80 + R)


def test_attend_ragged_lengths_and_empty():
    run_case(5, 200, 2, 4, 128, 32, seed=50, lengths=[200, 0, 1, 77, 13])


def test_attend_one_token_and_tiny_context():
    run_case(1, 1, 1, 4, 128, 32, seed=51)
    run_case(1, 7, 2, 2, 64, 16, seed=52)


def test_attend_long_context_many_splits():
    # one outer index and few heads: the context is split across many blocks
    run_case(1, 20000, 2, 4, 128, 32, seed=53)


def test_attend_peaked_scores():
    # large logits: the online softmax rescales often and the weights are
    # dominated by a few tokens
    run_case(2, 500, 2, 4, 128, 32, seed=54, qscale=8.0)


def test_attend_zero_query_averages_values():
    dev = device()
    L, T, H, R, D, G = 1, 64, 2, 4, 128, 32
    c = make_cache(L, T, H, D, G, 55, dev)
    q = torch.zeros((L, H * R, D), dtype=torch.float16, device=dev)
    kc, ks, lk = c["k"]
    vc, vs, lv = c["v"]
    out = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, c["s"], G)
    vhat = kvq.dequantize(vc, vs, lv, c["s"], G).to(torch.float64).mean(dim=1)          # [L, H, D]
    torch.cuda.synchronize()
    want = vhat.repeat_interleave(R, dim=1).cpu().numpy()
    # the fp16 dequantization adds up to half an fp16 ulp per row
    compare(out, want, lv, H, R, "zero query")


def test_attend_workspace_reuse_and_strided_cache():
    dev = device()
    L, T, H, R, D, G = 2, 120, 2, 4, 128, 32
    c = make_cache(L, T, H, D, G, 56, dev)
    kc, ks, lk = c["k"]
    vc, vs, lv = c["v"]
    # cache stored inside larger buffers (strided views)
    kbuf = torch.full((L, T + 5, H, D // 2 + 32), 0x77, dtype=torch.uint8, device=dev)
    kbuf[:, 2:2 + T, :, 16:16 + D // 2] = kc
    kcv = kbuf[:, 2:2 + T, :, 16:16 + D // 2]
    g = torch.Generator(device="cpu").manual_seed(57)
    q = torch.randn((L, H * R, D), generator=g).to(torch.float16).to(dev)
    ws = torch.full((kvq.attend_decode_workspace_bytes(L, T, H, D, R) + 64,), 0xFF, dtype=torch.uint8,
                    device=dev)
    o1 = kvq.attend_decode(q, kcv, ks, vc, vs, lk, lv, c["s"], G, workspace=ws)
    o2 = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, c["s"], G, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    out64 = oracle.attend_decode(bits(q), kc.cpu().numpy(), bits(ks), vc.cpu().numpy(), bits(vs),
                                 lk.cpu().numpy(), lv.cpu().numpy(), c["s"].cpu().numpy(), G, 1.0 / D ** 0.5)
    compare(o1, out64, lv, H, R, "strided cache")


def test_qwen3_8b_decode_step_full_size_sampled():
    """The decode-attention workload at full size, in the benchmark's launch
    configuration: the [36, 262144, 8, 128] K and V caches (written by the
    quantizer) read as 36 layers x 8 sequences of 32,768 tokens, 32 query
    heads per sequence (4 per KV head).  Parity on three seeded
    (sequence, KV head) pairs."""
    dev = device()
    cfg = synth.config("qwen3-8b")
    inp = synth.make_inputs(cfg, dev)
    caches = {}
    for name in ("K", "V"):
        codes, scales = kvq.quantize(inp[name], inp["lam_" + name], inp["signs"], cfg.G)
        del inp[name]
        torch.cuda.empty_cache()
        caches[name] = (codes, scales)
    B, Tq, R = 8, cfg.T // 8, 4
    L = cfg.L * B
    kc, ks = (t.view(L, Tq, cfg.H, -1) for t in caches["K"])
    vc, vs = (t.view(L, Tq, cfg.H, -1) for t in caches["V"])
    lk = inp["lam_K"].repeat_interleave(B, dim=0).contiguous()
    lv = inp["lam_V"].repeat_interleave(B, dim=0).contiguous()
    s = inp["signs"]
    g = torch.Generator(device="cpu").manual_seed(4321)
    q = torch.randn((L, cfg.H * R, cfg.D), generator=g).to(torch.float16).to(dev)
    out = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, s, cfg.G)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    for o, h in zip(rng.integers(0, L, 3), rng.integers(0, cfg.H, 3)):
        o, h = int(o), int(h)
        out64 = oracle.attend_decode(bits(q[o:o + 1, h * R:(h + 1) * R]),
                                     kc[o:o + 1, :, h:h + 1].cpu().numpy(), bits(ks[o:o + 1, :, h:h + 1]),
                                     vc[o:o + 1, :, h:h + 1].cpu().numpy(), bits(vs[o:o + 1, :, h:h + 1]),
                                     lk[o:o + 1, h:h + 1].cpu().numpy(), lv[o:o + 1, h:h + 1].cpu().numpy(),
                                     s.cpu().numpy(), cfg.G, 1.0 / cfg.D ** 0.5)
        compare(out[o:o + 1, h * R:(h + 1) * R], out64, lv[o:o + 1, h:h + 1], 1, R,
                "qwen3-8b decode step (outer %d, head %d)" % (o, h))


@pytest.mark.parametrize("stride_mb", [60, 70])
def test_attend_huge_token_stride(stride_mb):
    """K codes stored with a token stride of tens of MB: 60 MB keeps 32 token
    rows under 2^31 bytes (matrix-core kernel, 32-bit per-lane offsets near
    their limit); 70 MB goes past it, and the host must pick the VALU kernel.
    Both agree with the oracle."""
    dev = device()
    L, T, H, R, D, G = 1, 40, 1, 4, 128, 32
    c = make_cache(L, T, H, D, G, 60 + stride_mb, dev)
    kc, ks, lk = c["k"]
    vc, vs, lv = c["v"]
    st = stride_mb << 20
    buf = torch.zeros(T * st, dtype=torch.uint8, device=dev)
    big = buf.as_strided((L, T, H, D // 2), (T * st, st, D // 2, 1))
    big.copy_(kc)
    g = torch.Generator(device="cpu").manual_seed(stride_mb)
    q = torch.randn((L, H * R, D), generator=g).to(torch.float16).to(dev)
    out = kvq.attend_decode(q, big, ks, vc, vs, lk, lv, c["s"], G)
    ref = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, c["s"], G)
    torch.cuda.synchronize()
    out64 = oracle.attend_decode(bits(q), kc.cpu().numpy(), bits(ks), vc.cpu().numpy(), bits(vs),
                                 lk.cpu().numpy(), lv.cpu().numpy(), c["s"].cpu().numpy(), G, 1.0 / D ** 0.5)
    compare(out, out64, lv, H, R, "huge token stride %d MB" % stride_mb)
    if stride_mb == 60:
        assert torch.equal(out, ref)        # same kernel, same arithmetic
    del buf, big
    torch.cuda.empty_cache()


def _cache(x, lam, s, G):
    codes, scales = kvq.quantize(x, lam, s, G)
    return codes, scales


def test_attend_large_value_scales():
    """Values whose lambda-scaled magnitude is in the thousands (value
    scales far above 128): the matrix-core kernel keeps its fp16 value
    operand p * scale finite by moving the softmax reference to each such
    step's maximum (p <= 1).  Tolerance relative to the values' RMS."""
    dev = device()
    L, T, H, R, D, G = 2, 300, 2, 4, 128, 32
    g = torch.Generator(device="cpu").manual_seed(71)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    xk = torch.randn((L, T, H, D), generator=g).to(torch.float16).to(dev)
    xv = (torch.randn((L, T, H, D), generator=g) * 2000.0).to(torch.float16).to(dev)
    lk = torch.ones((L, H, D), dtype=torch.float32, device=dev)
    lv = torch.ones((L, H, D), dtype=torch.float32, device=dev)
    kc, ks = _cache(xk, lk, s, G)
    vc, vs = _cache(xv, lv, s, G)
    assert float(vs.float().max()) > 128.0
    q = (torch.randn((L, H * R, D), generator=g) * 3.0).to(torch.float16).to(dev)
    out = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, s, G)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    out64 = oracle.attend_decode(bits(q), kc.cpu().numpy(), bits(ks), vc.cpu().numpy(), bits(vs),
                                 lk.cpu().numpy(), lv.cpu().numpy(), s.cpu().numpy(), G, 1.0 / D ** 0.5)
    compare(out, out64, lv, H, R, "large value scales", unit=2000.0)


def test_attend_huge_rotated_queries():
    """A tiny key lambda makes the rotated query (q / lambda_K) exceed the
    fp16 range: the matrix-core kernel scales its query operand by a power
    of two and the scores back, exactly."""
    dev = device()
    L, T, H, R, D, G = 2, 300, 2, 4, 128, 32
    g = torch.Generator(device="cpu").manual_seed(72)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    xk = (torch.randn((L, T, H, D), generator=g) * 16.0).to(torch.float16).to(dev)
    xv = torch.randn((L, T, H, D), generator=g).to(torch.float16).to(dev)
    lk = torch.full((L, H, D), 2.0 ** -14, dtype=torch.float32, device=dev)
    lv = torch.ones((L, H, D), dtype=torch.float32, device=dev)
    kc, ks = _cache(xk, lk, s, G)
    vc, vs = _cache(xv, lv, s, G)
    q = (torch.randn((L, H * R, D), generator=g) * 10.0).to(torch.float16).to(dev)
    out = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, s, G)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    out64 = oracle.attend_decode(bits(q), kc.cpu().numpy(), bits(ks), vc.cpu().numpy(), bits(vs),
                                 lk.cpu().numpy(), lv.cpu().numpy(), s.cpu().numpy(), G, 1.0 / D ** 0.5)
    compare(out, out64, lv, H, R, "huge rotated queries")


def test_attend_seeded_shape_sweep():
    """Twenty seeded random shapes (head dims 64/128/256 with every group the
    kernels take, 1-16 KV heads, 1-9 query heads per KV head, short and
    ragged contexts, random lengths including zero) against the oracle: both
    kernel versions, every head-group size and pass count, partial steps."""
    rng = np.random.default_rng(2024)
    for case in range(20):
        D = int(rng.choice([64, 128, 256]))
        G = D // 4 if case % 2 == 0 else int(rng.choice([g for g in (8, 16, 32, 64, 128, 256) if g <= D]))
        H = int(rng.integers(1, 17))
        R = int(rng.integers(1, 10))
        L = int(rng.integers(1, 4))
        T = int(rng.integers(1, 400))
        lengths = [int(rng.integers(0, T + 1)) for _ in range(L)]
        if case % 5 == 0:
            lengths[0] = 0
        log("sweep case %d: L=%d T=%d H=%d R=%d D=%d G=%d lengths=%s" % (case, L, T, H, R, D, G, lengths))
        run_case(L, T, H, R, D, G, seed=900 + case, lengths=lengths)
