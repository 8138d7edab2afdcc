"""GPU parity of the SRFT variant of the fused int4 quantizer and its mirror
(real-packed unitary DFT as the rotation: D/2-point radix-2 FFT in registers
and DPP, Hermitian unpacking) against the fp64 oracle, through the C ABI via
the binding, under the same contract as the Walsh-Hadamard path: model-shaped
caches, every (head dim, group) pair in both work-item layouts, ragged,
degenerate and strided inputs, and the full-size Qwen3-8B-shaped K cache
(sampled)."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import oracle
import synth
from tests import parity
from tests.gpu_util import all_idx, bits, device, lam_rows, log, rows

pytestmark = pytest.mark.gpu


def run_srft(x, lam, s, G):
    codes, scales = kvq.quantize_srft(x, lam, s, G)
    out = kvq.dequantize_srft(codes, scales, lam, s, G)
    torch.cuda.synchronize()
    return codes, scales, out


def check(x, lam, s, G, codes, scales, out, idx, what):
    rep = parity.int4_parity(rows(x, idx), lam_rows(lam, idx), s.cpu().numpy(), G, rows(codes, idx),
                             rows(scales, idx), rows(out, idx), fourier=True)
    log(what, parity.summary(rep))
    return rep


def full(x, lam, s, G, what):
    L, T, H, D = x.shape
    codes, scales, out = run_srft(x, lam, s, G)
    return check(x, lam, s, G, codes, scales, out, all_idx(L, T, H), what)


def test_model_shaped_caches():
    dev = device()
    for name, T in (("tiny", None), ("qwen2.5-1.5b", None), ("gemma-3-1b", 1024)):
        cfg = synth.config(name, T=T) if T else synth.config(name)
        inp = synth.make_inputs(cfg, dev)
        for t in ("K", "V"):
            if t in inp:
                full(inp[t], inp["lam_" + t], inp["signs"], 32 if name == "tiny" else cfg.G,
                     "srft %s %s" % (name, t))


@pytest.mark.parametrize("D,G", [(64, 8), (64, 16), (64, 64), (128, 8), (128, 16), (128, 32), (128, 128),
                                 (256, 32), (256, 64), (256, 256)])
@pytest.mark.parametrize("H", [2, 3])
def test_every_shape(D, G, H):
    g = torch.Generator(device="cpu").manual_seed(D * 5 + G + H)
    dev = device()
    x = (torch.randn((2, 37, H, D), generator=g) * torch.exp(torch.randn((2, 1, H, D), generator=g))).to(
        torch.float16).to(dev)
    lam = torch.exp(0.3 * torch.randn((2, H, D), generator=g)).to(torch.float32).to(dev)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    full(x, lam, s, G, "srft D=%d G=%d H=%d" % (D, G, H))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_pure_tones_and_degenerate_vectors(D):
    """Impulses, pure cosines and sines at several frequencies (all the
    spectrum in one packed pair), the Nyquist alternation, zero and constant
    vectors, with lambda = 1 and s = 1 so that the rotated values are known in
    closed form; checked under the same contract.  One group per vector: the
    coordinates that are exactly zero in fp64 come out of an fp32 FFT as
    rounding noise, which in a group of their own would set a tiny non-zero
    scale where the exact one is zero."""
    dev = device()
    j = np.arange(D)
    vecs = [np.zeros(D), np.ones(D), (-1.0) ** j]
    for k in (1, 3, D // 4, D // 2 - 1):
        vecs.append(np.cos(2 * np.pi * k * j / D) * 4)
        vecs.append(np.sin(2 * np.pi * k * j / D) * 4)
    for p in (0, 1, D // 2, D - 1):
        e = np.zeros(D)
        e[p] = 3.0
        vecs.append(e)
    X = np.stack(vecs)
    n = len(X)
    x = torch.from_numpy(X.reshape(1, n, 1, D)).to(torch.float16).to(dev)
    lam = torch.ones((1, 1, D), dtype=torch.float32, device=dev)
    s = torch.ones((D,), dtype=torch.int8, device=dev)
    full(x, lam, s, D, "srft tones D=%d" % D)


def test_ragged_empty_and_strided():
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(7)
    L, T, H, D, G = 2, 45, 4, 128, 32
    x = torch.randn((L, T, H, D), generator=g).to(torch.float16).to(dev)
    lam = torch.exp(0.3 * torch.randn((L, H, D), generator=g)).to(torch.float32).to(dev)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    cbuf = torch.full((L, T + 2, H, D // 2 + 32), 0x5A, dtype=torch.uint8, device=dev)
    sbuf = torch.full((L, T + 2, H, D // G + 2), 7.0, dtype=torch.float16, device=dev)
    codes, scales = cbuf[:, 1:T + 1, :, 16:16 + D // 2], sbuf[:, 1:T + 1, :, 1:1 + D // G]
    kvq.quantize_srft(x, lam, s, G, codes=codes, scales=scales)
    out = kvq.dequantize_srft(codes, scales, lam, s, G)
    torch.cuda.synchronize()
    check(x, lam, s, G, codes, scales, out, all_idx(L, T, H), "srft strided ragged")
    assert (cbuf[:, 0] == 0x5A).all() and (cbuf[:, T + 1] == 0x5A).all()
    assert (cbuf[..., :16] == 0x5A).all() and (cbuf[..., 16 + D // 2:] == 0x5A).all()
    assert (sbuf[..., 0] == 7.0).all() and (sbuf[..., 1 + D // G:] == 7.0).all()
    e = torch.zeros((L, 0, H, D), dtype=torch.float16, device=dev)
    c0, s0 = kvq.quantize_srft(e, lam, s, G)
    assert c0.numel() == 0 and s0.numel() == 0


def test_srft_and_hadamard_differ_but_both_roundtrip():
    """The two rotations give different codes for the same input, and each
    dequantizer undoes only its own quantizer (a mix-up between the two
    paths would pass neither)."""
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(8)
    x = torch.randn((1, 64, 2, 128), generator=g).to(torch.float16).to(dev)
    lam = torch.ones((1, 2, 128), dtype=torch.float32, device=dev)
    s = (torch.randint(0, 2, (128,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    cf, sf = kvq.quantize_srft(x, lam, s, 32)
    ch, sh = kvq.quantize(x, lam, s, 32)
    of = kvq.dequantize_srft(cf, sf, lam, s, 32)
    oh = kvq.dequantize(ch, sh, lam, s, 32)
    cross = kvq.dequantize(cf, sf, lam, s, 32)
    torch.cuda.synchronize()
    assert not torch.equal(cf, ch)
    xf = x.float()
    ef, eh, ex = ((o.float() - xf).norm() / xf.norm() for o in (of, oh, cross))
    log("srft vs hadamard relative errors", float(ef), float(eh), float(ex))
    assert ef < 0.2 and eh < 0.2 and ex > 0.5


def test_qwen3_8b_full_size_sampled():
    """The Qwen3-8B-shaped K cache at full size through the SRFT kernels;
    parity on 24,576 sampled vectors."""
    dev = device()
    cfg = synth.config("qwen3-8b")
    inp = synth.make_inputs(cfg, dev, want_v=False)
    x, lam, s = inp["K"], inp["lam_K"], inp["signs"]
    codes, scales, out = run_srft(x, lam, s, cfg.G)
    idx = synth.sample_rows(cfg.L, cfg.T, cfg.H, 24576, 777).numpy()
    check(x, lam, s, cfg.G, codes, scales, out, idx, "srft qwen3-8b full-size K")
