"""GPU parity of the block-scaled E2M1 (MXFP4) variant of the fused
quantizer -- same rotation, 32-coordinate blocks with E8M0 power-of-two
scales, E2M1 elements via the gfx950 FP4 conversions -- against the fp64
oracle, through the C ABI via the binding: model-shaped caches, every head
dim in both work-item layouts, tiny and zero blocks, ragged and strided
views, and the full-size Qwen3-8B-shaped K cache (sampled)."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import synth
from tests import parity
from tests.gpu_util import all_idx, device, lam_rows, log, rows

pytestmark = pytest.mark.gpu


def run_mx(x, lam, s):
    codes, scales = kvq.quantize_mxfp4(x, lam, s)
    out = kvq.dequantize_mxfp4(codes, scales, lam, s)
    torch.cuda.synchronize()
    return codes, scales, out


def check(x, lam, s, codes, scales, out, idx, what):
    rep = parity.mxfp4_parity(rows(x, idx), lam_rows(lam, idx), s.cpu().numpy(), rows(codes, idx),
                              rows(scales, idx), rows(out, idx))
    log(what, parity.summary(rep))
    return rep


def full(x, lam, s, what):
    L, T, H, D = x.shape
    codes, scales, out = run_mx(x, lam, s)
    return check(x, lam, s, codes, scales, out, all_idx(L, T, H), what)


def test_model_shaped_caches():
    dev = device()
    for name, T in (("qwen2.5-1.5b", None), ("gemma-3-1b", 1024)):
        cfg = synth.config(name, T=T) if T else synth.config(name)
        inp = synth.make_inputs(cfg, dev)
        for t in ("K", "V"):
            full(inp[t], inp["lam_" + t], inp["signs"], "mxfp4 %s %s" % (name, t))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("H", [2, 3])
def test_every_head_dim(D, H):
    g = torch.Generator(device="cpu").manual_seed(D + H)
    dev = device()
    x = (torch.randn((2, 37, H, D), generator=g) * torch.exp(2 * torch.randn((2, 1, H, D), generator=g))).to(
        torch.float16).to(dev)
    lam = torch.exp(0.3 * torch.randn((2, H, D), generator=g)).to(torch.float32).to(dev)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    full(x, lam, s, "mxfp4 D=%d H=%d" % (D, H))


def test_zero_tiny_and_huge_blocks():
    dev = device()
    L, T, H, D = 1, 16, 4, 128
    g = torch.Generator(device="cpu").manual_seed(3)
    x = torch.randn((L, T, H, D), generator=g)
    x[0, 0] = 0.0                                           # all-zero vectors: E8M0 byte 0, codes 0
    x[0, 1] = torch.randn((H, D), generator=g) * 1e-6       # fp16 subnormal-range inputs
    x[0, 2] = torch.randn((H, D), generator=g) * 3e3        # large values
    x[0, 3, :, :] = 0.0
    x[0, 3, :, 5] = -1.0                                    # one non-zero coordinate
    x = x.to(torch.float16).to(dev)
    lam = torch.ones((L, H, D), dtype=torch.float32, device=dev)
    s = torch.ones((D,), dtype=torch.int8, device=dev)
    full(x, lam, s, "mxfp4 degenerate")


def test_ragged_and_strided():
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(5)
    L, T, H, D = 2, 45, 3, 128
    x = torch.randn((L, T, H, D), generator=g).to(torch.float16).to(dev)
    lam = torch.exp(0.3 * torch.randn((L, H, D), generator=g)).to(torch.float32).to(dev)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)
    cbuf = torch.full((L, T + 2, H, D // 2 + 32), 0x5A, dtype=torch.uint8, device=dev)
    sbuf = torch.full((L, T + 2, H, D // 32 + 3), 0xA5, dtype=torch.uint8, device=dev)
    codes, scales = cbuf[:, 1:T + 1, :, 16:16 + D // 2], sbuf[:, 1:T + 1, :, 1:1 + D // 32]
    kvq.quantize_mxfp4(x, lam, s, codes=codes, scales=scales)
    out = kvq.dequantize_mxfp4(codes, scales, lam, s)
    torch.cuda.synchronize()
    check(x, lam, s, codes, scales, out, all_idx(L, T, H), "mxfp4 strided ragged")
    assert (cbuf[:, 0] == 0x5A).all() and (cbuf[:, T + 1] == 0x5A).all()
    assert (cbuf[..., :16] == 0x5A).all() and (cbuf[..., 16 + D // 2:] == 0x5A).all()
    assert (sbuf[..., 0] == 0xA5).all() and (sbuf[..., 1 + D // 32:] == 0xA5).all()


def test_qwen3_8b_full_size_sampled():
    """The Qwen3-8B-shaped K cache at full size through the MXFP4 kernels, in
    the benchmark's launch configuration; parity on 24,576 sampled vectors."""
    dev = device()
    cfg = synth.config("qwen3-8b")
    inp = synth.make_inputs(cfg, dev, want_v=False)
    x, lam, s = inp["K"], inp["lam_K"], inp["signs"]
    codes, scales, out = run_mx(x, lam, s)
    idx = synth.sample_rows(cfg.L, cfg.T, cfg.H, 24576, 999).numpy()
    check(x, lam, s, codes, scales, out, idx, "mxfp4 qwen3-8b full-size K")
