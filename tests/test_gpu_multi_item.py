"""GPU parity of the quantize / dequantize kernels of every format (int4,
int8, MXFP4, SRFT) at shapes where each wavefront runs several consecutive
work items, so that the paths a one-item wavefront never takes are covered:
a run that crosses a lambda key (a layer for token-major items, a (layer,
head) for head-major ones) and reloads the multipliers mid-run, the
prefetch of the next item and the deferred stores of the loops without it
(token-major head_dim 256 dequantize, head_dim-256 SRFT), a partial last
item, and a ragged last wavefront.

Each case is checked two ways, through the C ABI via the binding:
  * against the fp64 oracle (contract in tests/parity.py) on every vector of
    every wavefront that holds a key boundary, the first and last
    wavefronts, and a seeded sample elsewhere;
  * on every vector, bit for bit, against calls over chunks of one layer's
    tokens small enough (at most 2048 items) to run one item per wavefront
    (the decomposition most other parity tests cover), which compute each
    vector with the same arithmetic.
Outputs are written into views of token-padded, sentinel-filled buffers, and
the padding must come back untouched."""
import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import synth
from tests import parity
from tests.gpu_util import device, lam_rows, log, rows

pytestmark = pytest.mark.gpu

PAD = 8                       # sentinel token rows after each layer's outputs

# (L, T, H, D, G): token-major and head-major items, every head dim, odd item
# counts per key (a wavefront straddles each key boundary), T not a multiple
# of the tokens per item (partial last item)
SHAPES = [
    (5, 80001, 2, 128, 32),   # token-major, 3 items per wavefront, ragged last wavefront
    (3, 65541, 3, 128, 16),   # head-major, 2 per wavefront, ragged last wavefront
    (3, 200003, 1, 256, 64),  # head_dim 256, one head (head-major items), ragged last wavefront
    (2, 87400, 3, 256, 32),   # head-major head_dim 256
    (2, 90001, 2, 256, 64),   # token-major head_dim 256 (dequantize without prefetch)
    (2, 70001, 4, 64, 8),     # head_dim 64, 4 tokens per item
]


def _fmt(name, G):
    """(quantize, dequantize, parity, code row bytes, scale row, scale dtype)."""
    if name == "int4":
        return (lambda x, l, s, c, sc: kvq.quantize(x, l, s, G, codes=c, scales=sc),
                lambda c, sc, l, s, o: kvq.dequantize(c, sc, l, s, G, out=o),
                lambda *a: parity.int4_parity(*a[:3], G, *a[3:]), 2, G, torch.float16, torch.uint8)
    if name == "srft":
        return (lambda x, l, s, c, sc: kvq.quantize_srft(x, l, s, G, codes=c, scales=sc),
                lambda c, sc, l, s, o: kvq.dequantize_srft(c, sc, l, s, G, out=o),
                lambda *a: parity.int4_parity(*a[:3], G, *a[3:], fourier=True), 2, G, torch.float16, torch.uint8)
    if name == "int8":
        return (lambda x, l, s, c, sc: kvq.quantize_int8(x, l, s, G, codes=c, scales=sc),
                lambda c, sc, l, s, o: kvq.dequantize_int8(c, sc, l, s, G, out=o),
                lambda *a: parity.int8_parity(*a[:3], G, *a[3:]), 1, G, torch.float16, torch.int8)
    if name == "mxfp4":
        return (lambda x, l, s, c, sc: kvq.quantize_mxfp4(x, l, s, codes=c, scales=sc),
                lambda c, sc, l, s, o: kvq.dequantize_mxfp4(c, sc, l, s, out=o),
                lambda *a: parity.mxfp4_parity(*a), 2, 32, torch.uint8, torch.uint8)
    raise KeyError(name)


def _geometry(L, T, H, D, inverse, fourier):
    tm, n_items, ipw = kvq.item_plan(L, T, H, D, inverse=inverse, fourier=fourier)
    tpi = 16 // H if tm else 16
    ipg = math.ceil(T / tpi)                   # items per lambda key
    assert n_items == (L if tm else L * H) * ipg
    return tm, n_items, ipw, tpi, ipg


def _item_rows(item, tm, tpi, ipg, T, H):
    key, k = divmod(item, ipg)
    t0 = k * tpi
    if tm:
        return [(key, t, h) for t in range(t0, min(t0 + tpi, T)) for h in range(H)]
    l, h = divmod(key, H)
    return [(l, t, h) for t in range(t0, min(t0 + 16, T))]


def boundary_rows(L, T, H, D, seed, fourier=False, n_sample=1024):
    """Every vector of the wavefronts that hold a key boundary, of the first
    and the last wavefront, in the quantize and in the dequantize plan (their
    runs differ), plus a seeded sample; and, per plan, the facts the shape
    was chosen for."""
    out, facts = [], {}
    for inverse in (False, True):
        tm, n_items, ipw, tpi, ipg = _geometry(L, T, H, D, inverse, fourier)
        n_waves = math.ceil(n_items / ipw)
        waves = {0, n_waves - 1}
        straddling = 0
        for b in range(ipg, n_items, ipg):         # first item of each key after the first
            w0, w1 = (b - 1) // ipw, b // ipw
            waves.update((w0, w1))
            straddling += w0 == w1
        for w in sorted(waves):
            for item in range(w * ipw, min((w + 1) * ipw, n_items)):
                out.extend(_item_rows(item, tm, tpi, ipg, T, H))
        facts["dequantize" if inverse else "quantize"] = {
            "token_major": tm, "items_per_wave": ipw, "straddling_waves": straddling,
            "partial_last_item": T % tpi != 0, "ragged_last_wave": n_items % ipw != 0}
    smp = synth.sample_rows(L, T, H, n_sample, seed).numpy()
    idx = np.unique(np.concatenate([np.array(out, dtype=np.int64), smp]), axis=0)
    return idx, facts


def _padded(L, T, H, row, dtype, fill, dev):
    buf = torch.empty((L, T + PAD, H, row), dtype=dtype, device=dev)
    if dtype == torch.float16:
        buf.view(torch.int16).fill_(fill)
    else:
        buf.view(torch.uint8).fill_(fill & 0xFF)
    return buf, buf[:, :T]


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4", "srft"])
@pytest.mark.parametrize("L,T,H,D,G", SHAPES)
def test_multi_item_wavefronts(fmt, L, T, H, D, G):
    dev = device()
    quant, dequant, check, cdiv, sgrp, sdt, cdt = _fmt(fmt, G)
    seed = L * 7919 + T + H * 31 + D + G
    log("multi-item %s shape=%s G=%d" % (fmt, (L, T, H, D), G))
    x = synth.draw(L, T, H, D, synth.Dist("normal", lognormal_channels=True), seed, seed + 1, dev)
    g = torch.Generator(device="cpu").manual_seed(seed + 2)
    lam = torch.exp(0.3 * torch.randn((L, H, D), generator=g)).to(torch.float32).to(dev)
    s = (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.int8).to(dev)

    idx, facts = boundary_rows(L, T, H, D, seed + 3, fourier=fmt == "srft")
    for f in facts.values():
        assert f["items_per_wave"] > 1 and f["straddling_waves"] > 0 and f["partial_last_item"], facts
    assert any(f["ragged_last_wave"] for f in facts.values()), facts
    tm = facts["quantize"]["token_major"]
    chunk = 2048 * (16 // H) if tm else 16 * (2048 // H)      # tokens per one-item-per-wave call
    for inverse in (False, True):
        assert kvq.item_plan(1, chunk, H, D, inverse=inverse, fourier=fmt == "srft")[2] == 1

    sfill = 0x7BFF if sdt == torch.float16 else 0xA5
    cbuf, codes = _padded(L, T, H, D // cdiv, cdt, 0x5A, dev)
    sbuf, scales = _padded(L, T, H, D // sgrp, sdt, sfill, dev)
    obuf, out = _padded(L, T, H, D, torch.float16, 0x7C01, dev)
    quant(x, lam, s, codes, scales)
    dequant(codes, scales, lam, s, out)
    torch.cuda.synchronize()

    for buf, fill in ((cbuf, 0x5A), (sbuf, sfill), (obuf, 0x7C01)):
        want, _ = _padded(L, 0, H, buf.shape[-1], buf.dtype, fill, dev)
        assert torch.equal(buf[:, T:].contiguous().view(torch.uint8), want.view(torch.uint8)), "padding overwritten"

    # oracle on the boundary wavefronts and the sample
    rep = check(rows(x, idx), lam_rows(lam, idx), s.cpu().numpy(), rows(codes, idx), rows(scales, idx),
                rows(out, idx))
    log("multi-item %s %s: %d rows %s; %s" % (fmt, (L, T, H, D, G), len(idx), facts, parity.summary(rep)))

    # every vector against token-chunked calls of one layer (one item per wavefront)
    c1 = torch.empty((1, chunk) + tuple(codes.shape[2:]), dtype=codes.dtype, device=dev)
    s1 = torch.empty((1, chunk) + tuple(scales.shape[2:]), dtype=scales.dtype, device=dev)
    o1 = torch.empty((1, chunk, H, D), dtype=torch.float16, device=dev)
    for l in range(L):
        lam1 = lam[l:l + 1].contiguous()
        for t0 in range(0, T, chunk):
            n = min(chunk, T - t0)
            quant(x[l:l + 1, t0:t0 + n], lam1, s, c1[:, :n], s1[:, :n])
            dequant(c1[:, :n], s1[:, :n], lam1, s, o1[:, :n])
            torch.cuda.synchronize()
            for a, b, what in ((codes[l:l + 1, t0:t0 + n], c1[:, :n], "codes"),
                               (scales[l:l + 1, t0:t0 + n], s1[:, :n], "scales"),
                               (out[l:l + 1, t0:t0 + n], o1[:, :n], "dequantized")):
                av = a.contiguous().view(torch.uint8)
                bv = b.contiguous().view(torch.uint8)
                if not torch.equal(av, bv):
                    bad = (av != bv).nonzero()[:5].tolist()
                    raise AssertionError("%s of layer %d, tokens %d.. differ from the one-item-per-wave run at %s"
                                         % (what, l, t0, bad))
