"""GPU parity of product VQ with one-byte indices (value codebooks of at most
256 centroids) against the fp64 oracle, through the C ABI via the binding:
every head dim, codebook sizes up to 256, duplicated centroids, strided
views, ragged and empty caches, index clamping, and the VecInfer-shaped value
cache at full size (sampled)."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import oracle
import synth
from tests import parity
from tests.gpu_util import all_idx, bits, device, lam_rows, log, rows
from tests.test_gpu_vq import rand_case

pytestmark = pytest.mark.gpu


def run8(x, lam, s, cb):
    idx = kvq.vq_encode_u8(x, lam, s, cb, 8)
    out = kvq.vq_decode_u8(idx, cb, lam, s, 8)
    torch.cuda.synchronize()
    return idx, out


def check(x, lam, s, cb, idx, out, sel, what):
    L, T, H, D = x.shape
    books = bits(cb).reshape(H, cb.shape[-2], 8)
    rep = parity.vq_parity(rows(x, sel), lam_rows(lam, sel), s.cpu().numpy(), books,
                           sel[:, 2].astype(np.int32), 8, rows(idx, sel), rows(out, sel))
    log(what, parity.summary(rep))
    return rep


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("K", [1, 100, 256])
def test_small_caches(D, K):
    x, lam, s, cb = rand_case(2, 37, 3, D, K, seed=3 * D + K)
    idx, out = run8(x, lam, s, cb)
    assert idx.dtype == torch.uint8
    check(x, lam, s, cb, idx, out, all_idx(2, 37, 3), "u8 D=%d K=%d" % (D, K))


def test_duplicate_centroids_resolve_to_lowest_index():
    x, lam, s, cb = rand_case(1, 48, 2, 128, 256, seed=77, dup=24)
    idx, out = run8(x, lam, s, cb)
    check(x, lam, s, cb, idx, out, all_idx(1, 48, 2), "u8 duplicates")
    assert int(idx.max()) < 24


def test_strided_views_ragged_and_empty():
    dev = device()
    x0, lam, s, cb = rand_case(2, 45, 3, 128, 256, seed=15)
    base = torch.zeros((2, 3, 45, 128), dtype=torch.float16, device=dev)
    base.copy_(x0.permute(0, 2, 1, 3))
    x = base.permute(0, 2, 1, 3)                                                   # head-major storage
    ibuf = torch.full((2, 47, 3, 24), 0xEE, dtype=torch.uint8, device=dev)
    idx = ibuf[:, 1:46, :, 4:20]
    kvq.vq_encode_u8(x, lam, s, cb, 8, idx=idx)
    out = kvq.vq_decode_u8(idx, cb, lam, s, 8)
    torch.cuda.synchronize()
    check(x, lam, s, cb, idx, out, all_idx(2, 45, 3), "u8 strided ragged")
    assert (ibuf[:, 0] == 0xEE).all() and (ibuf[:, 46] == 0xEE).all()
    assert (ibuf[..., :4] == 0xEE).all() and (ibuf[..., 20:] == 0xEE).all()
    e = torch.zeros((2, 0, 3, 128), dtype=torch.float16, device=dev)
    i2 = kvq.vq_encode_u8(e, lam, s, cb, 8)
    o2 = kvq.vq_decode_u8(i2, cb, lam, s, 8)
    torch.cuda.synchronize()
    assert i2.numel() == 0 and o2.numel() == 0


@pytest.mark.parametrize("D", [64, 128, 256])
def test_decode_random_indices_and_clamp(D):
    """Uniform random indices (every byte position), compared with the
    oracle's decode of the same indices; indices >= n_centroids decode as the
    last centroid."""
    K, L, T, H = 200, 2, 51, 3
    x, lam, s, cb = rand_case(L, T, H, D, K, seed=D + 1)
    g = torch.Generator(device="cpu").manual_seed(D)
    idx = torch.randint(0, K, (L, T, H, D // 8), generator=g, dtype=torch.int32).to(torch.uint8).to(x.device)
    out = kvq.vq_decode_u8(idx, cb, lam, s, 8)
    hi = idx.clone()
    hi[..., ::3] = 255
    lo = hi.clone()
    lo[lo >= K] = K - 1
    o_hi = kvq.vq_decode_u8(hi, cb, lam, s, 8)
    o_lo = kvq.vq_decode_u8(lo, cb, lam, s, 8)
    torch.cuda.synchronize()
    assert torch.equal(o_hi, o_lo)
    sel = all_idx(L, T, H)
    x64, _ = oracle.vq_decode(rows(idx, sel).astype(np.uint16), bits(cb).reshape(H, K, 8),
                              sel[:, 2].astype(np.int32), lam_rows(lam, sel), s.cpu().numpy(), 8)
    rep = parity.check_dequant(rows(out, sel), x64, lam_rows(lam, sel))
    log("u8 decode D=%d" % D, {k: v for k, v in rep.items() if k != "bad_mask"})
    assert rep["bad"] == 0


@pytest.mark.parametrize("D", [128, 256])
def test_multi_unit_blocks_ragged(D):
    """Encoder blocks that run several 64-token units, across (layer, head)
    boundaries, with a ragged last unit per (layer, head): [4, 6500, 8, D]
    gives 102 units per (layer, head) (the last one 36 tokens) and more units
    than the launch has blocks.  Checked on every vector of the first and
    last unit of every (layer, head) and a seeded sample elsewhere."""
    L, T, H = 4, 6500, 8
    x, lam, s, cb = rand_case(L, T, H, D, 256, seed=611 + D)
    idx, out = run8(x, lam, s, cb)
    edge = [(l, t, h) for l in range(L) for h in range(H)
            for t in list(range(0, 64)) + list(range(6400, T))]
    smp = synth.sample_rows(L, T, H, 1024, 612 + D).numpy()
    sel = np.unique(np.concatenate([np.array(edge, dtype=np.int64), smp]), axis=0)
    check(x, lam, s, cb, idx, out, sel, "u8 multi-unit D=%d" % D)


def test_vecinfer_values_full_size_sampled():
    """The VecInfer-shaped value cache at full size ([36, 8192, 8, 128],
    per-head 256-centroid fp16 codebooks, one-byte indices), in the
    benchmark's launch configuration; parity on a seeded sample of 2048
    vectors."""
    dev = device()
    cfg = synth.config("vq")
    inp = synth.make_inputs(cfg, dev)
    x, lam, s, cb = inp["V"], inp["lam_V"], inp["signs"], inp["codebook_V"]
    del inp["K"]
    idx, out = run8(x, lam, s, cb)
    sel = synth.sample_rows(cfg.L, cfg.T, cfg.H, 2048, 4343).numpy()
    check(x, lam, s, cb, idx, out, sel, "vecinfer values full-size")
