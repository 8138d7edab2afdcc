"""GPU parity of the product-VQ encode (MFMA nearest-centroid search) and
decode kernels against the fp64 oracle, through the C ABI via the binding:
the VecInfer-shaped key cache at full size (sampled), small caches at every
head dim, non-multiple-of-32 and multi-chunk codebook sizes, per-layer
codebooks, strided views, and codebooks full of exact duplicates (ties must
resolve to the lowest index)."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import oracle
import synth
from tests import parity
from tests.gpu_util import all_idx, bits, device, lam_rows, log, rows

pytestmark = pytest.mark.gpu


def run_vq(x, lam, s, cb, cb_layer_stride=0):
    idx = kvq.vq_encode(x, lam, s, cb, 8, codebook_layer_stride=cb_layer_stride)
    out = kvq.vq_decode(idx, cb, lam, s, 8, codebook_layer_stride=cb_layer_stride)
    torch.cuda.synchronize()
    return idx, out


def check(x, lam, s, cb, idx, out, sel, what, per_layer=False):
    """sel: [n, 3] (l, t, h) rows to check."""
    L, T, H, D = x.shape
    cbb = bits(cb)
    if per_layer:
        books = cbb.reshape(L * H, cbb.shape[-2], 8)
        book = (sel[:, 0] * H + sel[:, 2]).astype(np.int32)
    else:
        books = cbb.reshape(H, cbb.shape[-2], 8)
        book = sel[:, 2].astype(np.int32)
    rep = parity.vq_parity(rows(x, sel), lam_rows(lam, sel), s.cpu().numpy(), books, book, 8,
                           rows(idx, sel), rows(out, sel))
    log(what, parity.summary(rep))
    return rep


def rand_case(L, T, H, D, K, seed, dup=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = (torch.randn((L, T, H, D), generator=g) * torch.exp(0.5 * torch.randn((L, 1, H, D), generator=g)))
    lam = (1.0 / x[:, :16].pow(2).mean(dim=1).sqrt()).to(torch.float32)
    s = (torch.randint(0, 2, (D,), generator=g, dtype=torch.int8) * 2 - 1).to(torch.int8)
    if dup:
        base = torch.randn((H, dup, 8), generator=g)
        cb = base[:, torch.arange(K) % dup]          # centroid k == centroid k % dup
    else:
        cb = torch.randn((H, K, 8), generator=g)
    dev = device()
    return x.to(torch.float16).to(dev), lam.contiguous().to(dev), s.to(dev), cb.to(torch.float16).contiguous().to(dev)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("K", [1, 300, 4096])
def test_small_caches(D, K):
    x, lam, s, cb = rand_case(2, 37, 3, D, K, seed=D + K)
    idx, out = run_vq(x, lam, s, cb)
    L, T, H, _ = x.shape
    check(x, lam, s, cb, idx, out, all_idx(L, T, H), "D=%d K=%d" % (D, K))


def test_multi_chunk_codebook():
    """More centroids than one LDS chunk (4096): the running best must carry
    across chunks."""
    x, lam, s, cb = rand_case(1, 40, 2, 128, 9000, seed=5)
    idx, out = run_vq(x, lam, s, cb)
    check(x, lam, s, cb, idx, out, all_idx(1, 40, 2), "K=9000")
    assert bits(idx).max() >= 4096, "no index from the second LDS chunk was chosen"


@pytest.mark.parametrize("K,dup", [(512, 64), (5000, 1000)])
def test_duplicate_centroids_resolve_to_lowest_index(K, dup):
    """Every centroid has exact copies (centroid k == k mod dup), inside a
    tile, across tiles and across LDS chunks: every nearest-centroid search
    meets exact ties, which must go to the lowest index (< dup)."""
    x, lam, s, cb = rand_case(1, 48, 2, 128, K, seed=K + dup, dup=dup)
    idx, out = run_vq(x, lam, s, cb)
    got = bits(idx)
    assert got.max() < dup, "a tie resolved to a higher duplicate"
    check(x, lam, s, cb, idx, out, all_idx(1, 48, 2), "dup K=%d" % K)


@pytest.mark.parametrize("K,u8", [(33, False), (33, True), (4096 + 33, False), (1, False)])
def test_far_codebook_partial_last_tile(K, u8):
    """Every centroid lies far on the opposite side of every sub-vector
    (rotated keys near +1414 per coordinate, centroids near -70 per
    coordinate), so every score c.y - |c|^2/2 is about -8e5, far below any
    fixed padding score: the rows past the end of the codebook in the
    partial last tile (of the last LDS chunk) must never be chosen, and the
    index must be the oracle's.  lambda = 1, s = 1 and x = 16000 e_0 + small
    noise make every rotated coordinate about 16000 / sqrt(128)."""
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(K + 7 * u8)
    L, T, H, D = 1, 40, 2, 128
    x = torch.randn((L, T, H, D), generator=g) * 20.0
    x[..., 0] = 16000.0
    lam = torch.ones((L, H, D), dtype=torch.float32)
    s = torch.ones(D, dtype=torch.int8)
    cb = -70.0 + 2.0 * torch.randn((H, K, 8), generator=g)
    x, lam, s = x.to(torch.float16).to(dev), lam.to(dev), s.to(dev)
    cb = cb.to(torch.float16).contiguous().to(dev)
    if u8:
        idx = kvq.vq_encode_u8(x, lam, s, cb, 8)
        out = kvq.vq_decode_u8(idx, cb, lam, s, 8)
        torch.cuda.synchronize()
        assert int(idx.max()) < K
        idx = idx.to(torch.int16)
    else:
        idx, out = run_vq(x, lam, s, cb)
        assert int(bits(idx).max()) < K
    check(x, lam, s, cb, idx, out, all_idx(L, T, H), "far codebook K=%d u8=%s" % (K, u8))


def test_per_layer_codebooks_and_strided_views():
    dev = device()
    x0, lam, s, _ = rand_case(3, 21, 2, 128, 64, seed=9)
    g = torch.Generator(device="cpu").manual_seed(10)
    cbl = torch.randn((3, 2, 200, 8), generator=g).to(torch.float16).to(dev)      # [L, H, K, 8]
    base = torch.zeros((3, 2, 21, 128), dtype=torch.float16, device=dev)
    base.copy_(x0.permute(0, 2, 1, 3))
    x = base.permute(0, 2, 1, 3)                                                   # head-major storage
    ibuf = torch.full((3, 24, 2, 20), -1, dtype=torch.int16, device=dev)
    idx = ibuf[:, 1:22, :, 2:18]
    kvq.vq_encode(x, lam, s, cbl, 8, idx=idx, codebook_layer_stride=2 * 200 * 8)
    out = kvq.vq_decode(idx, cbl, lam, s, 8, codebook_layer_stride=2 * 200 * 8)
    torch.cuda.synchronize()
    check(x, lam, s, cbl, idx, out, all_idx(3, 21, 2), "per-layer strided", per_layer=True)
    assert (ibuf[:, 0] == -1).all() and (ibuf[:, 22:] == -1).all()
    assert (ibuf[..., :2] == -1).all() and (ibuf[..., 18:] == -1).all()


def test_ragged_and_empty():
    x, lam, s, cb = rand_case(2, 129, 1, 128, 100, seed=12)
    idx, out = run_vq(x, lam, s, cb)
    check(x, lam, s, cb, idx, out, all_idx(2, 129, 1), "ragged T=129")
    e = torch.zeros((2, 0, 1, 128), dtype=torch.float16, device=x.device)
    i2 = kvq.vq_encode(e, lam, s, cb, 8)
    o2 = kvq.vq_decode(i2, cb, lam, s, 8)
    torch.cuda.synchronize()
    assert i2.numel() == 0 and o2.numel() == 0


def test_decode_clamps_out_of_range_indices():
    x, lam, s, cb = rand_case(1, 16, 2, 128, 50, seed=13)
    idx = torch.full((1, 16, 2, 16), 49, dtype=torch.int16, device=x.device)
    ref = kvq.vq_decode(idx, cb, lam, s, 8)
    idx2 = idx.clone()
    idx2[..., ::2] = 4000                                  # beyond n_centroids
    out = kvq.vq_decode(idx2, cb, lam, s, 8)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("K,L,T,H,D", [
    (4096, 3, 1000, 3, 128),    # codebook staged in LDS; block ranges span (layer, head) segments
    (257, 2, 77, 8, 64),
    (4096, 1, 45, 1, 256),
    (5000, 2, 333, 2, 128),     # codebook above one LDS chunk: gathers from global memory, token-major
    (5000, 2, 50, 3, 256),      # ... head-major
    (4096, 3, 7, 2, 128),       # fewer than 16 tokens: the global-gather decoder at any codebook size
    (256, 2, 15, 3, 64),
    (4096, 2, 17, 2, 128),      # one full 16-token item, and a last item shifted back to end at token 16
])
def test_decode_random_indices(K, L, T, H, D):
    """Decode of indices drawn uniformly (not produced by the encoder), so
    every centroid position and both decode paths are exercised; each GPU
    output is compared with the oracle's decode of the same indices."""
    x, lam, s, cb = rand_case(L, T, H, D, K, seed=K + T)
    g = torch.Generator(device="cpu").manual_seed(K * 7 + T)
    idx = torch.randint(0, K, (L, T, H, D // 8), generator=g, dtype=torch.int32).to(torch.int16).to(x.device)
    out = kvq.vq_decode(idx, cb, lam, s, 8)
    torch.cuda.synchronize()
    sel = all_idx(L, T, H)
    cbb = bits(cb).reshape(H, K, 8)
    x64, _ = oracle.vq_decode(rows(idx, sel), cbb, sel[:, 2].astype(np.int32), lam_rows(lam, sel),
                              s.cpu().numpy(), 8)
    rep = parity.check_dequant(rows(out, sel), x64, lam_rows(lam, sel))
    log("decode K=%d [%d,%d,%d,%d]" % (K, L, T, H, D), {k: v for k, v in rep.items() if k != "bad_mask"})
    assert rep["bad"] == 0


def test_vecinfer_full_size_sampled():
    """The VecInfer-shaped key cache at full size ([36, 8192, 8, 128],
    per-head 4096-centroid fp16 codebooks), in the benchmark's launch
    configuration; parity on a seeded sample of 4,608 keys (73,728
    sub-vectors), 16 per (layer, head) on average, with the oracle run on
    disjoint shards in parallel."""
    dev = device()
    cfg = synth.config("vq")
    inp = synth.make_inputs(cfg, dev)
    x, lam, s, cb = inp["K"], inp["lam_K"], inp["signs"], inp["codebook"]
    idx, out = run_vq(x, lam, s, cb)
    sel = synth.sample_rows(cfg.L, cfg.T, cfg.H, 4608, 4242).numpy()
    xr, lr, ir, orow = rows(x, sel), lam_rows(lam, sel), rows(idx, sel), rows(out, sel)
    books = bits(cb).reshape(cfg.H, cfg.n_centroids, 8)
    book = sel[:, 2].astype(np.int32)
    sv = s.cpu().numpy()
    rep = parity.sharded(lambda k: parity.vq_parity(xr[k], lr[k], sv, books, book[k], 8, ir[k], orow[k]), len(sel))
    log("vecinfer full-size (%d keys, %d oracle threads)" % (len(sel), parity.workers()), parity.summary(rep))
