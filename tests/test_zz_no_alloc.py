"""kvq_attend_decode_noalloc -- decode attention with its partial states in
the library's static device scratch (for callers that cannot allocate) --
against kvq_attend_decode with a caller workspace, through the C ABI via the
binding: three calls in a row on the same device, each smaller than the one
before and each through a different kernel (matrix-core head_dim 128,
matrix-core head_dim 256, vector-ALU head_dim 64), so that the later calls
run over what the earlier ones left in the shared array.  The two entry
points run the same kernels under the same plan, so their outputs must be
identical bit for bit; the first call is also checked against the fp64
oracle."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_quantize_amd as kvq
import oracle
from tests.gpu_util import bits, device, log
from tests.test_gpu_attend import compare, make_cache

pytestmark = pytest.mark.gpu

CASES = [  # (L, T, H, R, D, G, lengths)
    (6, 3000, 8, 4, 128, 32, "ragged"),
    (4, 1500, 2, 2, 256, 64, None),
    (2, 300, 3, 1, 64, 16, "ragged"),
]


def test_noalloc_matches_workspace_entry_point():
    dev = device()
    for i, (L, T, H, R, D, G, lens) in enumerate(CASES):
        need = kvq.attend_decode_workspace_bytes(L, T, H, D, R)
        assert 0 < need <= 64 << 20, need
        c = make_cache(L, T, H, D, G, 100 + i, dev)
        g = torch.Generator(device="cpu").manual_seed(200 + i)
        q = torch.randn((L, H * R, D), generator=g).to(torch.float16).to(dev)
        ln = None
        if lens:
            ln = torch.randint(0, T + 1, (L,), generator=g, dtype=torch.int32)
            ln[0], ln[-1] = T, 0
            ln = ln.to(dev)
        kc, ks, lk = c["k"]
        vc, vs, lv = c["v"]
        want = kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, c["s"], G, lengths=ln)
        got = torch.full_like(q, float("nan"))
        kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, c["s"], G, lengths=ln, out=got, noalloc=True)
        torch.cuda.synchronize()
        log("noalloc call %d: [%d, %d, %d, %d] R=%d G=%d, %d workspace bytes" % (i, L, T, H, D, R, G, need))
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "call %d differs" % i
        if i == 0:
            out64 = oracle.attend_decode(bits(q), kc.cpu().numpy(), bits(ks), vc.cpu().numpy(), bits(vs),
                                         lk.cpu().numpy(), lv.cpu().numpy(), c["s"].cpu().numpy(), G,
                                         1.0 / D ** 0.5, None if ln is None else ln.cpu().numpy())
            compare(got, out64, lv, H, R, "noalloc call 0 vs oracle")
