"""Seeded synthetic KV-cache inputs shared by the tests, the smoke check and the
benchmark.

This module holds no quantizer arithmetic: it draws fp16 key/value tensors
shaped like the caches of the models the pages benchmark, calibrates the
smooth scale lambda from a separate small draw of the same distribution, draws
the +-1 sign vector and the product-VQ codebooks.  Both the HIP path and the
CPU oracle consume exactly the bytes produced here (the oracle reads them back
from the device), so neither side needs to regenerate them.

Seeds: seed(config i, purpose p) = 1000 * i + p with p = 1 K data, 2 V data,
3 K calibration, 4 V calibration, 5 signs, 6 outlier-channel / channel-scale
choice, 7 key codebook, 8 value codebook.

Calibration (input recipe, not part of the quantizer): for every (layer,
head, channel) lambda = 1 / sqrt(mean over 16 calibration tokens of x^2),
computed in fp64 from the fp16-rounded draw and stored as fp32; lambda = 1
where that mean is 0.  The per-channel smooth scale is described as
calibrated (or learned) per head and channel in the VecInfer blog post
("What VecInfer does") and in the gist.science explanation of arXiv
2605.05699 (Methodologie, section 2).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

CALIB_TOKENS = 16
P_KDATA, P_VDATA, P_KCAL, P_VCAL, P_SIGNS, P_CHAN, P_CODEBOOK, P_VCODEBOOK = 1, 2, 3, 4, 5, 6, 7, 8


def seed(config: int, purpose: int) -> int:
    return 1000 * config + purpose


def _gen(s: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    return g


def normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def student_t4(shape, g, device):
    """Student-t with 4 degrees of freedom: Z / sqrt(W / 4), W = -2 ln(U1 U2)."""
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    u1 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    u2 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    w = -2.0 * torch.log(u1 * u2)
    return z / torch.sqrt(w / 4.0)


def signs(D: int, s: int, device="cpu") -> torch.Tensor:
    g = _gen(s, "cpu")
    r = torch.randint(0, 2, (D,), generator=g, dtype=torch.int8)
    return (r * 2 - 1).to(torch.int8).to(device)


def calibrate_lambda(calib_f16: torch.Tensor) -> torch.Tensor:
    """calib [L, Tc, H, D] fp16 -> lambda [L, H, D] fp32 (1/RMS over tokens)."""
    c = calib_f16.to(torch.float64)
    ms = (c * c).mean(dim=1)
    lam = torch.where(ms > 0, 1.0 / torch.sqrt(ms), torch.ones_like(ms))
    return lam.to(torch.float32).contiguous()


# ------------------------------------------------------------ distributions
@dataclass
class Dist:
    """How one tensor of a config is drawn.

    kind: "normal" or "t4".  outliers: number of seeded outlier channels per
    (layer, head) and their multiplier.  lognormal_channels: per (layer, head,
    channel) LogNormal(0, 1) scale.
    """
    kind: str = "normal"
    outlier_channels: int = 0
    outlier_mult: float = 1.0
    fixed_outliers: tuple = ()       # explicit channel list (same for all l, h)
    lognormal_channels: bool = False


def _channel_mult(L, H, D, dist: Dist, chan_seed: int, device):
    """[L, 1, H, D] fp32 multiplier per channel, or None."""
    m = None
    if dist.fixed_outliers:
        m = torch.ones((L, 1, H, D), dtype=torch.float32)
        m[..., list(dist.fixed_outliers)] = dist.outlier_mult
    elif dist.outlier_channels:
        g = _gen(chan_seed, "cpu")
        m = torch.ones((L, 1, H, D), dtype=torch.float32)
        for l in range(L):
            for h in range(H):
                ch = torch.randperm(D, generator=g)[: dist.outlier_channels]
                m[l, 0, h, ch] = dist.outlier_mult
    if dist.lognormal_channels:
        g = _gen(chan_seed, "cpu")
        ln = torch.exp(torch.randn((L, 1, H, D), generator=g, dtype=torch.float32))
        m = ln if m is None else m * ln
    return None if m is None else m.to(device)


def draw(L, T, H, D, dist: Dist, data_seed: int, chan_seed: int, device="cpu",
         chunk_layers: int = 1) -> torch.Tensor:
    """fp16 tensor [L, T, H, D] drawn from `dist`, generated on `device`
    layer-chunk by layer-chunk (so a 19 GB tensor never needs an fp32 copy)."""
    out = torch.empty((L, T, H, D), dtype=torch.float16, device=device)
    mult = _channel_mult(L, H, D, dist, chan_seed, device)
    g = _gen(data_seed, device)
    for l0 in range(0, L, chunk_layers):
        l1 = min(L, l0 + chunk_layers)
        shape = (l1 - l0, T, H, D)
        v = normal(shape, g, device) if dist.kind == "normal" else student_t4(shape, g, device)
        if mult is not None:
            v = v * mult[l0:l1]
        out[l0:l1] = v.to(torch.float16)
        del v
    return out


# ------------------------------------------------------------------ configs
@dataclass
class Config:
    index: int
    name: str
    L: int
    T: int
    H: int
    D: int
    G: int
    k_dist: Dist
    v_dist: Dist | None            # None = keys only
    vq: bool = False
    n_centroids: int = 4096
    v_centroids: int = 256             # value codebooks (one-byte indices)
    sub_dim: int = 8
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def vectors(self) -> int:
        return self.L * self.T * self.H


def config(name: str, T: int | None = None) -> Config:
    """The five workloads: tiny, qwen2.5-1.5b, gemma-3-1b, qwen3-8b, vq."""
    if name == "tiny":
        return Config(0, name, 1, 64, 2, 128, 32,
                      Dist("normal", outlier_mult=20.0, fixed_outliers=(0, 1, 2, 3)), None,
                      notes="keys only; channels 0-3 x20")
    if name == "qwen2.5-1.5b":
        return Config(1, name, 28, 4096 if T is None else T, 2, 128, 32,
                      Dist("normal", outlier_channels=4, outlier_mult=15.0), Dist("normal"))
    if name == "gemma-3-1b":
        return Config(2, name, 26, 4096 if T is None else T, 1, 256, 64,
                      Dist("t4", outlier_channels=2, outlier_mult=25.0), Dist("normal"))
    if name == "qwen3-8b":
        return Config(3, name, 36, 8 * 32768 if T is None else T, 8, 128, 32,
                      Dist("normal", lognormal_channels=True),
                      Dist("normal", lognormal_channels=True))
    if name == "vq":
        return Config(4, name, 36, 8192 if T is None else T, 8, 128, 0,
                      Dist("normal", lognormal_channels=True), Dist("normal", lognormal_channels=True), vq=True,
                      notes="keys: 4096-centroid codebooks (12-bit); values: 256-centroid codebooks (8-bit)")
    raise KeyError(name)


CONFIG_NAMES = ("tiny", "qwen2.5-1.5b", "gemma-3-1b", "qwen3-8b", "vq")


def make_inputs(cfg: Config, device="cpu", want_v: bool = True) -> dict:
    """Draw one config: K (and V), their lambdas, the sign vector and, for the
    VQ config, the per-head key codebook [H, K, sub] and value codebook
    [H, 256, sub], fp16 ~ N(0, 1)."""
    i = cfg.index
    out = {"cfg": cfg}
    out["K"] = draw(cfg.L, cfg.T, cfg.H, cfg.D, cfg.k_dist, seed(i, P_KDATA), seed(i, P_CHAN), device)
    kc = draw(cfg.L, CALIB_TOKENS, cfg.H, cfg.D, cfg.k_dist, seed(i, P_KCAL), seed(i, P_CHAN), "cpu")
    out["lam_K"] = calibrate_lambda(kc).to(device)
    if cfg.v_dist is not None and want_v:
        # V channel structure uses its own stream (offset 100) so K and V differ.
        out["V"] = draw(cfg.L, cfg.T, cfg.H, cfg.D, cfg.v_dist, seed(i, P_VDATA), seed(i, P_CHAN) + 100, device)
        vc = draw(cfg.L, CALIB_TOKENS, cfg.H, cfg.D, cfg.v_dist, seed(i, P_VCAL), seed(i, P_CHAN) + 100, "cpu")
        out["lam_V"] = calibrate_lambda(vc).to(device)
    out["signs"] = signs(cfg.D, seed(i, P_SIGNS), device)
    if cfg.vq:
        g = _gen(seed(i, P_CODEBOOK), "cpu")
        cb = torch.randn((cfg.H, cfg.n_centroids, cfg.sub_dim), generator=g, dtype=torch.float32)
        out["codebook"] = cb.to(torch.float16).to(device)
        g = _gen(seed(i, P_VCODEBOOK), "cpu")
        cb = torch.randn((cfg.H, cfg.v_centroids, cfg.sub_dim), generator=g, dtype=torch.float32)
        out["codebook_V"] = cb.to(torch.float16).to(device)
    return out


def sample_rows(L: int, T: int, H: int, n: int, s: int) -> torch.Tensor:
    """Seeded sample of n (layer, token, head) triples [n, 3] (int64), with the
    first and last token of every layer's range always represented."""
    g = _gen(s, "cpu")
    l = torch.randint(0, L, (n,), generator=g)
    t = torch.randint(0, T, (n,), generator=g)
    h = torch.randint(0, H, (n,), generator=g)
    if n >= 4:
        t[0], t[1] = 0, T - 1
        l[0], l[1] = 0, L - 1
    return torch.stack([l, t, h], dim=1)
