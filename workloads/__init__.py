"""Seeded synthetic workloads for the Hyena order-N forward.

This module only draws random inputs; it holds none of the operator's
arithmetic, so both the HIP path and the float64 oracle can take their inputs
from it.  Every value is reproducible from (config seed, tensor id).

Workload shapes follow the five operator configurations the project measures
(orders 2 and 3, lengths 256 .. 1,048,576, fp32 or bf16 I/O).  The pages'
own workloads (language modelling at 2K context, the 64K speed point of the
Hyena Hierarchy explainer, the 1M-token DNA setting of the jisaku.com
glossary entry, order-3 at ~128K) need datasets and trained weights that are
not available, so seeded random tensors of the same shape and dtype stand in
for them:

  * v, x_1..x_N ~ N(0, 1) (torch generator seeded per tensor), rounded to
    bf16 (round-to-nearest-even) where the I/O dtype is bf16;
  * DNA-style v: tokens i.i.d. uniform over a 4-symbol alphabet, looked up in
    a 4 x D embedding table drawn from N(0, 1);
  * filter FFN weights ~ N(0, 1/fan_in) (numpy PCG64 per layer), biases 0,
    window rates alpha_d linearly spaced in [1, 10];
  * block around the operator: input u [B][L][D] ~ N(0, 1), projection
    weights W_in [(N+1)D][D] and W_out [D][D] ~ N(0, 1/D), short filters
    [(N+1)D][T] ~ N(0, 1/T), biases zero unless asked for; projection weights
    and u are rounded to bf16 where the I/O dtype is bf16;
  * grid convolutions (the HyenaND summary's images, volumes and periodic
    physics fields, whose datasets are not available): v, x_n ~ N(0, 1) on
    the grid (bf16-rounded for bf16 I/O); each kernel is a Gaussian window
    exp(-|o|^2 / (2 sigma_d^2)) over the offsets o (sigma_d linearly spaced
    from 1 to half the largest side over the channels; circular offsets
    taken as the nearest signed representative) times N(0, 1) values,
    scaled to unit Euclidean norm.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Config", "CONFIGS", "make_filter_params", "make_activations",
           "config_by_name", "make_block_params", "make_block_input", "bf16_round",
           "GridConfig", "GRID_CONFIGS", "make_grid_kernel", "make_grid_activations"]


@dataclass(frozen=True)
class Config:
    name: str
    N: int          # order
    B: int          # batch
    D: int          # channels
    L: int          # sequence length
    io: str         # "fp32" or "bf16"
    H: int          # FFN hidden width
    seed: int
    K: int = 8      # sin/cos frequencies in the positional features (dim 1+2K)
    v_kind: str = "normal"   # "normal" or "dna"
    desc: str = ""

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "C1": Config("C1", 2, 1, 16, 256, "fp32", 32, 1,
                 desc="order-2, B=1, D=16, L=256, fp32 (small parity case)"),
    "C2": Config("C2", 2, 4, 768, 2048, "fp32", 64, 2,
                 desc="order-2, B=4, D=768, L=2048, fp32 (2K-context LM shape)"),
    "C3": Config("C3", 2, 1, 768, 65536, "bf16", 64, 3,
                 desc="order-2, B=1, D=768, L=65536, bf16 I/O (64K long-context shape)"),
    "C4": Config("C4", 2, 1, 256, 1048576, "fp32", 64, 4, v_kind="dna",
                 desc="order-2, B=1, D=256, L=1048576, fp32, DNA-token v (1M-token shape)"),
    "C5a": Config("C5a", 3, 2, 1024, 131072, "bf16", 64, 5,
                  desc="order-3, B=2, D=1024, L=131072, bf16 I/O"),
    "C5b": Config("C5b", 3, 2, 1024, 100000, "bf16", 64, 6,
                  desc="order-3, B=2, D=1024, L=100000, bf16 I/O (non-power-of-two L)"),
}


def config_by_name(name: str) -> Config:
    return CONFIGS[name]


def _np_rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))


def make_filter_params(cfg: Config, bias_scale: float = 0.0) -> dict:
    """FFN weights (float32, row-major [out][in]) and window rates.

    W1 [H][1+2K] ~ N(0, 1/(1+2K)), W2 [H][H] ~ N(0, 1/H), W3 [N*D][H] ~ N(0, 1/H).
    Biases are zero unless ``bias_scale`` > 0 (tests use nonzero biases too).
    alpha_d = linspace(1, 10, D) (alpha = 1 when D = 1).
    """
    F = 1 + 2 * cfg.K
    H, ND = cfg.H, cfg.N * cfg.D
    r1, r2, r3, rb = (_np_rng(cfg.seed, 101), _np_rng(cfg.seed, 102),
                      _np_rng(cfg.seed, 103), _np_rng(cfg.seed, 104))
    W1 = (r1.standard_normal((H, F)) / np.sqrt(F)).astype(np.float32)
    W2 = (r2.standard_normal((H, H)) / np.sqrt(H)).astype(np.float32)
    W3 = (r3.standard_normal((ND, H)) / np.sqrt(H)).astype(np.float32)
    if bias_scale > 0:
        b1 = (bias_scale * rb.standard_normal(H)).astype(np.float32)
        b2 = (bias_scale * rb.standard_normal(H)).astype(np.float32)
        b3 = (bias_scale * rb.standard_normal(ND)).astype(np.float32)
    else:
        b1 = np.zeros(H, np.float32); b2 = np.zeros(H, np.float32); b3 = np.zeros(ND, np.float32)
    if cfg.D == 1:
        alpha = np.ones(1, np.float32)
    else:
        alpha = np.linspace(1.0, 10.0, cfg.D).astype(np.float32)
    return dict(D=cfg.D, N=cfg.N, K=cfg.K, H=H, W1=W1, b1=b1, W2=W2, b2=b2,
                W3=W3, b3=b3, alpha=alpha)


def make_activations(cfg: Config, device="cpu", B: int | None = None):
    """(v, [x_1..x_N]) as torch tensors [B][D][L] in the config's I/O dtype.

    Drawn with a torch generator on ``device`` (seeded per tensor), so large
    shapes are generated where they are used.  Values for a given device are
    reproducible; CPU and GPU generators give different streams.
    """
    import torch

    B = cfg.B if B is None else B
    dt = torch.float32 if cfg.io == "fp32" else torch.bfloat16
    dev = torch.device(device)

    def gen(tid: int):
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.seed * 1000 + tid)
        return g

    shape = (B, cfg.D, cfg.L)
    if cfg.v_kind == "dna":
        table = torch.from_numpy(_np_rng(cfg.seed, 200).standard_normal((4, cfg.D))
                                 .astype(np.float32)).to(dev)
        tokens = torch.randint(0, 4, (B, cfg.L), generator=gen(0), device=dev)
        # v[b, d, t] = table[tokens[b, t], d]  (embedding lookup, done upstream)
        v = table.t()[:, tokens].permute(1, 0, 2).contiguous()
    else:
        v = torch.randn(shape, generator=gen(0), device=dev, dtype=torch.float32)
    xs = [torch.randn(shape, generator=gen(1 + n), device=dev, dtype=torch.float32)
          for n in range(cfg.N)]
    v = v.to(dt).contiguous()
    xs = [x.to(dt).contiguous() for x in xs]
    return v, xs



def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), as float32."""
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def make_block_params(cfg: Config, T: int = 3, bias_scale: float = 0.0) -> dict:
    """Weights of the block around the operator (numpy float32; W_in and W_out
    hold bf16-representable values when the I/O dtype is bf16)."""
    D, C = cfg.D, (cfg.N + 1) * cfg.D
    r = [_np_rng(cfg.seed, 300 + i) for i in range(5)]
    W_in = (r[0].standard_normal((C, D)) / np.sqrt(D)).astype(np.float32)
    W_out = (r[1].standard_normal((D, D)) / np.sqrt(D)).astype(np.float32)
    w_short = (r[2].standard_normal((C, T)) / np.sqrt(T)).astype(np.float32)
    if cfg.io == "bf16":
        W_in, W_out = bf16_round(W_in), bf16_round(W_out)
    b_in = (bias_scale * r[3].standard_normal(C)).astype(np.float32) if bias_scale > 0 else None
    b_out = (bias_scale * r[4].standard_normal(D)).astype(np.float32) if bias_scale > 0 else None
    return dict(D=D, N=cfg.N, T=T, W_in=W_in, b_in=b_in, w_short=w_short, W_out=W_out, b_out=b_out)


def make_block_input(cfg: Config, device="cpu", B: int | None = None):
    """u [B][L][D] ~ N(0, 1) in the config's I/O dtype (torch, seeded)."""
    import torch

    B = cfg.B if B is None else B
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed * 1000 + 500)
    u = torch.randn((B, cfg.L, cfg.D), generator=g, device=dev, dtype=torch.float32)
    return u.to(torch.float32 if cfg.io == "fp32" else torch.bfloat16).contiguous()


# ------------------------------------------------------------------ grids

@dataclass(frozen=True)
class GridConfig:
    name: str
    N: int                  # order
    B: int                  # batch
    D: int                  # channels
    dims: tuple             # grid sides L_1..L_k (last axis contiguous)
    circular: bool
    io: str                 # "fp32" or "bf16"
    seed: int
    per_sample: bool = False
    desc: str = ""

    @property
    def ndim(self) -> int:
        return len(self.dims)

    @property
    def kernel_shape(self) -> tuple:
        return tuple(self.dims) if self.circular else tuple(2 * L - 1 for L in self.dims)

    def with_(self, **kw) -> "GridConfig":
        return replace(self, **kw)


GRID_CONFIGS = {
    "G1": GridConfig("G1", 2, 2, 4, (8, 8), False, "fp32", 21,
                     desc="order-2, B=2, D=4, 8x8 grid, non-circular, fp32 (small parity case)"),
    "G2": GridConfig("G2", 2, 8, 192, (56, 56), False, "bf16", 22,
                     desc="order-2, B=8, D=192, 56x56 image grid, non-circular, bf16 I/O"),
    "G3": GridConfig("G3", 2, 2, 128, (16, 16, 16), False, "bf16", 23,
                     desc="order-2, B=2, D=128, 16^3 volume, non-circular, bf16 I/O"),
    "GP": GridConfig("GP", 2, 16, 64, (128, 128), True, "fp32", 24,
                     desc="order-2, B=16, D=64, 128x128 periodic field, circular, fp32"),
    "G4": GridConfig("G4", 2, 4, 96, (224, 224), False, "bf16", 25,
                     desc="order-2, B=4, D=96, 224x224 pixel grid, non-circular, bf16 I/O (multi-pass)"),
    "GP2": GridConfig("GP2", 2, 2, 32, (512, 512), True, "fp32", 26,
                      desc="order-2, B=2, D=32, 512x512 periodic field, circular, fp32 (multi-pass)"),
    "G5": GridConfig("G5", 2, 2, 64, (32, 32, 32), False, "bf16", 27,
                     desc="order-2, B=2, D=64, 32^3 volume, non-circular, bf16 I/O (multi-pass)"),
}


def make_grid_kernel(cfg: GridConfig) -> np.ndarray:
    """Kernels [N][D][ext...] (or [B][N][D][ext...] per sample), float32.

    Offsets: non-circular extent 2L-1 per axis, index o + L - 1; circular
    extent L, index o mod L.
    """
    lead = (cfg.B, cfg.N, cfg.D) if cfg.per_sample else (cfg.N, cfg.D)
    rng = _np_rng(cfg.seed, 600)
    ext = cfg.kernel_shape
    offs = []
    for L, e in zip(cfg.dims, ext):
        o = np.arange(e) - (L - 1) if not cfg.circular else np.arange(e)
        if cfg.circular:
            o = np.where(o > L // 2, o - L, o)
        offs.append(o.astype(np.float64))
    r2 = np.zeros(ext)
    for a, o in enumerate(offs):
        shape = [1] * len(ext)
        shape[a] = len(o)
        r2 = r2 + (o ** 2).reshape(shape)
    smax = max(1.0, max(cfg.dims) / 2.0)
    sig = np.linspace(1.0, smax, cfg.D) if cfg.D > 1 else np.ones(1)
    win = np.exp(-r2[None] / (2.0 * sig.reshape((-1,) + (1,) * len(ext)) ** 2))     # [D, ext...]
    K = rng.standard_normal(lead + ext) * win
    norm = np.sqrt((K ** 2).sum(axis=tuple(range(-len(ext), 0)), keepdims=True))
    return (K / np.maximum(norm, 1e-30)).astype(np.float32)


def make_grid_activations(cfg: GridConfig, device="cpu", B: int | None = None):
    """(v, [x_1..x_N]) as torch tensors [B][D][L_1..L_k] in the I/O dtype."""
    import torch

    B = cfg.B if B is None else B
    dt = torch.float32 if cfg.io == "fp32" else torch.bfloat16
    dev = torch.device(device)
    shape = (B, cfg.D) + tuple(cfg.dims)

    def draw(tid: int):
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.seed * 1000 + tid)
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(dt).contiguous()

    return draw(0), [draw(1 + n) for n in range(cfg.N)]
