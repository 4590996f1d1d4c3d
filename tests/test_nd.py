"""GPU parity of the grid convolutions (2-D and 3-D, circular and
twice-padded) against the float64 oracle's nd_forward, through the C ABI.

Error metric as for the 1-D operator: per grid (b, d), max |y - y_ref| over
the grid divided by max |y_ref|; 1e-4 for fp32 I/O, 2e-2 for bf16 I/O.
"""
import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, channel_errors
from workloads import GRID_CONFIGS, GridConfig, make_grid_activations, make_grid_kernel

pytestmark = pytest.mark.gpu


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(cfg: GridConfig):
    v, xs = make_grid_activations(cfg, DEV)
    K = torch.from_numpy(make_grid_kernel(cfg)).to(DEV)
    spec = H.nd_filter_spectrum(K, cfg.dims, cfg.circular)
    y = H.nd_forward(v, xs, spec, cfg.circular, cfg.per_sample)
    torch.cuda.synchronize()
    return v, xs, K, y


def _errors(cfg, v, xs, K, y, pairs=None):
    ndim = cfg.ndim
    if pairs is None:
        ref = O.nd_forward(_np(v), [_np(x) for x in xs], _np(K), ndim, cfg.circular, cfg.per_sample)
        got = _np(y)
    else:
        ref, got = [], []
        for b, d in pairs:
            Kb = _np(K[b][:, d:d + 1]) if cfg.per_sample else _np(K[:, d:d + 1])
            r = O.nd_forward(_np(v[b:b + 1, d:d + 1]), [_np(x[b:b + 1, d:d + 1]) for x in xs], Kb, ndim,
                             cfg.circular)
            ref.append(r[0, 0])
            got.append(_np(y[b, d]))
        ref, got = np.stack(ref), np.stack(got)
    flat = lambda a: a.reshape(a.shape[:-ndim] + (-1,))
    assert np.all(np.isfinite(got)), "non-finite output"
    return channel_errors(flat(got), flat(ref))


def _tol(cfg):
    return 1e-4 if cfg.io == "fp32" else 2e-2


CASES = [
    # N, B, D, dims, circular, io, per_sample
    (2, 2, 3, (8, 8), False, "fp32", False),          # P = 16
    (2, 1, 2, (5, 7), False, "fp32", False),          # ragged, odd last side
    (1, 2, 2, (1, 9), False, "fp32", False),          # a single row
    (3, 1, 2, (16, 16), False, "fp32", False),        # P = 32
    (2, 1, 2, (13, 31), False, "fp32", False),        # P = 64, odd sides
    (2, 1, 2, (32, 32), False, "bf16", False),        # P = 64
    (2, 1, 2, (56, 56), False, "fp32", False),        # P = 128 (image grid)
    (2, 1, 1, (64, 63), False, "fp32", False),        # largest 2-D non-circular
    (2, 2, 2, (16, 16), True, "fp32", False),
    (2, 1, 2, (32, 32), True, "fp32", False),
    (1, 1, 2, (64, 64), True, "bf16", False),
    (2, 1, 2, (128, 128), True, "fp32", False),
    (2, 2, 2, (4, 4, 4), False, "fp32", False),       # P = 8
    (2, 1, 2, (3, 4, 2), False, "fp32", False),
    (2, 1, 2, (8, 8, 8), False, "fp32", False),       # P = 16
    (2, 1, 2, (5, 7, 3), False, "bf16", False),
    (2, 1, 2, (16, 16, 16), False, "fp32", False),    # P = 32
    (1, 1, 1, (9, 16, 11), False, "fp32", False),
    (2, 2, 2, (8, 8, 8), True, "fp32", False),
    (2, 1, 2, (16, 16, 16), True, "fp32", False),
    (1, 1, 2, (32, 32, 32), True, "fp32", False),
    (2, 3, 2, (12, 10), False, "fp32", True),         # per-sample kernels
    (2, 2, 2, (16, 16), True, "bf16", True),
    (2, 2, 1, (6, 5, 4), False, "fp32", True),
    # multi-pass 2-D grids (P >= 256): column and row passes over a workspace
    (2, 2, 2, (100, 130), False, "fp32", False),      # P = 256
    (3, 1, 2, (200, 255), False, "fp32", False),      # P = 512, odd last side
    (1, 1, 1, (300, 17), False, "fp32", False),       # P = 1024
    (2, 1, 2, (224, 224), False, "bf16", False),      # image grid
    (2, 1, 2, (256, 256), True, "fp32", False),
    (2, 1, 1, (512, 512), True, "fp32", False),
    (2, 2, 2, (120, 90), False, "fp32", True),        # per-sample kernels
    # multi-pass 3-D grids (P >= 64): column pass over the first axis, plane pass over the other two
    (2, 2, 2, (20, 24, 18), False, "fp32", False),    # P = 64
    (3, 1, 1, (32, 31, 17), False, "bf16", False),
    (1, 1, 2, (40, 9, 33), False, "fp32", False),     # P = 128
    (2, 1, 2, (64, 64, 64), True, "fp32", False),
    (1, 1, 1, (128, 128, 128), True, "fp32", False),
    (2, 2, 1, (17, 20, 19), False, "fp32", True),     # per-sample kernels
]


@pytest.mark.parametrize("N,B,D,dims,circ,io,ps", CASES)
def test_nd_forward_matches_oracle(N, B, D, dims, circ, io, ps):
    cfg = GridConfig("t", N, B, D, dims, circ, io, 31 + sum(dims), per_sample=ps)
    v, xs, K, y = _run(cfg)
    err = _errors(cfg, v, xs, K, y).max()
    assert err <= _tol(cfg), f"max normalised error {err:.3e}"


@pytest.mark.parametrize("name", ["G2", "G3", "GP", "G4", "GP2", "G5"])
def test_nd_configs_sampled(name):
    """The measured grid workloads at full size, checked on sampled grids."""
    cfg = GRID_CONFIGS[name]
    v, xs, K, y = _run(cfg)
    rng = np.random.default_rng(7)
    pairs = sorted({(0, 0), (cfg.B - 1, cfg.D - 1)} |
                   {(int(rng.integers(cfg.B)), int(rng.integers(cfg.D))) for _ in range(4)})
    err = _errors(cfg, v, xs, K, y, pairs).max()
    assert err <= _tol(cfg), f"max normalised error {err:.3e}"


def test_nd_g1_full():
    cfg = GRID_CONFIGS["G1"]
    v, xs, K, y = _run(cfg)
    assert _errors(cfg, v, xs, K, y).max() <= 1e-4


def test_nd_delta_kernel_gives_the_gate_product():
    """Kernel = delta at offset 0: y = v * x_1 * x_2 (exactly up to rounding)."""
    dims = (20, 24)
    cfg = GridConfig("d", 2, 2, 3, dims, False, "fp32", 5)
    v, xs = make_grid_activations(cfg, DEV)
    K = torch.zeros((2, 3, 39, 47), device=DEV)
    K[:, :, 19, 23] = 1.0
    spec = H.nd_filter_spectrum(K, dims)
    y = H.nd_forward(v, xs, spec)
    torch.cuda.synchronize()
    ref = v * xs[0] * xs[1]
    assert torch.max(torch.abs(y - ref)).item() <= 1e-5 * torch.max(torch.abs(ref)).item()


def test_nd_repeat_calls_identical():
    cfg = GridConfig("r", 2, 2, 4, (24, 24), False, "fp32", 8)
    v, xs = make_grid_activations(cfg, DEV)
    K = torch.from_numpy(make_grid_kernel(cfg)).to(DEV)
    spec = H.nd_filter_spectrum(K, cfg.dims)
    call = H.prepare_nd_forward(v, xs, spec)
    a = call().clone()
    b = call().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dims,grid_bytes", [((150, 150), 512 * 256 * 8), ((20, 20, 20), 64 * 64 * 32 * 8)])
def test_nd_multipass_small_workspace_matches(dims, grid_bytes):
    """A workspace smaller than the one asked for only splits the passes into
    more groups (single grids below B, whole channels of B grids above)."""
    cfg = GridConfig("w", 2, 3, 2, dims, False, "fp32", 9)
    v, xs = make_grid_activations(cfg, DEV)
    K = torch.from_numpy(make_grid_kernel(cfg)).to(DEV)
    spec = H.nd_filter_spectrum(K, cfg.dims)
    y_full = H.nd_forward(v, xs, spec).clone()
    for grids in (1, 2, 3, 4):
        ws = H._empty(grids * grid_bytes, dtype=torch.uint8, device=DEV)
        y_ws = H.nd_forward(v, xs, spec, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_full, y_ws), f"workspace of {grids} grids"


def test_nd_errors():
    dev = DEV
    K = torch.zeros((1, 1, 1025, 15), device=dev)
    with pytest.raises(H.HyenaError):           # needs P = 2048 > 1024
        H.nd_filter_spectrum(K, (513, 8))
    v = torch.zeros((1, 1, 32, 16), device=dev)
    with pytest.raises(H.HyenaError):           # circular needs equal power-of-two sides
        H.nd_filter_spectrum(torch.zeros((1, 1, 32, 16), device=dev), (32, 16), circular=True)
    K = torch.zeros((1, 1, 63, 31), device=dev)
    spec = H.nd_filter_spectrum(K, (32, 16))
    with pytest.raises(H.HyenaError):           # y aliases v
        H.nd_forward(v, [v], spec, out=v)
