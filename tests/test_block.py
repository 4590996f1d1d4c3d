"""GPU parity of the block around the operator (in-projection with the short
causal convolution, out-projection, the whole block) through the C ABI,
against the float64 oracle on the same inputs.

Tolerances, max |got - ref| / max |ref| per row: projections 2e-5 (fp32:
matrix-core fp32 products, fp32 accumulation over D terms) and 8e-3 (bf16:
the stored result is rounded to bf16, 2^-9 relative), rows being one
projected stream of one channel (in-projection) or one output time step
(out-projection); the block 1e-4 (fp32) and 2e-2 (bf16) per output channel
over time, the operator's own metric (its FFT rounding scales with a
channel's whole row, so single early time steps, where the output is small,
are not a fair denominator).
"""
import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, channel_errors, params_to_device
from workloads import CONFIGS, Config, make_block_input, make_block_params, make_filter_params

pytestmark = pytest.mark.gpu

TOL_PROJ = {"fp32": 2e-5, "bf16": 8e-3}
TOL_BLOCK = {"fp32": 1e-4, "bf16": 2e-2}


def _cfg(B, L, D, N, io, seed=21):
    return Config("blk", N, B, D, L, io, 32, seed)


def _bp_device(bp, io):
    dt = torch.float32 if io == "fp32" else torch.bfloat16
    out = {"D": bp["D"], "N": bp["N"], "T": bp["T"]}
    for k in ("W_in", "W_out"):
        out[k] = torch.from_numpy(bp[k]).to(DEV).to(dt).contiguous()
    out["w_short"] = torch.from_numpy(bp["w_short"]).to(DEV)
    for k in ("b_in", "b_out"):
        out[k] = None if bp[k] is None else torch.from_numpy(bp[k]).to(DEV)
    return out


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


IN_CASES = [
    # B, L, D, N, T, io
    (1, 5, 3, 1, 1, "fp32"), (2, 130, 16, 2, 3, "fp32"), (1, 257, 37, 2, 3, "fp32"),
    (2, 1000, 128, 3, 3, "fp32"), (1, 700, 64, 2, 16, "fp32"), (2, 300, 48, 2, 3, "bf16"),
    (1, 200, 20, 2, 5, "bf16"), (1, 3, 8, 8, 2, "fp32"), (4, 2048, 768, 2, 3, "fp32"),
    # bf16 with D % 8 == 0 and T <= 8: 128 x 256 tiles, short convolution on the
    # accumulators (strips of tiles; L % 4 != 0 stores element-wise; ragged k
    # slices, column blocks and strips)
    (2, 1000, 128, 2, 3, "bf16"), (1, 777, 192, 3, 4, "bf16"), (1, 4096, 768, 2, 3, "bf16"),
    (1, 129, 8, 1, 1, "bf16"), (1, 2050, 64, 2, 7, "bf16"), (2, 1500, 256, 1, 8, "bf16"),
    (1, 20000, 64, 2, 3, "bf16"), (3, 5000, 256, 3, 6, "bf16"), (1, 1, 16, 2, 2, "bf16"),
    (2, 6, 40, 2, 5, "bf16"), (1, 3001, 520, 2, 4, "bf16"),
    # bf16 beyond the wide path: 16 taps, D % 8 != 0
    (1, 700, 64, 2, 16, "bf16"), (1, 333, 36, 2, 3, "bf16"),
]


@pytest.mark.parametrize("B,L,D,N,T,io", IN_CASES)
def test_in_projection_matches_oracle(B, L, D, N, T, io):
    cfg = _cfg(B, L, D, N, io)
    bp = make_block_params(cfg, T=T, bias_scale=0.3)
    u = make_block_input(cfg, DEV)
    v, xs = H.in_projection(u, _bp_device(bp, io))
    torch.cuda.synchronize()
    rv, rxs = O.in_projection(_np(u), bp["W_in"], bp["b_in"], bp["w_short"], N)
    for got, ref in zip([v] + xs, [rv] + rxs):
        err = channel_errors(_np(got), ref)
        assert np.all(np.isfinite(_np(got)))
        assert err.max() <= TOL_PROJ[io], (err.max(), np.unravel_index(err.argmax(), err.shape))


def test_in_projection_full_width_sampled_columns():
    """The 64K-token block shape (B=1, L=65536, D=768, order 2, 3 taps, bf16):
    every time step of sampled projected columns against the oracle, among
    them the first and last column of each stream and the columns on either
    side of a 256-column block edge."""
    B, L, D, N, T = 1, 65536, 768, 2, 3
    cfg = _cfg(B, L, D, N, "bf16")
    bp = make_block_params(cfg, T=T, bias_scale=0.3)
    u = make_block_input(cfg, DEV)
    v, xs = H.in_projection(u, _bp_device(bp, "bf16"))
    torch.cuda.synchronize()
    streams = [v] + xs
    rs = np.random.default_rng(5)
    cols = sorted({0, D - 1, D, 2 * D - 1, 2 * D, 3 * D - 1, 255, 256, 511, 512, 1279, 1280,
                   *rs.integers(0, (N + 1) * D, 10).tolist()})
    ref = O.in_projection_columns(_np(u), bp["W_in"], bp["b_in"], bp["w_short"], cols)
    got = np.stack([_np(streams[c // D][:, c % D]) for c in cols], axis=1)
    err = channel_errors(got, ref)
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL_PROJ["bf16"], (err.max(), cols[int(np.argmax(err.max(axis=0)))])


OUT_CASES = [(1, 5, 3, "fp32"), (2, 130, 16, "fp32"), (1, 257, 37, "fp32"), (2, 1000, 128, "fp32"),
             (4, 2048, 768, "fp32"), (2, 300, 48, "bf16"), (1, 200, 20, "bf16"), (1, 4096, 256, "bf16")]


@pytest.mark.parametrize("B,L,D,io", OUT_CASES)
def test_out_projection_matches_oracle(B, L, D, io):
    cfg = _cfg(B, L, D, 2, io)
    bp = make_block_params(cfg, bias_scale=0.3)
    g = torch.Generator(device=DEV); g.manual_seed(77)
    y = torch.randn((B, D, L), generator=g, device=DEV).to(torch.float32 if io == "fp32" else torch.bfloat16)
    o = H.out_projection(y, _bp_device(bp, io))
    torch.cuda.synchronize()
    ref = O.out_projection(_np(y), bp["W_out"], bp["b_out"])
    err = channel_errors(_np(o), ref)                       # rows: (b, t)
    assert err.max() <= TOL_PROJ[io], err.max()


def _block_case(cfg, T, batches, bias=0.2):
    bp = make_block_params(cfg, T=T, bias_scale=bias)
    fp = make_filter_params(cfg)
    u = make_block_input(cfg, DEV)
    h = H.filter_gen(params_to_device(fp), cfg.L)
    spec = H.filter_spectrum(h)
    out = H.block_forward(u, _bp_device(bp, cfg.io), spec)
    torch.cuda.synchronize()
    ref = O.block_forward(_np(u)[batches], bp, _np(h))          # same filters h as the GPU
    return _np(out)[batches], ref, out, u, bp, spec


def _block_errors(got, ref):
    # per output channel over time, as for the operator: the long convolution's
    # rounding scales with a channel's whole-row magnitude, not with one step's
    return channel_errors(np.transpose(got, (0, 2, 1)), np.transpose(ref, (0, 2, 1)))


@pytest.mark.parametrize("B,L,D,N,T,io,batches", [(1, 256, 16, 2, 3, "fp32", [0]), (2, 1000, 40, 3, 4, "fp32", [0, 1]),
                                                   (2, 600, 64, 2, 3, "bf16", [0, 1]), (1, 20000, 32, 2, 3, "fp32", [0]),
                                                   (4, 2048, 768, 2, 3, "fp32", [3])])
def test_block_matches_oracle(B, L, D, N, T, io, batches):
    cfg = _cfg(B, L, D, N, io)
    got, ref, *_ = _block_case(cfg, T, batches)
    err = _block_errors(got, ref)
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL_BLOCK[io], err.max()


def test_block_equals_its_three_calls():
    cfg = _cfg(2, 500, 24, 2, "fp32")
    _, _, out, u, bp, spec = _block_case(cfg, 3, [0])
    bpd = _bp_device(bp, "fp32")
    v, xs = H.in_projection(u, bpd)
    y = H.forward(v, xs, spec)
    o2 = H.out_projection(y, bpd)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
