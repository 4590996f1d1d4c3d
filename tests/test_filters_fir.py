"""GPU parity of the other filter families and of the short-filter path:
Hyena-LI generation, Hyena-MR damping, the operator with LI filters on the
FFT path, and the recurrence with explicit short filters evaluated directly
(hyena_forward_fir), against the float64 oracle.

Tolerances (per row, max |got - ref| / max |ref|): generated filters 2e-6;
forward 1e-4 (fp32; the direct FIR sums Lh products in fp32) and 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, channel_errors
from workloads import Config, make_activations

pytestmark = pytest.mark.gpu

rng = np.random.default_rng(2024)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("N,D,S,L", [(1, 1, 1, 1), (2, 3, 4, 1000), (3, 5, 16, 65536), (2, 2, 64, 4097)])
def test_filter_gen_li_matches_oracle(N, D, S, L):
    R = rng.standard_normal((N * D, S)).astype(np.float32)
    lam = rng.uniform(-0.999, 0.9999, (N * D, S)).astype(np.float32)
    lam[0, 0] = 0.0
    h = H.filter_gen_li(torch.from_numpy(R).to(DEV), torch.from_numpy(lam).to(DEV), D, N, L)
    ref = O.filter_gen_li(R, lam, L).reshape(N, D, L)
    assert channel_errors(_np(h), ref).max() < 2e-6


def test_filter_gen_mr_matches_oracle():
    N, D, Lh = 3, 4, 200
    hhat = rng.standard_normal((N, D, Lh)).astype(np.float32)
    alpha = np.linspace(0.0, 0.1, D).astype(np.float32)
    h = H.filter_gen_mr(torch.from_numpy(hhat).to(DEV), torch.from_numpy(alpha).to(DEV))
    assert channel_errors(_np(h), O.filter_gen_mr(hhat, alpha, N)).max() < 2e-6


@pytest.mark.parametrize("L", [3000, 20000])
def test_forward_with_li_filters(L):
    # Hyena-LI filters through the spectrum and the FFT path, single and four-step
    N, B, D, S = 2, 2, 3, 8
    R = (rng.standard_normal((N * D, S)) / S).astype(np.float32)
    lam = rng.uniform(0.9, 0.99999, (N * D, S)).astype(np.float32)
    h = H.filter_gen_li(torch.from_numpy(R).to(DEV), torch.from_numpy(lam).to(DEV), D, N, L)
    v, xs = make_activations(Config("li", N, B, D, L, "fp32", 32, 8), DEV)
    y = H.forward(v, xs, H.filter_spectrum(h))
    torch.cuda.synchronize()
    ref = O.hyena_forward(_np(v), [_np(x) for x in xs], _np(h))
    assert channel_errors(_np(y), ref).max() < 1e-4


FIR_CASES = [
    # N, B, D, L, Lh, io
    (1, 1, 1, 1, 1, "fp32"), (2, 2, 3, 100, 3, "fp32"), (2, 1, 4, 5000, 7, "fp32"), (3, 2, 2, 4097, 14, "fp32"),
    (8, 1, 2, 3000, 5, "fp32"), (2, 1, 3, 2500, 256, "fp32"), (2, 2, 3, 1000, 4, "bf16"), (2, 1, 2, 9000, 128, "bf16"),
    (2, 1, 2, 7, 40, "fp32"),
    # tap counts that are not multiples of 4 over several orders and tiles
    (3, 2, 3, 6000, 6, "fp32"), (4, 1, 2, 5000, 9, "bf16"),
]


@pytest.mark.parametrize("N,B,D,L,Lh,io", FIR_CASES)
def test_forward_fir_matches_oracle(N, B, D, L, Lh, io):
    v, xs = make_activations(Config("fir", N, B, D, L, io, 32, 9), DEV)
    hs = (rng.standard_normal((N, D, Lh)) / np.sqrt(Lh)).astype(np.float32)
    y = H.forward_fir(v, xs, torch.from_numpy(hs).to(DEV))
    torch.cuda.synchronize()
    hp = np.zeros((N, D, L)); hp[..., :min(Lh, L)] = hs[..., :min(Lh, L)]
    ref = O.hyena_forward(_np(v), [_np(x) for x in xs], hp)
    err = channel_errors(_np(y), ref).max()
    assert err < (1e-4 if io == "fp32" else 2e-2), err
