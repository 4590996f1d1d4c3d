"""GPU parity of the circular mode (periodic convolution, M = L, no zero
padding) against the float64 oracle with circular_conv, on the single-pass
and four-step paths; tolerances as for the linear mode."""
import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, channel_errors, params_to_device
from workloads import Config, make_activations, make_filter_params

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    monkeypatch.delenv("HYENA_FORCE_PATH", raising=False)
    monkeypatch.delenv("HYENA_FOURSTEP_N1", raising=False)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


CASES = [
    # N, B, D, L, io, force, n1
    (2, 2, 3, 128, "fp32", None, None), (2, 1, 4, 2048, "fp32", None, None), (3, 2, 2, 16384, "fp32", None, None),
    (2, 1, 2, 32768, "fp32", None, None), (2, 1, 2, 65536, "fp32", None, None), (2, 2, 3, 4096, "bf16", None, None),
    (2, 1, 2, 2048, "fp32", "fourstep", "16"), (1, 2, 2, 8192, "fp32", "fourstep", "64"),
]


@pytest.mark.parametrize("N,B,D,L,io,force,n1", CASES)
def test_circular_forward_matches_oracle(N, B, D, L, io, force, n1, monkeypatch):
    if force:
        monkeypatch.setenv("HYENA_FORCE_PATH", force)
    if n1:
        monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    cfg = Config("circ", N, B, D, L, io, 32, 12)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    h = H.filter_gen(params_to_device(p), L)
    spec = H.filter_spectrum(h, circular=True)
    y = H.forward(v, xs, spec)
    torch.cuda.synchronize()
    ref = O.hyena_forward(_np(v), [_np(x) for x in xs], _np(h), conv=O.circular_conv)
    err = channel_errors(_np(y), ref).max()
    assert err <= (1e-4 if io == "fp32" else 2e-2), err
    # the spectrum is the plain L-point DFT of each filter
    got = H.spectrum_export(spec, D, N, L).cpu().numpy()
    refs = np.fft.rfft(_np(h), axis=-1)
    assert np.max(np.abs(got - refs)) / np.max(np.abs(refs)) < 5e-6


def test_circular_wraps_and_linear_does_not():
    # a filter that is a one-sample delay: circular output at t = 0 reads z[L-1]
    L, D, N = 256, 1, 1
    h = torch.zeros((N, D, L), device=DEV); h[0, 0, 1] = 1.0
    v = torch.arange(L, dtype=torch.float32, device=DEV).reshape(1, 1, L) + 1.0
    x = torch.ones_like(v)
    yc = H.forward(v, [x], H.filter_spectrum(h, circular=True))
    yl = H.forward(v, [x], H.filter_spectrum(h))
    torch.cuda.synchronize()
    assert abs(float(yc[0, 0, 0]) - float(L)) < 1e-3 and abs(float(yl[0, 0, 0])) < 1e-4
    assert torch.allclose(yc[0, 0, 1:], v[0, 0, :-1], atol=1e-3) and torch.allclose(yl[0, 0, 1:], v[0, 0, :-1], atol=1e-3)
