"""GPU parity of hyena_backward (single-pass lengths) against the float64
oracle's backward on the same inputs and the same filters.

Tolerances (per row, max |got - ref| / max |ref|): gv and gx_n 1e-4 for fp32,
2e-2 for bf16 (stored results rounded to bf16); gh 1e-4 (fp32 output, the
internal arithmetic is fp32 for both I/O dtypes).  Gradients of a channel
depend only on that channel's rows and filters, so the full-width shape is
checked exactly on a sample of channels."""
import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, channel_errors, params_to_device
from workloads import Config, make_activations, make_filter_params

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
TOL_GH = 1e-4


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


CASES = [
    # N, B, D, L, io
    (1, 1, 1, 1, "fp32"), (2, 1, 3, 17, "fp32"), (2, 3, 4, 100, "fp32"), (3, 2, 5, 1000, "fp32"),
    (2, 4, 8, 2048, "fp32"), (2, 1, 2, 8191, "fp32"), (8, 1, 2, 64, "fp32"), (1, 2, 3, 4096, "fp32"),
    (2, 2, 3, 300, "bf16"), (3, 1, 4, 4096, "bf16"), (2, 3, 2, 2047, "bf16"),
]


def _run(N, B, D, L, io, channels=None, seed=31):
    cfg = Config("bwd", N, B, D, L, io, 32, seed)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    g = torch.Generator(device=DEV); g.manual_seed(seed + 7)
    gy = torch.randn((B, D, L), generator=g, device=DEV).to(v.dtype)
    h = H.filter_gen(params_to_device(p), L)
    spec = H.filter_spectrum(h)
    gv, gxs, gh = H.backward(v, xs, spec, gy)
    torch.cuda.synchronize()
    ds = list(range(D)) if channels is None else channels
    hn = _np(h)[:, ds]
    rv, rxs, rgh = O.hyena_backward(_np(v)[:, ds], [_np(x)[:, ds] for x in xs], hn, _np(gy)[:, ds])
    return (_np(gv)[:, ds], [_np(t)[:, ds] for t in gxs], _np(gh)[:, ds]), (rv, rxs, rgh)


def _check(got, ref, io):
    gv, gxs, gh = got
    rv, rxs, rgh = ref
    assert all(np.all(np.isfinite(a)) for a in [gv, gh] + gxs)
    e = channel_errors(gv, rv).max()
    assert e <= TOL[io], ("gv", e)
    for n, (a, r) in enumerate(zip(gxs, rxs)):
        e = channel_errors(a, r).max()
        assert e <= TOL[io], (f"gx{n + 1}", e)
    e = channel_errors(gh, rgh).max()
    assert e <= TOL_GH, ("gh", e)


@pytest.mark.parametrize("N,B,D,L,io", CASES)
def test_backward_matches_oracle(N, B, D, L, io):
    got, ref = _run(N, B, D, L, io)
    _check(got, ref, io)


def test_backward_full_width_sampled_channels():
    # the 2K-context shape (order 2, B = 4, D = 768, L = 2048), 6 channels
    got, ref = _run(2, 4, 768, 2048, "fp32", channels=[0, 1, 100, 383, 700, 767], seed=2)
    _check(got, ref, "fp32")


def test_backward_deterministic():
    a, _ = _run(2, 3, 4, 500, "fp32", channels=[0])
    b, _ = _run(2, 3, 4, 500, "fp32", channels=[0])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


def test_backward_rejects_long_rows():
    cfg = Config("bwd", 2, 1, 2, 9000, "fp32", 32, 3)
    v, xs = make_activations(cfg, DEV)
    assert H.backward_workspace_bytes(1, 2, 2, 9000) == -1
    with pytest.raises(H.HyenaError):
        H.backward(v, xs, torch.zeros(16, dtype=torch.uint8, device=DEV), v.clone(),
                   workspace=torch.empty(1 << 20, dtype=torch.uint8, device=DEV))
