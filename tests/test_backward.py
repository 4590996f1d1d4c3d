"""GPU parity of hyena_backward (single-pass and four-step lengths) against
the float64 oracle's backward on the same inputs and the same filters.

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


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    monkeypatch.delenv("HYENA_FORCE_PATH", raising=False)
    monkeypatch.delenv("HYENA_FOURSTEP_N1", raising=False)


def _run(N, B, D, L, io, channels=None, seed=31, circular=False):
    cfg = Config("bwd", N, B, D, L, io, 32, seed)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    g = torch.Generator(device=DEV); g.manual_seed(seed + 7)
    gy = torch.randn((B, D, L), generator=g, device=DEV).to(v.dtype)
    h = H.filter_gen(params_to_device(p), L)
    spec = H.filter_spectrum(h, circular=circular)
    gv, gxs, gh = H.backward(v, xs, spec, gy)
    torch.cuda.synchronize()
    ds = list(range(D)) if channels is None else channels
    hn = _np(h)[:, ds]
    rv, rxs, rgh = O.hyena_backward(_np(v)[:, ds], [_np(x)[:, ds] for x in xs], hn, _np(gy)[:, ds],
                                    circular=circular)
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


@pytest.mark.parametrize("N,B,D,L,io", [(1, 1, 2, 128, "fp32"), (2, 3, 4, 256, "fp32"), (3, 2, 3, 2048, "fp32"),
                                        (2, 1, 2, 16384, "fp32"), (2, 2, 3, 1024, "bf16")])
def test_backward_circular_matches_oracle(N, B, D, L, io):
    """Periodic convolution (L = FFT length): the adjoint and the filter
    gradient are circular correlations."""
    got, ref = _run(N, B, D, L, io, circular=True)
    _check(got, ref, io)


@pytest.mark.parametrize("N,B,D,L,io", [(2, 2, 2, 32768, "fp32"), (2, 1, 2, 65536, "bf16"), (3, 1, 1, 131072, "fp32")])
def test_backward_circular_long_matches_oracle(N, B, D, L, io):
    """Periodic rows beyond the one-launch kernel: the four-step pipeline with
    the periodic reversal (32768 is planned on the single path forward, its
    spectrum rewritten into the four-step layout)."""
    got, ref = _run(N, B, D, L, io, circular=True)
    _check(got, ref, io)


def test_backward_full_width_sampled_channels():
    # the 2K-context shape (order 2, B = 4, D = 768, L = 2048), 6 channels
    got, ref = _run(2, 4, 768, 2048, "fp32", channels=[0, 1, 100, 383, 700, 767], seed=2)
    _check(got, ref, "fp32")


def test_backward_deterministic():
    a, _ = _run(2, 3, 4, 500, "fp32", channels=[0])
    b, _ = _run(2, 3, 4, 500, "fp32", channels=[0])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


LONG_CASES = [
    # N, B, D, L, io, forced path, forced n1 (four-step at small L: the oracle's direct sums stay fast)
    (2, 2, 3, 1000, "fp32", "fourstep", "16"), (3, 1, 2, 2048, "fp32", "fourstep", "64"),
    (1, 3, 2, 4096, "fp32", "fourstep", "32"), (2, 2, 2, 777, "bf16", "fourstep", "16"),
    (8, 1, 1, 512, "fp32", "fourstep", "16"),
    (2, 2, 2, 1000, "fp32", "fourstep", "25"), (2, 1, 3, 777, "bf16", "fourstep", "3"),   # odd column lengths
    (3, 2, 1, 2000, "fp32", "fourstep", "9"), (2, 2, 2, 1500, "fp32", "fourstep", "50"),
    (2, 2, 2, 12000, "fp32", None, None),     # single-path spectrum rewritten for the four-step backward
    (2, 1, 2, 20000, "fp32", None, None),     # four-step plan, ragged length
    (2, 1, 2, 65536, "bf16", None, None),     # the 64K shape's length
]


@pytest.mark.parametrize("N,B,D,L,io,force,n1", LONG_CASES)
def test_backward_long_matches_oracle(N, B, D, L, io, force, n1, monkeypatch):
    if force:
        monkeypatch.setenv("HYENA_FORCE_PATH", force)
    if n1:
        monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    got, ref = _run(N, B, D, L, io, seed=41 + N)
    _check(got, ref, io)


@pytest.mark.parametrize("B,D,L,circular,n1", [(3, 31, 2048, False, "16"), (2, 5, 32768, True, None),
                                               (2, 15, 6000, False, "25")])
def test_backward_long_several_pass_groups(B, D, L, circular, n1, monkeypatch):
    """A 1 MiB work budget splits the rows into several channel-major pass
    groups, the last one ragged: 93 rows of 16 KiB as 15 + 15 + 1 channels;
    10 periodic rows of 128 KiB as 2 + 2 + 1 channels; 30 rows of 50 KiB at
    an odd column length (25 x 256) as 7 + 7 + 1 channels.  Channels on both
    sides of every group boundary are checked."""
    monkeypatch.setenv("HYENA_WORK_MB", "1")
    if n1:
        monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
        monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    chans = sorted({0, 1, D // 2 - 1, D // 2, D - 2, D - 1} | ({14, 15, 29, 30} if D == 31 else set()))
    got, ref = _run(2, B, D, L, "fp32", channels=chans, seed=57, circular=circular)
    _check(got, ref, "fp32")


def test_backward_long_deterministic(monkeypatch):
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    monkeypatch.setenv("HYENA_FOURSTEP_N1", "16")
    a, _ = _run(2, 3, 2, 600, "fp32", channels=[1])
    b, _ = _run(2, 3, 2, 600, "fp32", channels=[1])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


@pytest.mark.parametrize("name,channels", [("C3", 3), ("C4", 2), ("C5b", 2)])
def test_backward_config_full_size_sampled(name, channels):
    """The backward on the full configuration shapes (the pass groups and
    column kernels the benchmark times: 64 x 1024 rows in two groups, 512 x
    2048 rows in eight, 50-point columns on lane pairs), checked on channels
    0, D - 1 and a seeded sample against the oracle's backward on the same
    inputs.  fp32 gradients beyond L = 64K against 5e-4, as the forward."""
    from workloads import CONFIGS
    cfg = CONFIGS[name]
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    g = torch.Generator(device=DEV); g.manual_seed(cfg.seed + 7)
    gy = torch.randn(v.shape, generator=g, device=DEV).to(v.dtype)
    h = H.filter_gen(params_to_device(p), cfg.L)
    spec = H.filter_spectrum(h)
    del h
    gv, gxs, gh = H.backward(v, xs, spec, gy)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.seed)
    ds = sorted({0, cfg.D - 1} | set(rng.choice(np.arange(1, cfg.D - 1), channels - 2, replace=False).tolist()
                                      if channels > 2 else set()))
    hn = O.filter_gen(p, cfg.L, channels=ds)
    sel = lambda t: t[:, ds].float().cpu().numpy().astype(np.float64)
    rv, rxs, rgh = O.hyena_backward(sel(v), [sel(x) for x in xs], hn, sel(gy))
    tol = TOL[cfg.io] if (cfg.io == "bf16" or cfg.L <= 65536) else 5e-4
    tol_gh = TOL_GH if cfg.L <= 65536 else 5e-4
    errs = [channel_errors(sel(gv), rv).max()] + [channel_errors(sel(a), r).max() for a, r in zip(gxs, rxs)]
    egh = channel_errors(gh[:, ds].cpu().numpy().astype(np.float64), rgh).max()
    print(f"{name} backward: channels {ds}, gv/gx max normalised error {max(errs):.3e}, gh {egh:.3e}")
    assert all(np.isfinite(errs)) and max(errs) <= tol, errs
    assert np.isfinite(egh) and egh <= tol_gh, egh
