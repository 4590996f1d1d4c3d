"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (per-channel max|y - y_ref| / max|y_ref|): 1e-4 for fp32 up to
L = 64K, 5e-4 for fp32 at L = 1M, 2e-2 for bf16 I/O (the oracle gets the same
bf16-rounded inputs, upcast exactly).
"""
import os

import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, channel_errors, check_rows, params_to_device, run_hip, sample_pairs
from workloads import CONFIGS, Config, make_activations, make_filter_params

pytestmark = pytest.mark.gpu

TOL_FP32, TOL_FP32_1M, TOL_BF16 = 1e-4, 5e-4, 2e-2


def _cfg(N, B, D, L, io="fp32", H_=32, seed=11, K=8):
    return Config("t", N, B, D, L, io, H_, seed, K=K)


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    monkeypatch.delenv("HYENA_FORCE_PATH", raising=False)
    monkeypatch.delenv("HYENA_FOURSTEP_N1", raising=False)


# ------------------------------------------------------------- filter_gen

@pytest.mark.parametrize("D,N,Hd,K,L,bias", [(16, 2, 32, 8, 256, 0.0), (5, 3, 64, 8, 1000, 0.5),
                                             (1, 1, 8, 0, 7, 0.3), (3, 2, 128, 16, 4096, 0.2),
                                             (7, 4, 16, 3, 333, 1.0)])
def test_filter_gen_matches_oracle(D, N, Hd, K, L, bias):
    cfg = _cfg(N, 1, D, L, H_=Hd, K=K)
    p = make_filter_params(cfg, bias_scale=bias)
    h = H.filter_gen(params_to_device(p), L).cpu().numpy()
    ref = O.filter_gen(p, L)
    err = np.max(np.abs(h - ref)) / np.max(np.abs(ref))
    assert err < 2e-6, err


# ------------------------------------------------------------- spectrum

@pytest.mark.parametrize("L,force,n1", [(1, None, None), (17, None, None), (256, None, None),
                                        (3000, None, None), (8192, None, None),
                                        (300, "fourstep", None), (1000, "fourstep", "64"),
                                        (5000, "fourstep", "256"), (20000, None, None)])
def test_spectrum_matches_oracle(L, force, n1, monkeypatch):
    if force:
        monkeypatch.setenv("HYENA_FORCE_PATH", force)
    if n1:
        monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    D, N = 3, 2
    cfg = _cfg(N, 1, D, L)
    p = make_filter_params(cfg, bias_scale=0.3)
    h = H.filter_gen(params_to_device(p), L)
    spec = H.filter_spectrum(h)
    got = H.spectrum_export(spec, D, N, L).cpu().numpy()
    M = H.plan(L)["M"]
    ref = O.filter_spectrum(h.cpu().numpy().astype(np.float64), M)   # same h: isolates the FFT
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err < 5e-6, err


def test_spectrum_window_only_closed_form():
    # W3 = 0, b3 = 1: h_t = a^t; spectrum is the geometric sum (closed form).
    L, D, N = 2048, 4, 1
    cfg = _cfg(N, 1, D, L)
    p = make_filter_params(cfg)
    p["W3"] = np.zeros_like(p["W3"]); p["b3"] = np.ones_like(p["b3"])
    h = H.filter_gen(params_to_device(p), L)
    got = H.spectrum_export(H.filter_spectrum(h), D, N, L).cpu().numpy()[0]
    M = H.plan(L)["M"]
    k = np.arange(M // 2 + 1)
    w = np.exp(-2j * np.pi * k / M)
    for d in range(D):
        a = np.exp(-float(p["alpha"][d]) / L)
        ref = (1 - (a * w) ** L) / (1 - a * w)
        assert np.max(np.abs(got[d] - ref)) / np.max(np.abs(ref)) < 5e-6


# ------------------------------------------------------------- forward, small shapes

SMALL = [
    # N, B, D, L, io
    (1, 1, 1, 1, "fp32"), (2, 1, 2, 2, "fp32"), (2, 1, 3, 3, "fp32"), (2, 2, 3, 17, "fp32"),
    (3, 3, 5, 100, "fp32"), (2, 1, 16, 256, "fp32"), (2, 4, 6, 1000, "fp32"), (4, 2, 4, 2048, "fp32"),
    (2, 3, 3, 4096, "fp32"), (2, 1, 4, 8192, "fp32"), (1, 2, 2, 8191, "fp32"), (8, 1, 2, 64, "fp32"),
    (2, 1, 5, 300, "bf16"), (3, 2, 4, 2048, "bf16"), (2, 3, 3, 8192, "bf16"),
]


@pytest.mark.parametrize("N,B,D,L,io", SMALL)
def test_forward_small_matches_oracle(N, B, D, L, io):
    cfg = _cfg(N, B, D, L, io=io)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    _, _, y = run_hip(p, L, v, xs)
    pairs = [(b, d) for b in range(B) for d in range(D)]
    check_rows(y, p, L, v, xs, pairs, TOL_FP32 if io == "fp32" else TOL_BF16)


FOURSTEP = [
    # N, B, D, L, io, n1
    (2, 1, 3, 1, "fp32", "16"), (2, 2, 3, 100, "fp32", "16"), (2, 1, 4, 1000, "fp32", "32"),
    (3, 3, 3, 3000, "fp32", "64"), (2, 2, 2, 5000, "fp32", "128"), (2, 1, 3, 8192, "fp32", "256"),
    (2, 1, 2, 2000, "fp32", "512"), (2, 2, 2, 4000, "fp32", "1024"), (2, 3, 5, 6000, "bf16", "16"),
    (1, 1, 1, 700, "bf16", "64"), (2, 2, 3, 4097, "fp32", "32"), (2, 1, 2, 999, "bf16", "16"),
]


@pytest.mark.parametrize("N,B,D,L,io,n1", FOURSTEP)
def test_forward_fourstep_matches_oracle(N, B, D, L, io, n1, monkeypatch):
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    cfg = _cfg(N, B, D, L, io=io)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    _, _, y = run_hip(p, L, v, xs)
    pairs = [(b, d) for b in range(B) for d in range(D)]
    check_rows(y, p, L, v, xs, pairs, TOL_FP32 if io == "fp32" else TOL_BF16)


@pytest.mark.parametrize("L", [9000, 20000])
def test_forward_long_auto_path(L):
    cfg = _cfg(2, 3, 3, L)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    _, _, y = run_hip(p, L, v, xs)
    check_rows(y, p, L, v, xs, [(b, d) for b in range(3) for d in range(3)], TOL_FP32)


@pytest.mark.slow
def test_forward_maximum_length():
    # Largest supported L = 2^22 (real FFT of 2^23 points); one channel pair.
    L = 1 << 22
    cfg = _cfg(2, 1, 2, L, H_=16)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, _, y = run_hip(p, L, v, xs)
    check_rows(y, p, L, v, xs, [(0, 1)], TOL_FP32_1M)


def test_small_workspace_still_correct():
    # A workspace for a single row forces one row per pass group.
    L, cfg = 20000, _cfg(2, 2, 3, 20000)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    h = H.filter_gen(params_to_device(p), L)
    spec = H.filter_spectrum(h)
    ws = H._empty(H.plan(L)["M"] // 2 * 8, dtype=torch.uint8, device=DEV)
    y = H.forward(v, xs, spec, workspace=ws)
    torch.cuda.synchronize()
    check_rows(y, p, L, v, xs, [(b, d) for b in range(2) for d in range(3)], TOL_FP32)


def test_fourstep_pass_groups_bitwise_equal(monkeypatch):
    """Pass groups of whole channels (all batch rows of each) or of single
    rows, whatever the workspace allows, compute every row the same way."""
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    monkeypatch.setenv("HYENA_FOURSTEP_N1", "16")
    cfg = _cfg(2, 3, 5, 3000)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, spec, y = run_hip(p, cfg.L, v, xs)
    check_rows(y, p, cfg.L, v, xs, [(0, 0), (1, 2), (2, 4)], TOL_FP32)
    row_bytes = H.plan(cfg.L)["M"] // 2 * 8
    for rows in (1, 2, 3, 4, 7):      # below B, one channel, one channel + spare, several channels
        ws = H._empty(rows * row_bytes, dtype=torch.uint8, device=DEV)
        y2 = H.forward(v, xs, spec, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"workspace of {rows} rows"


# ------------------------------------------------------------- robustness

def test_deterministic_bitwise():
    cfg = _cfg(2, 3, 5, 3000)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, spec, y1 = run_hip(p, cfg.L, v, xs)
    y2 = H.forward(v, xs, spec)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("L,io", [(1000, "fp32"), (20000, "bf16")])
def test_output_guard_regions_untouched(L, io):
    cfg = _cfg(2, 1, 3, L, io=io)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    h = H.filter_gen(params_to_device(p), L)
    spec = H.filter_spectrum(h)
    n = v.numel()
    pad = 4096
    big = torch.full((n + 2 * pad,), 12345.0, dtype=v.dtype, device=DEV)
    y = big[pad:pad + n].view_as(v)
    H.forward(v, xs, spec, out=y)
    torch.cuda.synchronize()
    assert torch.all(big[:pad] == 12345.0) and torch.all(big[pad + n:] == 12345.0)
    check_rows(y, p, L, v, xs, [(0, 0), (0, 2)], TOL_FP32 if io == "fp32" else TOL_BF16)


@pytest.mark.parametrize("L", [3000, 20000])
def test_rows_of_very_different_magnitude(L):
    # Rounding must stay relative to each row's own scale: neighbouring rows
    # (batch or channel) 1e4 times larger may not leak error into a small row.
    cfg = _cfg(2, 2, 4, L)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    v[0] *= 1e4
    v[1, 2] *= 1e-3
    _, _, y = run_hip(p, L, v, xs)
    check_rows(y, p, L, v, xs, [(b, d) for b in range(2) for d in range(4)], TOL_FP32)


def test_spectrum_reused_across_batches():
    cfg = _cfg(2, 4, 3, 1500)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, spec, y = run_hip(p, cfg.L, v, xs)
    y1 = H.forward(v[1:2].contiguous(), [x[1:2].contiguous() for x in xs], spec)
    torch.cuda.synchronize()
    check_rows(y1, p, cfg.L, v[1:2], [x[1:2] for x in xs], [(0, 0), (0, 1), (0, 2)], TOL_FP32)
    check_rows(y, p, cfg.L, v, xs, [(b, d) for b in range(4) for d in range(3)], TOL_FP32)


def test_bf16_intermediate_every_row_order2():
    """bf16 activations at order 2 keep the four-step intermediate as bf16
    pairs: every row of a 64K-length shape (two channel groups of the
    filter, batch rows sharing a channel) stays inside the bf16 bound; the
    same shape at order 3 (fp32 intermediate) too."""
    for N in (2, 3):
        cfg = Config("w", N, 2, 24, 65536, "bf16", 32, 41 + N)
        assert H.plan(cfg.L)["path"] == "fourstep"
        p = make_filter_params(cfg, bias_scale=0.2)
        v, xs = make_activations(cfg, DEV)
        _, _, y = run_hip(p, cfg.L, v, xs)
        check_rows(y, p, cfg.L, v, xs, [(b, d) for b in range(cfg.B) for d in range(cfg.D)], TOL_BF16)


# ------------------------------------------------------------- configurations

CFG_SAMPLES = {"C1": 16, "C2": 48, "C3": 6, "C4": 3, "C5a": 5, "C5b": 5}


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5a", "C5b"])
def test_config_full_size_sampled(name):
    cfg = CONFIGS[name]
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, spec, y = run_hip(p, cfg.L, v, xs)
    del spec
    if name == "C1":
        pairs = [(b, d) for b in range(cfg.B) for d in range(cfg.D)]
    else:
        pairs = sample_pairs(cfg.B, cfg.D, CFG_SAMPLES[name], seed=cfg.seed)
    if cfg.io == "bf16":
        tol = TOL_BF16
    else:
        tol = TOL_FP32_1M if cfg.L >= (1 << 20) else TOL_FP32
    err = check_rows(y, p, cfg.L, v, xs, pairs, tol)
    print(f"{name}: max normalised error {err:.3e} over {len(pairs)} rows")
