"""GPU parity of the four-step path at FFT lengths 2^a 3^b 5^c (column lengths
q = 3, 5, 9, 15, 25, 27 on one lane, or 2q on a lane pair exchanging through
DPP, with power-of-two rows): column lengths forced at
small L, where the oracle's direct sums are fast; the lengths the planner
itself sends there; spectra at those lengths; pass groups of any size; batch
rows sharing a channel (channel-major launches padded to whole XCD rounds);
and the backward.  Zero padding to any length >= 2L - 1 gives the same
causal convolution (gist.science HyenaND summary, section 手法: HyenaND)."""
import numpy as np
import pytest
import torch

import hyena_long_conv_amd as H
import oracle as O
from tests.gpu_helpers import DEV, check_rows, params_to_device, run_hip
from workloads import Config, make_activations, make_filter_params

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    for k in ("HYENA_FORCE_PATH", "HYENA_FOURSTEP_N1", "HYENA_WORK_MB"):
        monkeypatch.delenv(k, raising=False)


def _cfg(N, B, D, L, io="fp32", seed=23):
    return Config("s", N, B, D, L, io, 32, seed)


ODD = [
    # N, B, D, L, io, n1
    (2, 1, 3, 100, "fp32", "3"), (2, 2, 3, 1000, "fp32", "5"), (3, 3, 2, 2000, "fp32", "9"),
    (2, 1, 4, 3001, "fp32", "15"), (2, 2, 3, 5000, "fp32", "25"), (4, 1, 2, 4097, "fp32", "27"),
    (2, 3, 3, 6000, "bf16", "25"), (1, 1, 1, 1, "fp32", "5"), (2, 2, 2, 999, "bf16", "3"),
    (8, 1, 1, 512, "fp32", "27"), (2, 4, 5, 1500, "fp32", "9"),
    # lane-pair columns (2q)
    (2, 1, 3, 100, "fp32", "6"), (2, 2, 3, 1000, "fp32", "10"), (3, 3, 2, 2001, "fp32", "18"),
    (2, 1, 4, 3000, "bf16", "30"), (2, 2, 3, 5000, "fp32", "50"), (4, 1, 2, 4097, "fp32", "54"),
    (1, 1, 1, 1, "fp32", "6"), (2, 3, 2, 999, "bf16", "50"),
]


@pytest.mark.parametrize("N,B,D,L,io,n1", ODD)
def test_forward_odd_columns_match_oracle(N, B, D, L, io, n1, monkeypatch):
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    plan = H.plan(L)
    assert plan["n1"] == int(n1) and plan["M"] >= 2 * L and plan["n2"] & (plan["n2"] - 1) == 0
    cfg = _cfg(N, B, D, L, io)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    _, _, y = run_hip(p, L, v, xs)
    check_rows(y, p, L, v, xs, [(b, d) for b in range(B) for d in range(D)], TOL[io])


@pytest.mark.parametrize("L,n1,n2,B,D,io", [(16385, 9, 2048, 1, 3, "fp32"), (20000, 10, 2048, 2, 2, "fp32"),
                                            (50000, 25, 2048, 2, 2, "bf16"), (70000, 50, 2048, 1, 2, "fp32"),
                                            (100000, 50, 2048, 2, 3, "bf16")])
def test_planner_smooth_lengths_match_oracle(L, n1, n2, B, D, io):
    plan = H.plan(L)
    assert plan["path"] == "fourstep" and (plan["n1"], plan["n2"]) == (n1, n2)
    assert plan["M"] == 2 * n1 * n2 and 2 * L <= plan["M"] < 1 << (2 * L - 1).bit_length()
    cfg = _cfg(2, B, D, L, io)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    _, _, y = run_hip(p, L, v, xs)
    check_rows(y, p, L, v, xs, [(b, d) for b in range(B) for d in range(D)], TOL[io])


@pytest.mark.parametrize("L,n1", [(300, "3"), (1000, "15"), (5000, "25"), (700, "27"), (300, "6"), (2000, "50"),
                                  (999, "54")])
def test_spectrum_odd_columns_matches_oracle(L, n1, monkeypatch):
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    D, N = 3, 2
    p = make_filter_params(_cfg(N, 1, D, L), bias_scale=0.3)
    h = H.filter_gen(params_to_device(p), L)
    got = H.spectrum_export(H.filter_spectrum(h), D, N, L).cpu().numpy()
    M = H.plan(L)["M"]
    ref = O.filter_spectrum(h.cpu().numpy().astype(np.float64), M)
    assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) < 5e-6


@pytest.mark.parametrize("n1", ["25", "50"])
def test_odd_column_pass_groups_bitwise_equal(n1, monkeypatch):
    """Workspaces of 1..7 rows (below B, one channel, several channels, the
    last group ragged): every row computed the same way as in one group."""
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    monkeypatch.setenv("HYENA_FOURSTEP_N1", n1)
    cfg = _cfg(2, 3, 5, 3000)
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, spec, y = run_hip(p, cfg.L, v, xs)
    check_rows(y, p, cfg.L, v, xs, [(0, 0), (1, 2), (2, 4)], TOL["fp32"])
    row_bytes = H.plan(cfg.L)["M"] // 2 * 8
    for rows in (1, 2, 3, 4, 7):
        ws = H._empty(rows * row_bytes, dtype=torch.uint8, device=DEV)
        y2 = H.forward(v, xs, spec, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"workspace of {rows} rows"


def test_forward_work_budget_override_bitwise_equal(monkeypatch):
    """HYENA_WORK_MB splits the rows into several pass groups (here 2 rows
    of 800 KiB per 2 MiB group, one channel's batch rows; FFT length
    2 x 50 x 2048); results equal the one-group run."""
    cfg = _cfg(2, 2, 7, 100000, "bf16")
    p = make_filter_params(cfg)
    v, xs = make_activations(cfg, DEV)
    _, spec, y = run_hip(p, cfg.L, v, xs)
    monkeypatch.setenv("HYENA_WORK_MB", "2")
    y2 = H.forward(v, xs, spec)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    check_rows(y2, p, cfg.L, v, xs, [(0, 0), (1, 6), (1, 3)], TOL["bf16"])
