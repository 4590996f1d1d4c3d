"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding and compare it with the float64 oracle on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import hyena_long_conv_amd as H
import oracle as O

DEV = "cuda:0"


def params_to_device(params: dict) -> dict:
    return {k: (torch.from_numpy(v).to(DEV) if isinstance(v, np.ndarray) else v) for k, v in params.items()}


def run_hip(params: dict, L: int, v, xs, spec=None):
    """filter_gen -> filter_spectrum -> forward on the GPU; returns (h, spec, y)."""
    h = H.filter_gen(params_to_device(params), L)
    if spec is None:
        spec = H.filter_spectrum(h)
    y = H.forward(v, xs, spec)
    torch.cuda.synchronize()
    return h, spec, y


def channel_errors(y, yref):
    """Per-channel normalised max error max|y - yref| / max|yref| (rows on the last axis)."""
    y = np.asarray(y, np.float64)
    yref = np.asarray(yref, np.float64)
    num = np.max(np.abs(y - yref), axis=-1)
    den = np.max(np.abs(yref), axis=-1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num <= 1e-30, 0.0, np.inf))
    return out


def oracle_rows(params: dict, L: int, v, xs, pairs):
    """Oracle outputs for the (b, d) rows in ``pairs`` (inputs copied from the device)."""
    ds = sorted({d for _, d in pairs})
    href = O.filter_gen(params, L, channels=ds)          # [N, len(ds), L]
    col = {d: i for i, d in enumerate(ds)}
    out = []
    for b, d in pairs:
        vb = v[b, d].float().cpu().numpy().astype(np.float64)[None]
        xb = [x[b, d].float().cpu().numpy().astype(np.float64)[None] for x in xs]
        hb = href[:, [col[d]], :]
        out.append(O.hyena_forward(vb, xb, hb)[0])
    return np.stack(out)


def sample_pairs(B: int, D: int, k: int, seed: int):
    """Always (0, 0) and (B-1, D-1), plus a seeded uniform sample, k pairs in total."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (B - 1, D - 1)}
    while len(pairs) < min(k, B * D):
        pairs.add((int(rng.integers(B)), int(rng.integers(D))))
    return sorted(pairs)


def check_rows(y, params, L, v, xs, pairs, tol):
    ref = oracle_rows(params, L, v, xs, pairs)
    got = np.stack([y[b, d].float().cpu().numpy() for b, d in pairs])
    err = channel_errors(got, ref)
    worst = int(np.argmax(err))
    assert np.all(np.isfinite(got)), "non-finite output"
    assert err[worst] <= tol, f"max normalised error {err[worst]:.3e} at (b,d)={pairs[worst]} > {tol}"
    return float(err[worst])
