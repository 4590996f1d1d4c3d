"""Seeded random shapes through the C ABI against the float64 oracle: lengths
on both sides of every plan boundary (single pass / four-step, power of two
or padded, odd and prime L), orders 1-4, odd B and D, both I/O dtypes.
Forward on sampled (b, d) rows; backward (linear and circular) on the first
and last channel.  The shape of each case is in its test id."""
import random

import pytest
import torch

import hyena_long_conv_amd as H
from tests.gpu_helpers import check_rows, params_to_device, sample_pairs
from tests.test_backward import _check, _run
from workloads import Config, make_activations, make_filter_params

pytestmark = pytest.mark.gpu

_LF = [1, 2, 3, 5, 7, 31, 255, 256, 257, 1000, 1023, 1025, 2047, 2049, 4095, 4097, 8191, 8192, 8193,
       16383, 16384, 16385, 32767, 32769, 65535, 65537, 100003, 131071, 131073, 262145]


def _fwd_cases(n, seed):
    r = random.Random(seed)
    return [(r.choice([1, 2, 3, 4]), r.choice([1, 2, 3]), r.choice([1, 3, 8, 13]), r.choice(_LF),
             r.choice(["fp32", "bf16"])) for _ in range(n)]


def _bwd_cases(n, seed):
    r = random.Random(seed)
    out = []
    for _ in range(n):
        circ = r.random() < 0.35
        L = r.choice([128, 256, 2048, 8192, 16384, 32768] if circ else
                     [1, 3, 17, 255, 1000, 2047, 2048, 4097, 8193, 20000, 65536])
        out.append((r.choice([1, 2, 3]), r.choice([1, 2, 3]), r.choice([1, 2, 5]), L,
                    r.choice(["fp32", "bf16"]), circ))
    return out


@pytest.mark.parametrize("N,B,D,L,io", _fwd_cases(40, 20261203))
def test_forward_random_shape(N, B, D, L, io):
    cfg = Config("rand", N, B, D, L, io, 32, 1000 + L % 997 + 7 * N + D)
    p = make_filter_params(cfg)
    spec = H.filter_spectrum(H.filter_gen(params_to_device(p), L))
    v, xs = make_activations(cfg, "cuda:0")
    y = H.forward(v, xs, spec)
    torch.cuda.synchronize()
    tol = 2e-2 if io == "bf16" else 1e-4
    check_rows(y, p, L, v, xs, sample_pairs(B, D, 3, L + N), tol)


@pytest.mark.parametrize("N,B,D,L,io,circular", _bwd_cases(16, 777))
def test_backward_random_shape(N, B, D, L, io, circular):
    got, ref = _run(N, B, D, L, io, channels=[0, D - 1] if D > 2 else None, seed=500 + L % 89 + N,
                    circular=circular)
    _check(got, ref, io)


def _circ_cases(n, seed):
    r = random.Random(seed)
    return [(r.choice([1, 2, 3, 4]), r.choice([1, 2, 3]), r.choice([1, 2, 3]),
             r.choice([64, 128, 512, 1024, 4096, 8192, 16384, 32768, 65536]), r.choice(["fp32", "bf16"]))
            for _ in range(n)]


@pytest.mark.parametrize("N,B,D,L,io", _circ_cases(10, 4242))
def test_circular_forward_random_shape(N, B, D, L, io):
    import numpy as np

    import oracle as O
    from tests.gpu_helpers import channel_errors

    cfg = Config("randc", N, B, D, L, io, 32, 300 + L % 101 + N)
    p = make_filter_params(cfg, bias_scale=0.2)
    h = H.filter_gen(params_to_device(p), L)
    v, xs = make_activations(cfg, "cuda:0")
    y = H.forward(v, xs, H.filter_spectrum(h, circular=True))
    torch.cuda.synchronize()
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    ref = O.hyena_forward(f64(v), [f64(x) for x in xs], f64(h), conv=O.circular_conv)
    assert channel_errors(f64(y), ref).max() <= (1e-4 if io == "fp32" else 2e-2)
