"""hyena_forward_static (the forward whose four-step intermediate lives in the
library's static device scratch, for callers that cannot allocate) against
hyena_forward, through the C ABI: two calls in a row on the same GPU, the
second with a smaller input, each equal to hyena_forward's output and within
the operator's tolerance of the float64 oracle on sampled rows."""
import ctypes

import pytest
import torch

import hyena_long_conv_amd as H
from tests.gpu_helpers import DEV, check_rows, params_to_device
from workloads import Config, make_activations, make_filter_params

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    for k in ("HYENA_FORCE_PATH", "HYENA_FOURSTEP_N1", "HYENA_WORK_MB"):
        monkeypatch.delenv(k, raising=False)


def _static_call(v, xs, spec, y):
    lib = H.lib()
    B, D, L = v.shape
    io = 0 if v.dtype == torch.float32 else 1
    xp = (ctypes.c_void_p * len(xs))(*[x.data_ptr() for x in xs])
    code = lib.hyena_forward_static(ctypes.c_void_p(v.data_ptr()), xp, ctypes.c_void_p(spec.data_ptr()),
                                    ctypes.c_void_p(y.data_ptr()), B, D, len(xs), L, io,
                                    ctypes.c_void_p(torch.cuda.current_stream(v.device).cuda_stream))
    assert code == 0, H.lib().hyena_status_str(code)


def _case(N, B, D, L, io, seed):
    cfg = Config("na", N, B, D, L, io, 32, seed)
    p = make_filter_params(cfg, bias_scale=0.2)
    v, xs = make_activations(cfg, DEV)
    spec = H.filter_spectrum(H.filter_gen(params_to_device(p), L))
    ref = H.forward(v, xs, spec)                    # the existing entry point, with its workspace
    y = torch.full_like(v, float("nan"))
    _static_call(v, xs, spec, y)
    torch.cuda.synchronize()
    return p, v, xs, ref, y


def test_forward_static_two_calls_second_smaller():
    # 1st: 80 rows of L = 100000, bf16 (FFT length 204800, the intermediate as bf16 pairs: 400 KiB per
    # row, one pass group)
    p, v, xs, ref, y = _case(2, 2, 40, 100000, "bf16", 71)
    assert torch.equal(y, ref)
    check_rows(y, p, 100000, v, xs, [(0, 0), (1, 39), (1, 17)], 2e-2)
    # 2nd, smaller: 1 x 3 rows at L = 20000, fp32, reusing the scratch the first call left behind
    p, v, xs, ref, y = _case(2, 1, 3, 20000, "fp32", 72)
    assert torch.equal(y, ref)
    check_rows(y, p, 20000, v, xs, [(0, 0), (0, 1), (0, 2)], 1e-4)


def test_forward_static_more_rows_than_the_scratch_holds():
    # L = 1M rows are 8 MiB: 20 rows take two pass groups in 128 MiB
    p, v, xs, ref, y = _case(2, 1, 20, 1 << 20, "fp32", 73)
    assert torch.equal(y, ref)
    check_rows(y, p, 1 << 20, v, xs, [(0, 0), (0, 19)], 5e-4)


def test_forward_static_single_path_and_binding():
    p, v, xs, ref, y = _case(3, 2, 5, 2048, "fp32", 74)
    assert torch.equal(y, ref)
    y2 = H.forward_static(v, xs, H.filter_spectrum(H.filter_gen(params_to_device(p), 2048)), torch.empty_like(v))
    torch.cuda.synchronize()
    assert torch.equal(y2, ref)
