"""The odd-length register DFTs of the four-step column pass (csrc/fft_odd.hpp),
compiled for the host and checked against numpy's FFT in float64.  Runs on CPU."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hyena_long_conv_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("fft_odd") / "fft_odd_host")
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", CSRC,
           os.path.join(ROOT, "tests", "fft_odd_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, tmp, n, inv, x):
    src, dst = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
    x.astype(np.complex64).tofile(src)
    r = subprocess.run([exe, str(n), str(int(inv)), src, dst, str(x.shape[0])], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return np.fromfile(dst, dtype=np.complex64).reshape(x.shape)


@pytest.mark.parametrize("n", [3, 5, 9, 15, 25, 27])
@pytest.mark.parametrize("inv", [False, True])
def test_register_dft_matches_numpy(harness, tmp_path, n, inv):
    rng = np.random.default_rng(n * 2 + inv)
    x = (rng.standard_normal((64, n)) + 1j * rng.standard_normal((64, n))).astype(np.complex64)
    got = _run(harness, str(tmp_path), n, inv, x)
    xd = x.astype(np.complex128)
    ref = n * np.fft.ifft(xd, axis=1) if inv else np.fft.fft(xd, axis=1)
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err < 2e-6, err
    # unit impulses give the DFT matrix columns exactly up to float rounding
    eye = np.eye(n, dtype=np.complex64)
    cols = _run(harness, str(tmp_path), n, inv, eye)
    k = np.arange(n)
    W = np.exp((2j if inv else -2j) * np.pi * np.outer(k, k) / n)
    assert np.max(np.abs(cols - W)) < 1e-6


def test_inverse_undoes_forward(harness, tmp_path):
    rng = np.random.default_rng(7)
    for n in (3, 5, 9, 15, 25, 27):
        x = (rng.standard_normal((8, n)) + 1j * rng.standard_normal((8, n))).astype(np.complex64)
        y = _run(harness, str(tmp_path), n, False, x)
        z = _run(harness, str(tmp_path), n, True, y) / n
        assert np.max(np.abs(z - x)) < 1e-5 * np.max(np.abs(x))
