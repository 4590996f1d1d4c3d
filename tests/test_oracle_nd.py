"""Pins of the oracle's grid convolutions (the gist.science HyenaND summary,
"手法: HyenaND": native N-D convolution by the N-D FFT, circular boundaries
for periodic systems, twice-padded non-circular ones for images and volumes).

Each pin checks the oracle against something other than itself: a library
routine for a special case (scipy's N-D convolution, numpy's FFTs), the
oracle's own 1-D causal and circular convolutions (pinned in their own
files), closed forms (separable kernels, shifted deltas) and invariants.
"""
import numpy as np
import pytest
from scipy.signal import convolve

from oracle import hyena_oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _scipy_linear(K, z, ndim):
    """y[t] = sum_s K[t - s] z[s] via scipy's full convolution, cropped to the
    grid: the full output index of offset 0 is L - 1 on every axis."""
    Ls = z.shape[-ndim:]
    full = convolve(z, K, mode="full", method="direct")
    return full[tuple(slice(L - 1, 2 * L - 1) for L in Ls)]


@pytest.mark.parametrize("shape", [(5, 6), (8, 8), (1, 7), (3, 1), (4, 3, 5), (2, 2, 2)])
def test_linear_matches_scipy(shape):
    rng = _rng(sum(shape))
    ndim = len(shape)
    z = rng.standard_normal(shape)
    K = rng.standard_normal(tuple(2 * L - 1 for L in shape))
    ref = _scipy_linear(K, z, ndim)
    np.testing.assert_allclose(O.nd_conv_direct(K, z, ndim), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.nd_conv_fft(K, z, ndim), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(8, 4), (16, 16), (4, 8, 2), (8, 8, 8)])
def test_circular_matches_numpy_fft(shape):
    rng = _rng(3 * sum(shape))
    ndim = len(shape)
    z = rng.standard_normal((2,) + shape)
    K = rng.standard_normal(shape)
    axes = tuple(range(-ndim, 0))
    ref = np.fft.ifftn(np.fft.fftn(K, axes=axes) * np.fft.fftn(z, axes=axes), axes=axes).real
    np.testing.assert_allclose(O.nd_conv_direct(K, z, ndim, circular=True), ref, atol=1e-12)
    np.testing.assert_allclose(O.nd_conv_fft(K, z, ndim, circular=True), ref, atol=1e-12)


def test_ndfft_matches_numpy():
    rng = _rng(11)
    x = rng.standard_normal((3, 8, 16, 4)) + 1j * rng.standard_normal((3, 8, 16, 4))
    np.testing.assert_allclose(O.ndfft(x, 3), np.fft.fftn(x, axes=(1, 2, 3)), atol=1e-11)
    np.testing.assert_allclose(O.ndfft(x, 2, inverse=True), np.fft.ifftn(x, axes=(2, 3)), atol=1e-12)


def test_one_axis_reduces_to_the_causal_and_circular_convolutions():
    """With one axis and a kernel that is zero at negative offsets the grid
    convolution is the 1-D causal one; circular mode is the 1-D periodic one."""
    rng = _rng(5)
    L = 37
    h = rng.standard_normal((3, L))
    z = rng.standard_normal((2, 3, L))
    K = np.concatenate([np.zeros((3, L - 1)), h], axis=-1)     # index o + L - 1
    np.testing.assert_allclose(O.nd_conv_direct(K, z, 1), O.causal_conv_direct(h, z), atol=1e-12)
    Lc = 32
    hc = rng.standard_normal((3, Lc))
    zc = rng.standard_normal((2, 3, Lc))
    np.testing.assert_allclose(O.nd_conv_direct(hc, zc, 1, circular=True), O.circular_conv(hc, zc), atol=1e-12)


def test_separable_kernel_closed_form():
    """K = a (x) b and z = u (x) w give y = (a * u)_crop (x) (b * w)_crop."""
    rng = _rng(7)
    L1, L2 = 6, 9
    a, b = rng.standard_normal(2 * L1 - 1), rng.standard_normal(2 * L2 - 1)
    u, w = rng.standard_normal(L1), rng.standard_normal(L2)
    y1 = np.convolve(u, a)[L1 - 1:2 * L1 - 1]
    y2 = np.convolve(w, b)[L2 - 1:2 * L2 - 1]
    y = O.nd_conv_direct(np.outer(a, b), np.outer(u, w), 2)
    np.testing.assert_allclose(y, np.outer(y1, y2), atol=1e-12)


def test_shifted_delta_kernels():
    rng = _rng(9)
    L1, L2 = 5, 7
    z = rng.standard_normal((L1, L2))
    for o1, o2 in [(0, 0), (2, -3), (-4, 6), (1, 0)]:
        K = np.zeros((2 * L1 - 1, 2 * L2 - 1))
        K[o1 + L1 - 1, o2 + L2 - 1] = 1.0
        ref = np.zeros_like(z)
        for t1 in range(L1):
            for t2 in range(L2):
                s1, s2 = t1 - o1, t2 - o2
                if 0 <= s1 < L1 and 0 <= s2 < L2:
                    ref[t1, t2] = z[s1, s2]
        assert np.array_equal(O.nd_conv_direct(K, z, 2), ref)
        Kc = np.zeros((8, 8))
        Kc[o1 % 8, o2 % 8] = 1.0
        zc = rng.standard_normal((8, 8))
        assert np.array_equal(O.nd_conv_direct(Kc, zc, 2, circular=True), np.roll(zc, (o1, o2), axis=(0, 1)))


def test_circular_sum_invariant():
    """Periodic convolution multiplies the sums: sum_t y = sum K * sum z."""
    rng = _rng(13)
    K = rng.standard_normal((4, 8, 8))
    z = rng.standard_normal((4, 8, 8))
    y = O.nd_conv_direct(K, z, 3, circular=True)
    assert abs(y.sum() - K.sum() * z.sum()) < 1e-10


def test_non_power_of_two_circular_uses_brute_force():
    rng = _rng(17)
    K = rng.standard_normal((6, 5))
    z = rng.standard_normal((6, 5))
    ref = np.fft.ifft2(np.fft.fft2(K) * np.fft.fft2(z)).real
    np.testing.assert_allclose(O.nd_conv(K, z, 2, circular=True), ref, atol=1e-12)


def test_nd_forward_recurrence():
    rng = _rng(19)
    B, D, N, L1, L2 = 2, 3, 3, 4, 5
    v = rng.standard_normal((B, D, L1, L2))
    xs = [rng.standard_normal((B, D, L1, L2)) for _ in range(N)]
    # delta kernels: y = v * x_1 * x_2 * x_3
    K = np.zeros((N, D, 2 * L1 - 1, 2 * L2 - 1))
    K[:, :, L1 - 1, L2 - 1] = 1.0
    np.testing.assert_allclose(O.nd_forward(v, xs, K, 2), v * xs[0] * xs[1] * xs[2], atol=1e-14)
    # explicit order-2 form with scipy convolutions: y = x2 (K2 * (x1 (K1 * v)))
    K = rng.standard_normal((2, D, 2 * L1 - 1, 2 * L2 - 1))
    ref = np.empty_like(v)
    for b in range(B):
        for d in range(D):
            z2 = xs[0][b, d] * _scipy_linear(K[0, d], v[b, d], 2)
            ref[b, d] = xs[1][b, d] * _scipy_linear(K[1, d], z2, 2)
    np.testing.assert_allclose(O.nd_forward(v, xs[:2], K, 2), ref, atol=1e-11)
    # per-sample kernels: sample b uses its own K[b]
    Kb = rng.standard_normal((B, 2, D, 2 * L1 - 1, 2 * L2 - 1))
    y = O.nd_forward(v, xs[:2], Kb, 2, per_sample=True)
    for b in range(B):
        np.testing.assert_allclose(y[b], O.nd_forward(v[b:b + 1], [x[b:b + 1] for x in xs[:2]], Kb[b], 2)[0],
                                   atol=1e-12)


def test_nd_forward_is_linear_in_v():
    rng = _rng(23)
    B, D, L = 1, 2, 4
    v1, v2 = rng.standard_normal((2, B, D, L, L, L))
    xs = [rng.standard_normal((B, D, L, L, L)) for _ in range(2)]
    K = rng.standard_normal((2, D, 2 * L - 1, 2 * L - 1, 2 * L - 1))
    lhs = O.nd_forward(2.0 * v1 - 3.0 * v2, xs, K, 3)
    rhs = 2.0 * O.nd_forward(v1, xs, K, 3) - 3.0 * O.nd_forward(v2, xs, K, 3)
    np.testing.assert_allclose(lhs, rhs, atol=1e-10)
