"""CPU pins of the oracle's backward: central finite differences of a scalar
loss, the transposes of explicit dense Toeplitz matrices, numpy.correlate,
and agreement of the direct and FFT evaluations."""
import numpy as np
import pytest

import oracle as O

rng = np.random.default_rng(4321)


def _toeplitz(h, L):
    T = np.zeros((L, L))
    for t in range(L):
        for k in range(t + 1):
            T[t, t - k] = h[k]
    return T


def test_adjoint_is_the_matrix_transpose():
    L = 9
    h = rng.standard_normal(L); g = rng.standard_normal(L)
    assert np.allclose(O.causal_conv_adjoint(h, g), _toeplitz(h, L).T @ g, atol=1e-12)
    # <h conv z, g> == <z, adjoint(h, g)>
    z = rng.standard_normal(L)
    assert np.isclose(np.dot(O.causal_conv_direct(h, z), g), np.dot(z, O.causal_conv_adjoint(h, g)))


def test_filter_correlation_matches_numpy_correlate():
    L = 13
    g = rng.standard_normal(L); z = rng.standard_normal(L)
    ref = np.correlate(g, z, mode="full")[L - 1:]      # ref[k] = sum_t g[t + k] z[t]
    assert np.allclose(O.filter_correlation(g, z), ref, atol=1e-12)
    # <h conv z, g> is linear in h with gradient filter_correlation(g, z)
    h = rng.standard_normal(L)
    assert np.isclose(np.dot(O.causal_conv_direct(h, z), g), np.dot(h, O.filter_correlation(g, z)))


def test_fft_and_direct_paths_agree(monkeypatch):
    L = 300
    h = rng.standard_normal((2, L)); g = rng.standard_normal((2, L)); z = rng.standard_normal((2, L))
    a1, c1 = O.causal_conv_adjoint(h, g), O.filter_correlation(g, z)
    monkeypatch.setattr(O.hyena_oracle, "DIRECT_MAX_L", 16)
    a2, c2 = O.causal_conv_adjoint(h, g), O.filter_correlation(g, z)
    assert np.allclose(a1, a2, atol=1e-10) and np.allclose(c1, c2, atol=1e-10)


@pytest.mark.parametrize("N", [1, 2, 3])
def test_backward_matches_finite_differences(N):
    B, D, L = 2, 2, 7
    v = rng.standard_normal((B, D, L))
    xs = [rng.standard_normal((B, D, L)) for _ in range(N)]
    h = rng.standard_normal((N, D, L)) * 0.5
    gy = rng.standard_normal((B, D, L))
    loss = lambda v_, xs_, h_: float(np.sum(gy * O.hyena_forward(v_, xs_, h_, conv=O.causal_conv_direct)))
    gv, gxs, gh = O.hyena_backward(v, xs, h, gy, conv=O.causal_conv_direct)
    eps = 1e-6

    def fd(arr, idx, f):
        a0 = arr[idx]
        arr[idx] = a0 + eps; lp = f()
        arr[idx] = a0 - eps; lm = f()
        arr[idx] = a0
        return (lp - lm) / (2 * eps)

    for idx in [(0, 0, 0), (1, 1, 3), (0, 1, 6)]:
        assert np.isclose(gv[idx], fd(v, idx, lambda: loss(v, xs, h)), rtol=1e-6, atol=1e-8)
        for n in range(N):
            assert np.isclose(gxs[n][idx], fd(xs[n], idx, lambda: loss(v, xs, h)), rtol=1e-6, atol=1e-8)
    for idx in [(0, 0, 0), (N - 1, 1, 2), (0, 1, 6)]:
        assert np.isclose(gh[idx], fd(h, idx, lambda: loss(v, xs, h)), rtol=1e-6, atol=1e-8)


def test_backward_order2_by_dense_matrices():
    # y = X2 T2 X1 T1 v (X_n = diag x_n, T_n Toeplitz of h_n): gv = T1^T X1 T2^T X2 gy
    L = 6
    v = rng.standard_normal(L); x1 = rng.standard_normal(L); x2 = rng.standard_normal(L)
    h = rng.standard_normal((2, 1, L)); gy = rng.standard_normal(L)
    T1, T2 = _toeplitz(h[0, 0], L), _toeplitz(h[1, 0], L)
    X1, X2 = np.diag(x1), np.diag(x2)
    gv, gxs, gh = O.hyena_backward(v[None], [x1[None], x2[None]], h, gy[None], conv=O.causal_conv_direct)
    assert np.allclose(gv[0], T1.T @ X1 @ T2.T @ X2 @ gy, atol=1e-12)
    assert np.allclose(gxs[1][0], gy * (T2 @ X1 @ T1 @ v), atol=1e-12)
    assert np.allclose(gxs[0][0], (T2.T @ X2 @ gy) * (T1 @ v), atol=1e-12)


# ------------------------------------------------------------ circular mode

def _circulant(h, L):
    C = np.zeros((L, L))
    for t in range(L):
        for k in range(L):
            C[t, (t - k) % L] += h[k]
    return C


def test_circular_adjoint_is_the_circulant_transpose():
    L = 8
    h = rng.standard_normal(L); g = rng.standard_normal(L); z = rng.standard_normal(L)
    C = _circulant(h, L)
    assert np.allclose(O.circular_conv(h, z), C @ z, atol=1e-12)
    assert np.allclose(O.circular_conv_adjoint(h, g), C.T @ g, atol=1e-12)


def test_circular_correlation_against_numpy_fft():
    # out[k] = sum_t g[t] z[t - k mod L]: by the correlation theorem ifft(fft(g) * conj(fft(z)))
    L = 16
    g = rng.standard_normal(L); z = rng.standard_normal(L)
    ref = np.real(np.fft.ifft(np.fft.fft(g) * np.conj(np.fft.fft(z))))
    assert np.allclose(O.circular_filter_correlation(g, z), ref, atol=1e-12)
    h = rng.standard_normal(L)
    assert np.isclose(np.dot(O.circular_conv(h, z), g), np.dot(h, O.circular_filter_correlation(g, z)))


def test_circular_fft_and_direct_paths_agree(monkeypatch):
    L = 256
    h = rng.standard_normal((2, L)); g = rng.standard_normal((2, L)); z = rng.standard_normal((2, L))
    a1, c1 = O.circular_conv_adjoint(h, g), O.circular_filter_correlation(g, z)
    monkeypatch.setattr(O.hyena_oracle, "DIRECT_MAX_L", 16)
    a2, c2 = O.circular_conv_adjoint(h, g), O.circular_filter_correlation(g, z)
    assert np.allclose(a1, a2, atol=1e-10) and np.allclose(c1, c2, atol=1e-10)


@pytest.mark.parametrize("N", [1, 2])
def test_circular_backward_matches_finite_differences(N):
    B, D, L = 2, 2, 8
    v = rng.standard_normal((B, D, L))
    xs = [rng.standard_normal((B, D, L)) for _ in range(N)]
    h = rng.standard_normal((N, D, L)) * 0.5
    gy = rng.standard_normal((B, D, L))
    loss = lambda: float(np.sum(gy * O.hyena_forward(v, xs, h, conv=O.circular_conv)))
    gv, gxs, gh = O.hyena_backward(v, xs, h, gy, circular=True)
    eps = 1e-6

    def fd(arr, idx):
        a0 = arr[idx]
        arr[idx] = a0 + eps; lp = loss()
        arr[idx] = a0 - eps; lm = loss()
        arr[idx] = a0
        return (lp - lm) / (2 * eps)

    for idx in [(0, 0, 0), (1, 1, 3), (0, 1, 7)]:
        assert np.isclose(gv[idx], fd(v, idx), rtol=1e-6, atol=1e-8)
        for n in range(N):
            assert np.isclose(gxs[n][idx], fd(xs[n], idx), rtol=1e-6, atol=1e-8)
    for idx in [(0, 0, 0), (N - 1, 1, 5), (0, 1, 7)]:
        assert np.isclose(gh[idx], fd(h, idx), rtol=1e-6, atol=1e-8)
