"""CPU pins of the other filter families (Hyena-LI sum of real exponentials,
Hyena-MR damped explicit filter) and of the short-FIR evaluation of the
operator: geometric-series closed forms, a hand-worked value, brute force."""
import numpy as np

import oracle as O

rng = np.random.default_rng(99)


def test_li_single_exponential_and_closed_form_spectrum():
    L = 50
    R = np.array([[2.0]]); lam = np.array([[0.9]])
    h = O.filter_gen_li(R, lam, L)[0]
    assert np.allclose(h, 2.0 * 0.9 ** np.arange(L))
    # its DFT zero-padded to P is a finite geometric series
    P = 128
    H = O.filter_spectrum(h[None], P)[0]
    w = np.exp(-2j * np.pi * np.arange(P // 2 + 1) / P)
    assert np.allclose(H, 2.0 * (1 - (0.9 * w) ** L) / (1 - 0.9 * w), atol=1e-10)


def test_li_sum_negative_and_zero_rates():
    R = np.array([[1.0, -0.5, 3.0]]); lam = np.array([[0.5, -0.8, 0.0]])
    h = O.filter_gen_li(R, lam, 4)[0]
    # t=0: 1 - 0.5 + 3 (0**0 = 1); t=1: 0.5 + 0.4 + 0; t=2: 0.25 - 0.32; t=3: 0.125 + 0.256
    assert np.allclose(h, [3.5, 0.9, 0.25 - 0.32, 0.125 + 0.256])


def test_mr_damping():
    N, D, Lh = 2, 3, 9
    hhat = rng.standard_normal((N, D, Lh)); alpha = np.array([0.0, 0.1, 1.0])
    h = O.filter_gen_mr(hhat, alpha, N)
    assert np.array_equal(h[:, 0], hhat[:, 0])
    assert np.allclose(h[1, 2, 4], hhat[1, 2, 4] * np.exp(-4.0))


def test_short_fir_operator_equals_brute_force():
    # explicit filters of Lh taps act as length-L filters zero beyond Lh
    B, D, L, N, Lh = 2, 3, 40, 2, 5
    v = rng.standard_normal((B, D, L)); xs = [rng.standard_normal((B, D, L)) for _ in range(N)]
    hs = rng.standard_normal((N, D, Lh))
    hp = np.zeros((N, D, L)); hp[..., :Lh] = hs
    y = O.hyena_forward(v, xs, hp)
    z = v.copy()
    for n in range(N):
        c = np.zeros_like(z)
        for t in range(L):
            for k in range(min(Lh, t + 1)):
                c[..., t] += hs[n, :, k] * z[..., t - k]
        z = xs[n] * c
    assert np.allclose(y, z, atol=1e-12)


def test_circular_conv_matches_numpy_fft_and_roll():
    L = 64
    h = rng.standard_normal((2, L)); z = rng.standard_normal((2, L))
    got = O.circular_conv(h, z)
    ref = np.real(np.fft.ifft(np.fft.fft(h) * np.fft.fft(z)))
    assert np.allclose(got, ref, atol=1e-12)
    # a one-sample delay filter rotates the signal (wrap-around at t = 0)
    d = np.zeros(L); d[3] = 1.0
    assert np.allclose(O.circular_conv(d, z[0]), np.roll(z[0], 3))


def test_circular_equals_linear_when_halves_are_zero():
    # with filter and signal zero in their second halves nothing wraps
    L = 32
    h = np.zeros(L); z = np.zeros(L)
    h[:8] = rng.standard_normal(8); z[:16] = rng.standard_normal(16)
    assert np.allclose(O.circular_conv(h, z), O.causal_conv_direct(h, z), atol=1e-12)


def test_circular_fft_path(monkeypatch):
    L = 256
    h = rng.standard_normal(L); z = rng.standard_normal(L)
    a = O.circular_conv(h, z)
    monkeypatch.setattr(O.hyena_oracle, "DIRECT_MAX_L", 16)
    assert np.allclose(O.circular_conv(h, z), a, atol=1e-10)
