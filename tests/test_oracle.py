"""Pins for the float64 oracle, independent of the oracle itself.

Each check ties an oracle function to something the pages or mathematics fix:
a hand-worked example, the matrix (Toeplitz) view, a library routine that the
definition reduces to in a special case, a closed form, or an invariant
(linearity, causality).  They are chosen so that a dropped term, a wrong sign
or index, a swapped x/h pairing, a transposed weight or a mis-ordered feature
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# --------------------------------------------------------------- convolution

@pytest.mark.parametrize("L", [1, 2, 3, 7, 16, 64])
def test_direct_conv_matches_toeplitz_matrix(L):
    # Matrix view (Hyena Hierarchy explainer, section on the Toeplitz view;
    # homemade-llm operators page, section 2 index equation): the causal
    # convolution is a lower-triangular Toeplitz matrix T[t, s] = h[t - s].
    h = rng.standard_normal(L); z = rng.standard_normal(L)
    T = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            T[t, s] = h[t - s]
    np.testing.assert_allclose(O.causal_conv_direct(h, z), T @ z, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [1, 5, 33, 256, 1000])
def test_direct_conv_matches_numpy_convolve(L):
    # Special case reducing to a library routine: the first L samples of the
    # full linear convolution.
    h = rng.standard_normal(L); z = rng.standard_normal(L)
    np.testing.assert_allclose(O.causal_conv_direct(h, z), np.convolve(h, z)[:L],
                               rtol=0, atol=1e-10)


def test_direct_conv_batched_broadcast():
    h = rng.standard_normal((3, 50)); z = rng.standard_normal((2, 3, 50))
    got = O.causal_conv_direct(h, z)
    for b in range(2):
        for d in range(3):
            np.testing.assert_allclose(got[b, d], np.convolve(h[d], z[b, d])[:50], atol=1e-12)


@pytest.mark.parametrize("P", [1, 2, 4, 8, 64, 1024, 4096])
def test_fft_matches_numpy(P):
    x = rng.standard_normal(P) + 1j * rng.standard_normal(P)
    np.testing.assert_allclose(O.fft(x), np.fft.fft(x), rtol=0, atol=1e-9 * max(1, P))
    np.testing.assert_allclose(O.fft(x, inverse=True), np.fft.ifft(x), rtol=0, atol=1e-12)


def test_fft_definition_small():
    # Direct DFT sum for P = 8 written out (forward sign is negative).
    P = 8
    x = rng.standard_normal(P) + 1j * rng.standard_normal(P)
    ref = np.array([sum(x[n] * np.exp(-2j * np.pi * n * k / P) for n in range(P)) for k in range(P)])
    np.testing.assert_allclose(O.fft(x), ref, atol=1e-12)


def test_fft_parseval_and_roundtrip():
    P = 2 ** 14
    x = rng.standard_normal(P) + 1j * rng.standard_normal(P)
    X = O.fft(x)
    assert abs(np.sum(np.abs(X) ** 2) / P - np.sum(np.abs(x) ** 2)) < 1e-8 * np.sum(np.abs(x) ** 2)
    np.testing.assert_allclose(O.fft(X, inverse=True), x, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 64, 100, 257, 1000, 4096])
def test_fft_conv_matches_direct(L):
    h = rng.standard_normal(L); z = rng.standard_normal(L)
    a = O.causal_conv_fft(h, z); b = O.causal_conv_direct(h, z)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b))) * max(1, np.log2(L) + 1)


def test_fft_conv_matches_numpy_fft_large():
    # Long case on one channel: oracle FFT path vs numpy's rfft/irfft pipeline.
    L = 2 ** 16
    h = rng.standard_normal(L); z = rng.standard_normal(L)
    P = 2 * L
    ref = np.fft.irfft(np.fft.rfft(h, P) * np.fft.rfft(z, P), P)[:L]
    got = O.causal_conv_fft(h, z)
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_conv_closed_form_geometric():
    # h_t = a^t, z = 1: (h*z)[t] = sum_{k<=t} a^k = (1 - a^{t+1}) / (1 - a).
    L = 300; a = math.exp(-3.0 / L)
    h = a ** np.arange(L); z = np.ones(L)
    ref = (1 - a ** (np.arange(L) + 1)) / (1 - a)
    for f in (O.causal_conv_direct, O.causal_conv_fft):
        np.testing.assert_allclose(f(h, z), ref, rtol=1e-12)


def test_conv_closed_form_prefix_sum():
    # h = 1 everywhere: causal convolution is the running (prefix) sum.
    L = 77; z = rng.standard_normal(L)
    np.testing.assert_allclose(O.causal_conv_direct(np.ones(L), z), np.cumsum(z), atol=1e-12)


# ---------------------------------------------------------------- recurrence

def test_golden_tiny_order2():
    g = json.load(open(os.path.join(GOLDEN, "tiny_order2.json")))
    v = np.array(g["v"], float)
    xs = [np.array(g["x1"], float)[None], np.array(g["x2"], float)[None]]
    h = np.array([g["h1"], g["h2"]], float)[:, None, :]
    y = O.hyena_forward(v[None], xs, h)
    np.testing.assert_array_equal(y[0], np.array(g["y"], float))


def _rand_problem(N, B, D, L):
    v = rng.standard_normal((B, D, L))
    xs = [rng.standard_normal((B, D, L)) for _ in range(N)]
    h = rng.standard_normal((N, D, L)) * np.exp(-np.arange(L) / L)
    return v, xs, h


def test_explicit_order2_form():
    # y = x2 * (h2 conv (x1 * (h1 conv v))) written out with numpy.convolve.
    B, D, L = 2, 3, 40
    v, xs, h = _rand_problem(2, B, D, L)
    y = O.hyena_forward(v, xs, h)
    for b in range(B):
        for d in range(D):
            inner = xs[0][b, d] * np.convolve(h[0, d], v[b, d])[:L]
            ref = xs[1][b, d] * np.convolve(h[1, d], inner)[:L]
            np.testing.assert_allclose(y[b, d], ref, atol=1e-12)


def test_rejects_other_nesting():
    # The glossary page prints a different order-2 nesting (gate first, conv
    # last); the followed reading must NOT reproduce it on generic data.
    B, D, L = 1, 1, 30
    v, xs, h = _rand_problem(2, B, D, L)
    y = O.hyena_forward(v, xs, h)[0, 0]
    other = np.convolve(h[1, 0], xs[0][0, 0] * np.convolve(h[0, 0], xs[1][0, 0] * v[0, 0])[:L])[:L]
    assert np.max(np.abs(y - other)) > 1e-3


def test_delta_filter_gives_gated_product():
    N, B, D, L = 3, 2, 4, 25
    v, xs, _ = _rand_problem(N, B, D, L)
    h = np.zeros((N, D, L)); h[:, :, 0] = 1.0
    np.testing.assert_allclose(O.hyena_forward(v, xs, h), v * xs[0] * xs[1] * xs[2], atol=1e-12)
    ones = [np.ones_like(v)] * N
    np.testing.assert_allclose(O.hyena_forward(v, ones, h), v, atol=0)


def test_shifted_delta_shifts():
    B, D, L, k = 1, 2, 20, 3
    v = rng.standard_normal((B, D, L))
    h = np.zeros((1, D, L)); h[:, :, k] = 1.0
    y = O.hyena_forward(v, [np.ones_like(v)], h)
    ref = np.zeros_like(v); ref[..., k:] = v[..., :L - k]
    np.testing.assert_allclose(y, ref, atol=0)


def test_linearity():
    N, B, D, L = 2, 1, 2, 33
    v, xs, h = _rand_problem(N, B, D, L)
    v2, xs2, h2 = _rand_problem(N, B, D, L)
    a, b = 0.7, -1.3
    f = O.hyena_forward
    # linear in v
    np.testing.assert_allclose(f(a * v + b * v2, xs, h), a * f(v, xs, h) + b * f(v2, xs, h), atol=1e-11)
    # linear in each x_n separately
    for n in range(N):
        xa = list(xs); xb = list(xs); xc = list(xs)
        xb[n] = xs2[n]; xc[n] = a * xs[n] + b * xs2[n]
        np.testing.assert_allclose(f(v, xc, h), a * f(v, xa, h) + b * f(v, xb, h), atol=1e-11)
    # linear in each h_n separately
    for n in range(N):
        hb = h.copy(); hb[n] = h2[n]; hc = h.copy(); hc[n] = a * h[n] + b * h2[n]
        np.testing.assert_allclose(f(v, xs, hc), a * f(v, xs, h) + b * f(v, xs, hb), atol=1e-11)


def test_causality_direct_and_fft():
    N, B, D, L, t0 = 2, 1, 3, 64, 37
    v, xs, h = _rand_problem(N, B, D, L)
    y = O.hyena_forward(v, xs, h)
    v2 = v.copy(); v2[..., t0:] += 5.0
    xs2 = [x.copy() for x in xs]; xs2[0][..., t0:] -= 2.0; xs2[1][..., t0 + 3:] *= 3.0
    y2 = O.hyena_forward(v2, xs2, h)
    np.testing.assert_array_equal(y[..., :t0], y2[..., :t0])        # bitwise on the direct path
    assert np.max(np.abs(y[..., t0:] - y2[..., t0:])) > 1e-3
    yf = O.hyena_forward(v, xs, h, conv=O.causal_conv_fft)
    yf2 = O.hyena_forward(v2, xs2, h, conv=O.causal_conv_fft)
    assert np.max(np.abs(yf[..., :t0] - yf2[..., :t0])) <= 1e-12


def test_fft_and_direct_recurrence_agree():
    N, B, D, L = 3, 2, 2, 300
    v, xs, h = _rand_problem(N, B, D, L)
    a = O.hyena_forward(v, xs, h, conv=O.causal_conv_direct)
    b = O.hyena_forward(v, xs, h, conv=O.causal_conv_fft)
    assert np.max(np.abs(a - b)) <= 1e-11 * np.max(np.abs(a))


# ------------------------------------------------------------- filter gen

def test_positional_features_values():
    L, K = 16, 8
    e = O.positional_features(L, K)
    assert e.shape == (L, 1 + 2 * K)
    # t = 0: position 0, all sines 0, all cosines 1
    np.testing.assert_array_equal(e[0], np.r_[0.0, np.zeros(K), np.ones(K)])
    # t = L/4: position 1/4, sin(pi k/2) and cos(pi k/2) for k = 1..K
    k = np.arange(1, K + 1)
    np.testing.assert_allclose(e[L // 4], np.r_[0.25, np.sin(np.pi * k / 2), np.cos(np.pi * k / 2)], atol=1e-15)
    # column 0 is t/L for every t
    np.testing.assert_array_equal(e[:, 0], np.arange(L) / L)


def test_golden_tiny_filter():
    g = json.load(open(os.path.join(GOLDEN, "tiny_filter.json")))
    p = {k: np.array(g[k], float) for k in ("W1", "b1", "W2", "b2", "W3", "b3", "alpha")}
    p.update(D=1, N=1, K=1)
    h = O.filter_gen(p, g["L"])[0, 0]
    s = math.sin(math.sin(1.0))
    closed = [1.0, math.exp(-0.25) * (2 * s + 1), math.exp(-0.5), math.exp(-0.75) * (1 - 2 * s)]
    np.testing.assert_allclose(g["h"], closed, rtol=1e-15)
    np.testing.assert_allclose(h, closed, rtol=1e-13)


def _params(D=5, N=2, H=6, K=8, bias=True):
    F = 1 + 2 * K
    p = dict(D=D, N=N, K=K,
             W1=rng.standard_normal((H, F)) / np.sqrt(F), b1=rng.standard_normal(H) * bias,
             W2=rng.standard_normal((H, H)) / np.sqrt(H), b2=rng.standard_normal(H) * bias,
             W3=rng.standard_normal((N * D, H)) / np.sqrt(H), b3=rng.standard_normal(N * D) * bias,
             alpha=np.linspace(1, 10, D))
    return p


def test_filter_window_ratio_and_t0():
    L = 64
    p = _params()
    h = O.filter_gen(p, L)
    o = O.filter_ffn(O.positional_features(L, 8), p["W1"], p["b1"], p["W2"], p["b2"], p["W3"], p["b3"])
    t = np.arange(L)
    for n in range(p["N"]):
        for d in range(p["D"]):
            np.testing.assert_allclose(h[n, d] / o[:, n * p["D"] + d], np.exp(-p["alpha"][d] * t / L), rtol=1e-12)
            assert h[n, d, 0] == o[0, n * p["D"] + d]        # window is exactly 1 at t = 0


def test_filter_with_zero_W2_closed_form():
    L = 32
    p = _params(); p["W2"] = np.zeros_like(p["W2"])
    h = O.filter_gen(p, L)
    t = np.arange(L)
    for n in range(p["N"]):
        for d in range(p["D"]):
            j = n * p["D"] + d
            const = p["W3"][j] @ np.sin(p["b2"]) + p["b3"][j]
            np.testing.assert_allclose(h[n, d], np.exp(-p["alpha"][d] * t / L) * const, rtol=1e-12)


def test_filter_ffn_matches_torch_nn():
    # Library cross-check: torch.nn.Linear ([out][in] weights) with sin, float64.
    torch = pytest.importorskip("torch")
    L = 50
    p = _params(D=3, N=3, H=7)
    e = O.positional_features(L, 8)
    l1 = torch.nn.Linear(17, 7).double(); l2 = torch.nn.Linear(7, 7).double(); l3 = torch.nn.Linear(7, 9).double()
    with torch.no_grad():
        for l, W, b in ((l1, p["W1"], p["b1"]), (l2, p["W2"], p["b2"]), (l3, p["W3"], p["b3"])):
            l.weight.copy_(torch.from_numpy(W)); l.bias.copy_(torch.from_numpy(b))
        ref = l3(torch.sin(l2(torch.sin(l1(torch.from_numpy(e)))))).numpy()
    np.testing.assert_allclose(O.filter_ffn(e, p["W1"], p["b1"], p["W2"], p["b2"], p["W3"], p["b3"]), ref, atol=1e-13)


def test_filter_output_column_mapping():
    # Column j = n*D + d of the last layer feeds filter h_n of channel d.
    L, D, N, H = 16, 4, 3, 5
    p = _params(D=D, N=N, H=H, bias=False)
    p["W3"] = np.zeros((N * D, H)); p["b3"] = np.zeros(N * D)
    p["b3"][2 * D + 1] = 7.0                 # marker: order n=2 (third), channel d=1
    h = O.filter_gen(p, L)
    mask = np.zeros((N, D), bool); mask[2, 1] = True
    assert np.all(h[~mask] == 0)
    np.testing.assert_allclose(h[2, 1], 7.0 * np.exp(-p["alpha"][1] * np.arange(L) / L), rtol=1e-14)


def test_filter_channel_subset_matches_full():
    L = 40
    p = _params(D=6, N=2)
    full = O.filter_gen(p, L)
    sub = O.filter_gen(p, L, channels=[5, 0, 3])
    np.testing.assert_array_equal(sub, full[:, [5, 0, 3]])


# ----------------------------------------------------------------- spectrum

def test_spectrum_window_only_closed_form():
    # W3 = 0, b3 = 1: h_t = a^t with a = exp(-alpha/L); its zero-padded
    # P-point spectrum is the geometric sum (1 - (a w^k)^L) / (1 - a w^k).
    L, P, D = 256, 512, 3
    p = _params(D=D, N=1, bias=False)
    p["W3"] = np.zeros_like(p["W3"]); p["b3"] = np.ones(D)
    h = O.filter_gen(p, L)[0]
    S = O.filter_spectrum(h, P)
    k = np.arange(P // 2 + 1)
    w = np.exp(-2j * np.pi * k / P)
    for d in range(D):
        a = math.exp(-p["alpha"][d] / L)
        ref = (1 - (a * w) ** L) / (1 - a * w)
        np.testing.assert_allclose(S[d], ref, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S[d, 0], np.sum(h[d]), rtol=1e-13)


@pytest.mark.parametrize("L,P", [(256, 600), (100, 384), (300, 2 * 5 * 64), (37, 90)])
def test_spectrum_any_even_length_closed_form(L, P):
    # The same closed form at FFT lengths that are not powers of two (the
    # direct DFT branch), and numpy's real FFT of the zero-padded filter as a
    # library special case.
    D = 2
    p = _params(D=D, N=1, bias=False)
    p["W3"] = np.zeros_like(p["W3"]); p["b3"] = np.ones(D)
    h = O.filter_gen(p, L)[0]
    S = O.filter_spectrum(h, P)
    k = np.arange(P // 2 + 1)
    w = np.exp(-2j * np.pi * k / P)
    for d in range(D):
        a = math.exp(-p["alpha"][d] / L)
        ref = (1 - (a * w) ** L) / (1 - a * w)
        np.testing.assert_allclose(S[d], ref, rtol=1e-11, atol=1e-11)
    hr = O.filter_gen(_params(D=3, N=2), L)
    np.testing.assert_allclose(O.filter_spectrum(hr, P), np.fft.rfft(hr, n=P), rtol=1e-10, atol=1e-10)


def test_spectrum_direct_branch_matches_fft_branch():
    # A power of two through the radix-2 FFT equals the written-out sum.
    L, P = 50, 128
    h = O.filter_gen(_params(D=3, N=2), L)
    t = np.arange(L); k = np.arange(P // 2 + 1)
    direct = h @ np.exp(-2j * np.pi * np.outer(t, k) / P)
    np.testing.assert_allclose(O.filter_spectrum(h, P), direct, rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------- bf16 rounding

def test_bf16_rounding_is_rne():
    # The input generator rounds to bf16 with torch; check that it is
    # round-to-nearest-even on ties and exact on representable values.
    torch = pytest.importorskip("torch")
    def rne(x):
        u = np.array([x], np.float32).view(np.uint32)[0]
        r = ((int(u) + 0x7FFF + ((int(u) >> 16) & 1)) >> 16) << 16
        return np.array([r], np.uint32).view(np.float32)[0]
    vals = [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-39, 1.0e-40, 65504.0, 1.0 + 2 ** -7 + 2 ** -8]
    for x in vals:
        xf = float(np.float32(x))
        got = torch.tensor([xf], dtype=torch.float32).to(torch.bfloat16).float().item()
        assert got == float(rne(xf)), (x, got, rne(xf))
