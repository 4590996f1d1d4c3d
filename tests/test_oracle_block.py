"""CPU pins of the oracle's block functions (short convolution, in/out
projections, the block), each checked against something other than itself:
numpy.convolve, brute-force loops, a hand-worked fixture, reductions to the
bare operator, causality and linearity."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def test_short_conv_matches_numpy_convolve():
    z = rng.standard_normal((2, 5, 37))
    w = rng.standard_normal((5, 4))
    got = O.short_conv(z, w)
    for b in range(2):
        for c in range(5):
            ref = np.convolve(z[b, c], w[c])[:37]
            assert np.allclose(got[b, c], ref, rtol=0, atol=1e-12)


def test_short_conv_identity_and_shift():
    z = rng.standard_normal((3, 11))
    assert np.array_equal(O.short_conv(z, np.ones((3, 1))), z)
    w = np.zeros((3, 5)); w[:, 3] = 1.0                      # pure delay by 3
    got = O.short_conv(z, w)
    assert np.array_equal(got[:, 3:], z[:, :-3]) and np.all(got[:, :3] == 0)
    # taps longer than the sequence: only the first L taps can act
    w6 = rng.standard_normal((3, 6))
    got = O.short_conv(z[:, :2], w6)
    assert np.allclose(got[:, 0], w6[:, 0] * z[:, 0])
    assert np.allclose(got[:, 1], w6[:, 0] * z[:, 1] + w6[:, 1] * z[:, 0])


def _loops_in_projection(u, W_in, b_in, w_short, N):
    B, L, D = u.shape
    C, T = w_short.shape
    Z = np.zeros((B, L, C))
    for b in range(B):
        for t in range(L):
            for c in range(C):
                acc = b_in[c]
                for k in range(D):
                    acc += u[b, t, k] * W_in[c, k]
                Z[b, t, c] = acc
    S = np.zeros((B, C, L))
    for b in range(B):
        for c in range(C):
            for t in range(L):
                for j in range(T):
                    if t - j >= 0:
                        S[b, c, t] += w_short[c, j] * Z[b, t - j, c]
    return S


def test_in_projection_matches_loops():
    B, L, D, N, T = 2, 6, 3, 2, 3
    u = rng.standard_normal((B, L, D))
    W_in = rng.standard_normal(((N + 1) * D, D))
    b_in = rng.standard_normal((N + 1) * D)
    w = rng.standard_normal(((N + 1) * D, T))
    v, xs = O.in_projection(u, W_in, b_in, w, N)
    S = _loops_in_projection(u, W_in, b_in, w, N)
    assert np.allclose(v, S[:, :D], atol=1e-12)
    for n in range(N):
        assert np.allclose(xs[n], S[:, (n + 1) * D:(n + 2) * D], atol=1e-12)


def test_in_projection_columns_match_loops():
    """Column-sampled streams equal the loop definition at those columns (in
    any order, repeats and both ends included), with and without bias."""
    B, L, D, N, T = 2, 9, 4, 2, 4
    u = rng.standard_normal((B, L, D))
    W_in = rng.standard_normal(((N + 1) * D, D))
    b_in = rng.standard_normal((N + 1) * D)
    w = rng.standard_normal(((N + 1) * D, T))
    cols = [11, 0, 5, 5, 3, 8]
    for bias in (b_in, None):
        got = O.in_projection_columns(u, W_in, bias, w, cols)
        S = _loops_in_projection(u, W_in, np.zeros((N + 1) * D) if bias is None else bias, w, N)
        assert got.shape == (B, len(cols), L)
        assert np.allclose(got, S[:, cols], atol=1e-12)


def test_out_projection_matches_loops():
    B, D, L = 2, 4, 5
    y = rng.standard_normal((B, D, L))
    W = rng.standard_normal((D, D)); bo = rng.standard_normal(D)
    got = O.out_projection(y, W, bo)
    for b in range(B):
        for t in range(L):
            for e in range(D):
                assert abs(got[b, t, e] - (bo[e] + sum(W[e, d] * y[b, d, t] for d in range(D)))) < 1e-12


def test_golden_tiny_block():
    g = json.load(open(os.path.join(GOLDEN, "tiny_block.json")))
    u = np.array(g["u"], float).reshape(1, 3, 1)
    bp = {"W_in": np.array(g["W_in"], float), "b_in": np.array(g["b_in"], float),
          "w_short": np.array(g["w_short"], float), "W_out": np.array(g["W_out"], float),
          "b_out": np.array(g["b_out"], float)}
    h = np.array(g["h1"], float).reshape(1, 1, 3)
    out = O.block_forward(u, bp, h)
    assert np.allclose(out.reshape(-1), g["out"], atol=1e-12)


def test_block_reduces_to_operator():
    # identity projections, pass-through short filters: the block is the
    # operator on u^T with every gate equal to u^T
    B, L, D, N = 2, 40, 3, 2
    u = rng.standard_normal((B, L, D))
    h = rng.standard_normal((N, D, L))
    bp = {"W_in": np.vstack([np.eye(D)] * (N + 1)), "b_in": None,
          "w_short": np.tile([1.0, 0.0, 0.0], ((N + 1) * D, 1)), "W_out": np.eye(D), "b_out": None}
    got = O.block_forward(u, bp, h)
    ut = np.transpose(u, (0, 2, 1))
    ref = np.transpose(O.hyena_forward(ut, [ut] * N, h), (0, 2, 1))
    assert np.allclose(got, ref, atol=1e-12)


def test_stream_order_v_first():
    B, L, D, N = 1, 8, 2, 3
    u = rng.standard_normal((B, L, D))
    W = np.vstack([(s + 1.0) * np.eye(D) for s in range(N + 1)])
    v, xs = O.in_projection(u, W, None, np.ones(((N + 1) * D, 1)), N)
    ut = np.transpose(u, (0, 2, 1))
    assert np.allclose(v, ut)
    for n in range(N):
        assert np.allclose(xs[n], (n + 2.0) * ut)


def test_block_is_causal_and_projections_linear():
    B, L, D, N, T = 1, 64, 3, 2, 3
    u = rng.standard_normal((B, L, D))
    h = rng.standard_normal((N, D, L))
    bp = {"W_in": rng.standard_normal(((N + 1) * D, D)), "b_in": rng.standard_normal((N + 1) * D),
          "w_short": rng.standard_normal(((N + 1) * D, T)), "W_out": rng.standard_normal((D, D)),
          "b_out": rng.standard_normal(D)}
    y0 = O.block_forward(u, bp, h, conv=O.causal_conv_direct)
    u2 = u.copy(); u2[0, 40] += 1.0
    y1 = O.block_forward(u2, bp, h, conv=O.causal_conv_direct)
    assert np.array_equal(y0[:, :40], y1[:, :40]) and not np.allclose(y0[:, 40:], y1[:, 40:])
    # without biases the projections are linear in their input
    u3 = rng.standard_normal((B, L, D))
    a, b = 0.7, -1.3
    p1 = O.in_projection(a * u + b * u3, bp["W_in"], None, bp["w_short"], N)
    q1, q2 = O.in_projection(u, bp["W_in"], None, bp["w_short"], N), O.in_projection(u3, bp["W_in"], None, bp["w_short"], N)
    assert np.allclose(p1[0], a * q1[0] + b * q2[0])
    yy = rng.standard_normal((B, D, L))
    assert np.allclose(O.out_projection(a * yy, bp["W_out"], None), a * O.out_projection(yy, bp["W_out"], None))
