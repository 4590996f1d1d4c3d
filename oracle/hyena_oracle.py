"""Float64 CPU oracle for the Hyena order-N operator forward pass.

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP path (no kernels, helpers, tables or constants) and it
imports nothing from this repository.

Everything here is plain, slow and meant to be checked by eye against the
pages it follows.  Floating point is float64 throughout; fp32 or bf16 inputs
are upcast exactly before use.

Sources (web pages; cited below by key, page title and section):
  [P1] abeam-guide-lp.pages.dev, explainer of "Hyena Hierarchy: Towards Larger
       Convolutional Language Models" (Japanese).
  [P2] jisaku.com glossary entry "Hyena（ハイエナ）".
  [P3] imamachi-n.github.io homemade-llm, "02. 3つの Hyena 演算子"
       (StripedHyena 2 operators).
  [P4] irregular6612.github.io paper digest "Hyena Hierarchy - Towards Larger
       Convolutional Language Models" (Korean).
  [P5] gist.science summary of "Native Multi-Dimensional Subquadratic Operators
       via Input Dependent Long Convolutions" (HyenaND / nSubQ).

What the operator computes (restated):
  * [P1] section "Hyena 演算子の形" and [P4] section "방법 (Method)", framework
    figure: start from z_1 = v; for n = 1..N the next state is the elementwise
    product of the gate x_n with the long convolution of filter h_n and z_n;
    the output is y = z_{N+1}.
  * [P3] section 4 "FIR フィルタと効率的な生成", its causal-convolution equation:
    output sample t depends only on input samples at or before t, with the
    filter tap k weighting the input k steps back.  Here the filter spans the
    whole sequence (length L) and the output keeps the first L samples.
  * [P2] section "暗黙的畳み込みフィルタ": the filter is a window in t times an
    FFN evaluated on the normalised position t/L and sin/cos features of t;
    the window is an exponential decay and the FFN is a small MLP.
  * [P2] section "計算効率" and [P5] section "手法: HyenaND" (boundary handling):
    the long convolution is evaluated as FFT, pointwise product, inverse FFT,
    with the signals zero-padded to twice their length so that the circular
    convolution equals the linear one.  Any FFT length >= 2L-1 gives the same
    exact result; the oracle uses the next power of two >= 2L.

The block around the operator (restated):
  * [P4] framework figure: the input u (L x D) goes through one linear
    projection of width (N+1)D that yields v (the initial state) and the gates
    x_1..x_N; [P1] "計算方法" counts this dense work as the D in
    O(NDL(log L + D)).
  * [P3] section 2 "Hyena 演算子の構造": each projected stream is featurised by
    its own short convolution (h_T, h_H, h_K there), and the operator's output
    is mapped back by a dense matrix M.

Readings where the pages are silent (each listed in the design notes):
  positional features e(t) = [t/L, sin(2*pi*k*t/L) for k=1..K,
  cos(2*pi*k*t/L) for k=1..K]; FFN = affine -> sin -> affine -> sin -> affine
  (sin with unit frequency, "2-layer" counting hidden layers); output column
  j = n*D + d feeds filter h_n of channel d; window exp(-alpha_d * t / L) is
  the same for every order; no bias/skip term, no normalisation.
  Block: projection weights row-major [out][in] with output column c = s*D + d
  feeding stream s (s = 0 is v, s = n is x_n) of channel d; the short
  convolution is causal and depthwise (one T-tap filter per projected
  column, tap j weighting the sample j steps back, zero before t = 0); biases
  of both projections optional; the output projection has no activation.
  Circular mode ([P5] "手法: HyenaND", boundary handling: periodic systems
  use circular convolutions): c[t] = sum_{k<L} h[k] z[(t-k) mod L].
  Filter families ([P3] section 3): Hyena-LI's filter is a sum of real
  exponentials R_s * lambda_s^t over a small state of size S (the page
  indexes t from 1 with exponent t-1; here t = 0..L-1 with exponent t);
  Hyena-MR's explicit filter hhat_t is damped by exp(-alpha_d * t) (the
  page's lambda^(-alpha t) with the base folded into alpha_d); Hyena-SE's
  short explicit filters are used as given.
  Backward: the pages give no gradient formulas; they follow from the
  recurrence by the chain rule (the adjoint of a causal convolution is the
  correlation with the same filter), for a scalar loss whose gradient with
  respect to y is gy; filter gradients are summed over the batch.
  Grids ([P5] "手法: HyenaND", native N-D convolution and boundary
  handling): the same recurrence on a grid L_1 x .. x L_k, each long
  convolution a k-dimensional one with a global kernel K.  Non-circular
  mode: the kernel holds one value per offset o with |o_a| < L_a on every
  axis (both signs, so centred kernels are expressible; a causal one is
  zero at negative offsets) and y[t] = sum over grid points s of
  K[t - s] z[s] -- what zero-padding every axis to twice its size and
  keeping the first L_a samples computes.  Circular mode: K has the grid's
  own shape and offsets wrap, y[t] = sum_s K[(t - s) mod L] z[s].  The
  kernel may be shared by the batch or given per sample (the page's
  input-dependent kernels); how it is generated is not part of this
  operator.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "positional_features",
    "filter_ffn",
    "filter_gen",
    "causal_conv_direct",
    "fft",
    "causal_conv_fft",
    "causal_conv",
    "hyena_forward",
    "filter_spectrum",
    "short_conv",
    "in_projection",
    "in_projection_columns",
    "out_projection",
    "block_forward",
    "causal_conv_adjoint",
    "filter_correlation",
    "hyena_backward",
    "filter_gen_li",
    "filter_gen_mr",
    "circular_conv",
    "circular_conv_adjoint",
    "circular_filter_correlation",
    "ndfft",
    "nd_conv_direct",
    "nd_conv_fft",
    "nd_conv",
    "nd_forward",
    "DIRECT_MAX_L",
]

# Up to this length the convolution is the brute-force sum; beyond it the
# oracle's own radix-2 FFT is used (same exact result, O(L log L)).
DIRECT_MAX_L = 8192


# ---------------------------------------------------------------------------
# Implicit filter  ([P2] section "暗黙的畳み込みフィルタ"; [P1] section
# "フィルタの作り方"; [P4] framework figure, HyenaFilter node:
# positional encoding -> FFN -> window)
# ---------------------------------------------------------------------------

def positional_features(L: int, K: int = 8) -> np.ndarray:
    """e(t) for t = 0..L-1, shape [L, 1 + 2K], float64.

    Column 0 is the normalised position t/L; columns 1..K are sin(2*pi*k*t/L)
    and columns K+1..2K are cos(2*pi*k*t/L), k = 1..K ([P2] "暗黙的畳み込み
    フィルタ": t/L plus sin/cos frequency features).  The phase k*t/L is
    reduced modulo 1 with exact integer arithmetic before taking sin/cos.
    """
    t = np.arange(L, dtype=np.int64)
    feats = np.empty((L, 1 + 2 * K), dtype=np.float64)
    feats[:, 0] = t / L
    for k in range(1, K + 1):
        frac = np.mod(k * t, L) / L  # exact integer reduction, then one division
        feats[:, k] = np.sin(2.0 * np.pi * frac)
        feats[:, K + k] = np.cos(2.0 * np.pi * frac)
    return feats


def filter_ffn(e: np.ndarray, W1, b1, W2, b2, W3, b3, cols=None) -> np.ndarray:
    """FFN(e(t)) for every t: sin(W1 e + b1) -> sin(W2 . + b2) -> W3 . + b3.

    Weights are row-major [out][in] (W1 [H][1+2K], W2 [H][H], W3 [N*D][H]).
    Returns [L, len(cols)] (all N*D outputs when cols is None).  ``cols``
    selects output columns j = n*D + d so large shapes only evaluate the
    columns a test needs.
    """
    W1 = np.asarray(W1, np.float64); b1 = np.asarray(b1, np.float64)
    W2 = np.asarray(W2, np.float64); b2 = np.asarray(b2, np.float64)
    W3 = np.asarray(W3, np.float64); b3 = np.asarray(b3, np.float64)
    a1 = np.sin(e @ W1.T + b1)
    a2 = np.sin(a1 @ W2.T + b2)
    if cols is None:
        return a2 @ W3.T + b3
    cols = np.asarray(cols, dtype=np.int64)
    return a2 @ W3[cols].T + b3[cols]


def filter_gen(params: dict, L: int, channels=None) -> np.ndarray:
    """Filters h[n, d, t] = exp(-alpha_d * t / L) * FFN(e(t))[n*D + d].

    ``params`` holds D, N, K and the arrays W1, b1, W2, b2, W3, b3, alpha (any
    float dtype; upcast to float64).  Returns [N, D, L] float64, or
    [N, len(channels), L] when ``channels`` (a list of d) is given.
    """
    D, N, K = int(params["D"]), int(params["N"]), int(params.get("K", 8))
    chans = list(range(D)) if channels is None else [int(c) for c in channels]
    cols = [n * D + d for n in range(N) for d in chans]
    e = positional_features(L, K)
    o = filter_ffn(e, params["W1"], params["b1"], params["W2"], params["b2"],
                   params["W3"], params["b3"], cols=cols)          # [L, N*len(chans)]
    alpha = np.asarray(params["alpha"], np.float64)
    t = np.arange(L, dtype=np.float64)
    h = np.empty((N, len(chans), L), dtype=np.float64)
    for n in range(N):
        for i, d in enumerate(chans):
            window = np.exp(-alpha[d] * t / L)                      # exponential decay
            h[n, i] = window * o[:, n * len(chans) + i]
    return h


# ---------------------------------------------------------------------------
# Causal long convolution ([P3] section 4, causal FIR equation; [P1] section
# "なぜ attention っぽい表現力を持てるのか": a Toeplitz matrix)
# ---------------------------------------------------------------------------

def causal_conv_direct(h: np.ndarray, z: np.ndarray) -> np.ndarray:
    """c[..., t] = sum_{k=0..t} h[..., k] * z[..., t-k]  for t = 0..L-1.

    Brute force over the lag k.  ``h`` broadcasts against ``z`` on the
    leading axes; the last axis is time.
    """
    h = np.asarray(h, np.float64)
    z = np.asarray(z, np.float64)
    L = z.shape[-1]
    assert h.shape[-1] == L
    shape = np.broadcast_shapes(h.shape, z.shape)
    c = np.zeros(shape, dtype=np.float64)
    for k in range(L):
        c[..., k:] += h[..., k:k + 1] * z[..., :L - k]
    return c


def _bit_reverse_indices(n: int) -> np.ndarray:
    bits = n.bit_length() - 1
    idx = np.arange(n, dtype=np.int64)
    rev = np.zeros(n, dtype=np.int64)
    for b in range(bits):
        rev |= ((idx >> b) & 1) << (bits - 1 - b)
    return rev


def fft(x: np.ndarray, inverse: bool = False) -> np.ndarray:
    """The oracle's own iterative radix-2 Cooley-Tukey DFT along the last axis.

    Forward: X[k] = sum_n x[n] exp(-2*pi*i*n*k/P).  Inverse uses the opposite
    sign and divides by P.  P must be a power of two.  Decimation in time:
    bit-reverse the input, then merge sub-transforms of size m into 2m with
    X[k] = E[k] + w^k O[k], X[k+m] = E[k] - w^k O[k], w = exp(-+2*pi*i/(2m)).
    """
    a = np.asarray(x, dtype=np.complex128)
    P = a.shape[-1]
    assert P >= 1 and (P & (P - 1)) == 0, "power-of-two length required"
    lead = a.shape[:-1]
    a = a[..., _bit_reverse_indices(P)].copy()
    sign = 1.0 if inverse else -1.0
    m = 1
    while m < P:
        k = np.arange(m, dtype=np.float64)
        w = np.cos(np.pi * k / m) + sign * 1j * np.sin(np.pi * k / m)
        blocks = a.reshape(*lead, P // (2 * m), 2, m)
        even = blocks[..., 0, :]
        odd = blocks[..., 1, :] * w
        a = np.stack([even + odd, even - odd], axis=-2).reshape(*lead, P)
        m *= 2
    if inverse:
        a = a / P
    return a


def causal_conv_fft(h: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Same result as causal_conv_direct, by zero-padded FFT ([P2] "計算効率":
    transform, pointwise product, inverse transform; [P5] "手法: HyenaND":
    pad to twice the length so no circular wrap reaches the kept samples).
    """
    h = np.asarray(h, np.float64)
    z = np.asarray(z, np.float64)
    L = z.shape[-1]
    P = 1
    while P < 2 * L:
        P *= 2
    hp = np.zeros(h.shape[:-1] + (P,)); hp[..., :L] = h
    zp = np.zeros(z.shape[:-1] + (P,)); zp[..., :L] = z
    c = fft(fft(hp) * fft(zp), inverse=True)
    return c[..., :L].real


def causal_conv(h: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Direct sum for L <= DIRECT_MAX_L, FFT path beyond."""
    if np.asarray(z).shape[-1] <= DIRECT_MAX_L:
        return causal_conv_direct(h, z)
    return causal_conv_fft(h, z)


# ---------------------------------------------------------------------------
# The order-N recurrence ([P1] "Hyena 演算子の形"; [P4] framework figure)
# ---------------------------------------------------------------------------

def hyena_forward(v: np.ndarray, xs, h: np.ndarray, conv=causal_conv) -> np.ndarray:
    """y = z_{N+1} with z_1 = v and z_{n+1} = x_n * (h_n conv z_n).

    v: [..., D, L]; xs: sequence of N arrays shaped like v; h: [N, D, L].
    Gate x_n pairs with filter h_n at step n (figure of [P4]: the step that
    produces z2 uses x1 and h1).  Returns float64 with v's shape.
    """
    z = np.asarray(v, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    N = h.shape[0]
    assert len(xs) == N
    for n in range(N):
        c = conv(h[n], z)
        z = np.asarray(xs[n], dtype=np.float64) * c
    return z


def filter_spectrum(h: np.ndarray, P: int) -> np.ndarray:
    """Half spectrum H[..., k] = sum_{t<L} h[..., t] exp(-2*pi*i*k*t/P),
    k = 0..P/2, of the filter zero-padded to P points ([P2] "計算効率", first
    step applied to the filter; any even P >= 2L serves the zero-padded
    convolution, [P5] "手法: HyenaND", boundary handling).  A power-of-two P
    goes through the oracle's radix-2 FFT; any other P is the sum above
    evaluated as written, with the phase k*t reduced mod P in integers
    (O(L P) work: small cases only).
    """
    h = np.asarray(h, np.float64)
    L = h.shape[-1]
    assert P >= 2 * L and P % 2 == 0
    if P & (P - 1) == 0:
        hp = np.zeros(h.shape[:-1] + (P,)); hp[..., :L] = h
        return fft(hp)[..., : P // 2 + 1]
    t = np.arange(L, dtype=np.int64)
    out = np.empty(h.shape[:-1] + (P // 2 + 1,), np.complex128)
    for k0 in range(0, P // 2 + 1, 256):
        k = np.arange(k0, min(P // 2 + 1, k0 + 256), dtype=np.int64)
        ph = (np.outer(t, k) % P).astype(np.float64) * (2.0 * np.pi / P)
        out[..., k0:k0 + len(k)] = h @ np.exp(-1j * ph)
    return out


# ---------------------------------------------------------------------------
# The block around the operator ([P4] framework figure, projection node;
# [P3] section 2, featurisation by short convolutions and output matrix M)
# ---------------------------------------------------------------------------

def short_conv(z: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Causal depthwise FIR along the last axis: out[..., c, t] =
    sum_{j < T, j <= t} w[c, j] * z[..., c, t - j]  (z: [..., C, L], w: [C, T])."""
    z = np.asarray(z, np.float64)
    w = np.asarray(w, np.float64)
    C, T = w.shape
    L = z.shape[-1]
    out = np.zeros_like(z)
    for j in range(min(T, L)):
        out[..., j:] += w[:, j, None] * z[..., : L - j]
    return out


def in_projection(u: np.ndarray, W_in, b_in, w_short, N: int):
    """u [B, L, D] -> (v, [x_1..x_N]), each [B, D, L]: the (N+1)D-wide
    projection u W_in^T (+ b_in), then the short causal FIR of every projected
    column, split in blocks of D columns (v first)."""
    u = np.asarray(u, np.float64)
    W_in = np.asarray(W_in, np.float64)
    B, L, D = u.shape
    assert W_in.shape == ((N + 1) * D, D)
    Z = u @ W_in.T
    if b_in is not None:
        Z = Z + np.asarray(b_in, np.float64)
    S = short_conv(np.transpose(Z, (0, 2, 1)), w_short)          # [B, (N+1)D, L]
    return S[:, :D], [S[:, n * D:(n + 1) * D] for n in range(1, N + 1)]


def in_projection_columns(u: np.ndarray, W_in, b_in, w_short, cols) -> np.ndarray:
    """The streams of in_projection at chosen projected columns only:
    [B, len(cols), L], row i being column cols[i] of the (N+1)D-wide
    projection (stream cols[i] // D, channel cols[i] % D), by the same
    definition: the column's projection u W_in[c]^T (+ b_in[c]), then its
    short causal FIR with w_short[c]."""
    cols = np.asarray(cols, np.int64)
    u = np.asarray(u, np.float64)
    Z = u @ np.asarray(W_in, np.float64)[cols].T                   # [B, L, len(cols)]
    if b_in is not None:
        Z = Z + np.asarray(b_in, np.float64)[cols]
    return short_conv(np.transpose(Z, (0, 2, 1)), np.asarray(w_short, np.float64)[cols])


def out_projection(y: np.ndarray, W_out, b_out) -> np.ndarray:
    """y [B, D, L] -> [B, L, D]: out[b, t, e] = sum_d W_out[e, d] y[b, d, t] (+ b_out[e])."""
    o = np.transpose(np.asarray(y, np.float64), (0, 2, 1)) @ np.asarray(W_out, np.float64).T
    if b_out is not None:
        o = o + np.asarray(b_out, np.float64)
    return o


def block_forward(u: np.ndarray, bp: dict, h: np.ndarray, conv=causal_conv) -> np.ndarray:
    """u [B, L, D] -> [B, L, D]: in_projection, the order-N operator with
    filters h [N, D, L], out_projection.  bp holds W_in, b_in, w_short, W_out,
    b_out (biases may be None)."""
    N = h.shape[0]
    v, xs = in_projection(u, bp["W_in"], bp.get("b_in"), bp["w_short"], N)
    y = hyena_forward(v, xs, h, conv=conv)
    return out_projection(y, bp["W_out"], bp.get("b_out"))


# ---------------------------------------------------------------------------
# Backward of the recurrence (chain rule through [P1] "Hyena 演算子の形";
# [P3] section 4's causal FIR and its transpose)
# ---------------------------------------------------------------------------

def causal_conv_adjoint(h: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Transpose of c = h conv z (causal, length L) applied to g:
    out[..., s] = sum_{t >= s} h[..., t - s] * g[..., t]."""
    h = np.asarray(h, np.float64)
    g = np.asarray(g, np.float64)
    L = g.shape[-1]
    if L <= DIRECT_MAX_L:
        out = np.zeros(np.broadcast_shapes(h.shape[:-1], g.shape[:-1]) + (L,))
        for k in range(L):
            out[..., : L - k] += h[..., k:k + 1] * g[..., k:]
        return out
    P = 1
    while P < 2 * L:
        P *= 2
    hp = np.zeros(h.shape[:-1] + (P,)); hp[..., :L] = h
    gp = np.zeros(g.shape[:-1] + (P,)); gp[..., :L] = g
    return np.real(fft(np.conj(fft(hp)) * fft(gp), inverse=True))[..., :L]


def filter_correlation(g: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Gradient of c = h conv z with respect to h, contracted with g:
    out[..., k] = sum_{t >= k} g[..., t] * z[..., t - k]."""
    g = np.asarray(g, np.float64)
    z = np.asarray(z, np.float64)
    L = g.shape[-1]
    if L <= DIRECT_MAX_L:
        out = np.zeros(np.broadcast_shapes(g.shape, z.shape))
        for k in range(L):
            out[..., k] = np.sum(g[..., k:] * z[..., : L - k], axis=-1)
        return out
    P = 1
    while P < 2 * L:
        P *= 2
    gp = np.zeros(g.shape[:-1] + (P,)); gp[..., :L] = g
    zp = np.zeros(z.shape[:-1] + (P,)); zp[..., :L] = z
    return np.real(fft(np.conj(fft(zp)) * fft(gp), inverse=True))[..., :L]


def hyena_backward(v: np.ndarray, xs, h: np.ndarray, gy: np.ndarray, conv=causal_conv, circular: bool = False):
    """Gradients of a scalar loss with dloss/dy = gy through y = z_{N+1}:
    returns (gv, [gx_1..gx_N], gh) with gh [N, D, L] summed over the batch.

    Forward intermediates: z_1 = v, c_n = h_n conv z_n, z_{n+1} = x_n * c_n.
    Backward, n = N..1, with g = dloss/dz_{n+1}: gx_n = g * c_n;
    gc = g * x_n; gh_n = sum_b corr(gc, z_n); g <- adjoint conv of gc by h_n.
    circular: the convolution is periodic (conv defaults to circular_conv),
    and the adjoint and the correlation are the periodic ones.
    """
    if circular:
        if conv is causal_conv:
            conv = circular_conv
        adjoint, correlation = circular_conv_adjoint, circular_filter_correlation
    else:
        adjoint, correlation = causal_conv_adjoint, filter_correlation
    v = np.asarray(v, np.float64)
    h = np.asarray(h, np.float64)
    N = h.shape[0]
    zs, cs = [v], []
    for n in range(N):
        c = conv(h[n], zs[-1])
        cs.append(c)
        zs.append(np.asarray(xs[n], np.float64) * c)
    g = np.asarray(gy, np.float64)
    gxs = [None] * N
    gh = np.zeros_like(h)
    batch_axes = tuple(range(v.ndim - 2))
    for n in reversed(range(N)):
        x = np.asarray(xs[n], np.float64)
        gxs[n] = g * cs[n]
        gc = g * x
        gh[n] = np.sum(correlation(gc, zs[n]), axis=batch_axes) if batch_axes else correlation(gc, zs[n])
        g = adjoint(h[n], gc)
    return g, gxs, gh


# ---------------------------------------------------------------------------
# Other filter families ([P3] section 3: Hyena-LI, Hyena-SE, Hyena-MR)
# ---------------------------------------------------------------------------

def filter_gen_li(R: np.ndarray, lam: np.ndarray, L: int) -> np.ndarray:
    """Hyena-LI: h[f, t] = sum_s R[f, s] * lam[f, s]**t, t = 0..L-1 (0**0 = 1)."""
    R = np.asarray(R, np.float64)
    lam = np.asarray(lam, np.float64)
    t = np.arange(L, dtype=np.float64)
    return np.sum(R[..., None] * np.power(lam[..., None], t), axis=-2)


def filter_gen_mr(hhat: np.ndarray, alpha: np.ndarray, N: int) -> np.ndarray:
    """Hyena-MR: h[n, d, t] = hhat[n, d, t] * exp(-alpha[d] * t) (explicit
    filter of its own length, exponentially damped per channel)."""
    hhat = np.asarray(hhat, np.float64)
    alpha = np.asarray(alpha, np.float64)
    Lh = hhat.shape[-1]
    t = np.arange(Lh, dtype=np.float64)
    return hhat * np.exp(-alpha[None, :, None] * t)


def circular_conv(h: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Periodic convolution over the last axis ([P5] "手法: HyenaND", boundary
    handling): out[..., t] = sum_{k<L} h[..., k] * z[..., (t - k) mod L].
    Brute force for L <= DIRECT_MAX_L, else the oracle's FFT of length L
    (L a power of two)."""
    h = np.asarray(h, np.float64)
    z = np.asarray(z, np.float64)
    L = z.shape[-1]
    if L <= DIRECT_MAX_L:
        out = np.zeros(np.broadcast_shapes(h.shape[:-1], z.shape[:-1]) + (L,))
        for k in range(L):
            out += h[..., k:k + 1] * np.roll(z, k, axis=-1)
        return out
    return np.real(fft(fft(h) * fft(z), inverse=True))


def circular_conv_adjoint(h: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Transpose of the periodic convolution c = h conv z applied to g:
    out[..., s] = sum_t h[..., (t - s) mod L] * g[..., t]."""
    h = np.asarray(h, np.float64)
    g = np.asarray(g, np.float64)
    L = g.shape[-1]
    if L <= DIRECT_MAX_L:
        out = np.zeros(np.broadcast_shapes(h.shape[:-1], g.shape[:-1]) + (L,))
        for k in range(L):
            out += h[..., k:k + 1] * np.roll(g, -k, axis=-1)
        return out
    return np.real(fft(np.conj(fft(h)) * fft(g), inverse=True))


def circular_filter_correlation(g: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Gradient of the periodic c = h conv z with respect to h, contracted
    with g: out[..., k] = sum_t g[..., t] * z[..., (t - k) mod L]."""
    g = np.asarray(g, np.float64)
    z = np.asarray(z, np.float64)
    L = g.shape[-1]
    if L <= DIRECT_MAX_L:
        out = np.zeros(np.broadcast_shapes(g.shape, z.shape))
        for k in range(L):
            out[..., k] = np.sum(g * np.roll(z, k, axis=-1), axis=-1)
        return out
    return np.real(fft(np.conj(fft(z)) * fft(g), inverse=True))


# ---------------------------------------------------------------------------
# Convolution on k-dimensional grids ([P5] "手法: HyenaND": native N-D
# convolution through the N-D FFT; boundary handling, circular for periodic
# systems and twice-padded non-circular for images and volumes)
# ---------------------------------------------------------------------------

def _grid_shape(K: np.ndarray, ndim: int, circular: bool):
    ext = K.shape[-ndim:]
    if circular:
        return tuple(ext)
    assert all(e % 2 == 1 for e in ext), "non-circular kernels have odd extent 2L-1"
    return tuple((e + 1) // 2 for e in ext)


def ndfft(x: np.ndarray, ndim: int, inverse: bool = False) -> np.ndarray:
    """DFT over the last ``ndim`` axes: the k-dimensional DFT is the 1-D DFT
    applied along each axis in turn (the oracle's own radix-2 ``fft``)."""
    a = np.asarray(x, dtype=np.complex128)
    for ax in range(a.ndim - ndim, a.ndim):
        a = np.moveaxis(fft(np.moveaxis(a, ax, -1), inverse=inverse), -1, ax)
    return a


def nd_conv_direct(K: np.ndarray, z: np.ndarray, ndim: int, circular: bool = False) -> np.ndarray:
    """y[..., t] = sum_s K[..., t - s] z[..., s] over the last ``ndim`` axes,
    brute force over the kernel offsets o = t - s.

    Non-circular: K[..., o_1 + L_1 - 1, .., o_k + L_k - 1] for |o_a| < L_a,
    and only pairs with both t and s on the grid contribute.  Circular: K has
    the grid's shape and t - s is taken modulo L_a.  K broadcasts against z
    on the leading axes.
    """
    K = np.asarray(K, np.float64)
    z = np.asarray(z, np.float64)
    Ls = _grid_shape(K, ndim, circular)
    assert tuple(z.shape[-ndim:]) == Ls
    lead = np.broadcast_shapes(K.shape[:-ndim], z.shape[:-ndim])
    y = np.zeros(lead + Ls)
    for idx in np.ndindex(*K.shape[-ndim:]):
        w = K[(Ellipsis,) + idx][(Ellipsis,) + (None,) * ndim]
        if circular:
            y += w * np.roll(z, shift=idx, axis=tuple(range(-ndim, 0)))
            continue
        dst, src = [], []
        for a, i in enumerate(idx):
            o, L = i - (Ls[a] - 1), Ls[a]
            dst.append(slice(max(0, o), min(L, L + o)))      # t with t - o on the grid
            src.append(slice(max(0, -o), min(L, L - o)))     # s = t - o
        y[(Ellipsis,) + tuple(dst)] += w * z[(Ellipsis,) + tuple(src)]
    return y


def nd_conv_fft(K: np.ndarray, z: np.ndarray, ndim: int, circular: bool = False) -> np.ndarray:
    """Same result as nd_conv_direct by the k-dimensional FFT ([P5]): each
    axis padded to P_a, the next power of two >= 2 L_a (non-circular; the
    kernel's offset o lands at o mod P_a, z at its own index, zeros
    elsewhere) or P_a = L_a (circular, powers of two), transform, pointwise
    product, inverse transform, keep the grid."""
    K = np.asarray(K, np.float64)
    z = np.asarray(z, np.float64)
    Ls = _grid_shape(K, ndim, circular)
    if circular:
        assert all(L & (L - 1) == 0 for L in Ls), "circular FFT path needs power-of-two sides"
        Y = ndfft(ndfft(K, ndim) * ndfft(z, ndim), ndim, inverse=True)
        return Y.real
    Ps = []
    for L in Ls:
        P = 1
        while P < 2 * L:
            P *= 2
        Ps.append(P)
    Kp = np.zeros(K.shape[:-ndim] + tuple(Ps))
    for idx in np.ndindex(*K.shape[-ndim:]):
        dst = tuple((i - (Ls[a] - 1)) % Ps[a] for a, i in enumerate(idx))
        Kp[(Ellipsis,) + dst] = K[(Ellipsis,) + idx]
    zp = np.zeros(z.shape[:-ndim] + tuple(Ps))
    zp[(Ellipsis,) + tuple(slice(0, L) for L in Ls)] = z
    Y = ndfft(ndfft(Kp, ndim) * ndfft(zp, ndim), ndim, inverse=True)
    return Y[(Ellipsis,) + tuple(slice(0, L) for L in Ls)].real


def nd_conv(K: np.ndarray, z: np.ndarray, ndim: int, circular: bool = False) -> np.ndarray:
    """Brute force while the offset count times the grid is small, else FFT."""
    Ls = _grid_shape(np.asarray(K), ndim, circular)
    work = int(np.prod(np.asarray(K).shape[-ndim:])) * int(np.prod(Ls))
    pow2 = all(L & (L - 1) == 0 for L in Ls)
    if work <= (1 << 20) or (circular and not pow2):
        return nd_conv_direct(K, z, ndim, circular)
    return nd_conv_fft(K, z, ndim, circular)


def nd_forward(v: np.ndarray, xs, K: np.ndarray, ndim: int, circular: bool = False,
               per_sample: bool = False) -> np.ndarray:
    """The order-N recurrence of [P1]/[P4] with grid convolutions ([P5]).

    v: [B, D, L_1..L_k]; xs: N arrays shaped like v.  K: [N, D, ext...]
    shared by the batch, or [B, N, D, ext...] with per_sample (the kernel of
    each sample).  z_1 = v, z_{n+1} = x_n * (K_n conv z_n), y = z_{N+1}.
    """
    z = np.asarray(v, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    N = K.shape[1] if per_sample else K.shape[0]
    assert len(xs) == N
    for n in range(N):
        Kn = K[:, n] if per_sample else K[n]
        z = np.asarray(xs[n], dtype=np.float64) * nd_conv(Kn, z, ndim, circular)
    return z
