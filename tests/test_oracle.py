"""Pins for the float64 oracle, each from something other than the oracle.

* hand-derived p4 examples (tests/golden/p4_shift.txt)
* the dense block-circulant matrix of [pchao] §3.1 eq. (1), assembled and
  multiplied by numpy (the "naive EQ-Linear" of the pages)
* T = 1, where the layer is an ordinary linear layer (numpy matmul)
* one-hot inputs that fix the circulant direction
* the convolution theorem, [pchao] §3.1 eq. (3), evaluated with numpy.fft
* the p4 closed forms of [pchao] App. 6.2 eqs. (19)-(21)
* equivariance under every cyclic shift of the group axis ([pchao] §4.3)
* adjoint identities <dY, Y> = <dX, X> = <dWt, Wt> of the bilinear map, and
  brute-force chain rule through the assembled dense matrix
* numpy.fft.rfft for the spectrum
* the bias: the dense linear layer with b tiled over the group ([pchao]
  §3.1, below eq. (1)) and its gradient by torch autograd through that tiling
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p4_shift.txt")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def dense_weight(w):
    """Assemble the dense (D_T*T) x (C_T*T) block-circulant matrix.

    Channel index is c*T + g (group axis contiguous).  Block (g, h) of the
    matrix is Wt[:, :, (g - h) mod T]: row g of the block matrix of eq. (1)
    is a cyclic shift of row 0 by g positions.
    """
    D_T, C_T, T = w.shape
    W = np.zeros((D_T * T, C_T * T))
    for g in range(T):
        for h in range(T):
            W[g::T, h::T] = w[:, :, (g - h) % T]
    return W


SHAPES = [  # (N, C_T, D_T, T)
    (3, 2, 3, 1), (4, 3, 2, 2), (2, 3, 4, 3), (5, 4, 3, 4), (3, 2, 5, 5),
    (2, 3, 2, 8), (1, 1, 1, 4), (7, 5, 6, 6),
]


# ---------------------------------------------------------------- golden
def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, xs, ws, exp = [s.strip() for s in line.split("|")]
            rows.append((kind, xs, ws, exp))
    return rows


@pytest.mark.parametrize("row", _golden_rows())
def test_golden_p4(row):
    kind, xs, ws, exp = row
    w = np.array([float(v) for v in ws.split()]).reshape(1, 1, 4)
    e = np.array([float(v) for v in exp.split()])
    if kind == "forward":
        x = np.array([float(v) for v in xs.split()]).reshape(1, 1, 4)
        y = oracle.forward(x, w)
        np.testing.assert_array_equal(y.reshape(-1), e)
    else:
        s = oracle.spectrum(w)
        np.testing.assert_allclose(s.reshape(-1), e, atol=1e-14)


# ---------------------------------------------------------------- forward
@pytest.mark.parametrize("shape", SHAPES)
def test_forward_matches_dense_block_circulant(shape):
    N, C_T, D_T, T = shape
    x, w = rand((N, C_T, T), 1), rand((D_T, C_T, T), 2)
    ref = (x.reshape(N, -1) @ dense_weight(w).T).reshape(N, D_T, T)
    np.testing.assert_allclose(oracle.forward(x, w), ref, rtol=1e-12, atol=1e-12)


def test_t1_is_ordinary_linear():
    x, w = rand((9, 7, 1), 3), rand((5, 7, 1), 4)
    ref = x[:, :, 0] @ w[:, :, 0].T
    np.testing.assert_allclose(oracle.forward(x, w)[:, :, 0], ref, rtol=1e-13, atol=1e-13)
    dy = rand((9, 5, 1), 5)
    np.testing.assert_allclose(oracle.backward_input(dy, w)[:, :, 0],
                               dy[:, :, 0] @ w[:, :, 0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.backward_weight(x, dy)[:, :, 0],
                               dy[:, :, 0].T @ x[:, :, 0], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("T", [2, 3, 4, 5, 6, 7, 8])
def test_delta_fixes_direction(T):
    """One-hot X at (n0,c0,h0) and one-hot Wt at (d0,c0,m0) give a single
    one at Y[n0,d0,(h0+m0) mod T] (the weight shift moves h to h+m)."""
    N, C_T, D_T = 3, 4, 5
    for h0 in range(T):
        for m0 in range(T):
            x = np.zeros((N, C_T, T)); x[1, 2, h0] = 1.0
            w = np.zeros((D_T, C_T, T)); w[3, 2, m0] = 1.0
            y = oracle.forward(x, w)
            e = np.zeros((N, D_T, T)); e[1, 3, (h0 + m0) % T] = 1.0
            np.testing.assert_array_equal(y, e)


@pytest.mark.parametrize("shape", SHAPES)
def test_forward_convolution_theorem_fft(shape):
    """[pchao] §3.1 eq. (3): per frequency k, Yhat_k = Xhat_k . What_k^T."""
    N, C_T, D_T, T = shape
    x, w = rand((N, C_T, T), 6), rand((D_T, C_T, T), 7)
    xf = np.fft.fft(x, axis=2)
    wf = np.fft.fft(w, axis=2)
    yf = np.einsum("nck,dck->ndk", xf, wf)
    ref = np.fft.ifft(yf, axis=2)
    assert np.abs(ref.imag).max() < 1e-10
    np.testing.assert_allclose(oracle.forward(x, w), ref.real, rtol=1e-11, atol=1e-11)


def test_p4_closed_forms_eq19_to_21():
    """[pchao] App. 6.2: eq. (19) transform, eq. (20) products, eq. (21)
    inverse (coefficients 1/4, 1/2 as in the matrix of §3.2.2 step 4)."""
    N, C_T, D_T, T = 6, 5, 7, 4
    x, w = rand((N, C_T, T), 8), rand((D_T, C_T, T), 9)

    def eq19(v):
        v0, v1, v2, v3 = (v[..., i] for i in range(4))
        return v0 + v1 + v2 + v3, v0 - v2, v0 - v1 + v2 - v3, v3 - v1

    f0, f1, f2, f3 = eq19(x)
    w0, w1, w2, w3 = eq19(w)
    a0 = f0 @ w0.T
    a1 = f1 @ w1.T - f3 @ w3.T
    a2 = f2 @ w2.T
    a3 = f1 @ w3.T + f3 @ w1.T
    y = np.stack([a0 / 4 + a1 / 2 + a2 / 4,
                  a0 / 4 - a2 / 4 - a3 / 2,
                  a0 / 4 - a1 / 2 + a2 / 4,
                  a0 / 4 - a2 / 4 + a3 / 2], axis=-1)
    np.testing.assert_allclose(oracle.forward(x, w), y, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [2, 3, 4, 5, 6, 7, 8])
def test_equivariance_every_shift(T):
    x, w = rand((4, 3, T), 10), rand((5, 3, T), 11)
    y = oracle.forward(x, w)
    for s in range(T):
        ys = oracle.forward(np.roll(x, s, axis=2), w)
        np.testing.assert_allclose(ys, np.roll(y, s, axis=2), rtol=1e-12, atol=1e-12)


def test_row_selection_matches_full():
    x, w, dy = rand((11, 4, 4), 12), rand((6, 4, 4), 13), rand((11, 6, 4), 14)
    rows = [10, 0, 5, 5]
    np.testing.assert_array_equal(oracle.forward(x, w, rows=rows), oracle.forward(x, w)[rows])
    np.testing.assert_array_equal(oracle.backward_input(dy, w, rows=rows),
                                  oracle.backward_input(dy, w)[rows])
    ds = [5, 1]
    np.testing.assert_array_equal(oracle.backward_weight(x, dy, dsel=ds),
                                  oracle.backward_weight(x, dy)[ds])


# ---------------------------------------------------------------- gradients
@pytest.mark.parametrize("shape", SHAPES)
def test_adjoint_identities(shape):
    N, C_T, D_T, T = shape
    x, w, dy = rand((N, C_T, T), 15), rand((D_T, C_T, T), 16), rand((N, D_T, T), 17)
    y = oracle.forward(x, w)
    dx = oracle.backward_input(dy, w)
    dw = oracle.backward_weight(x, dy)
    a, b, c = np.sum(dy * y), np.sum(dx * x), np.sum(dw * w)
    scale = np.sqrt(np.sum(dy * dy) * np.sum(y * y)) + 1e-30
    assert abs(a - b) / scale < 1e-12
    assert abs(a - c) / scale < 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_gradients_brute_force_dense(shape):
    """dX = dY . W_dense; dWt = chain rule of W_dense(Wt): sum of dY^T X over
    the (g, h) blocks that carry shift m = (g - h) mod T."""
    N, C_T, D_T, T = shape
    x, w, dy = rand((N, C_T, T), 18), rand((D_T, C_T, T), 19), rand((N, D_T, T), 20)
    Wd = dense_weight(w)
    ref_dx = (dy.reshape(N, -1) @ Wd).reshape(N, C_T, T)
    np.testing.assert_allclose(oracle.backward_input(dy, w), ref_dx, rtol=1e-12, atol=1e-12)
    G = dy.reshape(N, -1).T @ x.reshape(N, -1)          # dL/dW_dense
    ref_dw = np.zeros((D_T, C_T, T))
    for g in range(T):
        for h in range(T):
            ref_dw[:, :, (g - h) % T] += G[g::T, h::T]
    np.testing.assert_allclose(oracle.backward_weight(x, dy), ref_dw, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [2, 3, 4, 5, 6, 7, 8])
def test_gradients_fft_route(T):
    """Correlation theorem: dXhat_k = dYhat_k conj(What_k);
    dWhat_k = sum_n dYhat_k conj(Xhat_k)."""
    N, C_T, D_T = 5, 3, 4
    x, w, dy = rand((N, C_T, T), 21), rand((D_T, C_T, T), 22), rand((N, D_T, T), 23)
    xf, wf, dyf = (np.fft.fft(a, axis=2) for a in (x, w, dy))
    dxf = np.einsum("ndk,dck->nck", dyf, np.conj(wf))
    dwf = np.einsum("ndk,nck->dck", dyf, np.conj(xf))
    np.testing.assert_allclose(oracle.backward_input(dy, w), np.fft.ifft(dxf, axis=2).real,
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(oracle.backward_weight(x, dy), np.fft.ifft(dwf, axis=2).real,
                               rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- spectrum
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_spectrum_matches_numpy_rfft(T):
    D_T, C_T = 6, 5
    w = rand((D_T, C_T, T), 24)
    r = np.fft.rfft(w, axis=2)                    # [D_T, C_T, T//2+1]
    planes = [r[:, :, 0].real]
    for k in range(1, (T - 1) // 2 + 1):
        planes += [r[:, :, k].real, r[:, :, k].imag]
    if T % 2 == 0 and T > 1:
        planes.append(r[:, :, T // 2].real)
    np.testing.assert_allclose(oracle.spectrum(w), np.stack(planes), rtol=1e-12, atol=1e-12)


def test_spectrum_p4_eq19():
    w = rand((4, 3, 4), 25)
    s = oracle.spectrum(w)
    w0, w1, w2, w3 = (w[..., i] for i in range(4))
    np.testing.assert_allclose(s[0], w0 + w1 + w2 + w3, atol=1e-13)
    np.testing.assert_allclose(s[1], w0 - w2, atol=1e-13)
    np.testing.assert_allclose(s[2], w3 - w1, atol=1e-13)
    np.testing.assert_allclose(s[3], w0 - w1 + w2 - w3, atol=1e-13)


def test_thread_count_does_not_change_results():
    """Each element is one sequential float64 sum: bitwise stable."""
    x, w = rand((33, 6, 4), 26), rand((7, 6, 4), 27)
    a = oracle.forward(x, w)
    b = np.concatenate([oracle.forward(x, w, rows=[i]) for i in range(33)])
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- bias
@pytest.mark.parametrize("shape", SHAPES)
def test_bias_is_tiled_dense_bias(shape):
    """With bias, Y is the naive layer XW^T + b where b in R^D tiles the
    group-shared bias over the T group components ([pchao] §3.1, eq. (7))."""
    N, C_T, D_T, T = shape
    x, w, b = rand((N, C_T, T), 40), rand((D_T, C_T, T), 41), rand((D_T,), 42)
    ref = x.reshape(N, -1) @ dense_weight(w).T + np.tile(b[:, None], (1, T)).reshape(-1)
    np.testing.assert_allclose(oracle.forward(x, w, bias=b), ref.reshape(N, D_T, T),
                               rtol=1e-12, atol=1e-12)
    rows = [N - 1, 0]
    np.testing.assert_array_equal(oracle.forward(x, w, rows=rows, bias=b),
                                  oracle.forward(x, w, bias=b)[rows])


@pytest.mark.parametrize("shape", SHAPES)
def test_bias_gradient_autograd(shape):
    """db from torch autograd (float64, CPU) through the tiled dense bias."""
    import torch
    N, C_T, D_T, T = shape
    x, w, b, dy = (rand((N, C_T, T), 43), rand((D_T, C_T, T), 44), rand((D_T,), 45),
                   rand((N, D_T, T), 46))
    bt = torch.tensor(b, requires_grad=True)
    y = torch.nn.functional.linear(torch.tensor(x.reshape(N, -1)), torch.tensor(dense_weight(w)),
                                   bt.repeat_interleave(T))
    y.backward(torch.tensor(dy.reshape(N, -1)))
    np.testing.assert_allclose(oracle.backward_bias(dy), bt.grad.numpy(), rtol=1e-12, atol=1e-12)
    # degenerate: no rows gives zeros
    np.testing.assert_array_equal(oracle.backward_bias(np.zeros((0, D_T, T))), np.zeros(D_T))
