"""Pins of the octic-group oracle (CPU only).

The octic group: quarter turns r and a reflection s, element g = a + 4 b for
r^a s^b.  Everything group-theoretic here is computed independently of the
oracle's C code, from the faithful representation of the group on the plane
(2x2 integer matrices R = quarter turn, S = reflection): products and inverses
by matrix arithmetic, and the irreducible representations for the Fourier
transform from their defining images of r and s.

Pins: the dense matrix of the layer assembled from that arithmetic (forward,
input gradient, weight gradient by the chain rule, bias), equivariance under
all eight elements, the rotation subgroup reducing to the cyclic layer of
order 4, the adjoint identities, hand-worked one-hot cases
(tests/golden/octic_onehot.txt), and the convolution theorem of the group
Fourier transform (Schur: the layer is a matrix product per irreducible
representation).
"""
import os

import numpy as np
import pytest

import oracle

R = np.array([[0, -1], [1, 0]])
S = np.array([[1, 0], [0, -1]])


def mat(u):
    a, b = u % 4, u // 4
    return np.linalg.matrix_power(R, a) @ np.linalg.matrix_power(S, b)


MATS = [mat(u) for u in range(8)]


def index_of(m):
    for u, mu in enumerate(MATS):
        if np.array_equal(mu, m):
            return u
    raise AssertionError("not a group element")


def mul(g, h):
    return index_of(MATS[g] @ MATS[h])


def inv(g):
    return index_of(np.round(np.linalg.inv(MATS[g])).astype(int))


def dense_weight_octic(w):
    """W[d*8+g, c*8+h] = Wt[d, c, h^-1 g]: the regular-representation layer."""
    D_T, C_T, _ = w.shape
    W = np.zeros((D_T * 8, C_T * 8))
    for g in range(8):
        for h in range(8):
            W[g::8, h::8] = w[:, :, mul(inv(h), g)]
    return W


def act(k, v):
    """Left regular action on the group axis: (k . v)[g] = v[k^-1 g]."""
    out = np.empty_like(v)
    for g in range(8):
        out[..., g] = v[..., mul(inv(k), g)]
    return out


CHI_R = [1, 1, -1, -1]
CHI_S = [1, -1, 1, -1]


def fourier(v):
    """Group Fourier transform along the last axis: 8 real planes
    (A1, A2, B1, B2, E11, E12, E21, E22) of sum_u v[u] rho(u), first axis."""
    out = []
    for j in range(4):
        coef = np.array([CHI_R[j] ** (u % 4) * CHI_S[j] ** (u // 4) for u in range(8)], float)
        out.append(v @ coef)
    for i in range(2):
        for k in range(2):
            coef = np.array([MATS[u][i, k] for u in range(8)], float)
            out.append(v @ coef)
    return np.stack(out)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol=1e-9):
    return a.shape == b.shape and np.allclose(a, b, rtol=tol, atol=tol)


def battery_octic(o):
    """Run the octic pins against oracle build ``o``; return failures."""
    failed = []
    for (N, C_T, D_T) in [(3, 2, 3), (2, 1, 4), (4, 3, 2)]:
        x, w, dy = rand((N, C_T, 8), 11), rand((D_T, C_T, 8), 12), rand((N, D_T, 8), 13)
        Wd = dense_weight_octic(w)
        y = o.octic_forward(x, w)
        if not _close(y, (x.reshape(N, -1) @ Wd.T).reshape(N, D_T, 8)):
            failed.append("dense_fwd")
        if not _close(o.octic_backward_input(dy, w), (dy.reshape(N, -1) @ Wd).reshape(N, C_T, 8)):
            failed.append("dense_dx")
        # weight gradient by the chain rule through the dense matrix
        G = dy.reshape(N, -1).T @ x.reshape(N, -1)
        ref = np.zeros((D_T, C_T, 8))
        for g in range(8):
            for h in range(8):
                ref[:, :, mul(inv(h), g)] += G[g::8, h::8]
        if not _close(o.octic_backward_weight(x, dy), ref):
            failed.append("dense_dw")
        b = rand((D_T,), 14)
        if not _close(o.octic_forward(x, w, bias=b), y + b[None, :, None]):
            failed.append("bias")
        # equivariance under every element
        for k in range(8):
            if not _close(o.octic_forward(act(k, x), w), act(k, y)):
                failed.append("equivariance_%d" % k)
                break
        # adjoint identities of the bilinear map
        dx = o.octic_backward_input(dy, w)
        dw = o.octic_backward_weight(x, dy)
        s = float(np.sum(dy * y))
        if not (np.isclose(s, float(np.sum(dx * x))) and np.isclose(s, float(np.sum(dw * w)))):
            failed.append("adjoint")
        # convolution theorem: Yhat_d(rho) = sum_c Xhat_c(rho) What_dc(rho)
        Xh, Yh, Wh = fourier(x), fourier(y), fourier(w)
        ok = all(np.allclose(Yh[j], Xh[j] @ Wh[j].T) for j in range(4))
        E = lambda F, i, k: F[4 + 2 * i + k]   # noqa: E731
        for i in range(2):
            for k in range(2):
                want = sum(E(Xh, i, m) @ E(Wh, m, k).T for m in range(2))
                ok = ok and np.allclose(E(Yh, i, k), want)
        if not ok:
            failed.append("convolution_theorem")
        if not _close(o.octic_spectrum(w), fourier(w)):
            failed.append("spectrum")
    # rotations only: the cyclic layer of order 4
    N, C_T, D_T = 3, 2, 3
    x, w = rand((N, C_T, 8), 15), rand((D_T, C_T, 8), 16)
    x[..., 4:] = 0.0
    w[..., 4:] = 0.0
    y = o.octic_forward(x, w)
    if not (_close(y[..., :4], o.forward(x[..., :4], w[..., :4])) and not np.any(y[..., 4:])):
        failed.append("rotation_subgroup")
    return failed


def test_group_table():
    """The matrix representation is a group of order 8 and faithful; r has
    order 4, s order 2, and s r s = r^-1 (the dihedral relations)."""
    assert len({m.tobytes() for m in MATS}) == 8
    for g in range(8):
        for h in range(8):
            for k in range(8):
                assert mul(mul(g, h), k) == mul(g, mul(h, k))
        assert mul(g, inv(g)) == 0
    assert mul(4, mul(1, 4)) == inv(1)


def test_fourier_is_invertible():
    """Plancherel for the real transform: 8 sum v^2 = sum_chi vhat^2 + 2 sum E_ik^2."""
    v = rand((5, 8), 21)
    F = fourier(v)
    lhs = 8 * np.sum(v * v, axis=1)
    rhs = np.sum(F[:4] ** 2, axis=0) + 2 * np.sum(F[4:] ** 2, axis=0)
    assert np.allclose(lhs, rhs)


def test_octic_oracle_pins():
    assert battery_octic(oracle._default()) == []


def read_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "octic_onehot.txt")
    cases = []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            u, h, g = (int(t) for t in line.split())
            cases.append((u, h, g))
    return cases


@pytest.mark.parametrize("case", read_golden())
def test_octic_onehot_golden(case):
    """One-hot weight at u and input at h: Y is one-hot at g = h u (worked by
    hand in the golden file)."""
    u, h, g = case
    x = np.zeros((1, 1, 8))
    x[0, 0, h] = 1.0
    w = np.zeros((1, 1, 8))
    w[0, 0, u] = 1.0
    y = oracle.octic_forward(x, w)
    want = np.zeros((1, 1, 8))
    want[0, 0, g] = 1.0
    np.testing.assert_array_equal(y, want)
