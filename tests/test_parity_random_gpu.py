"""GPU parity over seeded random shapes: every group (cyclic orders 2..8 and
the octic group), both dtypes, with and without bias, channel counts from 1
to a few hundred and row counts from 1 to several thousand, so that the host
plans (row tiles, half-width units, k-split kernels, element-granular
copies, weight-gradient splits, ring / narrow / producer-consumer kernels)
meet shapes no hand-picked case covers.  Each case compares sampled rows of
Y and dX, sampled output channels of dWt (all of them when cheap) and the
bias gradient with the float64 oracle, at the tolerances of the other
parity tests.
"""
import sys

import numpy as np
import pytest

import oracle
from group_wise_dft_amd.workloads import bias_input, custom_inputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "f16": (2e-3, None)}
CASES = 128       # small and mid sizes
LARGE = 32        # larger layers: many tiles, split weight gradients


def announce(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def E():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from group_wise_dft_amd import eqlinear
    return eqlinear


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.double().cpu().numpy()


def compare(got, ref, dt, what):
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 1.0
    mx = np.abs(got - ref).max() / max(rms, 1e-300) if ref.size else 0.0
    rtol, mtol = TOL[dt]
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert rel <= rtol, "%s: rel Frobenius %.3e > %.1e" % (what, rel, rtol)
    if mtol is not None:
        assert mx <= mtol, "%s: max-abs/RMS %.3e > %.1e" % (what, mx, mtol)


def draw_case(i):
    """Shape of case i: group, order, dtype, bias and sizes (log-uniform;
    cases from CASES on are the larger layers)."""
    rng = np.random.default_rng(7000 + i)
    octic = rng.random() < 0.2
    T = 8 if octic else int(rng.integers(2, 9))
    dt = "f32" if rng.random() < 0.5 else "f16"
    if i < CASES:
        n_lo, n_hi, c_lo, c_hi = 1.0, 6000.0, 1.0, 320.0
    else:
        n_lo, n_hi, c_lo, c_hi = 2000.0, 20000.0, 32.0, 600.0
    N = int(np.exp(rng.uniform(np.log(n_lo), np.log(n_hi))))
    C_T = int(np.exp(rng.uniform(np.log(c_lo), np.log(c_hi))))
    D_T = int(np.exp(rng.uniform(np.log(c_lo), np.log(c_hi))))
    bias = bool(rng.random() < 0.5)
    return octic, T, dt, max(1, N), max(1, C_T), max(1, D_T), bias


@pytest.mark.parametrize("i", range(CASES + LARGE))
def test_random_shape(E, i):
    octic, T, dt, N, C_T, D_T, use_bias = draw_case(i)
    announce("random %d: %s T=%d %s N=%d C_T=%d D_T=%d bias=%s" % (
        i, "octic" if octic else "cyclic", T, dt, N, C_T, D_T, use_bias))
    x, w, dy = custom_inputs(N, C_T, D_T, T, dt, seed=7100 + 10 * i)
    b = bias_input(D_T, dt, 7105 + 10 * i) if use_bias else None
    tx, tw, tdy = dev(x), dev(w), dev(dy)
    tb = dev(b) if use_bias else None
    if octic:
        what = E.eqlinear_octic_weight_spectrum(tw)
        y = E.eqlinear_octic_forward(tx, what, bias=tb)
        dx = E.eqlinear_octic_backward_input(tdy, what)
        dw = E.eqlinear_octic_backward_weight(tx, tdy)
        fwd, bwd_x, bwd_w = oracle.octic_forward, oracle.octic_backward_input, oracle.octic_backward_weight
    else:
        what = E.eqlinear_weight_spectrum(tw)
        y = E.eqlinear_forward(tx, what, bias=tb)
        dx = E.eqlinear_backward_input(tdy, what)
        dw = E.eqlinear_backward_weight(tx, tdy)
        fwd, bwd_x, bwd_w = oracle.forward, oracle.backward_input, oracle.backward_weight
    db = E.eqlinear_backward_bias(tdy)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7200 + i)
    rows = np.unique(np.concatenate([np.arange(min(4, N)), rng.choice(N, size=min(24, N), replace=False),
                                     np.arange(max(0, N - 4), N)]))
    idx = torch.from_numpy(rows).cuda()
    compare(host(y[idx]), fwd(x, w, rows=rows, bias=b), dt, "Y")
    compare(host(dx[idx]), bwd_x(dy, w, rows=rows), dt, "dX")
    if N * C_T * D_T * T * T <= 2e9:
        compare(host(dw), bwd_w(x, dy), dt, "dW (every entry)")
    else:
        dsel = np.unique(np.concatenate([[0, D_T - 1], rng.choice(D_T, size=min(8, D_T), replace=False)]))
        compare(host(dw[torch.from_numpy(dsel).cuda()]), bwd_w(x, dy, dsel=dsel), dt, "dW (sampled)")
    compare(host(db), oracle.backward_bias(dy), dt, "db")
