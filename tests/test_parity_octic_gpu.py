"""GPU parity of the octic-group layer: libeqlinear.so's eqlinear_octic_*
entry points (through the C ABI) against the float64 oracle's octic section.

Same inputs on both sides (for fp16 the oracle sees the fp16-rounded values
exactly) and the tolerances of the cyclic parity tests: relative Frobenius
error <= 1e-5 and max |gpu - oracle| <= 1e-4 * RMS(oracle) in fp32, relative
Frobenius error <= 2e-3 in fp16.  The octic transform has the same reach as
the order-8 DFT (entries of its planes are sums of eight terms with
coefficients +-1, 0), so the rounding budget of the cyclic tests carries
over.
"""
import sys

import numpy as np
import pytest

import oracle
from group_wise_dft_amd.workloads import OCTIC_WORKLOADS, bias_input, custom_inputs, inputs
from tests.test_oracle_octic import act, fourier

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "f16": (2e-3, None)}


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


def run_all(E, x, w, dy, bias=None):
    tx, tw, tdy = dev(x), dev(w), dev(dy)
    what = E.eqlinear_octic_weight_spectrum(tw)
    y = E.eqlinear_octic_forward(tx, what, bias=None if bias is None else dev(bias))
    dx = E.eqlinear_octic_backward_input(tdy, what)
    dw = E.eqlinear_octic_backward_weight(tx, tdy)
    torch.cuda.synchronize()
    return what, y, dx, dw


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("shape", [(40, 24), (8, 8), (33, 7)], ids=lambda s: "D%d_C%d" % s)
def test_octic_spectrum(E, shape, dt):
    """Part 0 holds the eight planes (A1, A2, B1, B2, E11, E12, E21, E22) of
    sum_u Wt[.,.,u] rho(u); part 1 the same with the E block transposed."""
    D_T, C_T = shape
    announce("octic spectrum D_T=%d C_T=%d %s" % (D_T, C_T, dt))
    _, w, _ = custom_inputs(1, C_T, D_T, 8, dt, seed=5)
    wh = E.eqlinear_octic_weight_spectrum(dev(w))
    assert wh.stored_planes == 8
    p0, p1 = wh.planes()
    ref = oracle.octic_spectrum(w.astype(np.float64))
    # independently of the oracle: the transform written from the
    # representation matrices
    assert np.allclose(ref, fourier(w.astype(np.float64)).reshape(8, D_T, C_T), rtol=1e-12, atol=1e-12)
    tol = 1e-6 if dt == "f32" else 1e-3
    got0 = host(p0)
    got1 = host(p1).transpose(0, 2, 1)[[0, 1, 2, 3, 4, 6, 5, 7]]
    for got in (got0, got1):
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= tol
    np.testing.assert_array_equal(got0, got1)
    n = wh.buf.numel()
    assert n * wh.buf.element_size() == E.eqlinear_octic_spectrum_size(C_T, D_T, wh.buf.dtype)
    # the padding of the blocked layout is zero
    assert torch.count_nonzero(wh.buf).item() == torch.count_nonzero(p0).item() + torch.count_nonzero(p1).item()


SMALL = [  # (N, C_T, D_T): several tiles in every direction plus ragged tails
    (1, 8, 8), (17, 8, 24), (300, 40, 72), (1000, 24, 136), (129, 264, 16), (70, 5, 13),
]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "N%d_C%d_D%d" % s)
def test_octic_small_full(E, shape, dt):
    N, C_T, D_T = shape
    announce("octic small N=%d C_T=%d D_T=%d %s seed=11" % (N, C_T, D_T, dt))
    x, w, dy = custom_inputs(N, C_T, D_T, 8, dt, seed=11)
    b = bias_input(D_T, dt, 14)
    _, y, dx, dw = run_all(E, x, w, dy, bias=b)
    compare(host(y), oracle.octic_forward(x, w, bias=b), dt, "Y")
    compare(host(dx), oracle.octic_backward_input(dy, w), dt, "dX")
    compare(host(dw), oracle.octic_backward_weight(x, dy), dt, "dW")


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    head = np.arange(min(8, n))
    tail = np.arange(max(0, n - 24), n)
    mid = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


def dw_select(D_T, seed):
    """The first and last output channel and one random channel in every run
    of 32: every weight-gradient tile, wave and 32-channel block is reached."""
    rng = np.random.default_rng(seed)
    picks = [b + int(rng.integers(0, min(32, D_T - b))) for b in range(0, D_T, 32)]
    return np.unique(np.array([0, D_T - 1] + picks))


def check_sampled(E, x, w, dy, dt, seed, full_dw_macs=2e10):
    N, C_T, _ = x.shape
    D_T = w.shape[0]
    tx, tw, tdy = dev(x), dev(w), dev(dy)
    what = E.eqlinear_octic_weight_spectrum(tw)
    y = E.eqlinear_octic_forward(tx, what)
    dx = E.eqlinear_octic_backward_input(tdy, what)
    dw = E.eqlinear_octic_backward_weight(tx, tdy)
    torch.cuda.synchronize()
    rows = sample_rows(N, 40, seed)
    idx = torch.from_numpy(rows).cuda()
    compare(host(y[idx]), oracle.octic_forward(x, w, rows=rows), dt, "Y")
    compare(host(dx[idx]), oracle.octic_backward_input(dy, w, rows=rows), dt, "dX")
    if N * D_T * C_T * 64 <= full_dw_macs:
        compare(host(dw), oracle.octic_backward_weight(x, dy), dt, "dW (every entry)")
    else:
        dsel = dw_select(D_T, seed + 1)
        compare(host(dw[torch.from_numpy(dsel).cuda()]), oracle.octic_backward_weight(x, dy, dsel=dsel), dt,
                "dW (%d of %d channels)" % (dsel.size, D_T))


GENERAL = [  # (N, C_T, D_T): many row tiles, split weight gradient, ragged tails
    (6000, 136, 264), (3001, 72, 520), (8001, 40, 200), (20000, 13, 100),
]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("shape", GENERAL, ids=lambda s: "N%d_C%d_D%d" % s)
def test_octic_general_sampled(E, shape, dt):
    N, C_T, D_T = shape
    announce("octic general N=%d C_T=%d D_T=%d %s seed=61" % (N, C_T, D_T, dt))
    x, w, dy = custom_inputs(N, C_T, D_T, 8, dt, seed=61)
    check_sampled(E, x, w, dy, dt, 62)


ROW_PLAN_EDGES = [  # (N, C_T, D_T): 128 and 189 row-kernel tiles at K >= 256 in one pass
                    # (the few-tile kernel in fp32, the row tiles in fp16) and more
                    # tiles or a shorter K in the other
    (2000, 270, 200), (4000, 300, 130),
]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("shape", ROW_PLAN_EDGES, ids=lambda s: "N%d_C%d_D%d" % s)
def test_octic_row_plan_edges(E, shape, dt):
    N, C_T, D_T = shape
    announce("octic row plan edge N=%d C_T=%d D_T=%d %s seed=71" % (N, C_T, D_T, dt))
    x, w, dy = custom_inputs(N, C_T, D_T, 8, dt, seed=71)
    b = bias_input(D_T, dt, 74)
    tx, tw, tdy = dev(x), dev(w), dev(dy)
    what = E.eqlinear_octic_weight_spectrum(tw)
    y = E.eqlinear_octic_forward(tx, what, bias=dev(b))
    dx = E.eqlinear_octic_backward_input(tdy, what)
    torch.cuda.synchronize()
    compare(host(y), oracle.octic_forward(x, w, bias=b), dt, "Y+b")
    compare(host(dx), oracle.octic_backward_input(dy, w), dt, "dX")


CASES = [(name, dt) for name, w in OCTIC_WORKLOADS.items() for dt in w.dtypes]


@pytest.mark.parametrize("name,dt", CASES, ids=["%s-%s" % c for c in CASES])
def test_octic_workload(E, name, dt):
    wl = OCTIC_WORKLOADS[name]
    announce("octic workload %s %s N=%d C_T=%d D_T=%d" % (name, dt, wl.N, wl.C_T, wl.D_T))
    x, w, dy = inputs(wl, dt)
    check_sampled(E, x, w, dy, dt, wl.seed(9))


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_octic_equivariance(E, dt):
    """Acting on the group axis of the input by any element k acts the same
    way on the output, acting on dY acts the same way on dX, and acting on
    X and dY together leaves dWt unchanged (Y[g] = sum_h Wt[h^-1 g] X[h]
    and its adjoints; checked on the GPU results against each other)."""
    N, C_T, D_T = 200, 24, 40
    announce("octic equivariance N=%d C_T=%d D_T=%d %s" % (N, C_T, D_T, dt))
    x, w, dy = custom_inputs(N, C_T, D_T, 8, dt, seed=31)
    what = E.eqlinear_octic_weight_spectrum(dev(w))
    y = host(E.eqlinear_octic_forward(dev(x), what))
    dx = host(E.eqlinear_octic_backward_input(dev(dy), what))
    dw = host(E.eqlinear_octic_backward_weight(dev(x), dev(dy)))
    for k in range(8):
        xk, dyk = act(k, x), act(k, dy)
        yk = host(E.eqlinear_octic_forward(dev(xk), what))
        compare(yk, act(k, y), dt, "equivariance under element %d" % k)
        dxk = host(E.eqlinear_octic_backward_input(dev(dyk), what))
        compare(dxk, act(k, dx), dt, "input gradient under element %d" % k)
        dwk = host(E.eqlinear_octic_backward_weight(dev(xk), dev(dyk)))
        compare(dwk, dw, dt, "weight gradient invariant under element %d" % k)


def test_octic_deterministic_and_empty(E):
    N, C_T, D_T = 5000, 40, 72
    announce("octic determinism N=%d C_T=%d D_T=%d f16" % (N, C_T, D_T))
    x, w, dy = custom_inputs(N, C_T, D_T, 8, "f16", seed=41)
    a = run_all(E, x, w, dy)
    b = run_all(E, x, w, dy)
    for u, v in zip(a[1:], b[1:]):
        assert torch.equal(u, v)
    # N = 0: forward and input gradient are no-ops, the weight gradient is zero
    x0 = torch.empty((0, C_T, 8), dtype=torch.float16, device="cuda")
    dy0 = torch.empty((0, D_T, 8), dtype=torch.float16, device="cuda")
    assert E.eqlinear_octic_forward(x0, a[0]).shape == (0, D_T, 8)
    assert E.eqlinear_octic_backward_input(dy0, a[0]).shape == (0, C_T, 8)
    dw = torch.full((D_T, C_T, 8), 7.0, dtype=torch.float16, device="cuda")
    E.eqlinear_octic_backward_weight(x0, dy0, dw=dw)
    torch.cuda.synchronize()
    assert not torch.any(dw)


def test_octic_and_cyclic_spectra_not_mixed(E):
    _, w, _ = custom_inputs(1, 8, 8, 8, "f32", seed=3)
    cyc = E.eqlinear_weight_spectrum(dev(w))
    with pytest.raises(ValueError):
        E.eqlinear_octic_forward(dev(np.zeros((4, 8, 8), np.float32)), cyc)
    # and the other way round
    oc = E.eqlinear_octic_weight_spectrum(dev(w))
    with pytest.raises(ValueError):
        E.eqlinear_forward(dev(np.zeros((4, 8, 8), np.float32)), oc)
    with pytest.raises(ValueError):
        E.eqlinear_backward_input(dev(np.zeros((4, 8, 8), np.float32)), oc)
    with pytest.raises(ValueError):
        E.eqlinear_weight_spectrum(dev(w), oc)


def test_octic_graph_capture_replay(E):
    """An octic training-step pass (spectrum, forward with bias, both
    gradients, bias gradient at T = 8) captured in a HIP graph: every replay,
    with eager work and a synchronisation in between, matches the eager
    results bit for bit (the weight gradient of this shape runs in split
    partials)."""
    N, C_T, D_T = 3000, 40, 72
    announce("octic graph capture N=%d C_T=%d D_T=%d f16" % (N, C_T, D_T))
    x, w, dy = custom_inputs(N, C_T, D_T, 8, "f16", seed=97)
    b = bias_input(D_T, "f16", 98)
    tx, tw, tdy, tb = dev(x), dev(w), dev(dy), dev(b)
    f16 = torch.float16
    assert E.eqlinear_octic_workspace_size(N, C_T, D_T, f16) > 0
    spec = E.new_octic_weight_spectrum(C_T, D_T, f16, tx.device)
    y = torch.empty((N, D_T, 8), dtype=f16, device="cuda")
    dx = torch.empty((N, C_T, 8), dtype=f16, device="cuda")
    dw = torch.empty((D_T, C_T, 8), dtype=f16, device="cuda")
    db = torch.empty((D_T,), dtype=f16, device="cuda")
    ws = torch.empty(E.eqlinear_octic_workspace_size(N, C_T, D_T, f16), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(16, E.eqlinear_bias_workspace_size(N, D_T, 8, f16)), dtype=torch.uint8, device="cuda")

    def step():
        E.eqlinear_octic_weight_spectrum(tw, spec)
        E.eqlinear_octic_forward(tx, spec, y, bias=tb)
        E.eqlinear_octic_backward_weight(tx, tdy, dw, ws)
        E.eqlinear_octic_backward_input(tdy, spec, dx)
        E.eqlinear_backward_bias(tdy, db, wsb)

    outs = (y, dx, dw, db)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for u, v, name in zip(ref, outs, ("Y", "dX", "dW", "db")):
            assert torch.equal(u, v), "replay %d: %s differs from eager" % (r, name)
    compare(host(y), oracle.octic_forward(x, w, bias=b), "f16", "Y (eager)")
    compare(host(dw), oracle.octic_backward_weight(x, dy), "f16", "dW (eager)")
