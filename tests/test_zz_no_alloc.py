"""eqlinear_backward_weight_noalloc (the weight gradient with the library's
static scratch) against eqlinear_backward_weight (caller's workspace).

Both use the same split plan and summation order, so their outputs are
compared bit for bit; the first call is also compared with the float64
oracle.  Two calls in a row on one GPU, the second with a smaller layer, so
the second runs on scratch that still holds the first call's partials.
"""
import sys

import numpy as np
import pytest

import oracle
from group_wise_dft_amd.workloads import custom_inputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("dt,T,first,second", [
    ("f16", 4, (12608, 192, 768), (3000, 64, 96)),     # 31.5 MiB of partials, then a small layer
    ("f32", 8, (16384, 128, 512), (5000, 40, 72)),
    ("f32", 4, (20000, 136, 200), (700, 13, 5)),       # ragged channels in the second call
])
def test_noalloc_matches_workspace_entry(E, dt, T, first, second):
    tdt = torch.float16 if dt == "f16" else torch.float32
    for call, (N, C_T, D_T) in enumerate((first, second)):
        announce("noalloc call %d N=%d C_T=%d D_T=%d T=%d %s seed=151" % (call, N, C_T, D_T, T, dt))
        need = E.eqlinear_workspace_size(N, C_T, D_T, T, tdt)
        assert 0 < need <= (64 << 20)
        x, _, dy = custom_inputs(N, C_T, D_T, T, dt, seed=151 + call)
        tx, tdy = dev(x), dev(dy)
        ref = E.eqlinear_backward_weight(tx, tdy)
        dw = torch.full((D_T, C_T, T), float("nan"), dtype=tdt, device="cuda")
        E.eqlinear_backward_weight_noalloc(tx, tdy, dw)
        torch.cuda.synchronize()
        assert torch.equal(dw, ref), "call %d differs from eqlinear_backward_weight" % call
        if call == 0:
            got = dw.double().cpu().numpy()
            want = oracle.backward_weight(x, dy, dsel=np.arange(0, D_T, 37))
            got = got[np.arange(0, D_T, 37)]
            rel = np.linalg.norm(got - want) / np.linalg.norm(want)
            assert rel <= (2e-3 if dt == "f16" else 1e-5), rel


def test_noalloc_rejects_oversized(E):
    """A layer whose partials exceed the scratch is rejected before any launch
    (the pointers are never dereferenced)."""
    announce("noalloc oversized")
    N, C_T, D_T, T = 65536, 2048, 2048, 8
    assert E.eqlinear_workspace_size(N, C_T, D_T, T, torch.float32) > (64 << 20)
    code = E.lib.eqlinear_backward_weight_noalloc(0x100000000, 0x900000000, 0x1100000000, N, C_T, D_T, T,
                                                  E.EQL_F32, None)
    assert code == 5   # EQL_ERR_WORKSPACE
