"""The oracle's pins must catch plausible mistakes (cyclic and octic layers).

Each case copies eqlinear_oracle.c, plants one mistake (a swapped circulant
index, a dropped term, a wrong sign, a transposed operand), builds the copy
with gcc into a temporary directory and runs the pin battery against it.  The
unmodified source must pass every pin; every mutant must fail at least one.
All of this runs on the CPU.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests.test_oracle import dense_weight
from tests.test_oracle_octic import battery_octic

SRC = os.path.join(os.path.dirname(oracle.__file__), "eqlinear_oracle.c")

MUTANTS = {
    "control": None,
    "fwd_correlation_index": ("w[(d * C_T + c) * T + wrap(g - h, T)] *\n                         x[",
                              "w[(d * C_T + c) * T + wrap(h - g, T)] *\n                         x["),
    "fwd_dropped_group_term": ("for (int64_t h = 0; h < T; ++h)\n                    s += w[(d * C_T + c) * T + wrap(g - h, T)] *\n                         x[",
                               "for (int64_t h = 1; h < T; ++h)\n                    s += w[(d * C_T + c) * T + wrap(g - h, T)] *\n                         x["),
    "fwd_transposed_weight": ("w[(d * C_T + c) * T + wrap(g - h, T)] *\n                         x[",
                              "w[(c * D_T + d) * T + wrap(g - h, T)] *\n                         x["),
    "dx_index_sign": ("w[(d * C_T + c) * T + wrap(g - h, T)] *\n                         dy[",
                      "w[(d * C_T + c) * T + wrap(h - g, T)] *\n                         dy["),
    "dx_dropped_channel": ("for (int64_t d = 0; d < D_T; ++d)\n                for (int64_t g = 0; g < T; ++g)",
                           "for (int64_t d = 1; d < D_T; ++d)\n                for (int64_t g = 0; g < T; ++g)"),
    "dw_shift_sign": ("dy[(n * D_T + d) * T + wrap(h + m, T)]",
                      "dy[(n * D_T + d) * T + wrap(h - m, T)]"),
    "dw_dropped_row": ("for (int64_t n = 0; n < N; ++n)\n                for (int64_t h = 0; h < T; ++h)",
                       "for (int64_t n = 0; n + 1 < N; ++n)\n                for (int64_t h = 0; h < T; ++h)"),
    "bias_dropped": ("yrow[d * T + g] = b ? s + b[d] : s;", "yrow[d * T + g] = s;"),
    "bias_wrong_channel": ("yrow[d * T + g] = b ? s + b[d] : s;", "yrow[d * T + g] = b ? s + b[g % D_T] : s;"),
    "dbias_dropped_group_term": ("for (int64_t g = 0; g < T; ++g)\n                s += dy[(n * D_T + d) * T + g];",
                                 "for (int64_t g = 1; g < T; ++g)\n                s += dy[(n * D_T + d) * T + g];"),
    "dbias_dropped_row": ("for (int64_t n = 0; n < N; ++n)\n            for (int64_t g = 0; g < T; ++g)\n                s += dy[",
                          "for (int64_t n = 1; n < N; ++n)\n            for (int64_t g = 0; g < T; ++g)\n                s += dy["),
    "spectrum_imag_sign": ("im -= wv[m] * sin(ang);", "im += wv[m] * sin(ang);"),
    # the octic group (battery_octic)
    "octic_fwd_right_product": ("w[(d * C_T + c) * 8 + oct_mul(oct_inv(h), g)] * x[",
                                "w[(d * C_T + c) * 8 + oct_mul(g, oct_inv(h))] * x["),
    "octic_reflection_inverse": ("return (g >> 2) ? g : wrap(-g, 4);", "return (g >> 2) ? wrap(-g, 4) + 4 : wrap(-g, 4);"),
    "octic_twist_sign": ("int64_t rot = b ? a - c : a + c;", "int64_t rot = a + c;"),
    "octic_dx_missing_inverse": ("w[(d * C_T + c) * 8 + oct_mul(oct_inv(h), g)] * dy[",
                                 "w[(d * C_T + c) * 8 + oct_mul(h, g)] * dy["),
    "octic_dw_order": ("dy[(n * D_T + d) * 8 + oct_mul(h, u)] * x[", "dy[(n * D_T + d) * 8 + oct_mul(u, h)] * x["),
    "octic_bias_dropped": ("yrow[d * 8 + g] = b ? s + b[d] : s;", "yrow[d * 8 + g] = s;"),
    "octic_spectrum_E_transposed": ("out[(4 + 2 * i + k) * plane_sz + off] = s;", "out[(4 + 2 * k + i) * plane_sz + off] = s;"),
    "spectrum_plane_swap": ("out[(2 * k - 1) * plane_sz + off] = re;\n                    out[(2 * k) * plane_sz + off] = im;",
                            "out[(2 * k - 1) * plane_sz + off] = im;\n                    out[(2 * k) * plane_sz + off] = re;"),
}


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol=1e-9):
    return a.shape == b.shape and np.allclose(a, b, rtol=tol, atol=tol)


def battery(o):
    """Run the independent pins against oracle build ``o``; return failures."""
    failed = []
    # dense block-circulant (forward, dX, dWt by chain rule), several shapes
    for (N, C_T, D_T, T) in [(3, 2, 3, 4), (2, 3, 2, 8), (4, 3, 5, 3), (3, 4, 2, 2)]:
        x, w, dy = rand((N, C_T, T), 1), rand((D_T, C_T, T), 2), rand((N, D_T, T), 3)
        Wd = dense_weight(w)
        if not _close(o.forward(x, w), (x.reshape(N, -1) @ Wd.T).reshape(N, D_T, T)):
            failed.append("dense_fwd")
        if not _close(o.backward_input(dy, w), (dy.reshape(N, -1) @ Wd).reshape(N, C_T, T)):
            failed.append("dense_dx")
        G = dy.reshape(N, -1).T @ x.reshape(N, -1)
        ref = np.zeros((D_T, C_T, T))
        for g in range(T):
            for h in range(T):
                ref[:, :, (g - h) % T] += G[g::T, h::T]
        if not _close(o.backward_weight(x, dy), ref):
            failed.append("dense_dw")
        # dense linear layer with the bias tiled over the group ([pchao] §3.1)
        b = rand((D_T,), 4)
        yb = x.reshape(N, -1) @ Wd.T + np.repeat(b, T)[None, :]
        if not _close(o.forward(x, w, bias=b), yb.reshape(N, D_T, T)):
            failed.append("dense_fwd_bias")
        # tiled-bias gradient: column sums of dY folded over the group
        if not _close(o.backward_bias(dy), dy.reshape(N, -1).sum(0).reshape(D_T, T).sum(1)):
            failed.append("dense_dbias")
        r = np.fft.rfft(w, axis=2)
        planes = [r[:, :, 0].real]
        for k in range(1, (T - 1) // 2 + 1):
            planes += [r[:, :, k].real, r[:, :, k].imag]
        if T % 2 == 0:
            planes.append(r[:, :, T // 2].real)
        if not _close(o.spectrum(w), np.stack(planes)):
            failed.append("rfft")
    # one-hot direction
    x = np.zeros((1, 1, 4)); x[0, 0, 1] = 1
    w = np.zeros((1, 1, 4)); w[0, 0, 2] = 1
    e = np.zeros((1, 1, 4)); e[0, 0, 3] = 1
    if not _close(o.forward(x, w), e):
        failed.append("delta")
    return sorted(set(failed))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    src = open(SRC).read()
    mut = MUTANTS[name]
    if mut is not None:
        old, new = mut
        assert src.count(old) == 1, "mutation anchor not unique/absent: " + name
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "m.c")
        with open(c, "w") as f:
            f.write(src)
        so = oracle.build(force=True, src=c, out=os.path.join(td, "m.so"))
        o = oracle.Oracle(so)
        failed = battery(o) + battery_octic(o)
    if mut is None:
        assert failed == []
    else:
        assert failed, "planted mistake %s passed every pin" % name
