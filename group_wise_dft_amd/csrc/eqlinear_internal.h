// eqlinear_internal.h -- declarations shared by the C-ABI layer and the
// kernel launchers of libeqlinear.so (not installed, not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// How the weight gradient splits the sum over rows: `splits` chunks of
// `chunk` rows each (the last one shorter) for each of `tiles` output tiles.
// A pure function of the shape, so the workspace size and the summation
// order never depend on the device.
struct DwPlan {
    int tiles;
    int splits;
    int chunk;
};
DwPlan dw_plan(int64_t N, int64_t C_T, int64_t D_T, int T, int elem_bytes);

// dt: 0 = fp32, 1 = fp16.  Shapes are validated by the caller.
hipError_t eqk_spectrum(const void *wt, void *what, int CT, int DT, int T, int dt, hipStream_t st);
hipError_t eqk_forward(const void *x, const void *what, void *y, int N, int CT, int DT, int T, int dt,
                       hipStream_t st);
hipError_t eqk_backward_input(const void *dy, const void *what, void *dx, int N, int CT, int DT, int T,
                              int dt, hipStream_t st);
hipError_t eqk_backward_weight(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                               int T, int dt, hipStream_t st);
