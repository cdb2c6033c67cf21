// eqlinear_internal.h -- declarations shared by the C-ABI layer and the
// kernel launchers of libeqlinear.so (not installed, not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// How the weight gradient splits the sum over rows: `splits` chunks of
// `chunk` rows each (the last one shorter) for each of `tiles` output tiles
// (of BR row channels x BC column channels).
// A pure function of the shape, so the workspace size and the summation
// order never depend on the device.
struct DwPlan {
    int tiles;
    int splits;
    int chunk;
    int swap;    // tile rows are c (and columns d) instead of d (and c)
    int ring;    // the ring-staged kernel (small grids) instead of the register-staged one
    int narrow;  // the narrow tiles of the register-staged kernel (DwCfgN)
    int pc;      // the producer/consumer kernel (one workgroup per CU)
};

// Compute units of one MI355X (the split plans assume this many).
constexpr int MI355X_CUS = 256;
// grp = 1: the octic group (T = 8), which always takes the producer/consumer
// kernel.
DwPlan dw_plan(int64_t N, int64_t C_T, int64_t D_T, int T, int elem_bytes, int grp = 0);

// Planes the weight spectrum stores per (column, k): T, or with Gauss's
// three-multiplication products T + (T - 1) / 2 (three per complex
// frequency instead of two; plus one zero plane at T = 8, 12 in all).  Fixed
// per (T, dtype); defined with the kernels.
int spectrum_planes(int T, int elem_bytes);

// Blocked layout of the cached weight spectrum (both orientations).  A part
// for NC output columns and a contraction length K is
//     [ceil(NC/32)][ceil(K/KC)][TP][32][KC]  elements, zero padded,
// KC = 16 (fp16) or 8 (fp32): one MFMA k slice; TP = spectrum_planes.  Part 0
// serves the forward (columns d, k = c), part 1 the input gradient (columns
// c, k = d).  For the octic group (grp = 1, T = 8) TP = 8.
struct SpecLayout {
    int64_t kc, tp;
    int64_t nb0, kb0, nb1, kb1;   // blocks of part 0 (NC = D_T, K = C_T) and part 1
    int64_t elems0, elems1;       // elements of each part
};
inline SpecLayout spec_layout(int64_t C_T, int64_t D_T, int64_t T, int elem_bytes, int grp = 0) {
    SpecLayout L;
    L.kc = elem_bytes == 2 ? 16 : 8;
    L.tp = grp ? T : spectrum_planes((int)T, elem_bytes);   // the octic group stores its 8 planes
    L.nb0 = (D_T + 31) / 32;
    L.kb0 = (C_T + L.kc - 1) / L.kc;
    L.nb1 = (C_T + 31) / 32;
    L.kb1 = (D_T + L.kc - 1) / L.kc;
    L.elems0 = L.nb0 * L.kb0 * L.tp * 32 * L.kc;
    L.elems1 = L.nb1 * L.kb1 * L.tp * 32 * L.kc;
    return L;
}

// How the bias gradient splits the sum over rows.
struct BiasPlan {
    int splits;
    int chunk;
};
BiasPlan bias_plan(int64_t N, int64_t D_T, int T, int elem_bytes);

// dt: 0 = fp32, 1 = fp16.  Shapes are validated by the caller.
hipError_t eqk_spectrum(const void *wt, void *what, int CT, int DT, int T, int dt, hipStream_t st);
hipError_t eqk_forward(const void *x, const void *what, const void *bias, void *y, int N, int CT, int DT,
                       int T, int dt, hipStream_t st);
hipError_t eqk_backward_bias(const void *dy, void *db, void *ws, int N, int DT, int T, int dt,
                             hipStream_t st);
hipError_t eqk_backward_input(const void *dy, const void *what, void *dx, int N, int CT, int DT, int T,
                              int dt, hipStream_t st);
hipError_t eqk_backward_weight(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                               int T, int dt, hipStream_t st);

// The octic group (quarter turns and reflections, T = 8 components per
// tuple); the spectrum layout is spec_layout(.., 8, .., 1), the weight
// gradient's plan dw_plan(.., 8, .., 1).
hipError_t eqk_octic_spectrum(const void *wt, void *what, int CT, int DT, int dt, hipStream_t st);
hipError_t eqk_octic_forward(const void *x, const void *what, const void *bias, void *y, int N, int CT, int DT,
                             int dt, hipStream_t st);
hipError_t eqk_octic_backward_input(const void *dy, const void *what, void *dx, int N, int CT, int DT, int dt,
                                    hipStream_t st);
hipError_t eqk_octic_backward_weight(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                                     int dt, hipStream_t st);
