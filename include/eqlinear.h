/*
 * eqlinear.h -- C ABI of libeqlinear.so: Flash EQ-Linear on AMD MI355X (gfx950).
 *
 * The layer (equivariant linear layer over the cyclic group of order T):
 *
 *     Y[n,d,g] = sum_{c<C_T} sum_{h<T} Wt[d,c,(g-h) mod T] * X[n,c,h]
 *
 * i.e. the block-circulant matrix of the pages' §3.1 eq. (1) applied to each
 * row, read as the circular convolution along the group axis that eq. (3)
 * diagonalises.  It is computed the way the pages' Algorithm 1 (§3.2.1)
 * describes: a real DFT along the group axis, one contraction over channels
 * per non-redundant frequency (real at k=0 and k=T/2, complex in between),
 * conjugate-symmetric recovery, and an inverse real DFT.
 *
 * Sources cited below:
 *   [pchao]     "Flash EQ-Linear: accelerating equivariant linear layers via
 *               group-wise DFT", Chinese translation at pchao.org
 *   [paperpeel] the English text of a later revision at paperpeel.com
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All array arguments are DEVICE pointers to dense row-major buffers of
 *    the call's dtype, with the group axis contiguous ([paperpeel] App. A.3,
 *    "Memory layout and weight caching"): X and dX are [N][C_T][T], Y and dY
 *    are [N][D_T][T], Wt and dWt are [D_T][C_T][T].  The flat channel index
 *    of a row is c*T + g.
 *  - The weight spectrum w_hat holds T real planes of What_k[d,c] =
 *    sum_m Wt[d,c,m] exp(-2 pi i k m / T), unnormalised ([pchao] §3.2.1
 *    eq. (4)), in the plane order
 *        plane 0          Re What_0
 *        plane 2k-1, 2k   Re What_k, Im What_k       (0 < k < T/2)
 *        plane T-1        Re What_{T/2}              (T even)
 *    (for odd T the last pair, k = (T-1)/2, fills planes T-2 and T-1).
 *    It is the cached "frequency-domain weight planes" of [paperpeel] App.
 *    A.3; the caller owns it and must recompute it after changing Wt.  It is
 *    stored twice, in the blocked order in which the kernels stream it
 *    (KC = 16 for EQL_F16, 8 for EQL_F32), as P planes per (column, k):
 *        part 0  [ceil(D_T/32)][ceil(C_T/KC)][P][32][KC]:
 *                element (db, kb, p, i, j) = stored plane p at d = 32*db + i,
 *                c = KC*kb + j            (read by the forward)
 *        part 1  [ceil(C_T/32)][ceil(D_T/KC)][P][32][KC]:
 *                element (cb, kb, p, i, j) = stored plane p at c = 32*cb + i,
 *                d = KC*kb + j            (read by the input gradient)
 *    with zeros outside 0 <= d < D_T, 0 <= c < C_T.  With EQL_F16, and with
 *    EQL_F32 at T = 2, 3, 5, 7, the stored planes are the T planes above
 *    (P = T; both parts hold the same values).  With EQL_F32 at T = 4, 6, 8
 *    the kernels use three real products per complex frequency (Gauss; the
 *    complex products of [pchao] §3.2.1 eq. (5) rearranged) and the parts
 *    store, with re/im the real and imaginary plane of What_k in part 0 and
 *    of conj(What_k) in part 1:
 *        plane 0                 Re What_0
 *        plane 3k-2, 3k-1, 3k    re, im - re, re + im     (0 < k < T/2)
 *        plane T + (T-1)/2 - 1   Re What_{T/2}
 *    (P = T + (T-1)/2, plus one zero plane at T = 8: P = 12).  Its size in
 *    bytes is eqlinear_spectrum_size(C_T, D_T, T, dtype).
 *  - dtype: EQL_F32 (IEEE binary32) or EQL_F16 (IEEE binary16) for every
 *    array of the call.  Accumulation is always fp32; with EQL_F16 the
 *    group-DFT coordinates fed to the matrix cores are rounded to fp16
 *    ([paperpeel] App. A.3: half-precision tiles, fp32 accumulators).
 *  - Supported: 2 <= T <= 8; 0 <= N < 2^30; 1 <= C_T, D_T <= 65536, with a
 *    spectrum (eqlinear_spectrum_size) below 2^31 bytes.  Any other shape
 *    returns EQL_ERR_UNSUPPORTED (or EQL_ERR_SHAPE for negative sizes).
 *    Ragged tails of every size are masked inside the kernels.  Layers whose
 *    activation rows (C_T * T or D_T * T elements) are a whole number of
 *    16-byte chunks take the fastest copy path; others (for example an odd
 *    C_T at T = 4 in EQL_F16) copy those rows in smaller pieces, with the same
 *    results.  N == 0 is a valid no-op for forward/backward_input and
 *    zero-fills dWt (db) for backward_weight (backward_bias).
 *  - Every pointer must be 16-byte aligned (EQL_ERR_ALIGN otherwise).
 *  - Outputs are overwritten (not accumulated into) and must not overlap any
 *    input of the same call (EQL_ERR_ALIAS otherwise).
 *  - stream: a hipStream_t passed as void*; NULL means the default stream.
 *    Every call only enqueues work on that stream: it never allocates device
 *    memory, never synchronises, and returns before the work is done.  The
 *    buffers must stay valid until the stream reaches the enqueued work.
 *  - Errors: arguments are validated before any HIP call; on a validation
 *    error nothing is launched and no output is touched.  EQL_ERR_HIP means
 *    a kernel launch failed (hipGetLastError); the outputs are then undefined.
 *  - Results are bitwise deterministic for a given shape, dtype and GPU model
 *    (no atomics; every reduction has a fixed order).
 *  - The calls are safe to make from several host threads at once.
 */
#ifndef EQLINEAR_H
#define EQLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EQL_F32 = 0, /* binary32 in, binary32 out */
    EQL_F16 = 1  /* binary16 in, binary16 out, fp32 accumulation */
} eql_dtype;

typedef enum {
    EQL_OK = 0,
    EQL_ERR_NULL = 1,        /* a required pointer is NULL                    */
    EQL_ERR_SHAPE = 2,       /* a size is negative                            */
    EQL_ERR_UNSUPPORTED = 3, /* T, dtype or channel counts not supported      */
    EQL_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned              */
    EQL_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required    */
    EQL_ERR_ALIAS = 6,       /* an output overlaps an input                   */
    EQL_ERR_HIP = 7          /* a HIP launch failed                           */
} eql_status;

/*
 * Weight spectrum: w_hat <- the T real planes of the group DFT of Wt
 * ([pchao] §3.2.1 eq. (4), step 1 of Algorithm 1 on the weight side; for
 * T=4 this is [pchao] App. 6.2 eq. (19) applied to Wt).
 *   w_tilde  in   [D_T][C_T][T]
 *   w_hat    out  eqlinear_spectrum_size(C_T, D_T, T, dtype) bytes, the
 *                 blocked layout above
 * The transform (and the sums of the three-multiplication planes) is
 * computed in fp32 and rounded once to the dtype.
 */
eql_status eqlinear_weight_spectrum(const void *w_tilde, void *w_hat,
                                    int64_t C_T, int64_t D_T, int32_t T,
                                    eql_dtype dtype, void *stream);

/*
 * Forward: y <- EQ-Linear(x) + bias ([pchao] §3.2.1 Algorithm 1 steps 1-4,
 * eq. (7); [paperpeel] App. A.3 "Fused forward kernel").  One fused kernel:
 * the group DFT of x tiles in registers, per-frequency contractions on the
 * matrix cores against w_hat, the inverse DFT and the bias in the epilogue.
 *   x      in   [N][C_T][T]
 *   w_hat  in   from eqlinear_weight_spectrum (same C_T, D_T, T, dtype)
 *   bias   in   [D_T], shared by the group: y[n,d,g] += bias[d] for every
 *               n and g; NULL for no bias
 *   y      out  [N][D_T][T]
 */
eql_status eqlinear_forward(const void *x, const void *w_hat, const void *bias,
                            void *y, int64_t N, int64_t C_T, int64_t D_T,
                            int32_t T, eql_dtype dtype, void *stream);

/*
 * Input gradient: dx[n,c,h] = sum_{d,g} Wt[d,c,(g-h) mod T] dy[n,d,g], the
 * adjoint of the forward.  Per frequency dXhat_k = dYhat_k . conj(What_k)
 * ([paperpeel] App. A.3 "Forward and backward passes": the output gradient
 * in the same frequency coordinates times the transposed structured weight,
 * mapped back by the inverse transform).
 *   dy     in   [N][D_T][T]
 *   w_hat  in   from eqlinear_weight_spectrum (same C_T, D_T, T, dtype)
 *   dx     out  [N][C_T][T]
 */
eql_status eqlinear_backward_input(const void *dy, const void *w_hat, void *dx,
                                   int64_t N, int64_t C_T, int64_t D_T,
                                   int32_t T, eql_dtype dtype, void *stream);

/*
 * Weight gradient in the original parameterisation ([paperpeel] App. A.3):
 *   dw[d,c,m] = sum_{n,h} dy[n,d,(h+m) mod T] x[n,c,h]
 * computed as dWhat_k = sum_n dYhat_k conj(Xhat_k) followed by the inverse
 * DFT over k.  The sum over n is split into fixed chunks whose fp32 partial
 * spectra go to the workspace and are then added in a fixed order.  With
 * EQL_F32 at T = 4, 6, 8 the complex products use three real products
 * (Gauss), as in the forward.
 *   x          in   [N][C_T][T]
 *   dy         in   [N][D_T][T]
 *   dw_tilde   out  [D_T][C_T][T]
 *   workspace  scratch device memory of at least
 *              eqlinear_workspace_size(N, C_T, D_T, T, dtype) bytes
 *              (may be NULL when that size is 0); must not overlap any
 *              other argument; its contents on entry are ignored.
 */
eql_status eqlinear_backward_weight(const void *x, const void *dy, void *dw_tilde,
                                    void *workspace, size_t workspace_bytes,
                                    int64_t N, int64_t C_T, int64_t D_T,
                                    int32_t T, eql_dtype dtype, void *stream);

/*
 * Weight gradient without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, result and summation order as eqlinear_backward_weight (the
 * output is bit-identical), but the fp32 split partials go to a static
 * device array of EQL_NOALLOC_SCRATCH_BYTES bytes inside the library: each
 * GPU the library runs on holds one such array until the process ends.
 *   x          in   [N][C_T][T]
 *   dy         in   [N][D_T][T]
 *   dw_tilde   out  [D_T][C_T][T]
 * Returns EQL_ERR_WORKSPACE, before any HIP call, when the shape needs more
 * than EQL_NOALLOC_SCRATCH_BYTES of partials (eqlinear_workspace_size tells
 * how much), and EQL_ERR_HIP if the array's device address cannot be found.
 * The array is shared by every call on that GPU and keeps the last call's
 * contents: calls that overlap in time on one GPU (several streams, several
 * host threads) race on it and must be serialised by the caller.
 */
#define EQL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

eql_status eqlinear_backward_weight_noalloc(const void *x, const void *dy, void *dw_tilde,
                                            int64_t N, int64_t C_T, int64_t D_T,
                                            int32_t T, eql_dtype dtype, void *stream);

/*
 * Bias gradient: db[d] = sum_{n,g} dy[n,d,g], the gradient of the
 * group-shared bias of eq. (7) ([pchao] §3.2.1; the "backward bias grad" of
 * [pchao] §4 Table 4).  The sum over n is split into fixed chunks whose fp32
 * partial sums go to the workspace and are then added in a fixed order.
 *   dy         in   [N][D_T][T]
 *   db         out  [D_T]
 *   workspace  scratch device memory of at least
 *              eqlinear_bias_workspace_size(N, D_T, T, dtype) bytes (may be
 *              NULL when that size is 0); must not overlap any other
 *              argument; its contents on entry are ignored.
 * D_T, T and N follow the same rules as the other calls.
 */
eql_status eqlinear_backward_bias(const void *dy, void *db, void *workspace,
                                  size_t workspace_bytes, int64_t N, int64_t D_T,
                                  int32_t T, eql_dtype dtype, void *stream);

/*
 * Bytes of the cached weight spectrum w_hat for this shape (a pure function of
 * the arguments; 0 for unsupported or negative shapes).
 */
size_t eqlinear_spectrum_size(int64_t C_T, int64_t D_T, int32_t T, eql_dtype dtype);

/*
 * Bytes of workspace eqlinear_backward_weight needs for this shape (a pure
 * function of the arguments; 0 for unsupported or negative shapes).
 */
size_t eqlinear_workspace_size(int64_t N, int64_t C_T, int64_t D_T, int32_t T,
                               eql_dtype dtype);

/*
 * Bytes of workspace eqlinear_backward_bias needs for this shape (a pure
 * function of the arguments; 0 for unsupported or negative shapes).
 */
size_t eqlinear_bias_workspace_size(int64_t N, int64_t D_T, int32_t T, eql_dtype dtype);

/*
 * The octic group
 * ---------------
 * The same layer over the group of order 8 made of the quarter turns and the
 * reflections of the square: the octic group D8 of [paperpeel] App. A.2
 * ("Relation to Isotypic-Basis Equivariant Architectures": Schur's lemma
 * block-diagonalises the layer; D8's two-dimensional irreducible
 * representation is of real type, for 5.33x fewer FLOPs than dense) and
 * App. A.4 ("Comparison with Quick ViTs"); [paperpeel] §5 names other
 * groups as the next step.  Group element u = a + 4 b
 * (0 <= a < 4, 0 <= b < 2) stands for r^a s^b, r the quarter turn and s the
 * reflection, with r^a s^b . r^c s^d = r^(a + (-1)^b c) s^(b + d); the layer
 * is the group convolution of the regular representation,
 *
 *     Y[n,d,g] = sum_{c<C_T} sum_{h<8} Wt[d,c,h^-1 g] * X[n,c,h]   (+ bias[d])
 *
 * with the layouts above at T = 8.  It is computed as for the cyclic layer,
 * with the group Fourier transform in place of the DFT (by Schur's lemma the
 * layer becomes one matrix product per irreducible representation): four
 * one-dimensional characters A1, A2, B1, B2 (r -> 1, 1, -1, -1; s -> 1, -1,
 * 1, -1) give four real channel contractions, and the two-dimensional
 * representation E (r -> [[0,-1],[1,0]], s -> [[1,0],[0,-1]]) gives a 2 x 2
 * block product of four real planes: 12 real contractions per layer against
 * 64 for the assembled dense matrix.  The spectrum holds the eight planes
 * What(rho)[d,c] = sum_u Wt[d,c,u] rho(u), in the order
 *        0 A1   1 A2   2 B1   3 B2   4 E11   5 E12   6 E21   7 E22
 * in both dtypes, blocked like the cyclic spectrum (P = 8), except that part
 * 1 (read by the input gradient) holds the E block transposed (planes 5 and
 * 6 exchanged).  Its size is eqlinear_octic_spectrum_size(C_T, D_T, dtype).
 * Shapes, alignment, aliasing, errors, streams and determinism follow the
 * conventions above.  The bias gradient is eqlinear_backward_bias with T = 8
 * (the bias is shared by the group as for the cyclic layer).
 */

/* w_hat <- the eight planes of the octic Fourier transform of w_tilde
 * ([D_T][C_T][8]), computed in fp32 and rounded once to the dtype. */
eql_status eqlinear_octic_weight_spectrum(const void *w_tilde, void *w_hat,
                                          int64_t C_T, int64_t D_T,
                                          eql_dtype dtype, void *stream);

/* y ([N][D_T][8]) <- octic layer of x ([N][C_T][8]) + bias ([D_T] or NULL):
 * the Fourier transform of x tiles in registers, the four character products
 * and the E block product on the matrix cores, and the inverse transform and
 * the bias in the epilogue, in one kernel. */
eql_status eqlinear_octic_forward(const void *x, const void *w_hat, const void *bias,
                                  void *y, int64_t N, int64_t C_T, int64_t D_T,
                                  eql_dtype dtype, void *stream);

/* dx ([N][C_T][8]) <- dx[n,c,h] = sum_{d,g} Wt[d,c,h^-1 g] dy[n,d,g], the
 * adjoint of the forward: per representation dXhat(rho) = dYhat(rho) times
 * the transposed weight block. */
eql_status eqlinear_octic_backward_input(const void *dy, const void *w_hat, void *dx,
                                         int64_t N, int64_t C_T, int64_t D_T,
                                         eql_dtype dtype, void *stream);

/* dw_tilde ([D_T][C_T][8]) <- dw[d,c,u] = sum_{n,h} dy[n,d,h u] x[n,c,h],
 * computed as dWhat(rho) = sum_n Xhat(rho)^T dYhat(rho) per representation
 * and the inverse transform.  The workspace holds the fp32 split partials
 * (at least eqlinear_octic_workspace_size bytes; may be NULL when that is
 * 0), as for eqlinear_backward_weight. */
eql_status eqlinear_octic_backward_weight(const void *x, const void *dy, void *dw_tilde,
                                          void *workspace, size_t workspace_bytes,
                                          int64_t N, int64_t C_T, int64_t D_T,
                                          eql_dtype dtype, void *stream);

/* Bytes of the octic weight spectrum, and of the octic weight gradient's
 * workspace, for this shape (pure functions; 0 for unsupported shapes). */
size_t eqlinear_octic_spectrum_size(int64_t C_T, int64_t D_T, eql_dtype dtype);
size_t eqlinear_octic_workspace_size(int64_t N, int64_t C_T, int64_t D_T, eql_dtype dtype);

/* Static, NUL-terminated description of a status code. */
const char *eqlinear_status_string(eql_status s);

#ifdef __cplusplus
}
#endif

#endif /* EQLINEAR_H */
