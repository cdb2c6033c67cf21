/*
 * eqlinear_oracle.c -- float64 CPU oracle for the equivariant linear layer
 * (EQ-Linear) and its two gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * Sources (two web pages on the same paper):
 *   [pchao]     "Flash EQ-Linear: accelerating equivariant linear layers via
 *               group-wise DFT", Chinese translation at pchao.org.
 *   [paperpeel] the English text of a later revision at paperpeel.com.
 *
 * What is computed.  The pages state that the Fourier algorithm is exact: it
 * reaches the naive block-circulant result up to rounding ([pchao] §3.4,
 * [paperpeel] §3.2 "Properties (i)").  So this oracle does not use any DFT for
 * the layer itself; it writes out the plain definition as a direct sum:
 *
 *   Y[n,d,g]  = sum_{c<C_T} sum_{h<T} Wt[d,c,(g-h) mod T] * X[n,c,h]
 *
 * which is the block-circulant product of [pchao] §3.1 eq. (1) with the
 * circulant index taken so that the convolution theorem of [pchao] §3.1
 * eq. (3) and the kernel formulas of [pchao] App. 6.2 eqs. (19)-(21) hold
 * (the index order printed inside eq. (2) is the transpose of that; the
 * reading taken is the convolution one, in which a one-hot weight at shift m
 * moves group component h to h+m).
 *
 * An optional bias b[D_T] is shared by the group: it is added to every
 * sample and every group component, Y[n,d,g] += b[d] ([pchao] §3.2.1 step 4,
 * eq. (7), the last step of Algorithm 1).
 *
 * The gradients are the adjoints of that map "in the original
 * parameterisation" ([paperpeel] App. A.3, "Forward and backward passes"):
 *
 *   dX[n,c,h]  = sum_{d<D_T} sum_{g<T} Wt[d,c,(g-h) mod T] * dY[n,d,g]
 *   dWt[d,c,m] = sum_{n<N}   sum_{h<T} dY[n,d,(h+m) mod T] * X[n,c,h]
 *   db[d]      = sum_{n<N}   sum_{g<T} dY[n,d,g]
 *
 * (the bias gradient is the one in the pages' accuracy table, [pchao] §4
 * Table 4, the adjoint of the broadcast over samples and group components).
 *
 * The weight spectrum is the group DFT of [pchao] §3.2.1 eq. (4) applied to
 * Wt along its last axis, unnormalised, with kernel e^{-i 2 pi k m / T}, for
 * k = 0..floor(T/2), stored as T real planes (see oracle_spectrum).
 *
 * Layouts (row-major, the group axis contiguous, [paperpeel] App. A.3
 * "Memory layout"):  X [N][C_T][T],  Wt [D_T][C_T][T],  Y/dY [N][D_T][T],
 * dX [N][C_T][T],  dWt [D_T][C_T][T].
 *
 * The same file holds the layer over the octic group (quarter turns and
 * reflections, [paperpeel] App. A.2), in the section marked below.
 *
 * Threads: OpenMP over the outermost output index; every output element is a
 * plain left-to-right float64 sum, so the result does not depend on the
 * thread count.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>

static int64_t wrap(int64_t a, int64_t T)
{
    int64_t r = a % T;
    return r < 0 ? r + T : r;
}

/* One output row Y[n,:,:] of the forward definition (b may be NULL). */
static void forward_row(const double *x, const double *w, const double *b, double *yrow,
                        int64_t n, int64_t C_T, int64_t D_T, int64_t T)
{
    for (int64_t d = 0; d < D_T; ++d)
        for (int64_t g = 0; g < T; ++g) {
            double s = 0.0;
            for (int64_t c = 0; c < C_T; ++c)
                for (int64_t h = 0; h < T; ++h)
                    s += w[(d * C_T + c) * T + wrap(g - h, T)] *
                         x[(n * C_T + c) * T + h];
            yrow[d * T + g] = b ? s + b[d] : s;
        }
}

/* One input-gradient row dX[n,:,:]. */
static void backward_input_row(const double *dy, const double *w, double *dxrow,
                               int64_t n, int64_t C_T, int64_t D_T, int64_t T)
{
    for (int64_t c = 0; c < C_T; ++c)
        for (int64_t h = 0; h < T; ++h) {
            double s = 0.0;
            for (int64_t d = 0; d < D_T; ++d)
                for (int64_t g = 0; g < T; ++g)
                    s += w[(d * C_T + c) * T + wrap(g - h, T)] *
                         dy[(n * D_T + d) * T + g];
            dxrow[c * T + h] = s;
        }
}

/* One weight-gradient slice dWt[d,:,:]. */
static void backward_weight_slice(const double *x, const double *dy, double *dwrow,
                                  int64_t d, int64_t N, int64_t C_T, int64_t D_T,
                                  int64_t T)
{
    for (int64_t c = 0; c < C_T; ++c)
        for (int64_t m = 0; m < T; ++m) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t h = 0; h < T; ++h)
                    s += dy[(n * D_T + d) * T + wrap(h + m, T)] *
                         x[(n * C_T + c) * T + h];
            dwrow[c * T + m] = s;
        }
}

/*
 * Forward.  rows == NULL: all N rows, y is [N][D_T][T].
 * rows != NULL: only rows[0..nrows), y is [nrows][D_T][T] in that order.
 * b == NULL: no bias.
 */
void oracle_forward(const double *x, const double *w, const double *b, double *y,
                    int64_t N, int64_t C_T, int64_t D_T, int64_t T,
                    const int64_t *rows, int64_t nrows)
{
    int64_t cnt = rows ? nrows : N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t n = rows ? rows[i] : i;
        forward_row(x, w, b, y + i * D_T * T, n, C_T, D_T, T);
    }
}

/* Bias gradient db[d] = sum over samples and group components of dY[n,d,g]. */
void oracle_backward_bias(const double *dy, double *db, int64_t N, int64_t D_T, int64_t T)
{
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D_T; ++d) {
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < T; ++g)
                s += dy[(n * D_T + d) * T + g];
        db[d] = s;
    }
}

/* Input gradient; rows as for oracle_forward, dx is [cnt][C_T][T]. */
void oracle_backward_input(const double *dy, const double *w, double *dx,
                           int64_t N, int64_t C_T, int64_t D_T, int64_t T,
                           const int64_t *rows, int64_t nrows)
{
    int64_t cnt = rows ? nrows : N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t n = rows ? rows[i] : i;
        backward_input_row(dy, w, dx + i * C_T * T, n, C_T, D_T, T);
    }
}

/*
 * Weight gradient.  dsel == NULL: all D_T output channels, dw is
 * [D_T][C_T][T].  dsel != NULL: only channels dsel[0..nd), dw is
 * [nd][C_T][T] in that order.
 */
void oracle_backward_weight(const double *x, const double *dy, double *dw,
                            int64_t N, int64_t C_T, int64_t D_T, int64_t T,
                            const int64_t *dsel, int64_t nd)
{
    int64_t cnt = dsel ? nd : D_T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t d = dsel ? dsel[i] : i;
        backward_weight_slice(x, dy, dw + i * C_T * T, d, N, C_T, D_T, T);
    }
}

/*
 * Weight spectrum, [pchao] §3.2.1 eq. (4) along the group axis of Wt:
 *   What_k[d,c] = sum_{m<T} Wt[d,c,m] * exp(-i 2 pi k m / T),  k = 0..floor(T/2)
 * stored as T real planes, each [D_T][C_T]:
 *   plane 0         = Re What_0
 *   plane 2k-1, 2k  = Re What_k, Im What_k     for 0 < k < T/2
 *   plane T-1       = Re What_{T/2}             (T even)
 * For odd T the last complex pair (k = (T-1)/2) fills planes T-2, T-1 and
 * there is no Nyquist plane.  T = 1 has the single plane Re What_0.
 * out is [T][D_T][C_T].
 */
void oracle_spectrum(const double *w, double *out, int64_t C_T, int64_t D_T, int64_t T)
{
    const double two_pi = 6.283185307179586476925286766559;
    int64_t plane_sz = D_T * C_T;
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D_T; ++d)
        for (int64_t c = 0; c < C_T; ++c) {
            const double *wv = w + (d * C_T + c) * T;
            for (int64_t k = 0; k <= T / 2; ++k) {
                double re = 0.0, im = 0.0;
                for (int64_t m = 0; m < T; ++m) {
                    double ang = two_pi * (double)((k * m) % T) / (double)T;
                    re += wv[m] * cos(ang);
                    im -= wv[m] * sin(ang);
                }
                int64_t off = d * C_T + c;
                if (k == 0) {
                    out[0 * plane_sz + off] = re;
                } else if (2 * k == T) {
                    out[(T - 1) * plane_sz + off] = re;
                } else {
                    out[(2 * k - 1) * plane_sz + off] = re;
                    out[(2 * k) * plane_sz + off] = im;
                }
            }
        }
}

/*
 * The octic group (rotations by multiples of 90 degrees and reflections, the
 * group of order 8 of [paperpeel] App. A.2 and A.4; [pchao] §3 treats the
 * rotation part).  Element g = a + 4 b stands for r^a s^b (a < 4 quarter
 * turns, b < 2 reflections), with r^a s^b . r^c s^d = r^(a + (-1)^b c) s^(b+d).
 *
 * The layer is the group convolution of the regular representation, the
 * same form as the cyclic layer above (whose (g - h) mod T is h^-1 g there):
 *
 *   Y[n,d,g]   = sum_{c<C_T} sum_{h<8} Wt[d,c,h^-1 g] * X[n,c,h]   (+ b[d])
 *   dX[n,c,h]  = sum_{d<D_T} sum_{g<8} Wt[d,c,h^-1 g] * dY[n,d,g]
 *   dWt[d,c,u] = sum_{n<N}   sum_{h<8} dY[n,d,h u] * X[n,c,h]
 *
 * Layouts as above with T = 8 (group axis contiguous).
 */
static int64_t oct_mul(int64_t g, int64_t h)
{
    int64_t a = g & 3, b = g >> 2, c = h & 3, d = h >> 2;
    int64_t rot = b ? a - c : a + c;
    return wrap(rot, 4) + 4 * (b ^ d);
}

static int64_t oct_inv(int64_t g)
{
    return (g >> 2) ? g : wrap(-g, 4);
}

static void oct_forward_row(const double *x, const double *w, const double *b, double *yrow,
                            int64_t n, int64_t C_T, int64_t D_T)
{
    for (int64_t d = 0; d < D_T; ++d)
        for (int64_t g = 0; g < 8; ++g) {
            double s = 0.0;
            for (int64_t c = 0; c < C_T; ++c)
                for (int64_t h = 0; h < 8; ++h)
                    s += w[(d * C_T + c) * 8 + oct_mul(oct_inv(h), g)] * x[(n * C_T + c) * 8 + h];
            yrow[d * 8 + g] = b ? s + b[d] : s;
        }
}

void oracle_octic_forward(const double *x, const double *w, const double *b, double *y,
                          int64_t N, int64_t C_T, int64_t D_T, const int64_t *rows, int64_t nrows)
{
    int64_t cnt = rows ? nrows : N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < cnt; ++i)
        oct_forward_row(x, w, b, y + i * D_T * 8, rows ? rows[i] : i, C_T, D_T);
}

void oracle_octic_backward_input(const double *dy, const double *w, double *dx,
                                 int64_t N, int64_t C_T, int64_t D_T, const int64_t *rows, int64_t nrows)
{
    int64_t cnt = rows ? nrows : N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t n = rows ? rows[i] : i;
        for (int64_t c = 0; c < C_T; ++c)
            for (int64_t h = 0; h < 8; ++h) {
                double s = 0.0;
                for (int64_t d = 0; d < D_T; ++d)
                    for (int64_t g = 0; g < 8; ++g)
                        s += w[(d * C_T + c) * 8 + oct_mul(oct_inv(h), g)] * dy[(n * D_T + d) * 8 + g];
                dx[(i * C_T + c) * 8 + h] = s;
            }
    }
}

void oracle_octic_backward_weight(const double *x, const double *dy, double *dw,
                                  int64_t N, int64_t C_T, int64_t D_T, const int64_t *dsel, int64_t nd)
{
    int64_t cnt = dsel ? nd : D_T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t d = dsel ? dsel[i] : i;
        for (int64_t c = 0; c < C_T; ++c)
            for (int64_t u = 0; u < 8; ++u) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t h = 0; h < 8; ++h)
                        s += dy[(n * D_T + d) * 8 + oct_mul(h, u)] * x[(n * C_T + c) * 8 + h];
                dw[(i * C_T + c) * 8 + u] = s;
            }
    }
}

/*
 * Group Fourier transform of Wt over the octic group, by definition
 *   What(rho)[d,c] = sum_{u<8} Wt[d,c,u] rho(u)
 * for the four one-dimensional representations chi (r -> +-1, s -> +-1) and
 * the two-dimensional one E (r -> quarter turn [[0,-1],[1,0]], s ->
 * [[1,0],[0,-1]]), rho(r^a s^b) = rho(r)^a rho(s)^b.  Eight real planes, each
 * [D_T][C_T]:
 *   0 A1 (r -> 1, s -> 1)   1 A2 (1, -1)   2 B1 (-1, 1)   3 B2 (-1, -1)
 *   4 E11   5 E12   6 E21   7 E22
 * out is [8][D_T][C_T].
 */
void oracle_octic_spectrum(const double *w, double *out, int64_t C_T, int64_t D_T)
{
    /* rho(u) for every element u, built from the generators */
    double chi[4][8], E[8][2][2];
    const double chr[4] = {1, 1, -1, -1}, chs[4] = {1, -1, 1, -1};
    const double R[2][2] = {{0, -1}, {1, 0}}, S[2][2] = {{1, 0}, {0, -1}};
    for (int u = 0; u < 8; ++u) {
        int a = u & 3, b = u >> 2;
        for (int j = 0; j < 4; ++j) chi[j][u] = pow(chr[j], a) * pow(chs[j], b);
        double m[2][2] = {{1, 0}, {0, 1}};
        for (int t = 0; t < a; ++t) {
            double q[2][2];
            for (int i = 0; i < 2; ++i)
                for (int k = 0; k < 2; ++k) q[i][k] = m[i][0] * R[0][k] + m[i][1] * R[1][k];
            for (int i = 0; i < 2; ++i)
                for (int k = 0; k < 2; ++k) m[i][k] = q[i][k];
        }
        if (b) {
            double q[2][2];
            for (int i = 0; i < 2; ++i)
                for (int k = 0; k < 2; ++k) q[i][k] = m[i][0] * S[0][k] + m[i][1] * S[1][k];
            for (int i = 0; i < 2; ++i)
                for (int k = 0; k < 2; ++k) m[i][k] = q[i][k];
        }
        for (int i = 0; i < 2; ++i)
            for (int k = 0; k < 2; ++k) E[u][i][k] = m[i][k];
    }
    int64_t plane_sz = D_T * C_T;
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D_T; ++d)
        for (int64_t c = 0; c < C_T; ++c) {
            const double *wv = w + (d * C_T + c) * 8;
            int64_t off = d * C_T + c;
            for (int j = 0; j < 4; ++j) {
                double s = 0.0;
                for (int u = 0; u < 8; ++u) s += wv[u] * chi[j][u];
                out[j * plane_sz + off] = s;
            }
            for (int i = 0; i < 2; ++i)
                for (int k = 0; k < 2; ++k) {
                    double s = 0.0;
                    for (int u = 0; u < 8; ++u) s += wv[u] * E[u][i][k];
                    out[(4 + 2 * i + k) * plane_sz + off] = s;
                }
        }
}

/* Number of OpenMP threads a parallel region here would use (1 without OpenMP). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
