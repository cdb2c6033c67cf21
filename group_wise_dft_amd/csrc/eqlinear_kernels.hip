// eqlinear_kernels.hip -- gfx950 (MI355X) kernels for Flash EQ-Linear.
//
// Sources:
//   [pchao]     "Flash EQ-Linear: accelerating equivariant linear layers via
//               group-wise DFT", Chinese translation at pchao.org
//   [paperpeel] the English text of a later revision at paperpeel.com
//
// The layer is a circular convolution along the group axis combined with a
// channel contraction ([pchao] §3.1 eqs. (1)-(3)).  Every kernel here works
// in the real-DFT coordinates of the group axis: T real "planes" per
// (row, channel),
//     plane 0         Re F_0
//     plane 2k-1, 2k  Re F_k, Im F_k      (0 < k < T/2)
//     plane T-1       Re F_{T/2}
// of F_k = sum_t v_t exp(-2 pi i k t / T) ([pchao] §3.2.1 eq. (4)).  The
// remaining frequencies are conjugates and are never formed (eq. (6)).
//
// Matrix-core mapping (gfx950, wave64).  All contractions use the 16x16
// MFMA family with fp32 accumulators:
//   fp16: v_mfma_f32_16x16x32_f16   (one instruction per 32-wide k slice)
//   fp32: v_mfma_f32_16x16x4_f32    (four instructions per 16-wide k slice)
// Lane l supplies operand row/column (l % 16) and a run of KL consecutive k
// values at k = (l / 16) * KL (KL = 8 for fp16, 4 for fp32).  A and B use the
// same lane->k assignment, so the sum over k is independent of how the
// hardware orders k inside an instruction.  Lane l receives result rows
// 4 * (l / 16) + e (e = 0..3) of column l % 16.
//
// Three kernel families:
//   row_kernel   forward (A = X rows, B = What) and input gradient
//                (A = dY rows, B = conj What transposed).  Each wave owns a
//                strip of rows; its lanes read KL consecutive channel groups
//                of one row straight from HBM into VGPRs (T*16 bytes), run
//                the group DFT in fp32 and build the A fragments of all T
//                planes in registers -- activations never pass through LDS
//                ([paperpeel] App. A.3 stage (i): transform on load).  The
//                weight planes of the tile are double-buffered in LDS.  The
//                epilogue applies the inverse group DFT to the T accumulator
//                planes of each output and stores the T group components
//                together ([pchao] App. 6.2 eq. (21) for T = 4).
//   dw_kernel    weight gradient dWhat_k = sum_n dYhat_k conj(Xhat_k): the
//                contraction runs over rows n, so both operands are staged
//                n-contiguous in LDS after the group DFT.  Rows are split into
//                fixed chunks; each workgroup writes fp32 partial spectra, and
//                dw_finalize adds them in a fixed order and applies the
//                inverse DFT (or the kernel does it directly when there is a
//                single chunk).
//   spectrum_kernel  What = group DFT of Wt (weight side of step 1).
//
// Complex products per non-redundant frequency 0 < k < T/2 ([pchao] App. 6.2
// eq. (20) for T = 4), with a = A operand planes and b = B operand planes:
//   forward (A . B):        re += a_r b_r - a_i b_i ; im += a_r b_i + a_i b_r
//   conj-B  (A . conj B):   re += a_r b_r + a_i b_i ; im += a_i b_r - a_r b_i
// The minus sign is carried by a negated copy of one A fragment.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "eqlinear_internal.h"

namespace eqk {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Real group DFT of length T and its inverse (with the 1/T factor).
// ---------------------------------------------------------------------------
template <int T> struct Dft;

template <> struct Dft<2> {
    __device__ static inline void fwd(const float *x, float *f) {
        f[0] = x[0] + x[1];
        f[1] = x[0] - x[1];
    }
    __device__ static inline void inv(const float *f, float *y) {
        y[0] = 0.5f * (f[0] + f[1]);
        y[1] = 0.5f * (f[0] - f[1]);
    }
};

// p4: [pchao] App. 6.2 eq. (19) (f0, f1 = Re F1, f3 = Im F1, f2 = F2 in the
// page's naming) and eq. (21) (coefficients 1/4 and 1/2).
template <> struct Dft<4> {
    __device__ static inline void fwd(const float *x, float *f) {
        const float s02 = x[0] + x[2], s13 = x[1] + x[3];
        f[0] = s02 + s13;
        f[1] = x[0] - x[2];
        f[2] = x[3] - x[1];
        f[3] = s02 - s13;
    }
    __device__ static inline void inv(const float *f, float *y) {
        const float a = 0.25f * (f[0] + f[3]), b = 0.25f * (f[0] - f[3]);
        const float r = 0.5f * f[1], i = 0.5f * f[2];
        y[0] = a + r;
        y[1] = b - i;
        y[2] = a - r;
        y[3] = b + i;
    }
};

// C8: one radix-2 split into sums s_t = x_t + x_{t+4} (even frequencies,
// a length-4 DFT) and differences d_t = x_t - x_{t+4} (odd frequencies,
// twiddles exp(-i pi t / 4) with the constant sqrt(1/2)).
template <> struct Dft<8> {
    static constexpr float R = 0.70710678118654752440f;
    __device__ static inline void fwd(const float *x, float *f) {
        const float s0 = x[0] + x[4], s1 = x[1] + x[5], s2 = x[2] + x[6], s3 = x[3] + x[7];
        const float d0 = x[0] - x[4], d1 = x[1] - x[5], d2 = x[2] - x[6], d3 = x[3] - x[7];
        const float p = R * (d1 - d3), q = R * (d1 + d3);
        f[0] = (s0 + s2) + (s1 + s3);      // Re F0
        f[1] = d0 + p;                     // Re F1
        f[2] = -(q + d2);                  // Im F1
        f[3] = s0 - s2;                    // Re F2
        f[4] = s3 - s1;                    // Im F2
        f[5] = d0 - p;                     // Re F3
        f[6] = d2 - q;                     // Im F3
        f[7] = (s0 + s2) - (s1 + s3);      // Re F4
    }
    __device__ static inline void inv(const float *f, float *y) {
        const float a04 = f[0] + f[7], b04 = f[0] - f[7];
        const float e0 = a04 + 2.0f * f[3], e2 = a04 - 2.0f * f[3];
        const float e1 = b04 - 2.0f * f[4], e3 = b04 + 2.0f * f[4];
        const float o0 = 2.0f * (f[1] + f[5]);
        const float o1 = (2.0f * R) * ((f[1] - f[5]) - (f[2] + f[6]));
        const float o2 = 2.0f * (f[6] - f[2]);
        const float o3 = (2.0f * R) * ((f[5] - f[1]) - (f[2] + f[6]));
        y[0] = 0.125f * (e0 + o0);
        y[1] = 0.125f * (e1 + o1);
        y[2] = 0.125f * (e2 + o2);
        y[3] = 0.125f * (e3 + o3);
        y[4] = 0.125f * (e0 - o0);
        y[5] = 0.125f * (e1 - o1);
        y[6] = 0.125f * (e2 - o2);
        y[7] = 0.125f * (e3 - o3);
    }
};

// ---------------------------------------------------------------------------
// Element-type traits: MFMA fragment and instruction per I/O dtype.
// ---------------------------------------------------------------------------
template <typename IO> struct Mma;

template <> struct Mma<f16> {
    static constexpr int KL = 8;  // consecutive k per lane and fragment
    typedef f16x8 frag;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KL = 4;
    typedef f32x4 frag;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

// T consecutive I/O elements (one group tuple), for loads and stores.
template <typename IO, int T> struct Tuple {
    typedef IO type __attribute__((ext_vector_type(T)));
};

// ---------------------------------------------------------------------------
// Workgroup -> tile order.  Consecutive workgroup ids are dealt round-robin
// to the 8 XCDs of an MI355X; remap so that each XCD receives a contiguous
// run of tile ids (tiles that share activation rows then share one L2).
// The map is a bijection on [0, n) for any n.
// ---------------------------------------------------------------------------
__device__ inline int xcd_tile(int b, int n) {
    const int xcd = b & 7, local = b >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd < rem ? xcd * (per + 1) + local
                     : rem * (per + 1) + (xcd - rem) * per + local;
}

// Per-frequency products of one (row block, column block, k slice).
template <int T, typename IO, bool CONJ>
__device__ inline void freq_mma(f32x4 *acc, const typename Mma<IO>::frag *a,
                                const typename Mma<IO>::frag *na,
                                const typename Mma<IO>::frag *b) {
    acc[0] = Mma<IO>::mma(a[0], b[0], acc[0]);
    acc[T - 1] = Mma<IO>::mma(a[T - 1], b[T - 1], acc[T - 1]);
#pragma unroll
    for (int k = 1; k < T / 2; ++k) {
        const int re = 2 * k - 1, im = 2 * k;
        acc[re] = Mma<IO>::mma(a[re], b[re], acc[re]);
        if (!CONJ) {
            acc[re] = Mma<IO>::mma(na[k - 1], b[im], acc[re]);   // - a_i b_i
            acc[im] = Mma<IO>::mma(a[re], b[im], acc[im]);
            acc[im] = Mma<IO>::mma(a[im], b[re], acc[im]);
        } else {
            acc[re] = Mma<IO>::mma(a[im], b[im], acc[re]);
            acc[im] = Mma<IO>::mma(a[im], b[re], acc[im]);
            acc[im] = Mma<IO>::mma(na[k - 1], b[im], acc[im]);   // - a_r b_i
        }
    }
}

// ===========================================================================
// Row kernel: out[m, col, :] = IDFT_k( sum_k' A_k[m, k'] op B_k[k', col] ).
//   act   [M][K][T]          rows of X (forward) or dY (input gradient)
//   what  [T][DT][CT]        weight planes
//   out   [M][NC][T]
//   BT = false: B[k][col] = what[p][col][k]   (forward: K = CT, NC = DT)
//   BT = true:  B[k][col] = what[p][k][col]   (input grad: K = DT, NC = CT)
//   CONJ: use conj(B) (input gradient).
// Tile: BM = WM*RB*16 rows x BN = WN*CB*16 columns, KC = KS*4*KL k per stage.
// ===========================================================================
template <int T, typename IO, bool CONJ, bool BT, int WM, int WN, int RB, int CB, int KS>
__global__ __launch_bounds__(WM *WN * 64) void row_kernel(
    const IO *__restrict__ act, const IO *__restrict__ what, IO *__restrict__ out,
    int M, int K, int NC, int DT, int CT) {
    typedef typename Mma<IO>::frag frag;
    constexpr int KL = Mma<IO>::KL;
    constexpr int KSUB = 4 * KL;
    constexpr int KC = KS * KSUB;
    constexpr int VL = 16 / sizeof(IO);       // elements per 16-byte chunk
    constexpr int PAD = VL;                   // 16 bytes of LDS row padding
    constexpr int LDK = KC + PAD;
    constexpr int NT = WM * WN * 64;
    constexpr int BM = WM * RB * 16, BN = WN * CB * 16;
    static_assert(VL == KL, "one fragment is one 16-byte chunk");

    __shared__ __attribute__((aligned(16))) IO sB[2][T][BN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 15, lg = lane >> 4;

    const int tiles_n = (NC + BN - 1) / BN;
    const int tiles = ((M + BM - 1) / BM) * tiles_n;
    const int tile = xcd_tile(blockIdx.x, tiles);
    const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
    const int nstage = (K + KC - 1) / KC;
    const size_t plane = (size_t)DT * CT;

    // ---- A: raw rows of the activation, loaded straight into VGPRs ----
    u32x4 rawA[RB][KS][T];
    auto load_a = [&](int ks) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int row = m0 + (wm * RB + i) * 16 + lr;
                const int k = ks * KC + s * KSUB + lg * KL;
                if (row < M && k < K) {
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(act + ((size_t)row * K + k) * T);
#pragma unroll
                    for (int t = 0; t < T; ++t) rawA[i][s][t] = src[t];
                } else {
#pragma unroll
                    for (int t = 0; t < T; ++t) rawA[i][s][t] = u32x4{0u, 0u, 0u, 0u};
                }
            }
    };

    frag aF[RB][KS][T];
    frag aN[RB][KS][T / 2 > 1 ? T / 2 - 1 : 1];
    auto transform_a = [&]() {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const IO *v = reinterpret_cast<const IO *>(&rawA[i][s][0]);
#pragma unroll
                for (int j = 0; j < KL; ++j) {
                    float x[T], f[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) x[t] = (float)v[j * T + t];
                    Dft<T>::fwd(x, f);
#pragma unroll
                    for (int p = 0; p < T; ++p) aF[i][s][p][j] = (IO)f[p];
                }
#pragma unroll
                for (int k = 1; k < T / 2; ++k)
                    aN[i][s][k - 1] = -(CONJ ? aF[i][s][2 * k - 1] : aF[i][s][2 * k]);
            }
    };

    // ---- B: weight planes, global -> VGPR -> LDS ----
    constexpr int BCH = BT ? T * (KC / VL) * (BN / VL) : T * BN * (KC / VL);  // chunks or blocks
    constexpr int BPER = (BCH + NT - 1) / NT;
    constexpr int BROWS = BT ? VL : 1;
    u32x4 rawB[BPER][BROWS];
    auto load_b = [&](int ks) {
#pragma unroll
        for (int it = 0; it < BPER; ++it) {
            const int u = it * NT + tid;
            if (BT) {
                const int cb = u % (BN / VL), kb = (u / (BN / VL)) % (KC / VL), p = u / ((BN / VL) * (KC / VL));
                const int k = ks * KC + kb * VL, col = n0 + cb * VL;
                const bool ok = (u < BCH) && (k < K) && (col < NC);
#pragma unroll
                for (int v = 0; v < BROWS; ++v)
                    rawB[it][v] = ok ? *reinterpret_cast<const u32x4 *>(what + p * plane + (size_t)(k + v) * CT + col)
                                     : u32x4{0u, 0u, 0u, 0u};
            } else {
                const int kc = u % (KC / VL), col = (u / (KC / VL)) % BN, p = u / ((KC / VL) * BN);
                const int k = ks * KC + kc * VL;
                const bool ok = (u < BCH) && (k < K) && (n0 + col < NC);
                rawB[it][0] = ok ? *reinterpret_cast<const u32x4 *>(what + p * plane + (size_t)(n0 + col) * CT + k)
                                 : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_b = [&](int buf) {
#pragma unroll
        for (int it = 0; it < BPER; ++it) {
            const int u = it * NT + tid;
            if (u >= BCH) continue;
            if (BT) {
                const int cb = u % (BN / VL), kb = (u / (BN / VL)) % (KC / VL), p = u / ((BN / VL) * (KC / VL));
                // transpose the VL x VL block: row v (k) x column w (col)
#pragma unroll
                for (int w = 0; w < VL; ++w) {
                    IO col_vals[VL];
#pragma unroll
                    for (int v = 0; v < VL; ++v) col_vals[v] = reinterpret_cast<const IO *>(&rawB[it][v])[w];
                    *reinterpret_cast<u32x4 *>(&sB[buf][p][cb * VL + w][kb * VL]) =
                        *reinterpret_cast<const u32x4 *>(col_vals);
                }
            } else {
                const int kc = u % (KC / VL), col = (u / (KC / VL)) % BN, p = u / ((KC / VL) * BN);
                *reinterpret_cast<u32x4 *>(&sB[buf][p][col][kc * VL]) = rawB[it][0];
            }
        }
    };

    f32x4 acc[RB][CB][T];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int p = 0; p < T; ++p) acc[i][j][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nstage > 0) {
        load_a(0);
        load_b(0);
        store_b(0);
        transform_a();
        __syncthreads();
    }
    for (int ks = 0; ks < nstage; ++ks) {
        const int buf = ks & 1;
        const bool more = ks + 1 < nstage;
        if (more) {
            load_a(ks + 1);
            load_b(ks + 1);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                frag bF[T];
                const int col = (wn * CB + j) * 16 + lr;
#pragma unroll
                for (int p = 0; p < T; ++p)
                    bF[p] = *reinterpret_cast<const frag *>(&sB[buf][p][col][s * KSUB + lg * KL]);
#pragma unroll
                for (int i = 0; i < RB; ++i) freq_mma<T, IO, CONJ>(acc[i][j], aF[i][s], aN[i][s], bF);
            }
        if (more) {
            store_b(buf ^ 1);
            transform_a();
        }
        __syncthreads();
    }

    // ---- epilogue: inverse group DFT of the T accumulator planes ----
    typedef typename Tuple<IO, T>::type tup;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + (wm * RB + i) * 16 + lg * 4 + e;
                const int col = n0 + (wn * CB + j) * 16 + lr;
                if (row < M && col < NC) {
                    float f[T], y[T];
#pragma unroll
                    for (int p = 0; p < T; ++p) f[p] = acc[i][j][p][e];
                    Dft<T>::inv(f, y);
                    tup o;
#pragma unroll
                    for (int t = 0; t < T; ++t) o[t] = (IO)y[t];
                    *reinterpret_cast<tup *>(out + ((size_t)row * NC + col) * T) = o;
                }
            }
}

// ===========================================================================
// Weight-gradient kernel: for its tile (d rows x c columns) and its chunk of
// rows n, acc_k[d, c] = sum_n dYhat_k[n, d] conj(Xhat_k[n, c]).
//   x   [N][CT][T], dy [N][DT][T]
//   DIRECT: one chunk; apply the inverse DFT and write dw [DT][CT][T].
//   else:   write fp32 planes to ws[split][T][DT][CT].
// ===========================================================================
template <int T, typename IO, int WM, int WN, int RB, int CB, int KS, bool DIRECT>
__global__ __launch_bounds__(WM *WN * 64) void dw_kernel(
    const IO *__restrict__ x, const IO *__restrict__ dy, float *__restrict__ ws,
    IO *__restrict__ dw, int N, int CT, int DT, int chunk) {
    typedef typename Mma<IO>::frag frag;
    constexpr int KL = Mma<IO>::KL;
    constexpr int KSUB = 4 * KL;
    constexpr int KC = KS * KSUB;
    constexpr int VL = 16 / sizeof(IO);
    constexpr int LDK = KC + VL;
    constexpr int NT = WM * WN * 64;
    constexpr int BM = WM * RB * 16, BN = WN * CB * 16;
    static_assert(VL == KL, "one fragment is one 16-byte chunk");

    __shared__ __attribute__((aligned(16))) IO sA[T][BM][LDK];
    __shared__ __attribute__((aligned(16))) IO sB[T][BN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 15, lg = lane >> 4;

    const int tiles_n = (CT + BN - 1) / BN;
    const int tiles = ((DT + BM - 1) / BM) * tiles_n;
    const int t_all = xcd_tile(blockIdx.x, gridDim.x);
    const int split = t_all / tiles, tile = t_all % tiles;
    const int d0 = (tile / tiles_n) * BM, c0 = (tile % tiles_n) * BN;
    const int nbeg = split * chunk;
    const int nend = min(N, nbeg + chunk);
    const int nstage = (nend - nbeg + KC - 1) / KC;

    typedef typename Tuple<IO, T>::type tup;
    // staging units: (channel within the tile, run of VL rows)
    constexpr int UA = (BM * (KC / VL) + NT - 1) / NT;
    constexpr int UB = (BN * (KC / VL) + NT - 1) / NT;
    tup rawA[UA][VL], rawB[UB][VL];

    auto load = [&](int ks) {
#pragma unroll
        for (int it = 0; it < UA; ++it) {
            const int u = it * NT + tid, dl = u % BM, nb = u / BM;
#pragma unroll
            for (int v = 0; v < VL; ++v) {
                const int n = nbeg + ks * KC + nb * VL + v;
                const bool ok = (u < BM * (KC / VL)) && (n < nend) && (d0 + dl < DT);
                tup z;
#pragma unroll
                for (int t = 0; t < T; ++t) z[t] = (IO)0.0f;
                rawA[it][v] = ok ? *reinterpret_cast<const tup *>(dy + ((size_t)n * DT + d0 + dl) * T) : z;
            }
        }
#pragma unroll
        for (int it = 0; it < UB; ++it) {
            const int u = it * NT + tid, cl = u % BN, nb = u / BN;
#pragma unroll
            for (int v = 0; v < VL; ++v) {
                const int n = nbeg + ks * KC + nb * VL + v;
                const bool ok = (u < BN * (KC / VL)) && (n < nend) && (c0 + cl < CT);
                tup z;
#pragma unroll
                for (int t = 0; t < T; ++t) z[t] = (IO)0.0f;
                rawB[it][v] = ok ? *reinterpret_cast<const tup *>(x + ((size_t)n * CT + c0 + cl) * T) : z;
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int it = 0; it < UA; ++it) {
            const int u = it * NT + tid, dl = u % BM, nb = u / BM;
            if (u >= BM * (KC / VL)) continue;
            frag pl[T];
#pragma unroll
            for (int v = 0; v < VL; ++v) {
                float xv[T], f[T];
#pragma unroll
                for (int t = 0; t < T; ++t) xv[t] = (float)rawA[it][v][t];
                Dft<T>::fwd(xv, f);
#pragma unroll
                for (int p = 0; p < T; ++p) pl[p][v] = (IO)f[p];
            }
#pragma unroll
            for (int p = 0; p < T; ++p) *reinterpret_cast<frag *>(&sA[p][dl][nb * VL]) = pl[p];
        }
#pragma unroll
        for (int it = 0; it < UB; ++it) {
            const int u = it * NT + tid, cl = u % BN, nb = u / BN;
            if (u >= BN * (KC / VL)) continue;
            frag pl[T];
#pragma unroll
            for (int v = 0; v < VL; ++v) {
                float xv[T], f[T];
#pragma unroll
                for (int t = 0; t < T; ++t) xv[t] = (float)rawB[it][v][t];
                Dft<T>::fwd(xv, f);
#pragma unroll
                for (int p = 0; p < T; ++p) pl[p][v] = (IO)f[p];
            }
#pragma unroll
            for (int p = 0; p < T; ++p) *reinterpret_cast<frag *>(&sB[p][cl][nb * VL]) = pl[p];
        }
    };

    f32x4 acc[RB][CB][T];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int p = 0; p < T; ++p) acc[i][j][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nstage > 0) load(0);
    for (int ks = 0; ks < nstage; ++ks) {
        __syncthreads();  // previous stage's fragment reads are done
        store();
        __syncthreads();
        if (ks + 1 < nstage) load(ks + 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            frag bF[CB][T];
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int p = 0; p < T; ++p)
                    bF[j][p] = *reinterpret_cast<const frag *>(&sB[p][(wn * CB + j) * 16 + lr][s * KSUB + lg * KL]);
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                frag aF[T], aN[T / 2 > 1 ? T / 2 - 1 : 1];
#pragma unroll
                for (int p = 0; p < T; ++p)
                    aF[p] = *reinterpret_cast<const frag *>(&sA[p][(wm * RB + i) * 16 + lr][s * KSUB + lg * KL]);
#pragma unroll
                for (int k = 1; k < T / 2; ++k) aN[k - 1] = -aF[2 * k - 1];
#pragma unroll
                for (int j = 0; j < CB; ++j) freq_mma<T, IO, true>(acc[i][j], aF, aN, bF[j]);
            }
        }
    }

#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = d0 + (wm * RB + i) * 16 + lg * 4 + e;
                const int c = c0 + (wn * CB + j) * 16 + lr;
                if (d < DT && c < CT) {
                    if (DIRECT) {
                        float f[T], y[T];
#pragma unroll
                        for (int p = 0; p < T; ++p) f[p] = acc[i][j][p][e];
                        Dft<T>::inv(f, y);
                        tup o;
#pragma unroll
                        for (int t = 0; t < T; ++t) o[t] = (IO)y[t];
                        *reinterpret_cast<tup *>(dw + ((size_t)d * CT + c) * T) = o;
                    } else {
#pragma unroll
                        for (int p = 0; p < T; ++p)
                            ws[(((size_t)split * T + p) * DT + d) * CT + c] = acc[i][j][p][e];
                    }
                }
            }
}

// dw[d, c, :] = IDFT( sum_{s < S} ws[s, :, d, c] ), s in increasing order.
template <int T, typename IO>
__global__ __launch_bounds__(256) void dw_finalize(const float *__restrict__ ws, IO *__restrict__ dw,
                                                   int CT, int DT, int S) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t plane = (size_t)DT * CT;
    if (idx >= plane) return;
    float f[T], y[T];
#pragma unroll
    for (int p = 0; p < T; ++p) f[p] = 0.0f;
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int p = 0; p < T; ++p) f[p] += ws[((size_t)s * T + p) * plane + idx];
    Dft<T>::inv(f, y);
    typedef typename Tuple<IO, T>::type tup;
    tup o;
#pragma unroll
    for (int t = 0; t < T; ++t) o[t] = (IO)y[t];
    *reinterpret_cast<tup *>(dw + idx * T) = o;
}

// what[p, d, c] = plane p of the group DFT of wt[d, c, :].
template <int T, typename IO>
__global__ __launch_bounds__(256) void spectrum_kernel(const IO *__restrict__ wt, IO *__restrict__ what,
                                                       int CT, int DT) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t plane = (size_t)DT * CT;
    if (idx >= plane) return;
    typedef typename Tuple<IO, T>::type tup;
    const tup v = *reinterpret_cast<const tup *>(wt + idx * T);
    float x[T], f[T];
#pragma unroll
    for (int t = 0; t < T; ++t) x[t] = (float)v[t];
    Dft<T>::fwd(x, f);
#pragma unroll
    for (int p = 0; p < T; ++p) what[p * plane + idx] = (IO)f[p];
}

// ===========================================================================
// Launch configurations (a fixed rule on T and dtype) and host launchers.
// ===========================================================================
template <int T, typename IO> struct RowCfg;      // forward / input gradient
template <> struct RowCfg<2, f16>   { enum { WM = 4, WN = 1, RB = 2, CB = 8, KS = 1 }; };
template <> struct RowCfg<4, f16>   { enum { WM = 4, WN = 1, RB = 2, CB = 4, KS = 1 }; };
template <> struct RowCfg<8, f16>   { enum { WM = 4, WN = 1, RB = 2, CB = 2, KS = 1 }; };
template <> struct RowCfg<2, float> { enum { WM = 4, WN = 1, RB = 2, CB = 8, KS = 1 }; };
template <> struct RowCfg<4, float> { enum { WM = 4, WN = 1, RB = 2, CB = 4, KS = 1 }; };
template <> struct RowCfg<8, float> { enum { WM = 4, WN = 1, RB = 2, CB = 2, KS = 1 }; };

template <int T, typename IO> struct DwCfg;       // weight gradient
template <> struct DwCfg<2, f16>   { enum { WM = 2, WN = 2, RB = 4, CB = 4, KS = 1 }; };
template <> struct DwCfg<4, f16>   { enum { WM = 2, WN = 2, RB = 4, CB = 2, KS = 1 }; };
template <> struct DwCfg<8, f16>   { enum { WM = 2, WN = 2, RB = 2, CB = 2, KS = 1 }; };
template <> struct DwCfg<2, float> { enum { WM = 2, WN = 2, RB = 4, CB = 4, KS = 1 }; };
template <> struct DwCfg<4, float> { enum { WM = 2, WN = 2, RB = 4, CB = 2, KS = 1 }; };
template <> struct DwCfg<8, float> { enum { WM = 2, WN = 2, RB = 2, CB = 2, KS = 1 }; };

template <int T, typename IO, bool CONJ, bool BT>
static hipError_t launch_row(const void *act, const void *what, void *out, int M, int K, int NC,
                             int DT, int CT, hipStream_t st) {
    typedef RowCfg<T, IO> C;
    constexpr int BM = C::WM * C::RB * 16, BN = C::WN * C::CB * 16;
    if (M == 0) return hipSuccess;
    const int tiles = ((M + BM - 1) / BM) * ((NC + BN - 1) / BN);
    hipLaunchKernelGGL((row_kernel<T, IO, CONJ, BT, C::WM, C::WN, C::RB, C::CB, C::KS>), dim3(tiles),
                       dim3(C::WM * C::WN * 64), 0, st, (const IO *)act, (const IO *)what, (IO *)out, M,
                       K, NC, DT, CT);
    return hipGetLastError();
}

template <int T, typename IO>
static hipError_t launch_spectrum(const void *wt, void *what, int CT, int DT, hipStream_t st) {
    const size_t n = (size_t)CT * DT;
    hipLaunchKernelGGL((spectrum_kernel<T, IO>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const IO *)wt, (IO *)what, CT, DT);
    return hipGetLastError();
}

template <int T, typename IO>
static hipError_t launch_dw(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                            hipStream_t st) {
    typedef DwCfg<T, IO> C;
    const DwPlan pl = dw_plan(N, CT, DT, T, sizeof(IO));
    const size_t n = (size_t)CT * DT;
    if (pl.splits == 0) {  // N == 0: the gradient is zero
        hipLaunchKernelGGL((dw_finalize<T, IO>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           (const float *)ws, (IO *)dw, CT, DT, 0);
        return hipGetLastError();
    }
    const int grid = pl.tiles * pl.splits;
    if (pl.splits == 1) {
        hipLaunchKernelGGL((dw_kernel<T, IO, C::WM, C::WN, C::RB, C::CB, C::KS, true>), dim3(grid),
                           dim3(C::WM * C::WN * 64), 0, st, (const IO *)x, (const IO *)dy, (float *)ws,
                           (IO *)dw, N, CT, DT, pl.chunk);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((dw_kernel<T, IO, C::WM, C::WN, C::RB, C::CB, C::KS, false>), dim3(grid),
                       dim3(C::WM * C::WN * 64), 0, st, (const IO *)x, (const IO *)dy, (float *)ws,
                       (IO *)dw, N, CT, DT, pl.chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dw_finalize<T, IO>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float *)ws, (IO *)dw, CT, DT, pl.splits);
    return hipGetLastError();
}

// Tile sizes of the weight-gradient kernel, for the split plan.
template <int T, typename IO> static void dw_tile(int *bm, int *bn, int *kc) {
    typedef DwCfg<T, IO> C;
    *bm = C::WM * C::RB * 16;
    *bn = C::WN * C::CB * 16;
    *kc = C::KS * 4 * Mma<IO>::KL;
}

}  // namespace eqk

// ---------------------------------------------------------------------------
// Internal entry points (declared in eqlinear_internal.h).
// ---------------------------------------------------------------------------
#define EQK_DISPATCH(T_, DT_, CALL)                                        \
    do {                                                                   \
        if ((DT_) == 0) {                                                  \
            if ((T_) == 2) { typedef float IO; constexpr int T = 2; CALL; } \
            if ((T_) == 4) { typedef float IO; constexpr int T = 4; CALL; } \
            if ((T_) == 8) { typedef float IO; constexpr int T = 8; CALL; } \
        } else {                                                           \
            if ((T_) == 2) { typedef eqk::f16 IO; constexpr int T = 2; CALL; } \
            if ((T_) == 4) { typedef eqk::f16 IO; constexpr int T = 4; CALL; } \
            if ((T_) == 8) { typedef eqk::f16 IO; constexpr int T = 8; CALL; } \
        }                                                                  \
        return hipErrorInvalidValue;                                       \
    } while (0)

DwPlan dw_plan(int64_t N, int64_t C_T, int64_t D_T, int T, int elem_bytes) {
    int bm = 0, bn = 0, kc = 0;
    if (elem_bytes == 4) {
        if (T == 2) eqk::dw_tile<2, float>(&bm, &bn, &kc);
        else if (T == 4) eqk::dw_tile<4, float>(&bm, &bn, &kc);
        else eqk::dw_tile<8, float>(&bm, &bn, &kc);
    } else {
        if (T == 2) eqk::dw_tile<2, eqk::f16>(&bm, &bn, &kc);
        else if (T == 4) eqk::dw_tile<4, eqk::f16>(&bm, &bn, &kc);
        else eqk::dw_tile<8, eqk::f16>(&bm, &bn, &kc);
    }
    DwPlan p;
    p.tiles = (int)(((D_T + bm - 1) / bm) * ((C_T + bn - 1) / bn));
    if (N <= 0) {
        p.splits = 0;
        p.chunk = 0;
        return p;
    }
    // Aim for about one workgroup per compute unit of an MI355X (256), with
    // every chunk a whole number of k stages.
    const int64_t target = 256;
    int64_t s = (target + p.tiles - 1) / p.tiles;
    const int64_t stages = (N + kc - 1) / kc;
    if (s > stages) s = stages;
    if (s < 1) s = 1;
    int64_t chunk = ((N + s - 1) / s + kc - 1) / kc * kc;
    p.chunk = (int)chunk;
    p.splits = (int)((N + chunk - 1) / chunk);
    return p;
}

hipError_t eqk_spectrum(const void *wt, void *what, int CT, int DT, int T, int dt, hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_spectrum<T, IO>(wt, what, CT, DT, st)));
}

hipError_t eqk_forward(const void *x, const void *what, void *y, int N, int CT, int DT, int T, int dt,
                       hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_row<T, IO, false, false>(x, what, y, N, CT, DT, DT, CT, st)));
}

hipError_t eqk_backward_input(const void *dy, const void *what, void *dx, int N, int CT, int DT, int T,
                              int dt, hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_row<T, IO, true, true>(dy, what, dx, N, DT, CT, DT, CT, st)));
}

hipError_t eqk_backward_weight(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                               int T, int dt, hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_dw<T, IO>(x, dy, dw, ws, N, CT, DT, st)));
}
