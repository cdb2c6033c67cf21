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
// Matrix-core mapping (gfx950, wave64).  All contractions run on 32x32 MFMA
// blocks with fp32 accumulators (M32):
//   fp16: v_mfma_f32_32x32x16_f16   (one instruction per 16-wide k slice)
//   fp32: v_mfma_f32_32x32x2_f32    (four instructions per 8-wide k slice)
// Lane l supplies operand row/column (l % 32) and a run of KL consecutive k
// values at k = (l / 32) * KL (KL = 8 for fp16, 4 for fp32): one 16-byte
// chunk of k-contiguous data.  A and B use the same lane->k assignment, so
// the sum over k does not depend on how the hardware orders k inside an
// instruction.
//
// Memory access.  Every global access goes through a buffer resource whose
// range covers only the valid part of the tile: loads outside it return
// zeros and stores outside it are dropped, so ragged tails need no branches
// in the hot loops.  Lanes whose k (or column) is past the end use an offset
// beyond every range (OOB).
//
// Kernel families:
//   row_kernel   forward (A = X rows, B = What) and input gradient (A = dY
//                rows, B = conj What, from the channel-major copy of the
//                spectrum).  Each stage's raw activation tuples and weight
//                planes are copied HBM -> LDS by the buffer unit into a ring
//                (no VGPR staging); each wave reads its rows' tuples, runs the
//                group DFT in fp32 into the A fragments of all T planes
//                ([paperpeel] App. A.3 stage (i): transform on load), and
//                multiplies.  The epilogue applies the inverse group DFT to
//                the T accumulator planes of each output and stores the T
//                group components together ([pchao] App. 6.2 eq. (21) for
//                T = 4).  rowk_kernel is the variant for layers with few
//                output tiles (k range of each stage split over the waves).
//   dw_kernel    weight gradient dWhat_k = sum_n dYhat_k conj(Xhat_k): the
//                contraction runs over rows n, so both operands are
//                transformed and staged n-contiguous in LDS.  Rows are split
//                into fixed chunks; each workgroup writes fp32 partial
//                spectra, and dw_finalize adds them in a fixed order and
//                applies the inverse DFT (or the kernel does it directly when
//                there is a single chunk).  dwr_kernel is the variant with a
//                copy ring for small grids, dwp_kernel the producer/consumer
//                variant (order 8, the octic group, order 2 in fp16 and
//                order 4 outside the narrow and ring plans; see dw_plan).
//   spectrum_kernel  What = group DFT of Wt (weight side of step 1), written
//                in two orientations, blocked for the row kernels' copies.
//   bias_partial / bias_finalize  the bias gradient.
//
// Complex products per non-redundant frequency 0 < k < T/2 ([pchao] App. 6.2
// eq. (20) for T = 4), with a = A operand planes and b = B operand planes:
//   plain (A . B):          re += a_r b_r - a_i b_i ; im += a_r b_i + a_i b_r
//   conj-B (A . conj B):    re += a_r b_r + a_i b_i ; im += a_i b_r - a_r b_i
// The minus sign is carried by a negated copy of one A fragment.  In fp32 at
// orders 4, 6, 8 the row kernels and the weight gradient use Gauss's three
// products instead (see Gauss below): the planes staged and multiplied are
// then the sums a_r + a_i, a_r, a_i against b_r, b_i - b_r, b_r + b_i (of
// conj b where the product takes the conjugate), and the diagonal plane
// products give Re = K1 - K3, Im = K1 + K2.
//
// The octic group (quarter turns and reflections, the group D8 of
// [paperpeel] App. A.2 and A.4): the template parameter GRP = 1 of the row,
// spectrum and producer/consumer weight-gradient kernels replaces the
// order-8 DFT by the octic Fourier transform (struct Octic: the four real
// characters and the 2 x 2 real representation E, eight planes) and the
// per-frequency products by the representation products (oct_mma_row,
// oct_mma_dw: four diagonal character products plus the E-block matrix
// product); tiles, rings and launch plans are those of order 8.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "eqlinear_internal.h"

namespace eqk {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Offset that is outside every buffer range used here (ranges stay below
// 2^31 bytes, enforced by the host layer).
constexpr uint32_t OOB = 0x80000000u;

// Buffer cache policy of the row kernels' output stores: non-temporal
// (streaming).  Each output tile is written once and never read by the
// kernel; the hint keeps the output stream from evicting the activation rows
// that the other column tiles of the same row block still read from L2.
constexpr int CP_NT = 2;

// Buffer resource over [base, base + bytes): gfx9 raw buffer, no stride.
__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// ---------------------------------------------------------------------------
// Real group DFT of length T and its inverse (with the 1/T factor), fp32.
// Planes: 0 = Re F0; 2k-1, 2k = Re F_k, Im F_k for 0 < k < T/2; T-1 = Re F_{T/2}
// when T is even.  F_k = sum_t x_t exp(-2 pi i k t / T) ([pchao] §3.2.1
// eq. (4)); the inverse is [pchao] eq. (7) with the conjugate symmetry of
// eq. (6).  Orders 2, 4 and 8 have the hand-written forms below; any other
// order uses the direct sums with compile-time twiddles.
// ---------------------------------------------------------------------------
// cos(2 pi m / T) and sin(2 pi m / T) evaluated at compile time (Taylor series
// in double on the reduced angle).
constexpr double cx_poly(double x, bool sine) {
    double term = sine ? x : 1.0, sum = term;
    for (int n = 1; n < 30; ++n) {
        const int a = sine ? 2 * n : 2 * n - 1, b = sine ? 2 * n + 1 : 2 * n;
        term *= -x * x / ((double)a * (double)b);
        sum += term;
    }
    return sum;
}
constexpr double cx_twiddle(int m, int T, bool sine) {
    const double pi = 3.14159265358979323846264338327950288;
    int r = m % T;
    if (r < 0) r += T;
    double x = 2.0 * pi * (double)r / (double)T;
    if (x > pi) x -= 2.0 * pi;
    return cx_poly(x, sine);
}
template <int T> struct Dft {
    // Components j and T - j share cos(2 pi j k / T) and have opposite sines,
    // so the sums run over the H = (T-1)/2 pairs s_j = x_j + x_{T-j},
    // d_j = x_j - x_{T-j} (plus the middle component x_{T/2} for even T):
    //   Re F_k = x_0 + sum_j cos(2 pi j k / T) s_j (+ (-1)^k x_{T/2})
    //   Im F_k =     - sum_j sin(2 pi j k / T) d_j
    // and the inverse pairs outputs t and T - t the same way.
    static constexpr int H = (T - 1) / 2;
    static constexpr bool EVEN = T % 2 == 0;
    __device__ static inline float cs(int m) { return (float)cx_twiddle(m, T, false); }
    __device__ static inline float sn(int m) { return (float)cx_twiddle(m, T, true); }
    __device__ static inline void fwd(const float *x, float *f) {
        float sp[H + 1], dp[H + 1];
#pragma unroll
        for (int j = 1; j <= H; ++j) {
            sp[j] = x[j] + x[T - j];
            dp[j] = x[j] - x[T - j];
        }
        const float mid = EVEN ? x[T / 2] : 0.0f;
        float s0 = x[0];
#pragma unroll
        for (int j = 1; j <= H; ++j) s0 += sp[j];
        f[0] = EVEN ? s0 + mid : s0;
#pragma unroll
        for (int k = 1; k <= H; ++k) {
            float re = x[0], im = 0.0f;
#pragma unroll
            for (int j = 1; j <= H; ++j) {
                re = __builtin_fmaf(cs(j * k), sp[j], re);
                im = __builtin_fmaf(-sn(j * k), dp[j], im);
            }
            if (EVEN) re += (k % 2 ? -mid : mid);
            f[2 * k - 1] = re;
            f[2 * k] = im;
        }
        if (EVEN) {
            float a = x[0];
#pragma unroll
            for (int j = 1; j <= H; ++j) a += (j % 2 ? -sp[j] : sp[j]);
            f[T - 1] = a + ((T / 2) % 2 ? -mid : mid);
        }
    }
    __device__ static inline void inv(const float *f, float *y) {
        constexpr float S = 1.0f / (float)T;
        const float nq = EVEN ? f[T - 1] : 0.0f;
        float r0 = 0.0f;
#pragma unroll
        for (int k = 1; k <= H; ++k) r0 += f[2 * k - 1];
        y[0] = (f[0] + nq + 2.0f * r0) * S;
#pragma unroll
        for (int t = 1; t <= H; ++t) {
            float pc = 0.0f, qs = 0.0f;
#pragma unroll
            for (int k = 1; k <= H; ++k) {
                pc = __builtin_fmaf(cs(k * t), f[2 * k - 1], pc);
                qs = __builtin_fmaf(sn(k * t), f[2 * k], qs);
            }
            const float base = EVEN ? f[0] + (t % 2 ? -nq : nq) : f[0];
            y[t] = (base + 2.0f * (pc - qs)) * S;
            y[T - t] = (base + 2.0f * (pc + qs)) * S;   // (-1)^(T-t) = (-1)^t for even T
        }
        if (EVEN) {
            float rm = 0.0f;
#pragma unroll
            for (int k = 1; k <= H; ++k) rm += (k % 2 ? -f[2 * k - 1] : f[2 * k - 1]);
            y[T / 2] = (f[0] + ((T / 2) % 2 ? -nq : nq) + 2.0f * rm) * S;
        }
    }
};

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
// Element-type traits: the 16-byte MFMA operand fragment (KL consecutive k
// of one row or column) per I/O dtype, shared by every kernel; M32 below adds
// the 32x32 instructions.
// ---------------------------------------------------------------------------
template <typename IO> struct Mma;

template <> struct Mma<f16> {
    static constexpr int KL = 8;  // consecutive k per lane and fragment
    typedef f16x8 frag;
    __device__ static inline frag neg(frag a) {  // flip the sign bits
        u32x4 u = __builtin_bit_cast(u32x4, a);
        u ^= 0x80008000u;
        return __builtin_bit_cast(frag, u);
    }
};

template <> struct Mma<float> {
    static constexpr int KL = 4;
    typedef f32x4 frag;
    __device__ static inline frag neg(frag a) { return -a; }
};

// 32x32 output blocks (the higher-throughput MFMA shape on gfx950).  Lane l
// supplies row/column (l % 32) and the k-run of KL values at (l / 32) * KL
// of a 2*KL-wide k slice; it receives rows (r % 4) + 4 * (l / 32) + 8 * (r / 4)
// (r = 0..15) of column l % 32.
//   fp16: v_mfma_f32_32x32x16_f16  (one instruction per slice)
//   fp32: v_mfma_f32_32x32x2_f32   (four instructions; instruction m takes
//                                   element m of each lane's run)
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <typename IO> struct M32;
template <> struct M32<f16> {
    static constexpr int KL = 8;
    typedef f16x8 frag;
    typedef f32x16 acc_t;
    __device__ static inline acc_t mma(frag a, frag b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag neg(frag a) { return Mma<f16>::neg(a); }
};
template <> struct M32<float> {
    static constexpr int KL = 4;
    typedef f32x4 frag;
    typedef f32x16 acc_t;
    __device__ static inline acc_t mma(frag a, frag b, acc_t c) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    __device__ static inline frag neg(frag a) { return -a; }
};

// T consecutive I/O elements (one group tuple), for loads and stores.
template <typename IO, int T> struct Tuple {
    typedef IO type __attribute__((ext_vector_type(T)));
};

// Raw buffer load / store of N bytes (N in {4, 8, 16, 32}).
template <int BYTES> struct Raw;

// One element of 2 (fp16) or 4 (fp32) bytes.
template <typename IO> struct Elem;
template <> struct Elem<f16> {
    __device__ static inline f16 load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(f16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    }
    template <int AUX = 0>
    __device__ static inline void store(f16 v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, off, 0, AUX);
    }
};
template <> struct Elem<float> {
    __device__ static inline float load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
    template <int AUX = 0>
    __device__ static inline void store(float v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, off, 0, AUX);
    }
};

// Group orders with a vector type of their own size (2, 4, 8) move a tuple in
// one access; the others (3, 5, 6, 7) move it one element at a time.
template <int T> struct Pow2 { static constexpr bool value = (T & (T - 1)) == 0; };
// Largest power of two that divides n, at most 16.
__host__ __device__ constexpr int pow2_part16(int n) { return (n & -n) > 16 ? 16 : (n & -n); }
template <typename IO, int T> struct Elems { IO v[T]; };
template <> struct Raw<4> {
    typedef unsigned int type;
    __device__ static inline type load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    template <int AUX = 0>
    __device__ static inline void store(type v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, AUX);
    }
};
template <> struct Raw<8> {
    typedef u32x2 type;
    __device__ static inline type load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
    template <int AUX = 0>
    __device__ static inline void store(type v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, AUX);
    }
};
template <> struct Raw<16> {
    typedef u32x4 type;
    __device__ static inline type load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
    template <int AUX = 0>
    __device__ static inline void store(type v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
    }
};
template <> struct Raw<32> {   // two 16-byte halves (fp32 tuples of T = 8)
    struct type { u32x4 lo, hi; };

    __device__ static inline type load(rsrc_t r, uint32_t off) {
        return {__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0),
                __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0)};
    }
    template <int AUX = 0>
    __device__ static inline void store(type v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b128(v.lo, r, off, 0, AUX);
        __builtin_amdgcn_raw_buffer_store_b128(v.hi, r, off + 16, 0, AUX);
    }
};

// One group tuple (T elements) through a buffer resource.
template <typename IO, int T, bool P2 = Pow2<T>::value> struct TupleLd {
    typedef typename Raw<T * (int)sizeof(IO)>::type type;
    __device__ static inline type load(rsrc_t r, uint32_t off) { return Raw<T * (int)sizeof(IO)>::load(r, off); }
};
template <typename IO, int T> struct TupleLd<IO, T, false> {
    typedef Elems<IO, T> type;
    __device__ static inline type load(rsrc_t r, uint32_t off) {
        type v;
#pragma unroll
        for (int t = 0; t < T; ++t) v.v[t] = Elem<IO>::load(r, off + (uint32_t)(t * sizeof(IO)));
        return v;
    }
};

// N dwords to a buffer at a 4-byte aligned offset: 16-byte accesses plus one
// of 12, 8 or 4 bytes.
template <int N, int AUX = 0>
__device__ inline void store_dwords(const unsigned int *w, rsrc_t r, uint32_t off) {
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[i], w[i + 1], w[i + 2], w[i + 3]}, r, off + 4u * i, 0, AUX);
    constexpr int I = N / 4 * 4;
    if constexpr (N - I == 3) {
        typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
        __builtin_amdgcn_raw_buffer_store_b96(u32x3{w[I], w[I + 1], w[I + 2]}, r, off + 4u * I, 0, AUX);
    } else if constexpr (N - I == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[I], w[I + 1]}, r, off + 4u * I, 0, AUX);
    } else if constexpr (N - I == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(w[I], r, off + 4u * I, 0, AUX);
    }
}

// Inverse group DFT of T fp32 planes (plus a bias b on every component, as
// T*b on the zero-frequency plane) stored as one tuple at byte offset off,
// for the orders without a vector type of their own (3, 5, 6, 7).
//   Tuples of whole dwords (T = 6 in fp16, every order in fp32): dword
//   accesses (one or two per tuple) when aligned4 (the buffer base is 4-byte
//   aligned; tuple offsets are multiples of the tuple size).
//   Odd T in fp16 (tuples of 2T bytes): with pairs, consecutive lanes hold
//   consecutive columns and every even lane's tuple starts 4-byte aligned
//   (an even column count and an aligned base); the even lane then stores
//   its tuple plus the first element of its odd neighbour's (fetched with a
//   quad permutation) as (T + 1) / 2 dwords, and the odd lane the rest of its
//   own as (T - 1) / 2 dwords from 2 bytes in: two accesses per pair of
//   tuples instead of 2T.  Every lane of the wave must take part (the
//   permutation reads the neighbour's register).
//   Otherwise one access per element.
template <typename IO, int T, int AUX = 0>
__device__ inline void store_tuple_inv(const float *f, float b, rsrc_t r, uint32_t off, bool aligned4, bool pairs,
                                       int lane) {
    constexpr int TB = T * (int)sizeof(IO);
    float g[T], y[T];
#pragma unroll
    for (int t = 0; t < T; ++t) g[t] = f[t];
    g[0] += (float)T * b;
    Dft<T>::inv(g, y);
    IO v[T];
#pragma unroll
    for (int t = 0; t < T; ++t) v[t] = (IO)y[t];
    if constexpr (TB % 4 == 0) {
        if (aligned4) {
            unsigned int w[TB / 4];
            __builtin_memcpy(w, v, TB);
            store_dwords<TB / 4, AUX>(w, r, off);
            return;
        }
    } else if constexpr (sizeof(IO) == 2) {
        if (pairs) {
            unsigned short h[T];
            __builtin_memcpy(h, v, TB);
            const unsigned int nb = (unsigned int)__builtin_amdgcn_mov_dpp((int)h[0], 0xF5, 0xF, 0xF, true);
            if ((lane & 1) == 0) {
                unsigned int w[(T + 1) / 2];
#pragma unroll
                for (int i = 0; i < (T + 1) / 2; ++i) {
                    const unsigned int lo = h[2 * i], hi = 2 * i + 1 < T ? h[2 * i + 1] : (nb & 0xFFFFu);
                    w[i] = lo | (hi << 16);
                }
                store_dwords<(T + 1) / 2, AUX>(w, r, off);
            } else {
                unsigned int w[(T - 1) / 2];
#pragma unroll
                for (int i = 0; i < (T - 1) / 2; ++i) w[i] = (unsigned int)h[2 * i + 1] | ((unsigned int)h[2 * i + 2] << 16);
                store_dwords<(T - 1) / 2, AUX>(w, r, off + 2u);
            }
            return;
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) Elem<IO>::template store<AUX>(v[t], r, off + (uint32_t)(t * sizeof(IO)));
}

// Group DFT of KL tuples (KL*T consecutive I/O values) into the T plane
// fragments of one k-run: F[p][j] = plane p of tuple j.
template <int T, typename IO> struct Frags {
    __device__ static inline void build(const IO *v, typename Mma<IO>::frag *F) {
        constexpr int KL = Mma<IO>::KL;
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            float x[T], f[T];
#pragma unroll
            for (int t = 0; t < T; ++t) x[t] = (float)v[j * T + t];
            Dft<T>::fwd(x, f);
#pragma unroll
            for (int p = 0; p < T; ++p) F[p][j] = (IO)f[p];
        }
    }
};

// p4 in fp16, written out for the VALU: per pair of tuples (a = x0|x1,
// b = x2|x3 of each tuple)
//   s02 = x0 + x2, s13 = x1 + x3   exact in fp32 (v_fma_mix_f32 reads the
//                                  halves directly)
//   f0 = s02 + s13, f3 = s02 - s13 rounded once to fp16 straight into the
//                                  low / high half of the plane register
//                                  (v_fma_mix{lo,hi}_f16)
//   (f1, f2) = (x0 - x2, x3 - x1)  one packed fp16 subtraction of exact
//                                  operands, i.e. the same single rounding
// then one byte permute per plane gathers the pair into a register.
__device__ inline void p4_pair(uint32_t a0, uint32_t b0, uint32_t a1, uint32_t b1, uint32_t &f0,
                               uint32_t &f1, uint32_t &f2, uint32_t &f3) {
    float s02a, s13a, s02b, s13b;
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,1]" : "=v"(s02a) : "v"(a0), "v"(b0));
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(s13a) : "v"(a0), "v"(b0));
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,1]" : "=v"(s02b) : "v"(a1), "v"(b1));
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(s13b) : "v"(a1), "v"(b1));
    uint32_t r0, r3, da, db;
    asm("v_fma_mixlo_f16 %0, %1, 1.0, %2" : "=v"(r0) : "v"(s02a), "v"(s13a));
    asm("v_fma_mixhi_f16 %0, %1, 1.0, %2" : "+v"(r0) : "v"(s02b), "v"(s13b));
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2" : "=v"(r3) : "v"(s13a), "v"(s02a));
    asm("v_fma_mixhi_f16 %0, %1, -1.0, %2" : "+v"(r3) : "v"(s13b), "v"(s02b));
    asm("v_pk_add_f16 %0, %1, %2 neg_lo:[0,1] neg_hi:[1,0]" : "=v"(da) : "v"(a0), "v"(b0));
    asm("v_pk_add_f16 %0, %1, %2 neg_lo:[0,1] neg_hi:[1,0]" : "=v"(db) : "v"(a1), "v"(b1));
    f0 = r0;
    f3 = r3;
    f1 = __builtin_amdgcn_perm(db, da, 0x05040100u);   // (da.lo, db.lo)
    f2 = __builtin_amdgcn_perm(db, da, 0x07060302u);   // (da.hi, db.hi)
}

template <> struct Frags<4, f16> {
    __device__ static inline void build(const f16 *v, f16x8 *F) {
        uint32_t w[16];   // 2 words per tuple (a copy: no type punning through pointers)
        __builtin_memcpy(w, v, sizeof(w));
        uint32_t P[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            p4_pair(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3], P[0][q], P[1][q], P[2][q],
                    P[3][q]);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            F[p] = __builtin_bit_cast(f16x8, u32x4{P[p][0], P[p][1], P[p][2], P[p][3]});
    }
};

template <int T, typename IO>
__device__ inline void tuples_to_frags(const IO *v, typename Mma<IO>::frag *F) {
    Frags<T, IO>::build(v, F);
}

// Raw loaded tuples -> I/O values.  A copy, not a pointer cast: reading a
// scalar raw type (the 4-byte tuples of T = 2 in fp16) through an IO pointer
// is type punning that the optimizer may assume never aliases.  The copy
// stays in registers.
template <typename IO, typename R, int N>
__device__ inline void raw_to_io(const R (&r)[N], IO *v) {
    __builtin_memcpy(v, r, sizeof(r));
}

// Inverse group DFT of one output's T fp32 planes, rounded to the I/O type.
// b: a value added to every group component (the bias); adding T*b to the
// zero-frequency plane before the inverse transform does exactly that.
template <int T, typename IO> struct Out {
    typedef typename Tuple<IO, T>::type tup;
    __device__ static inline tup build(const float *f, float b) {
        float g[T], y[T];
#pragma unroll
        for (int t = 0; t < T; ++t) g[t] = f[t];
        g[0] += (float)T * b;
        Dft<T>::inv(g, y);
        tup o;
#pragma unroll
        for (int t = 0; t < T; ++t) o[t] = (IO)y[t];
        return o;
    }
};

// p4 in fp16 ([pchao] App. 6.2 eq. (21)): u = (f0 + f3) / 4 + b, v = (f0 - f3) / 4 + b,
// y0 = u + f1/2, y2 = u - f1/2, y1 = v - f2/2, y3 = v + f2/2, each output
// one fused multiply-add rounded once to fp16 into its half register.
template <> struct Out<4, f16> {
    typedef Tuple<f16, 4>::type tup;
    __device__ static inline tup build(const float *f, float b) {
        const float u = __builtin_fmaf(0.25f, f[0] + f[3], b), v = __builtin_fmaf(0.25f, f[0] - f[3], b);
        uint32_t lo, hi;
        asm("v_fma_mixlo_f16 %0, 0.5, %1, %2" : "=v"(lo) : "v"(f[1]), "v"(u));
        asm("v_fma_mixhi_f16 %0, -0.5, %1, %2" : "+v"(lo) : "v"(f[2]), "v"(v));
        asm("v_fma_mixlo_f16 %0, -0.5, %1, %2" : "=v"(hi) : "v"(f[1]), "v"(u));
        asm("v_fma_mixhi_f16 %0, 0.5, %1, %2" : "+v"(hi) : "v"(f[2]), "v"(v));
        return __builtin_bit_cast(tup, u32x2{lo, hi});
    }
};

// Per-frequency products of one (row block, column block, k slice).
//   a: T plane fragments of A; na: the negated copies (Im planes for plain
//   products, Re planes for conjugate products); b: T plane fragments of B.
// FIRST: the accumulators start from these products (no prior sum).
// ---------------------------------------------------------------------------
// The octic group (quarter turns r and reflections s; [paperpeel] App. A.2:
// the regular representation splits into four one-dimensional irreducible
// representations and two copies of a two-dimensional one of real type).
// Group component u = a + 4 b of a tuple stands for r^a s^b.  The real group
// Fourier transform of a tuple v is
//     f_chi = sum_u v_u chi(u)     for chi = A1, A2, B1, B2 (r -> 1,1,-1,-1;
//                                  s -> 1,-1,1,-1)
//     F_E   = sum_u v_u E(u)       E(r) = [[0,-1],[1,0]], E(s) = [[1,0],[0,-1]]
// stored as eight planes A1, A2, B1, B2, E11, E12, E21, E22.  The layer is a
// product per representation: Yhat(rho) = Xhat(rho) What(rho), summed over
// channels (the group convolution Y[g] = sum_h Wt[h^-1 g] X[h]); the inverse
// is v_g = (1/8) (sum_chi chi(g) f_chi + 2 sum_ik E(g)_ik F_E,ik).
// GRP selects the group of a kernel: 0 the cyclic group of order T, 1 the
// octic group (T = 8 components per tuple).
// ---------------------------------------------------------------------------
struct Octic {
    __device__ static inline void fwd(const float *x, float *f) {
        const float rp = (x[0] + x[2]) + (x[1] + x[3]), rm = (x[4] + x[6]) + (x[5] + x[7]);
        const float ap = (x[0] + x[2]) - (x[1] + x[3]), am = (x[4] + x[6]) - (x[5] + x[7]);
        f[0] = rp + rm;                          // A1
        f[1] = rp - rm;                          // A2
        f[2] = ap + am;                          // B1
        f[3] = ap - am;                          // B2
        f[4] = (x[0] - x[2]) + (x[4] - x[6]);    // E11
        f[5] = (x[3] - x[1]) + (x[5] - x[7]);    // E12
        f[6] = (x[1] - x[3]) + (x[5] - x[7]);    // E21
        f[7] = (x[0] - x[2]) - (x[4] - x[6]);    // E22
    }
    __device__ static inline void inv(const float *f, float *y) {
        const float pq = f[0] + f[1], pmq = f[0] - f[1];
        const float uv = f[2] + f[3], umv = f[2] - f[3];
        const float ed = 2.0f * (f[4] + f[7]), es = 2.0f * (f[6] - f[5]);
        const float fd = 2.0f * (f[4] - f[7]), fs = 2.0f * (f[5] + f[6]);
        y[0] = 0.125f * ((pq + uv) + ed);
        y[1] = 0.125f * ((pq - uv) + es);
        y[2] = 0.125f * ((pq + uv) - ed);
        y[3] = 0.125f * ((pq - uv) - es);
        y[4] = 0.125f * ((pmq + umv) + fd);
        y[5] = 0.125f * ((pmq - umv) + fs);
        y[6] = 0.125f * ((pmq + umv) - fd);
        y[7] = 0.125f * ((pmq - umv) - fs);
    }
};
template <int T, int GRP> struct GrpT {
    __device__ static inline void fwd(const float *x, float *f) { Dft<T>::fwd(x, f); }
    __device__ static inline void inv(const float *f, float *y) { Dft<T>::inv(f, y); }
};
template <> struct GrpT<8, 1> {
    __device__ static inline void fwd(const float *x, float *f) { Octic::fwd(x, f); }
    __device__ static inline void inv(const float *f, float *y) { Octic::inv(f, y); }
};
// Output tuple of the T planes f plus a bias b on every component (T*b on
// the plane of the trivial representation), for either group.
template <int T, typename IO, int GRP>
__device__ inline typename Tuple<IO, T>::type grp_out(const float *f, float b) {
    if constexpr (GRP == 0) {
        return Out<T, IO>::build(f, b);
    } else {
        float g[T], y[T];
#pragma unroll
        for (int t = 0; t < T; ++t) g[t] = f[t];
        g[0] += (float)T * b;
        GrpT<T, GRP>::inv(g, y);
        typename Tuple<IO, T>::type o;
#pragma unroll
        for (int t = 0; t < T; ++t) o[t] = (IO)y[t];
        return o;
    }
}
// Group transform of KL tuples into T plane fragments, for either group.
template <int T, typename IO, int GRP>
__device__ inline void grp_frags(const IO *v, typename Mma<IO>::frag *F) {
    if constexpr (GRP == 0) {
        tuples_to_frags<T, IO>(v, F);
    } else {
        constexpr int KL = Mma<IO>::KL;
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            float x[T], f[T];
#pragma unroll
            for (int t = 0; t < T; ++t) x[t] = (float)v[j * T + t];
            GrpT<T, GRP>::fwd(x, f);
#pragma unroll
            for (int p = 0; p < T; ++p) F[p][j] = (IO)f[p];
        }
    }
}
// Octic products of one k slice for the row kernels: Yhat = Xhat What per
// representation (the input gradient uses the same table with the E blocks
// of its spectrum part stored transposed, giving dYhat What^T).
template <class MM, bool FIRST = false>
__device__ inline void oct_mma_row(typename MM::acc_t *acc, const typename MM::frag *a,
                                   const typename MM::frag *b) {
    typedef typename MM::acc_t acc_t;
    const acc_t z = {};
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[p] = MM::mma(a[p], b[p], FIRST ? z : acc[p]);
    acc[4] = MM::mma(a[5], b[6], MM::mma(a[4], b[4], FIRST ? z : acc[4]));   // x11 w11 + x12 w21
    acc[5] = MM::mma(a[5], b[7], MM::mma(a[4], b[5], FIRST ? z : acc[5]));   // x11 w12 + x12 w22
    acc[6] = MM::mma(a[7], b[6], MM::mma(a[6], b[4], FIRST ? z : acc[6]));   // x21 w11 + x22 w21
    acc[7] = MM::mma(a[7], b[7], MM::mma(a[6], b[5], FIRST ? z : acc[7]));   // x21 w12 + x22 w22
}
// Octic products of the weight gradient, dWhat_dc = Xhat_c^T dYhat_d per
// representation.  Rows d, columns c (A = dYhat, B = Xhat), or with SWAP rows
// c, columns d (A = Xhat, B = dYhat); either way the planes come out as dWhat.
template <class MM, bool SWAP>
__device__ inline void oct_mma_dw(typename MM::acc_t *acc, const typename MM::frag *a,
                                  const typename MM::frag *b) {
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[p] = MM::mma(a[p], b[p], acc[p]);
    acc[4] = MM::mma(a[6], b[6], MM::mma(a[4], b[4], acc[4]));
    acc[7] = MM::mma(a[7], b[7], MM::mma(a[5], b[5], acc[7]));
    if constexpr (SWAP) {   // dw_ik = sum_m x_mi y_mk with x = A, y = B
        acc[5] = MM::mma(a[6], b[7], MM::mma(a[4], b[5], acc[5]));
        acc[6] = MM::mma(a[7], b[6], MM::mma(a[5], b[4], acc[6]));
    } else {                // x = B, y = A
        acc[5] = MM::mma(a[7], b[6], MM::mma(a[5], b[4], acc[5]));
        acc[6] = MM::mma(a[6], b[7], MM::mma(a[4], b[5], acc[6]));
    }
}

template <int T, class MM, bool CONJ, bool FIRST = false>
__device__ inline void freq_mma(typename MM::acc_t *acc, const typename MM::frag *a,
                                const typename MM::frag *na, const typename MM::frag *b) {
    typedef typename MM::acc_t acc_t;
    const acc_t z = {};
    acc[0] = MM::mma(a[0], b[0], FIRST ? z : acc[0]);
    if (T % 2 == 0) acc[T - 1] = MM::mma(a[T - 1], b[T - 1], FIRST ? z : acc[T - 1]);   // Nyquist
#pragma unroll
    for (int k = 1; k <= (T - 1) / 2; ++k) {
        const int re = 2 * k - 1, im = 2 * k;
        acc[re] = MM::mma(a[re], b[re], FIRST ? z : acc[re]);
        if (!CONJ) {
            acc[re] = MM::mma(na[k - 1], b[im], acc[re]);   // - a_i b_i
            acc[im] = MM::mma(a[re], b[im], FIRST ? z : acc[im]);
            acc[im] = MM::mma(a[im], b[re], acc[im]);
        } else {
            acc[re] = MM::mma(a[im], b[im], acc[re]);
            acc[im] = MM::mma(a[im], b[re], FIRST ? z : acc[im]);
            acc[im] = MM::mma(na[k - 1], b[im], acc[im]);   // - a_r b_i
        }
    }
}

template <int T, class MM, bool CONJ>
__device__ inline void make_neg(const typename MM::frag *a, typename MM::frag *na) {
#pragma unroll
    for (int k = 1; k <= (T - 1) / 2; ++k) na[k - 1] = MM::neg(a[CONJ ? 2 * k - 1 : 2 * k]);
}

// ---------------------------------------------------------------------------
// Gauss's three-multiplication complex products.  For each
// complex frequency 0 < k < T/2 the product of a = a_r + i a_i (activation
// side) and b = b_r + i b_i (weight side) is formed from three real
// products instead of four:
//     K1 = (a_r + a_i) b_r,   K2 = a_r (b_i - b_r),   K3 = a_i (b_r + b_i),
//     Re(ab) = K1 - K3,       Im(ab) = K1 + K2,
// the complex products of [pchao] §3.2.1 eq. (5) and App. 6.2 eq. (20)
// rearranged.  The weight-side sums live in the cached spectrum (computed
// once per weight, in fp32 and rounded once), the activation-side sum is one
// more plane of the group DFT, and every product becomes diagonal: plane p
// of A times plane p of B into accumulator p, with no negated copies.  The
// input gradient's conjugate products use b_i -> -b_i in the stored planes.
// Plane order (TP = T + (T - 1) / 2 planes):
//     0                       real plane k = 0
//     3k - 2, 3k - 1, 3k      the three products of frequency k
//     TP - 1                  real plane k = T/2 (even T)
// Chosen per (order, dtype) at compile time (Gauss<T, IO>), by measurement
// on MI355X (row kernels, forward / input gradient, us, 4M -> 3M):
//   fp32  order 4 (N=12608, 384 -> 1152)   60.4 -> 54.1 / 70.6 -> 63.4
//         order 6 (N=12608, 768 -> 3072)  184.2 -> 178.0 / 199.7 -> 170.8
//         order 8 (N=16384, 1024 -> 4096) 319.6 -> 295.4 / 301.0 -> 265.9
//   fp16  slower at every order (ViT-B fc1 41.5 -> 155.0): the extra
//         accumulator planes push the fp16 tiles past the register file.
// The weight gradient uses them too (dw_frags3 below): there both operands
// are transformed on the fly, so each side forms its own sums.
// ---------------------------------------------------------------------------
template <int T, typename IO> struct Gauss { static constexpr bool V = false; };
template <> struct Gauss<4, float> { static constexpr bool V = true; };
template <> struct Gauss<6, float> { static constexpr bool V = true; };
template <> struct Gauss<8, float> { static constexpr bool V = true; };
// Planes multiplied (accumulators, activation fragments) ...
template <int T, typename IO> constexpr int math_planes() { return Gauss<T, IO>::V ? T + (T - 1) / 2 : T; }
// ... and planes stored per (column, k) in the cached spectrum: order 8 pads
// its 11 to 12 (a zero plane, never multiplied) so that a row-kernel stage of
// one 64-column tile is a whole number of 256-thread copy rounds.
template <int T, typename IO> constexpr int stored_planes() {
    return Gauss<T, IO>::V && T == 8 ? math_planes<T, IO>() + 1 : math_planes<T, IO>();
}

// Activation-side planes g[TP] from the T group-DFT planes f.
template <int T> __device__ inline void gauss_a(const float *f, float *g) {
    constexpr int H = (T - 1) / 2;
    g[0] = f[0];
#pragma unroll
    for (int k = 1; k <= H; ++k) {
        g[3 * k - 2] = f[2 * k - 1] + f[2 * k];
        g[3 * k - 1] = f[2 * k - 1];
        g[3 * k] = f[2 * k];
    }
    if (T % 2 == 0) g[T + H - 1] = f[T - 1];
}
// Weight-side planes g[TP] from the T planes f of What; conj: the planes of
// conj(What) (input gradient).
template <int T> __device__ inline void gauss_b(const float *f, float *g, bool conj) {
    constexpr int H = (T - 1) / 2;
    g[0] = f[0];
#pragma unroll
    for (int k = 1; k <= H; ++k) {
        const float re = f[2 * k - 1], im = conj ? -f[2 * k] : f[2 * k];
        g[3 * k - 2] = re;
        g[3 * k - 1] = im - re;
        g[3 * k] = re + im;
    }
    if (T % 2 == 0) g[T + H - 1] = f[T - 1];
}
// The T planes f of the product from the TP accumulators g.
template <int T> __device__ inline void gauss_out(const float *g, float *f) {
    constexpr int H = (T - 1) / 2;
    f[0] = g[0];
#pragma unroll
    for (int k = 1; k <= H; ++k) {
        f[2 * k - 1] = g[3 * k - 2] - g[3 * k];
        f[2 * k] = g[3 * k - 2] + g[3 * k - 1];
    }
    if (T % 2 == 0) f[T - 1] = g[T + H - 1];
}
// Group DFT of KL tuples into the TP activation-side plane fragments.
template <int T, typename IO>
__device__ inline void tuples_to_frags3(const IO *v, typename Mma<IO>::frag *F) {
    constexpr int KL = Mma<IO>::KL, TP = T + (T - 1) / 2;
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        float x[T], f[T], g[TP];
#pragma unroll
        for (int t = 0; t < T; ++t) x[t] = (float)v[j * T + t];
        Dft<T>::fwd(x, f);
        gauss_a<T>(f, g);
#pragma unroll
        for (int p = 0; p < TP; ++p) F[p][j] = (IO)g[p];
    }
}

// Row-kernel products of one k slice: 4M (freq_mma) or, with G3, the
// diagonal three-multiplication products over the TP stored planes.
template <int T, class MM, bool CONJ, bool G3, bool FIRST = false>
__device__ inline void plane_mma(typename MM::acc_t *acc, const typename MM::frag *a,
                                 const typename MM::frag *na, const typename MM::frag *b) {
    if constexpr (G3) {
        typedef typename MM::acc_t acc_t;
        const acc_t z = {};
#pragma unroll
        for (int p = 0; p < T + (T - 1) / 2; ++p) acc[p] = MM::mma(a[p], b[p], FIRST ? z : acc[p]);
    } else {
        freq_mma<T, MM, CONJ, FIRST>(acc, a, na, b);
    }
}
// Activation fragments of one k-run: T planes (+ negated copies) or TP planes.
template <int T, typename IO, class MM, bool CONJ, bool G3>
__device__ inline void act_frags(const IO *io, typename MM::frag *a, typename MM::frag *na) {
    if constexpr (G3) {
        tuples_to_frags3<T, IO>(io, a);
    } else {
        tuples_to_frags<T, IO>(io, a);
        make_neg<T, MM, CONJ>(a, na);
    }
}

// Row-kernel activation fragments and products for either group.
template <int T, typename IO, class MM, bool CONJ, bool G3, int GRP>
__device__ inline void act_frags_g(const IO *io, typename MM::frag *a, typename MM::frag *na) {
    if constexpr (GRP == 0) act_frags<T, IO, MM, CONJ, G3>(io, a, na);
    else grp_frags<T, IO, GRP>(io, a);
}
template <int T, class MM, bool CONJ, bool G3, int GRP, bool FIRST = false>
__device__ inline void plane_mma_g(typename MM::acc_t *acc, const typename MM::frag *a,
                                   const typename MM::frag *na, const typename MM::frag *b) {
    if constexpr (GRP == 0) plane_mma<T, MM, CONJ, G3, FIRST>(acc, a, na, b);
    else oct_mma_row<MM, FIRST>(acc, a, b);
}

// Weight-gradient operand planes with Gauss's products: the row operand a
// takes the activation-side planes of gauss_a, the column operand b the
// weight-side planes of conj(b) (gauss_b), so that the diagonal plane
// products summed over n give a * conj(b) through gauss_out.
template <int T, typename IO, bool COL>
__device__ inline void dw_frags3(const IO *v, typename Mma<IO>::frag *F) {
    constexpr int KL = Mma<IO>::KL, TP = T + (T - 1) / 2;
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        float x[T], f[T], g[TP];
#pragma unroll
        for (int t = 0; t < T; ++t) x[t] = (float)v[j * T + t];
        Dft<T>::fwd(x, f);
        if constexpr (COL) gauss_b<T>(f, g, true);
        else gauss_a<T>(f, g);
#pragma unroll
        for (int p = 0; p < TP; ++p) F[p][j] = (IO)g[p];
    }
}
// Operand planes of one weight-gradient staging unit: T group-DFT planes, or
// with Gauss's products the TP planes above.
template <int T, typename IO, bool COL>
__device__ inline void dw_frags(const IO *v, typename Mma<IO>::frag *F) {
    if constexpr (Gauss<T, IO>::V) dw_frags3<T, IO, COL>(v, F);
    else tuples_to_frags<T, IO>(v, F);
}

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

// LDS slot swizzle for tiles stored as rows of KCH 16-byte chunks: chunk g of
// row r lives in physical chunk g ^ swz(r), so that the 16 lanes reading one
// chunk of 16 consecutive rows hit 16 distinct 16-byte bank groups.  With G
// the largest power of two dividing KCH (at most 16), rows r and r + 16/G
// start in the same bank group of a 256-byte line; XOR-ing the chunk with
// (r / (16/G)) % G (< G, so the chunk stays inside the row) separates them
// (G = pow2_part16(KCH)).
template <int KCH> __device__ constexpr int swz(int r) {
    return (r / (16 / pow2_part16(KCH))) % pow2_part16(KCH);
}

// ===========================================================================
// Row kernel: out[m, col, :] = IDFT_k( sum_k' A_k[m, k'] op B_k[k', col] ).
//   act  [M][K][T]      rows of X (forward) or dY (input gradient)
//   bpl  weight planes in the blocked spectrum layout [NC/32][K/KC][T][32][KC]
//        (part 0 of the spectrum for the forward: columns d, k = c; part 1
//        for the input gradient: columns c, k = d), so that one stage of one
//        32-column block is T*32*KC contiguous elements
//   out  [M][NC][T]
//   CONJ: use conj(B) (input gradient).
// Tile: BM = WM*32 rows x BN = WN*CB*32 columns; wave (wm, wn) owns rows
// wm*32.. and CB 32-column blocks.  One stage is KS MFMA k slices of KC = 2*KL
// k values each.  The stages stream through an NS-deep LDS ring filled by the
// buffer unit directly (HBM -> LDS, no VGPRs): per stage the raw activation
// tuples of the tile's rows and the weight-plane blocks of its columns.
// Every wave then reads its own rows' raw tuples from LDS, runs the group DFT
// into MFMA fragments, and multiplies them with the weight fragments.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that the 16 lanes of one
// ds_read_b128 phase hit 16 distinct bank groups):
//   A: row r of the tile, chunk q of its stage segment -> slot r*RCH + (q ^ swz(r))
//   B: column block jb, k slice s, plane p, column c, k-run h
//                                  -> slot ACH + (jb*KS + s)*64*T + (p*32 + c)*2 + (h ^ swz<2>(c))
// ===========================================================================
// Workgroup barrier that waits for this wave's LDS reads but not for its
// buffer->LDS copies.  __syncthreads() also orders global memory, which makes
// every outstanding copy finish before the barrier and so caps the copy
// pipeline at one stage.  The ring loop below instead waits for exactly the
// copies it needs (s_waitcnt vmcnt) and then meets here; the "memory"
// clobber keeps the compiler from moving LDS accesses across the barrier.
__device__ inline void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt immediate for "vmcnt <= v" (gfx9 encoding, other counters free).
__device__ constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

// One stage of buffer->LDS copies for one thread: LPS 16-byte chunks, the
// first ACH chunks of a stage from the activation resource, the rest from the
// weight resource.  Stage offsets (st_a / st_b) are wave-uniform and go in the
// scalar offset; only a tail stage (full == false) checks each chunk's k.
template <int LPS, int NW, int ACH>
__device__ inline void dma_stage(rsrc_t ra, rsrc_t rb, u32x4 *dst, const uint32_t *l_off,
                                 const int *l_kk, int wave, uint32_t st_a, uint32_t st_b, bool full,
                                 int k0, int K, int KP) {
    if (full) {
#pragma unroll
        for (int li = 0; li < LPS; ++li) {
            const bool isA = (li * NW + wave) * 64 < ACH;   // wave-uniform
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                isA ? ra : rb, (__attribute__((address_space(3))) void *)&dst[(li * NW + wave) * 64], 16,
                l_off[li], isA ? st_a : st_b, 0, 0);
        }
    } else {
#pragma unroll
        for (int li = 0; li < LPS; ++li) {
            const bool isA = (li * NW + wave) * 64 < ACH;
            const uint32_t off = k0 + l_kk[li] >= (isA ? K : KP) ? OOB : l_off[li];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                isA ? ra : rb, (__attribute__((address_space(3))) void *)&dst[(li * NW + wave) * 64], 16,
                off, isA ? st_a : st_b, 0, 0);
        }
    }
}

// One stage of copies for layers whose activation rows are not a whole
// number of 16-byte chunks (K * T * sizeof(IO) not a multiple of 16): the
// weight chunks still go HBM -> LDS by the buffer unit, the activation chunks
// go through registers in pieces of `gran` bytes (the largest power of two
// dividing the row length, at most 8, so a piece never straddles two rows) and
// are written to the same LDS slots.  A piece at or past the row end
// (rowbytes) reads as zero.  l_qb: the chunk's byte offset within its row's
// stage segment.  The weight copies are issued first and the stage ends with
// every copy of this thread complete, so the ring's vmcnt waits hold.
template <typename IO, int LPS, int NW, int ACH>
__device__ inline void el_stage(rsrc_t ra, rsrc_t rb, u32x4 *dst, const uint32_t *l_off, const uint32_t *l_qb,
                                const int *l_kk, int wave, int lane, uint32_t st_a, uint32_t st_b, bool full,
                                int k0, int KP, uint32_t rowbytes, int gran) {
#pragma unroll
    for (int li = 0; li < LPS; ++li) {
        if ((li * NW + wave) * 64 < ACH) continue;
        const uint32_t off = full || k0 + l_kk[li] < KP ? l_off[li] : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void *)&dst[(li * NW + wave) * 64],
                                                 16, off, st_b, 0, 0);
    }
    u32x4 v[LPS];
#pragma unroll
    for (int li = 0; li < LPS; ++li) {
        if ((li * NW + wave) * 64 >= ACH) continue;
        const uint32_t off = l_off[li] + st_a, pos = st_a + l_qb[li];
        uint32_t w[4];
        if (gran == 8) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const u32x2 t = Raw<8>::load(ra, pos + 8 * i < rowbytes ? off + 8 * i : OOB);
                w[2 * i] = t[0];
                w[2 * i + 1] = t[1];
            }
        } else if (gran == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = Raw<4>::load(ra, pos + 4 * i < rowbytes ? off + 4 * i : OOB);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(ra, pos + 4 * i < rowbytes ? off + 4 * i : OOB, 0, 0);
                const uint32_t hi =
                    __builtin_amdgcn_raw_buffer_load_b16(ra, pos + 4 * i + 2 < rowbytes ? off + 4 * i + 2 : OOB, 0, 0);
                w[i] = (lo & 0xffffu) | (hi << 16);
            }
        }
        v[li] = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int li = 0; li < LPS; ++li)
        if ((li * NW + wave) * 64 < ACH) dst[(li * NW + wave) * 64 + lane] = v[li];
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

template <int T, typename IO, bool CONJ, int WM, int WN, int CB, int KS, int NS, int OCC, bool PIPE, bool EL,
          int GRP = 0>
__global__ __launch_bounds__(WM *WN * 64, OCC) void row_kernel(const IO *__restrict__ act,
                                                               const IO *__restrict__ bpl,
                                                               IO *__restrict__ out, int M, int K,
                                                               int NC, uint32_t bpl_bytes,
                                                               const IO *__restrict__ bias, int nbig,
                                                               int gran) {
    typedef M32<IO> MM;
    typedef typename MM::frag frag;
    typedef typename MM::acc_t acc_t;
    constexpr int ES = sizeof(IO), KL = MM::KL, KC = 2 * KL, TB = T * ES;
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int BM = WM * 32, BN = WN * CB * 32;
    constexpr int KSTG = KS * KC;          // k per stage
    constexpr int LCH = KL * TB / 16;      // chunks of one lane's k-run in one slice
    constexpr int RCH = KS * 2 * LCH;      // chunks of one activation row per stage
    constexpr int ACH = BM * RCH;          // activation chunks per stage
    constexpr bool G3 = Gauss<T, IO>::V && GRP == 0;   // three-multiplication products
    constexpr int TP = GRP ? T : math_planes<T, IO>();     // planes multiplied
    constexpr int TPS = GRP ? T : stored_planes<T, IO>();  // weight planes stored per (column, k)
    constexpr int BCH = TPS * BN * 2 * KS; // weight chunks per stage
    constexpr int SCH = ACH + BCH;
    constexpr int LPS = SCH / NT;          // buffer->LDS loads per thread per stage
    constexpr int NNEG = (T - 1) / 2 > 0 ? (T - 1) / 2 : 1;
    static_assert(ACH % 64 == 0 && BCH % 64 == 0 && SCH % NT == 0, "tile shape");
    static_assert(KL * ES == 16, "one fragment is one 16-byte chunk");
    static_assert((NS - 1) * LPS < 64 && NS >= 2, "vmcnt range");

    __shared__ __attribute__((aligned(16))) u32x4 ring[NS][SCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 31, lh = lane >> 5;

    // Column space in half-width units of BN/2 columns: hn per row block,
    // paired into fpr = hn/2 whole BN-wide tiles ("pairs", npairs in all),
    // plus one odd half unit per row block when hn is odd.  Workgroups
    // [0, nbig) take pairs 0 .. nbig-1 as whole tiles.  The workgroups after
    // them take single half units, each wave owning CB/2 column blocks: first
    // both halves of every remaining pair (so that the last, partial round of
    // resident workgroups holds twice as many workgroups of half the work),
    // then the odd units (no MFMA work on columns past the end).  When no
    // pair is split and hn is odd, the order is row-block major instead.
    // Without halves (CB odd), nbig is the grid and tiles are whole.
    constexpr bool CAN_HALF = CB % 2 == 0;
    const int rblocks = (M + BM - 1) / BM;
    bool half = false;
    int m0 = 0, n0 = 0;
    if constexpr (CAN_HALF) {
        const int hn = (NC + BN / 2 - 1) / (BN / 2), fpr = hn / 2;
        const int npairs = rblocks * fpr;
        half = (int)blockIdx.x >= nbig;
        if (nbig == npairs && (hn & 1)) {
            // No split, one odd unit per row block: the grid is row-block
            // major (fpr pairs, then the odd unit), so that each row block's
            // workgroups are consecutive and share an XCD (and its L2).
            const int it = xcd_tile(blockIdx.x, gridDim.x);
            const int r = it / (fpr + 1), w = it % (fpr + 1);
            m0 = r * BM;
            half = w == fpr;
            n0 = w * BN;
        } else if (!half) {
            const int pr = xcd_tile(blockIdx.x, nbig);
            m0 = (pr / fpr) * BM;
            n0 = (pr % fpr) * BN;
        } else {
            const int sg = xcd_tile(blockIdx.x - nbig, gridDim.x - nbig);   // halves of a pair share an XCD
            const int nsplit = 2 * (npairs - nbig);
            if (sg < nsplit) {
                const int pr = nbig + (sg >> 1);
                m0 = (pr / fpr) * BM;
                n0 = (pr % fpr) * BN + (sg & 1) * (BN / 2);
            } else {
                m0 = (sg - nsplit) * BM;
                n0 = fpr * BN;
            }
        }
    } else {
        const int tiles_n = (NC + BN - 1) / BN;
        const int tile = xcd_tile(blockIdx.x, gridDim.x);
        m0 = (tile / tiles_n) * BM;
        n0 = (tile % tiles_n) * BN;
    }
    const int rows = min(BM, M - m0);
    const int nks = (K + KC - 1) / KC;     // k slices (k blocks of the spectrum part)
    const int nst = (K + KSTG - 1) / KSTG;
    const int KP = nks * KC;               // K padded to whole slices (B validity)

    const rsrc_t ra = make_rsrc(act + (size_t)m0 * K * T, (uint32_t)rows * K * TB);
    const rsrc_t rb = make_rsrc(bpl, bpl_bytes);
    const int nbk = (NC + 31) / 32;      // column blocks of the spectrum part
    const rsrc_t ro = make_rsrc(out + (size_t)m0 * NC * T, (uint32_t)rows * NC * TB);
    // tuple stores of orders 3, 5, 6, 7 (store_tuple_inv): dword accesses
    // need a 4-byte aligned row base, lane pairs also an even column count
    [[maybe_unused]] const bool aligned4 = ((uintptr_t)(out + (size_t)m0 * NC * T) & 3u) == 0;
    [[maybe_unused]] const bool pairs = aligned4 && NC % 2 == 0;

    // ---- per-thread load slots ----
    // l_off: the lane's chunk offset for stage 0 (OOB for a column block past
    // the spectrum part); a stage adds a wave-uniform offset (st_a / st_b)
    // that goes into the instruction's scalar offset.  l_kk: index of the
    // chunk's first k within the stage, checked only in the tail stage.
    uint32_t l_off[LPS], l_qb[LPS];
    int l_kk[LPS];
    // A chunk index is (li * NW + wave) * 64 + lane: a wave-uniform multiple
    // of 64 plus the lane.  When a row's chunk count RCH divides 16 (orders
    // 2, 4, 8), every block size below divides or is a multiple of 64, so
    // each index splits into a uniform part (scalar arithmetic) and a lane
    // part computed once; otherwise (RCH = 2*KS*T for orders 3, 5, 6, 7) the
    // activation slots take the row and chunk from the whole index.
    constexpr bool ASPLIT = RCH <= 16 && 16 % RCH == 0;
    const uint32_t lane_a_row = ASPLIT ? (uint32_t)(lane / RCH) * K * TB : 0u;   // row within 64 chunks
    const int lane_b = ((lane / 2) * KC + ((lane % 2) ^ swz<2>(lane / 2)) * KL) * ES;
#pragma unroll
    for (int li = 0; li < LPS; ++li) {
        const int u = (li * NW + wave) * 64;   // wave-uniform
        if (u < ACH && ASPLIT) {
            // row r = u / RCH + lane / RCH, chunk q = lane % RCH, swizzled by
            // swz(r) = (r / (16 / RCH)) % RCH = (u / 16 + lane / 16) % RCH
            const int q = (lane % RCH) ^ ((u / 16 + lane / 16) % RCH);
            l_off[li] = (uint32_t)(u / RCH) * K * TB + lane_a_row + q * 16;
            l_kk[li] = q * 16 / TB;
            l_qb[li] = q * 16;
        } else if (u < ACH) {
            // slot u + lane holds chunk q of row r; a lane's k-run of KL
            // tuples is LCH whole chunks, so q * 16 / TB lies in the run of
            // the chunk's first byte and the tail check stays per run
            const int r = (u + lane) / RCH, q = ((u + lane) % RCH) ^ swz<RCH>(r);
            l_off[li] = (uint32_t)r * K * TB + q * 16;
            l_kk[li] = q * 16 / TB;
            l_qb[li] = q * 16;
        } else {
            // column block jb, k slice sl and plane p are uniform; column
            // lane / 2 and k-run half (lane % 2) come from the lane
            const int sb = u - ACH;
            const int jb = sb / (64 * TPS * KS), g = sb % (64 * TPS * KS);
            const int sl = g / (64 * TPS), p = (g % (64 * TPS)) / 64;
            const int cb = n0 / 32 + jb;
            const bool used = cb < nbk && (!half || jb < WN * CB / 2);
            const uint32_t base =
                used ? (uint32_t)(((cb * nks + sl) * TPS * 32 * KC + p * 32 * KC) * ES) : OOB;
            l_off[li] = base + lane_b;   // OOB + lane_b stays past the buffer
            l_kk[li] = sl * KC;
            l_qb[li] = 0;
        }
    }

    auto issue = [&](int st) {
        if (st >= nst) return;
        const int k0 = st * KSTG;
        if constexpr (EL)
            el_stage<IO, LPS, NW, ACH>(ra, rb, ring[st % NS], l_off, l_qb, l_kk, wave, lane, (uint32_t)k0 * TB,
                                       (uint32_t)st * KS * TPS * 32 * KC * ES, k0 + KSTG <= K, k0, KP,
                                       (uint32_t)K * TB, gran);
        else
            dma_stage<LPS, NW, ACH>(ra, rb, ring[st % NS], l_off, l_kk, wave, (uint32_t)k0 * TB,
                                    (uint32_t)st * KS * TPS * 32 * KC * ES, k0 + KSTG <= K, k0, K, KP);
    };

    const int arow = wm * 32 + lr;
    // The main loop and epilogue for CBE column blocks per wave (CB for a
    // whole tile, CB / 2 for a half tile).
    auto run = [&](auto cbe_tag) {
        constexpr int CBE = decltype(cbe_tag)::value;
        acc_t acc[CBE][TP];
        // Fragments of the stage being multiplied; the next stage's fragments are
        // read from LDS and transformed while these products run on the matrix
        // cores (the MFMAs are issued first and only read registers).
        frag aF[KS][TP], aN[KS][NNEG], bF[KS][CBE][TP];
        auto load_frags = [&](const u32x4 *buf) {
#pragma unroll
            for (int sl = 0; sl < KS; ++sl) {
                // A: this lane's k-run of raw tuples -> group DFT -> plane fragments
                u32x4 rawA[LCH];
#pragma unroll
                for (int c = 0; c < LCH; ++c)
                    rawA[c] = buf[arow * RCH + (((sl * 2 + lh) * LCH + c) ^ swz<RCH>(arow))];
                IO io[KL * T];
                raw_to_io(rawA, io);
                act_frags_g<T, IO, MM, CONJ, G3, GRP>(io, aF[sl], aN[sl]);
#pragma unroll
                for (int j = 0; j < CBE; ++j)
#pragma unroll
                    for (int p = 0; p < TP; ++p)
                        bF[sl][j][p] = __builtin_bit_cast(
                            frag, buf[ACH + ((wn * CBE + j) * KS + sl) * 64 * TPS + (p * 32 + lr) * 2 +
                                      (lh ^ swz<2>(lr))]);
            }
        };
        auto mma_stage = [&](bool first) {
#pragma unroll
            for (int sl = 0; sl < KS; ++sl)
#pragma unroll
                for (int j = 0; j < CBE; ++j) {
                    if (first && sl == 0) plane_mma_g<T, MM, CONJ, G3, GRP, true>(acc[j], aF[sl], aN[sl], bF[sl][j]);
                    else plane_mma_g<T, MM, CONJ, G3, GRP, false>(acc[j], aF[sl], aN[sl], bF[sl][j]);
                }
        };

        // Small T: the first stage starts the accumulators (no zeroing pass);
        // T = 8 zeroes them instead, which keeps one copy of the product code.
        constexpr bool PEEL = T <= 4;
        if (!PEEL) {
#pragma unroll
            for (int j = 0; j < CBE; ++j)
#pragma unroll
                for (int p = 0; p < TP; ++p) acc[j][p] = acc_t{};
        }
        // Ring of NS stages: stage s lives in ring[s % NS].  Stages 0..NS-1 are
        // requested up front; stage ks + NS goes into stage ks's slot once every
        // wave has read stage ks (the barrier of iteration ks).
#pragma unroll
        for (int st = 0; st < NS; ++st) issue(st);
        if (NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * LPS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        ring_barrier();
        load_frags(ring[0]);
        if constexpr (!PIPE) {
            // nst >= 1 always (K >= 8)
            for (int ks = 0; ks < nst; ++ks) {
                if (PEEL && ks == 0) mma_stage(true);
                else mma_stage(false);
                if (ks + 1 < nst) {
                    // stage ks+1 in LDS: at most the stages after it stay in flight
                    if (ks + NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
                    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    ring_barrier();   // every wave is done reading stage ks
                    issue(ks + NS);
                    load_frags(ring[(ks + 1) % NS]);
                }
            }
        } else {
            // Pipelined order: wait for stage ks+1 and pass the barrier first,
            // read its raw activation tuples, then issue stage ks's products
            // and, in the same block, the group DFT of stage ks+1 into a
            // second set of A fragments, so the scheduler can place the VALU
            // work between the matrix instructions.  Stage ks+1's weight
            // fragments are read into the same registers after the products.
            // The two A sets alternate (the loop is unrolled by two).
            frag aG[KS][TP], aM[KS][NNEG];
            auto step = [&](int ks, auto &cA, auto &cN, auto &nA, auto &nN) {
                const bool more = ks + 1 < nst;
                const u32x4 *buf = ring[(ks + 1) % NS];
                u32x4 rawA[KS][LCH];
                if (more) {
                    if (ks + NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
                    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    ring_barrier();   // every wave is done reading stage ks
                    issue(ks + NS);
#pragma unroll
                    for (int sl = 0; sl < KS; ++sl)
#pragma unroll
                        for (int c = 0; c < LCH; ++c)
                            rawA[sl][c] = buf[arow * RCH + (((sl * 2 + lh) * LCH + c) ^ swz<RCH>(arow))];
                }
#pragma unroll
                for (int sl = 0; sl < KS; ++sl)
#pragma unroll
                    for (int j = 0; j < CBE; ++j) {
                        if (PEEL && ks == 0 && sl == 0)
                            plane_mma_g<T, MM, CONJ, G3, GRP, true>(acc[j], cA[sl], cN[sl], bF[sl][j]);
                        else plane_mma_g<T, MM, CONJ, G3, GRP, false>(acc[j], cA[sl], cN[sl], bF[sl][j]);
                    }
                if (more) {
#pragma unroll
                    for (int sl = 0; sl < KS; ++sl) {
                        IO io[KL * T];
                        raw_to_io(rawA[sl], io);
                        act_frags_g<T, IO, MM, CONJ, G3, GRP>(io, nA[sl], nN[sl]);
#pragma unroll
                        for (int j = 0; j < CBE; ++j)
#pragma unroll
                            for (int p = 0; p < TP; ++p)
                                bF[sl][j][p] = __builtin_bit_cast(
                                    frag, buf[ACH + ((wn * CBE + j) * KS + sl) * 64 * TPS + (p * 32 + lr) * 2 +
                                              (lh ^ swz<2>(lr))]);
                    }
                }
            };
            for (int ks = 0; ks < nst; ks += 2) {
                step(ks, aF, aN, aG, aM);
                if (ks + 1 < nst) step(ks + 1, aG, aM, aF, aN);
            }
        }

        // ---- epilogue: inverse group DFT of the T accumulator planes ----
        // The whole output offset stays in the VGPR: the range check of a raw
        // buffer (stride 0) compares only the VGPR offset (plus the instruction
        // offset) with the range, not the scalar offset, so a row offset carried
        // in the scalar offset would let stores for rows past M (the last row
        // block's tail) escape the check and land past the output buffer.  With
        // the offset in the VGPR, rows past M fall outside the range and are
        // dropped.  (The copies of the main loop may carry the stage offset in
        // the scalar offset: their tails are masked through the VGPR offset.)
        // A bias b[col] adds T*b to the k = 0 plane: its inverse DFT is b in every
        // group component ([pchao] §3.2.1 eq. (7) with the bias of Algorithm 1).
        // A column past NC gets offset OOB; adding a row offset (< 2^31) keeps it
        // past the buffer, so those stores are dropped without a select.
#pragma unroll
        for (int j = 0; j < CBE; ++j) {
            const int col = n0 + (wn * CBE + j) * 32 + lr;
            const uint32_t lane_off = col < NC ? ((uint32_t)(wm * 32 + 4 * lh) * NC + col) * TB : OOB;
            const float bv = bias && col < NC ? (float)bias[col] : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t row_off = (uint32_t)((e & 3) + 8 * (e >> 2)) * NC * TB;
                float f[T];
                if constexpr (G3) {
                    float g[TP];
#pragma unroll
                    for (int p = 0; p < TP; ++p) g[p] = acc[j][p][e];
                    gauss_out<T>(g, f);
                } else {
#pragma unroll
                    for (int p = 0; p < T; ++p) f[p] = acc[j][p][e];
                }
                if constexpr (Pow2<T>::value) {
                    const typename Raw<TB>::type o =
                        __builtin_bit_cast(typename Raw<TB>::type, grp_out<T, IO, GRP>(f, bv));
                    Raw<TB>::template store<CP_NT>(o, ro, lane_off + row_off);
                } else {
                    store_tuple_inv<IO, T, CP_NT>(f, bv, ro, lane_off + row_off, aligned4, pairs, lane);
                }
            }
        }
    };
    if constexpr (CAN_HALF) {
        if (half) {
            run(std::integral_constant<int, CB / 2>{});
            return;
        }
    }
    run(std::integral_constant<int, CB>{});
}

// ===========================================================================
// Row kernel for layers with few output tiles (few rows, or few columns):
// the same product as row_kernel on 32-row x 32-column tiles, with the k
// range of each stage split over the workgroup's 4 waves.  A stage holds
// KW = 4 MFMA k slices; wave w multiplies slice w of every stage into its
// own accumulators, so a stage carries 4x the k of row_kernel's and a long
// K takes 4x fewer stages (the stage loop is latency-bound when there are
// too few tiles to fill the GPU).  After the last stage the four partial
// spectra are added in wave order through LDS and each wave applies the
// inverse DFT to a quarter of the tile.
// LDS layouts (16-byte chunks):
//   A: row r of the tile, chunk q of its stage segment (slice q / SRCH) ->
//      slot r*RCH + (q ^ (r % SWM)), SWM = 16 when a row holds a multiple of
//      16 chunks (then the 16 lanes of one ds_read_b128 phase, 16 rows at the
//      same chunk, land in 16 distinct bank groups), else 8 (orders 3, 5, 7:
//      at most two lanes share a bank group)
//   B: slice w, plane p, column c, k-run h -> slot ACH + w*64*T + (p*32 + c)*2
//      + (h ^ swz<2>(c)) (as in row_kernel, per slice)
// ===========================================================================
template <int T, typename IO, bool CONJ, int NS, bool EL, int KW, int GRP = 0>
__global__ __launch_bounds__(KW * 64, 1) void rowk_kernel(const IO *__restrict__ act, const IO *__restrict__ bpl,
                                                      IO *__restrict__ out, int M, int K, int NC,
                                                      uint32_t bpl_bytes, const IO *__restrict__ bias,
                                                      int col_major, int gran) {
    typedef M32<IO> MM;
    typedef typename MM::frag frag;
    typedef typename MM::acc_t acc_t;
    constexpr int NW = KW;
    constexpr int ES = sizeof(IO), KL = MM::KL, KC = 2 * KL, TB = T * ES;
    constexpr int LCH = KL * TB / 16;      // chunks of one lane's k-run in one slice
    constexpr int SRCH = 2 * LCH;          // chunks of one row in one slice
    constexpr int RCH = KW * SRCH;         // chunks of one row per stage
    constexpr int ACH = 32 * RCH;          // activation chunks per stage
    constexpr bool G3 = Gauss<T, IO>::V && GRP == 0;   // three-multiplication products
    constexpr int TP = GRP ? T : math_planes<T, IO>(), TPS = GRP ? T : stored_planes<T, IO>();
    constexpr int BCH = KW * TPS * 64;     // weight chunks per stage
    constexpr int SCH = ACH + BCH;
    constexpr int LPS = SCH / (KW * 64);   // buffer->LDS loads per thread per stage
    constexpr int KSTG = KW * KC;          // k per stage
    constexpr int NNEG = (T - 1) / 2 > 0 ? (T - 1) / 2 : 1;
    constexpr int SWM = RCH % 16 == 0 ? 16 : 8;
    static_assert(SCH % (KW * 64) == 0 && RCH % SWM == 0 && KW >= 4, "tile shape");
    static_assert(KL * ES == 16, "one fragment is one 16-byte chunk");
    static_assert((NS - 1) * LPS < 64 && NS >= 2, "vmcnt range");
    // partial spectra are added through the ring in groups of PG planes
    constexpr int PG = (NS * SCH * 16) / (KW * 16 * 64 * 4) < TP ? (NS * SCH * 16) / (KW * 16 * 64 * 4) : TP;
    static_assert(PG >= 1, "one plane of partials fits in the ring");

    __shared__ __attribute__((aligned(16))) u32x4 ring[NS][SCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;

    const int tiles_m = (M + 31) / 32, tiles_n = (NC + 31) / 32;
    const int tile = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    // consecutive tiles (one XCD) share the larger operand
    const int tm = col_major ? tile % tiles_m : tile / tiles_n;
    const int tn = col_major ? tile / tiles_m : tile % tiles_n;
    const int m0 = tm * 32, n0 = tn * 32, cb = tn;
    const int rows = min(32, M - m0);
    const int nks = (K + KC - 1) / KC;
    const int nst = (K + KSTG - 1) / KSTG;
    const int KP = nks * KC;

    const rsrc_t ra = make_rsrc(act + (size_t)m0 * K * T, (uint32_t)rows * K * TB);
    const rsrc_t rb = make_rsrc(bpl, bpl_bytes);
    const rsrc_t ro = make_rsrc(out + (size_t)m0 * NC * T, (uint32_t)rows * NC * TB);
    // tuple stores of orders 3, 5, 6, 7 (store_tuple_inv): dword accesses
    // need a 4-byte aligned row base, lane pairs also an even column count
    [[maybe_unused]] const bool aligned4 = ((uintptr_t)(out + (size_t)m0 * NC * T) & 3u) == 0;
    [[maybe_unused]] const bool pairs = aligned4 && NC % 2 == 0;

    // ---- per-thread load slots: chunk index (li * NW + wave) * 64 + lane ----
    uint32_t l_off[LPS], l_qb[LPS];
    int l_kk[LPS];
#pragma unroll
    for (int li = 0; li < LPS; ++li) {
        const int sidx = (li * NW + wave) * 64 + lane;
        l_qb[li] = 0;
        if (sidx < ACH) {
            const int r = sidx / RCH, q = (sidx % RCH) ^ (r % SWM);
            const int w = q / SRCH, q2 = q % SRCH;
            l_off[li] = (uint32_t)r * K * TB + (uint32_t)(w * KC * TB + q2 * 16);
            l_kk[li] = w * KC + q2 * 16 / TB;
            l_qb[li] = (uint32_t)(w * KC * TB + q2 * 16);
        } else {
            const int sb = sidx - ACH;
            const int w = sb / (64 * TPS), g = sb % (64 * TPS);
            const int p = g / 64, c = (g / 2) % 32, h = (g % 2) ^ swz<2>(c);
            l_off[li] = (uint32_t)(((cb * nks + w) * TPS * 32 * KC + (p * 32 + c) * KC + h * KL) * ES);
            l_kk[li] = w * KC;
        }
    }
    auto issue = [&](int st) {
        if (st >= nst) return;
        const int k0 = st * KSTG;
        if constexpr (EL)
            el_stage<IO, LPS, NW, ACH>(ra, rb, ring[st % NS], l_off, l_qb, l_kk, wave, lane, (uint32_t)k0 * TB,
                                       (uint32_t)st * KW * TPS * 32 * KC * ES, k0 + KSTG <= K, k0, KP,
                                       (uint32_t)K * TB, gran);
        else
            dma_stage<LPS, NW, ACH>(ra, rb, ring[st % NS], l_off, l_kk, wave, (uint32_t)k0 * TB,
                                    (uint32_t)st * KW * TPS * 32 * KC * ES, k0 + KSTG <= K, k0, K, KP);
    };

    acc_t acc[TP];
    frag aF[TP], aN[NNEG], bF[TP];
    auto load_frags = [&](const u32x4 *buf) {
        u32x4 rawA[LCH];
#pragma unroll
        for (int c = 0; c < LCH; ++c) rawA[c] = buf[lr * RCH + ((wave * SRCH + lh * LCH + c) ^ (lr % SWM))];
        IO io[KL * T];
        raw_to_io(rawA, io);
        act_frags_g<T, IO, MM, CONJ, G3, GRP>(io, aF, aN);
#pragma unroll
        for (int p = 0; p < TP; ++p)
            bF[p] = __builtin_bit_cast(frag, buf[ACH + wave * 64 * TPS + (p * 32 + lr) * 2 + (lh ^ swz<2>(lr))]);
    };

    constexpr bool PEEL = T <= 4;
    if (!PEEL) {
#pragma unroll
        for (int p = 0; p < TP; ++p) acc[p] = acc_t{};
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(st);
    if (NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * LPS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    ring_barrier();
    load_frags(ring[0]);
    for (int ks = 0; ks < nst; ++ks) {
        if (PEEL && ks == 0) plane_mma_g<T, MM, CONJ, G3, GRP, true>(acc, aF, aN, bF);
        else plane_mma_g<T, MM, CONJ, G3, GRP, false>(acc, aF, aN, bF);
        if (ks + 1 < nst) {
            if (ks + NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            ring_barrier();
            issue(ks + NS);
            load_frags(ring[(ks + 1) % NS]);
        }
    }

    // ---- the KW partial spectra, added in wave order ----
    // Per group of PG planes: red[w][p - p0][j][lane] holds elements
    // e = 4j .. 4j+3 of wave w's plane p; wave w < 4 finishes elements
    // e = 4w .. 4w+3 (rows 4*lh + 8*w + i, column lr).
    u32x4 *red = &ring[0][0];
    float f[4][T], g[4][TP];
#pragma unroll
    for (int p0 = 0; p0 < TP; p0 += PG) {
        ring_barrier();   // every wave is done reading the ring (or the previous group)
#pragma unroll
        for (int p = p0; p < p0 + PG && p < TP; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[((wave * PG + p - p0) * 4 + j) * 64 + lane] = __builtin_bit_cast(
                    u32x4, f32x4{acc[p][4 * j], acc[p][4 * j + 1], acc[p][4 * j + 2], acc[p][4 * j + 3]});
        ring_barrier();
        if (wave < 4) {
#pragma unroll
            for (int p = p0; p < p0 + PG && p < TP; ++p) {
                f32x4 v = __builtin_bit_cast(f32x4, red[((0 * PG + p - p0) * 4 + wave) * 64 + lane]);
#pragma unroll
                for (int w = 1; w < KW; ++w)
                    v += __builtin_bit_cast(f32x4, red[((w * PG + p - p0) * 4 + wave) * 64 + lane]);
#pragma unroll
                for (int i = 0; i < 4; ++i) g[i][p] = v[i];
            }
        }
    }
    if (wave >= 4) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (G3) {
            gauss_out<T>(g[i], f[i]);
        } else {
#pragma unroll
            for (int p = 0; p < T; ++p) f[i][p] = g[i][p];
        }
    }
    const int col = n0 + lr;
    const float bv = bias && col < NC ? (float)bias[col] : 0.0f;
    const uint32_t lane_off = col < NC ? ((uint32_t)(8 * wave + 4 * lh) * NC + col) * TB : OOB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (Pow2<T>::value) {
            const typename Raw<TB>::type o =
                __builtin_bit_cast(typename Raw<TB>::type, grp_out<T, IO, GRP>(f[i], bv));
            Raw<TB>::template store<CP_NT>(o, ro, lane_off + (uint32_t)i * NC * TB);
        } else {
            store_tuple_inv<IO, T, CP_NT>(f[i], bv, ro, lane_off + (uint32_t)i * NC * TB, aligned4, pairs, lane);
        }
    }
}

// Weight-gradient epilogue of one wave: its CB 32x32 blocks of all T planes,
// at tile rows rb.. (channels of the row operand) and columns cb.. (CB * 32
// channels of the column operand).  SWAP (rows c, columns d) holds
// conj(dWhat): the imaginary planes change sign.  DIRECT applies the inverse
// DFT and writes dw [DT][CT][T]; otherwise the fp32 planes go to split
// `split` of the workspace, in [DT][CT] order or [CT][DT] (SWAP) order.
template <int T, typename IO, int CB, bool SWAP, bool DIRECT, int NP = T, int GRP = 0>
__device__ inline void dw_epilogue(const typename M32<IO>::acc_t (&acc)[CB][NP], int rb, int cb, int lh, int lr,
                                   int NR, int NCc, int CT, int DT, int split, float *__restrict__ ws,
                                   IO *__restrict__ dw) {
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int rch = rb + (e & 3) + 4 * lh + 8 * (e >> 2);
            const int cch = cb + j * 32 + lr;
            if (rch < NR && cch < NCc) {
                const int d = SWAP ? cch : rch, c = SWAP ? rch : cch;
                float f[T];
                if constexpr (NP != T) {   // Gauss's products: K1, K2, K3 -> Re, Im
                    float g[NP];
#pragma unroll
                    for (int p = 0; p < NP; ++p) g[p] = acc[j][p][e];
                    gauss_out<T>(g, f);
                } else {
#pragma unroll
                    for (int p = 0; p < T; ++p) f[p] = acc[j][p][e];
                }
                if (SWAP && GRP == 0) {   // conj: Im planes change sign
#pragma unroll
                    for (int k = 1; k <= (T - 1) / 2; ++k) f[2 * k] = -f[2 * k];
                }
                if (DIRECT) {
                    if constexpr (Pow2<T>::value) {
                        typedef typename Tuple<IO, T>::type tup;
                        *reinterpret_cast<tup *>(dw + ((size_t)d * CT + c) * T) = grp_out<T, IO, GRP>(f, 0.0f);
                    } else {
                        float y[T];
                        Dft<T>::inv(f, y);
#pragma unroll
                        for (int t = 0; t < T; ++t) dw[((size_t)d * CT + c) * T + t] = (IO)y[t];
                    }
                } else {
                    const size_t at = SWAP ? ((size_t)split * CT + c) * DT + d : ((size_t)split * DT + d) * CT + c;
                    if constexpr (Pow2<T>::value) {
                        typedef float ftup __attribute__((ext_vector_type(T)));
                        ftup o;
#pragma unroll
                        for (int p = 0; p < T; ++p) o[p] = f[p];
                        *reinterpret_cast<ftup *>(ws + at * T) = o;
                    } else {
#pragma unroll
                        for (int p = 0; p < T; ++p) ws[at * T + p] = f[p];
                    }
                }
            }
        }
}

// Channels per weight-gradient load unit: CP adjacent channels' tuples move
// in one access (or one short run of dword accesses).  Tuples of 2, 4, 8
// bytes: CP*TB up to 16 bytes, when the U single-channel units of a stage
// still divide into whole rounds of the NT threads (halves the column
// operand's load instructions at T = 4, fp16).  Tuples whose size is not a
// multiple of 4 bytes (odd orders in fp16): CP = 2, so that a unit row is
// whole dwords, when the units still fill whole waves -- some waves then
// carry one more unit than others, which the removed per-element loads
// (T of them per tuple) more than pay for.
__host__ __device__ constexpr int dw_cpl(int TB, int U, int NT) {
    int best = 1;
    if ((TB & (TB - 1)) == 0) {
        for (int c = 2; c * TB <= 16; c *= 2)
            if (16 % (c * TB) == 0 && U % c == 0 && (U / c) % NT == 0) best = c;
    } else if (TB % 4 != 0 && U % 2 == 0 && (U / 2) % 64 == 0) {
        best = 2;
    }
    return best;
}

// N dwords from a buffer at a 4-byte aligned offset: 16-byte accesses plus
// one of 12, 8 or 4 bytes.
template <int N> struct Dwords {
    unsigned int w[N];
    __device__ static inline Dwords load(rsrc_t r, uint32_t off) {
        Dwords d;
#pragma unroll
        for (int i = 0; i + 4 <= N; i += 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4u * i, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) d.w[i + e] = v[e];
        }
        constexpr int I = N / 4 * 4;
        if constexpr (N - I == 3) {
            typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
            const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4u * I, 0, 0);
#pragma unroll
            for (int e = 0; e < 3; ++e) d.w[I + e] = v[e];
        } else if constexpr (N - I == 2) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4u * I, 0, 0);
            d.w[I] = v[0];
            d.w[I + 1] = v[1];
        } else if constexpr (N - I == 1) {
            d.w[I] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4u * I, 0, 0);
        }
        return d;
    }
};
template <typename R> struct IsDwords { static constexpr bool value = false; };
template <int N> struct IsDwords<Dwords<N>> { static constexpr bool value = true; };

// LDS placement of the weight-gradient stage (rows of RUNS 16-byte chunks, one
// row per channel).  On gfx950 a ds_write_b128 serves 8 lanes per clock from
// 128 bytes of banks and a ds_read_b128 16 lanes per clock from 256 bytes
// (measured with the bank-conflict counter), so with RUNS = 4 (64-byte rows):
//  - the fragment reads (16 consecutive rows, one chunk) need the chunk XOR
//    to take 4 distinct values over bits 2-3 of the row for each value of bits
//    0-1;
//  - the writes of single-channel units (8 consecutive rows, one chunk) need
//    4 distinct values over bits 1-2 for each value of bit 0;
//  - units of two adjacent channels write rows 2 apart; dw_row moves every
//    second group of 8 channels to the rows of the other parity, so that the 8
//    lanes of a write cover both parities and the condition above applies.
// x = ((b3 ^ b1) << 1) | (b2 ^ b1) meets both conditions; other row widths
// keep the generic swizzle.
template <int RUNS> __device__ constexpr int dw_swz(int r) {
    return RUNS == 4 ? ((((r >> 3) ^ (r >> 1)) & 1) << 1) | (((r >> 2) ^ (r >> 1)) & 1) : swz<RUNS>(r);
}
template <int CP> __device__ constexpr int dw_row(int c) { return CP == 2 ? c ^ ((c >> 3) & 1) : c; }

// Register type of one weight-gradient load unit row: CP adjacent tuples.
// Orders 2, 4, 8 use the power-of-two accesses of Raw; other orders whole
// dwords when CP tuples are (per-element loads otherwise).
template <typename IO, int T, int CP, bool P2 = Pow2<T>::value,
          bool DW = (CP * T * (int)sizeof(IO)) % 4 == 0>
struct DwUnit { typedef typename Raw<CP * T * (int)sizeof(IO)>::type type; };
template <typename IO, int T> struct DwUnit<IO, T, 1, true, true> { typedef typename TupleLd<IO, T>::type type; };
template <typename IO, int T> struct DwUnit<IO, T, 1, true, false> { typedef typename TupleLd<IO, T>::type type; };
template <typename IO, int T, int CP> struct DwUnit<IO, T, CP, false, true> {
    typedef Dwords<CP * T * (int)sizeof(IO) / 4> type;
};
template <typename IO, int T, int CP> struct DwUnit<IO, T, CP, false, false> { typedef typename TupleLd<IO, T>::type type; };

// ===========================================================================
// Weight-gradient kernel: dWhat_k[d, c] = sum_n dYhat_k[n, d] conj(Xhat_k[n, c])
// for its tile of channels and its chunk of rows n.
//   x [N][CT][T], dy [N][DT][T]
// The tile is BR "row" channels x BC "column" channels: rows are d and
// columns c, or (SWAP) rows c and columns d -- whichever divides the layer
// into whole tiles.  The contraction runs over n, so both operands are
// staged n-contiguous in LDS after the group DFT: a thread loads KL
// consecutive rows of one channel (one tuple each) -- or of CP adjacent
// channels, CP tuples in one access, where tuples are narrower than 16 bytes
// (WIDE; at ViT-B FFN size this cut the kernel by about a tenth, the load
// instructions rather than their bytes being the cost) -- transforms them,
// and writes one 16-byte chunk per plane and channel.  Products on 32x32
// MFMA blocks with A = row operand, B = column operand, A . conj(B); SWAP
// gives conj(dWhat) and the epilogue flips the imaginary planes back.  With
// Gauss's products (fp32, orders 4, 6, 8) the staged planes are those of
// dw_frags3 and the products diagonal; the epilogue forms Re, Im first.
//   DIRECT: one chunk; the epilogue applies the inverse DFT and writes
//           dw [DT][CT][T].
//   else:   fp32 plane values go to ws[split][...][T]: [DT][CT] order, or
//           [CT][DT] (SWAP) so that consecutive lanes write consecutive
//           addresses; dw_finalize adds the splits in order.
// Stage = KS MFMA k slices (KSTG = KS * 2 * KL rows n), single LDS buffer.
// LDS layout: plane p, channel ch, run q (KL rows) -> slot ch*RUNS + (q ^ swz(ch)).
// ===========================================================================
template <int T, typename IO, int WM, int WN, int CB, int KS, bool SWAP, bool DIRECT, int OCC, bool WIDE>
__global__ __launch_bounds__(WM *WN * 64, OCC) void dw_kernel(
    const IO *__restrict__ x, const IO *__restrict__ dy, float *__restrict__ ws,
    IO *__restrict__ dw, int N, int CT, int DT, int chunk) {
    typedef M32<IO> MM;
    typedef typename MM::frag frag;
    typedef typename MM::acc_t acc_t;
    constexpr int ES = sizeof(IO), KL = MM::KL, TB = T * ES;
    constexpr int RUNS = KS * 2;                 // KL-row runs per stage
    constexpr int KSTG = RUNS * KL;
    constexpr int NT = WM * WN * 64;
    constexpr int BR = WM * 32, BC = WN * CB * 32;
    // staging units: KL rows of CPR (CPC) adjacent channels; WIDE only when
    // the channel counts are multiples of them, so that a unit never straddles
    // the end of a row
    constexpr int CPR = WIDE ? dw_cpl(TB, BR * RUNS, NT) : 1, CPC = WIDE ? dw_cpl(TB, BC * RUNS, NT) : 1;
    constexpr int UR = BR * RUNS / CPR, UC = BC * RUNS / CPC;
    constexpr int GR = BR / CPR, GC = BC / CPC;     // channel groups per run
    constexpr int PR = (UR + NT - 1) / NT, PC = (UC + NT - 1) / NT;
    constexpr int NNEG = (T - 1) / 2 > 0 ? (T - 1) / 2 : 1;
    constexpr bool G3 = Gauss<T, IO>::V;        // Gauss's three products
    constexpr int TP = math_planes<T, IO>();     // planes staged and multiplied
    static_assert(KL * ES == 16, "one fragment is one 16-byte chunk");

    __shared__ __attribute__((aligned(16))) u32x4 sR[TP][BR * RUNS];
    __shared__ __attribute__((aligned(16))) u32x4 sC[TP][BC * RUNS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 31, lh = lane >> 5;

    const IO *src_r = SWAP ? x : dy;
    const IO *src_c = SWAP ? dy : x;
    const int NR = SWAP ? CT : DT, NCc = SWAP ? DT : CT;
    const int tiles_c = (NCc + BC - 1) / BC;
    const int tiles = ((NR + BR - 1) / BR) * tiles_c;
    const int t_all = xcd_tile(blockIdx.x, gridDim.x);
    const int split = t_all / tiles, tile = t_all % tiles;
    const int r0 = (tile / tiles_c) * BR, c0 = (tile % tiles_c) * BC;
    const int nbeg = split * chunk;
    const int nrows = min(N, nbeg + chunk) - nbeg;
    const int nst = (nrows + KSTG - 1) / KSTG;

    // rows past the chunk end fall outside these ranges and read as zero
    const rsrc_t rr = make_rsrc(src_r + (size_t)nbeg * NR * T, (uint32_t)nrows * NR * TB);
    const rsrc_t rc = make_rsrc(src_c + (size_t)nbeg * NCc * T, (uint32_t)nrows * NCc * TB);

    typedef typename TupleLd<IO, T>::type rawt;
    static_assert(sizeof(rawt) == TB, "tuples are packed");
    typedef typename DwUnit<IO, T, CPR>::type rawr_t;
    typedef typename DwUnit<IO, T, CPC>::type rawc_t;
    rawr_t rawR[PR][KL];
    rawc_t rawC[PC][KL];
    auto ld = [&](auto &dst, rsrc_t r, uint32_t off) {
        typedef typename std::remove_reference<decltype(dst)>::type R;
        if constexpr (IsDwords<R>::value) dst = R::load(r, off);
        else if constexpr (sizeof(R) == TB) dst = TupleLd<IO, T>::load(r, off);
        else dst = Raw<(int)sizeof(R)>::load(r, off);
    };
    auto load = [&](int ks) {
#pragma unroll
        for (int it = 0; it < PR; ++it) {
            const int u = it * NT + tid, ch = (u % GR) * CPR, run = u / GR;
            if (UR % NT != 0 && u >= UR) continue;   // whole waves without a unit
            const bool ok = (u < UR) && (r0 + ch < NR);
            const uint32_t base = ((uint32_t)(ks * KSTG + run * KL) * NR + r0 + ch) * TB;
#pragma unroll
            for (int v = 0; v < KL; ++v) ld(rawR[it][v], rr, ok ? base + (uint32_t)v * NR * TB : OOB);
        }
#pragma unroll
        for (int it = 0; it < PC; ++it) {
            const int u = it * NT + tid, ch = (u % GC) * CPC, run = u / GC;
            if (UC % NT != 0 && u >= UC) continue;
            const bool ok = (u < UC) && (c0 + ch < NCc);
            const uint32_t base = ((uint32_t)(ks * KSTG + run * KL) * NCc + c0 + ch) * TB;
#pragma unroll
            for (int v = 0; v < KL; ++v) ld(rawC[it][v], rc, ok ? base + (uint32_t)v * NCc * TB : OOB);
        }
    };
    // Transform one unit's KL x CP tuples and write CP chunks per plane.
    auto store = [&]() {
#pragma unroll
        for (int it = 0; it < PR; ++it) {
            const int u = it * NT + tid, ch = (u % GR) * CPR, run = u / GR;
            if (UR % NT != 0 && u >= UR) continue;
            IO all[KL * CPR * T];
            raw_to_io(rawR[it], all);
#pragma unroll
            for (int j = 0; j < CPR; ++j) {
                IO v[KL * T];
#pragma unroll
                for (int r = 0; r < KL; ++r)
#pragma unroll
                    for (int t = 0; t < T; ++t) v[r * T + t] = all[(r * CPR + j) * T + t];
                frag pl[TP];
                dw_frags<T, IO, false>(v, pl);
                const int lrow = dw_row<CPR>(ch + j);
#pragma unroll
                for (int p = 0; p < TP; ++p)
                    sR[p][lrow * RUNS + (run ^ dw_swz<RUNS>(lrow))] = __builtin_bit_cast(u32x4, pl[p]);
            }
        }
#pragma unroll
        for (int it = 0; it < PC; ++it) {
            const int u = it * NT + tid, ch = (u % GC) * CPC, run = u / GC;
            if (UC % NT != 0 && u >= UC) continue;
            IO all[KL * CPC * T];
            raw_to_io(rawC[it], all);
#pragma unroll
            for (int j = 0; j < CPC; ++j) {
                IO v[KL * T];
#pragma unroll
                for (int r = 0; r < KL; ++r)
#pragma unroll
                    for (int t = 0; t < T; ++t) v[r * T + t] = all[(r * CPC + j) * T + t];
                frag pl[TP];
                dw_frags<T, IO, true>(v, pl);
                const int lrow = dw_row<CPC>(ch + j);
#pragma unroll
                for (int p = 0; p < TP; ++p)
                    sC[p][lrow * RUNS + (run ^ dw_swz<RUNS>(lrow))] = __builtin_bit_cast(u32x4, pl[p]);
            }
        }
    };

    acc_t acc[CB][TP];
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int p = 0; p < TP; ++p) acc[j][p] = acc_t{};

    const int ar = dw_row<CPR>(wm * 32 + lr);
    if (nst > 0) load(0);
    for (int ks = 0; ks < nst; ++ks) {
        __syncthreads();  // previous stage's fragment reads are done
        store();
        __syncthreads();
        if (ks + 1 < nst) load(ks + 1);
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
            const int q = sl * 2 + lh;
            frag aF[TP], aN[NNEG];
#pragma unroll
            for (int p = 0; p < TP; ++p) aF[p] = __builtin_bit_cast(frag, sR[p][ar * RUNS + (q ^ dw_swz<RUNS>(ar))]);
            if constexpr (!G3) make_neg<T, MM, true>(aF, aN);
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int bc = dw_row<CPC>((wn * CB + j) * 32 + lr);
                if constexpr (G3) {   // diagonal plane products, one column fragment at a time
#pragma unroll
                    for (int p = 0; p < TP; ++p)
                        acc[j][p] = MM::mma(aF[p], __builtin_bit_cast(frag, sC[p][bc * RUNS + (q ^ dw_swz<RUNS>(bc))]),
                                            acc[j][p]);
                } else {
                    frag bF[T];
#pragma unroll
                    for (int p = 0; p < T; ++p)
                        bF[p] = __builtin_bit_cast(frag, sC[p][bc * RUNS + (q ^ dw_swz<RUNS>(bc))]);
                    freq_mma<T, MM, true>(acc[j], aF, aN, bF);
                }
            }
        }
    }

    dw_epilogue<T, IO, CB, SWAP, DIRECT, TP>(acc, r0 + wm * 32, c0 + wn * CB * 32, lh, lr, NR, NCc, CT, DT, split,
                                         ws, dw);
}

// ===========================================================================
// Weight-gradient kernel with producer and consumer waves: the product of
// dw_kernel (same tile, same LDS plane layout, same epilogue) on one
// 512-thread workgroup per CU.  Waves 0-3 are consumers: a 2 x 2 grid of
// 32 x (CB * 32) MFMA blocks that only read plane fragments from LDS and
// multiply.  Waves 4-7 are producers: each thread loads the raw tuples of its
// staging units (KL consecutive rows n of one channel, or of CPC adjacent
// column channels as in dw_kernel) P stages ahead into a register ring, applies the group DFT and writes one 16-byte chunk per plane
// into the LDS stage buffer the consumers read next.  The stage buffers are
// double-buffered, so in every step the producers fill stage s + 1 while the
// consumers multiply stage s, with a single workgroup barrier per stage.
// Waves are spread over the CU's four SIMDs in id order, so every SIMD runs
// one producer and one consumer: the group-DFT VALU work of one overlaps the
// matrix work of the other.  With one workgroup per CU instead of two, a
// layer needs half as many row splits to fill the GPU, which halves the fp32
// partial spectra written to the workspace and read back by dw_finalize.
// The producers' register ring is unrolled (UNR steps) so every slot index
// is a compile-time constant, and every step is unconditional so the
// compiler's vmcnt waits count exactly the loads of later stages.  The
// barrier (ring_barrier) waits for LDS traffic only: those loads stay in
// flight.  dw_plan dispatches it for order 8 and the octic group, for
// order 2 in fp16, and for order 4 unless the narrow or ring-staged plan
// runs.
// ===========================================================================
template <int T, typename IO, int CB, int KS, int P, bool SWAP, bool DIRECT, bool WIDE, int GRP = 0>
__global__ __launch_bounds__(512, 1) void dwp_kernel(const IO *__restrict__ x, const IO *__restrict__ dy,
                                                     float *__restrict__ ws, IO *__restrict__ dw, int N, int CT,
                                                     int DT, int chunk) {
    typedef M32<IO> MM;
    typedef typename MM::frag frag;
    typedef typename MM::acc_t acc_t;
    constexpr int ES = sizeof(IO), KL = MM::KL, TB = T * ES;
    constexpr int WM = 2, WN = 2;
    constexpr int RUNS = KS * 2;                 // KL-row runs per stage
    constexpr int KSTG = RUNS * KL;              // rows n per stage
    constexpr int BR = WM * 32, BC = WN * CB * 32;
    constexpr int NP = 256;                      // producer threads
    // staging units: KL rows of one row-operand channel, or of CPC adjacent
    // column-operand channels (one access of CPC tuples per row; WIDE only
    // when the column channel count is a multiple of CPC)
    constexpr int CPC = WIDE ? dw_cpl(TB, BC * RUNS, NP) : 1;
    constexpr int UR = BR * RUNS, UC = BC * RUNS / CPC;
    // Each operand part is whole rounds of the NP producer threads, or else
    // (MIXED) the two parts together are, each part being whole waves: then a
    // producer wave stages one operand or the other.
    constexpr bool MIXED = !(UR % NP == 0 && UC % NP == 0);
    constexpr int UROW = MIXED ? 0 : UR / NP, UCOL = MIXED ? 0 : UC / NP;   // units per producer thread
    constexpr int UMIX = MIXED ? (UR + UC) / NP : 0;
    constexpr int SR = BR * RUNS;                 // slots of the row part (column part follows)
    constexpr int UNR = P % 2 == 0 ? P : 2 * P;  // producer steps per unrolled loop body
    constexpr int NNEG = (T - 1) / 2 > 0 ? (T - 1) / 2 : 1;
    constexpr bool G3 = Gauss<T, IO>::V && GRP == 0;   // Gauss's three products
    constexpr int TP = GRP ? T : math_planes<T, IO>();     // planes staged and multiplied
    static_assert(KL * ES == 16, "one fragment is one 16-byte chunk");
    static_assert(!MIXED || (CPC == 1 && (UR + UC) % NP == 0 && UR % 64 == 0),
                  "operand parts are whole rounds of producer units, or whole waves of one round");
    static_assert(Pow2<T>::value, "one load per tuple");

    // [buffer][plane][slot]: row part slots [0, SR), column part [SR, SR + BC * RUNS)
    __shared__ __attribute__((aligned(16))) u32x4 sbuf[2][TP][(BR + BC) * RUNS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;

    const IO *src_r = SWAP ? x : dy;
    const IO *src_c = SWAP ? dy : x;
    const int NR = SWAP ? CT : DT, NCc = SWAP ? DT : CT;
    const int tiles_c = (NCc + BC - 1) / BC;
    const int tiles = ((NR + BR - 1) / BR) * tiles_c;
    const int t_all = xcd_tile(blockIdx.x, gridDim.x);
    const int split = t_all / tiles, tile = t_all % tiles;
    const int r0 = (tile / tiles_c) * BR, c0 = (tile % tiles_c) * BC;
    const int nbeg = split * chunk;
    const int nrows = min(N, nbeg + chunk) - nbeg;
    const int nst = (nrows + KSTG - 1) / KSTG;
    const int nstp = (nst + UNR - 1) / UNR * UNR;   // steps run by both roles

    if (wave >= 4) {
        // ---------------- producers ----------------
        // Row-operand units it * NP + (wave - 4) * 64 + lane for it < UROW,
        // column-operand units likewise for it < UCOL: compile-time loops
        // after unrolling (no branch around the loads).
        const int pw = (wave - 4) * 64;
        const uint32_t rsr = (uint32_t)NR * TB, rsc = (uint32_t)NCc * TB;   // bytes per row n
        typedef typename DwUnit<IO, T, 1>::type rawr_t;
        typedef typename DwUnit<IO, T, CPC>::type rawc_t;
        // per unit: byte offset of its first row within a stage and its LDS
        // slots.  A channel past the end of the layer reads whatever the
        // range check gives (the next row's channels, or zeros): its planes
        // only reach outputs the epilogue drops.  Rows past the chunk read
        // zeros (the stage's resource ends at the chunk's last row, and the
        // whole offset is in the VGPR, which the range check covers).
        uint32_t r_off[UROW > 0 ? UROW : 1], c_off[UCOL > 0 ? UCOL : 1], m_off[UMIX > 0 ? UMIX : 1];
        int r_slot[UROW > 0 ? UROW : 1], c_slot[UCOL > 0 ? UCOL : 1][CPC], m_slot[UMIX > 0 ? UMIX : 1];
        bool m_row[UMIX > 0 ? UMIX : 1];   // wave-uniform: the unit belongs to the row operand
#pragma unroll
        for (int it = 0; it < UMIX; ++it) {
            const int u = it * NP + pw + lane;
            m_row[it] = it * NP + pw < UR;
            if (m_row[it]) {
                const int ch = u % BR, run = u / BR;
                m_off[it] = ((uint32_t)(run * KL) * NR + r0 + ch) * TB;
                m_slot[it] = ch * RUNS + (run ^ dw_swz<RUNS>(ch));
            } else {
                const int u2 = u - UR, ch = u2 % BC, run = u2 / BC;
                m_off[it] = ((uint32_t)(run * KL) * NCc + c0 + ch) * TB;
                m_slot[it] = SR + ch * RUNS + (run ^ dw_swz<RUNS>(ch));
            }
        }
#pragma unroll
        for (int it = 0; it < UROW; ++it) {
            const int u = it * NP + pw + lane, ch = u % BR, run = u / BR;
            r_off[it] = ((uint32_t)(run * KL) * NR + r0 + ch) * TB;
            r_slot[it] = ch * RUNS + (run ^ dw_swz<RUNS>(ch));
        }
#pragma unroll
        for (int it = 0; it < UCOL; ++it) {
            const int u = it * NP + pw + lane, ch = (u % (BC / CPC)) * CPC, run = u / (BC / CPC);
            c_off[it] = ((uint32_t)(run * KL) * NCc + c0 + ch) * TB;
#pragma unroll
            for (int jj = 0; jj < CPC; ++jj) {
                const int lrow = dw_row<CPC>(ch + jj);
                c_slot[it][jj] = SR + lrow * RUNS + (run ^ dw_swz<RUNS>(lrow));
            }
        }
        // Per-row VGPR offsets of each unit inside a stage, fixed for the
        // whole loop; each stage's loads go through a resource whose base
        // is that stage's first row and whose range ends at the chunk's
        // last row (empty past it), so rows past the chunk still read zeros
        // and no address arithmetic runs per load (N = 8192 at 1024 -> 4096
        // steady-state step 147.5 -> 143.8 us, ViT-B fc1 / fc2 and the other
        // layers of this kernel 0.5-1% faster, results bit-identical).
        uint32_t r_offv[UROW > 0 ? UROW : 1][KL], c_offv[UCOL > 0 ? UCOL : 1][KL], m_offv[UMIX > 0 ? UMIX : 1][KL];
#pragma unroll
        for (int v = 0; v < KL; ++v) {
#pragma unroll
            for (int it = 0; it < UROW; ++it) r_offv[it][v] = r_off[it] + (uint32_t)v * rsr;
#pragma unroll
            for (int it = 0; it < UCOL; ++it) c_offv[it][v] = c_off[it] + (uint32_t)v * rsc;
#pragma unroll
            for (int it = 0; it < UMIX; ++it) m_offv[it][v] = m_off[it] + (uint32_t)v * (m_row[it] ? rsr : rsc);
        }
        auto stage_rsrc = [&](int st, bool row) {
            const int left = nrows - st * KSTG;
            const IO *p = row ? src_r + ((size_t)nbeg + (size_t)st * KSTG) * NR * T
                              : src_c + ((size_t)nbeg + (size_t)st * KSTG) * NCc * T;
            return make_rsrc(p, left > 0 ? (uint32_t)left * (row ? rsr : rsc) : 0u);
        };
        rawr_t rawR[P][UROW > 0 ? UROW : 1][KL];
        rawc_t rawC[P][UCOL > 0 ? UCOL : 1][KL];
        rawr_t rawM[P][UMIX > 0 ? UMIX : 1][KL];
        auto load = [&](int slot, int st) {
            const rsrc_t sr = stage_rsrc(st, true), sc = stage_rsrc(st, false);
#pragma unroll
            for (int it = 0; it < UMIX; ++it) {
#pragma unroll
                for (int v = 0; v < KL; ++v)
                    rawM[slot][it][v] = TupleLd<IO, T>::load(m_row[it] ? sr : sc, m_offv[it][v]);
            }
#pragma unroll
            for (int it = 0; it < UROW; ++it) {
#pragma unroll
                for (int v = 0; v < KL; ++v) rawR[slot][it][v] = TupleLd<IO, T>::load(sr, r_offv[it][v]);
            }
#pragma unroll
            for (int it = 0; it < UCOL; ++it) {
#pragma unroll
                for (int v = 0; v < KL; ++v) {
                    if constexpr (CPC == 1) rawC[slot][it][v] = TupleLd<IO, T>::load(sc, c_offv[it][v]);
                    else rawC[slot][it][v] = Raw<CPC * TB>::load(sc, c_offv[it][v]);
                }
            }
        };
        // One step's transform and reloads, unit by unit: each unit's planes
        // are written to LDS and its register slot reloaded with stage `st`
        // right away, so that the next unit's transform overlaps these loads
        // (the four producer waves share the CU's address path, and issuing
        // a whole step's loads in one burst after the whole transform kept
        // each wave ~700 cycles a stage at issue; ViT-B fc1 / fc2 steps
        // 149 -> 144 / 144 -> 140 us, D8 at ViT-B fc1 143 -> 137, C8 fp16
        // 233 -> 226, fp32 unchanged, results bit-identical).
        auto store_load = [&](int slot, int b, int st) {
            const rsrc_t sr = stage_rsrc(st, true), sc = stage_rsrc(st, false);
#pragma unroll
            for (int it = 0; it < UMIX; ++it) {
                {
                    frag pl[TP];
                    IO v[KL * T];
                    raw_to_io(rawM[slot][it], v);
                    if constexpr (GRP != 0) grp_frags<T, IO, GRP>(v, pl);
                    else if (m_row[it]) dw_frags<T, IO, false>(v, pl);
                    else dw_frags<T, IO, true>(v, pl);
#pragma unroll
                    for (int p = 0; p < TP; ++p) sbuf[b][p][m_slot[it]] = __builtin_bit_cast(u32x4, pl[p]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int v = 0; v < KL; ++v)
                    rawM[slot][it][v] = TupleLd<IO, T>::load(m_row[it] ? sr : sc, m_offv[it][v]);
            }
#pragma unroll
            for (int it = 0; it < UROW; ++it) {
                {
                    frag pl[TP];
                    IO v[KL * T];
                    raw_to_io(rawR[slot][it], v);
                    if constexpr (GRP != 0) grp_frags<T, IO, GRP>(v, pl);
                    else dw_frags<T, IO, false>(v, pl);
#pragma unroll
                    for (int p = 0; p < TP; ++p) sbuf[b][p][r_slot[it]] = __builtin_bit_cast(u32x4, pl[p]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int v = 0; v < KL; ++v) rawR[slot][it][v] = TupleLd<IO, T>::load(sr, r_offv[it][v]);
            }
#pragma unroll
            for (int it = 0; it < UCOL; ++it) {
                {
                    IO all[KL * CPC * T];
                    raw_to_io(rawC[slot][it], all);
#pragma unroll
                    for (int jj = 0; jj < CPC; ++jj) {
                        IO v[KL * T];
#pragma unroll
                        for (int r = 0; r < KL; ++r)
#pragma unroll
                            for (int t = 0; t < T; ++t) v[r * T + t] = all[(r * CPC + jj) * T + t];
                        frag pl[TP];
                        if constexpr (GRP != 0) grp_frags<T, IO, GRP>(v, pl);
                        else dw_frags<T, IO, true>(v, pl);
#pragma unroll
                        for (int p = 0; p < TP; ++p) sbuf[b][p][c_slot[it][jj]] = __builtin_bit_cast(u32x4, pl[p]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int v = 0; v < KL; ++v) {
                    if constexpr (CPC == 1) rawC[slot][it][v] = TupleLd<IO, T>::load(sc, c_offv[it][v]);
                    else rawC[slot][it][v] = Raw<CPC * TB>::load(sc, c_offv[it][v]);
                }
            }
        };
        // Every step is unconditional (stages past the chunk load zeros through
        // the range check), so the number of loads issued after any slot's
        // loads is the same on every path and the compiler's vmcnt waits are
        // exact: (P - 1) stages of loads, within the counter's range.
        // prologue: stages 0 .. P-1 requested, stage 0 transformed, its slots
        // refilled with stage P
        // (scheduling barriers keep the compiler from hoisting a unit's
        // reload above its transform, which would hold P + 1 stages of
        // tuples in registers)
#pragma unroll
        for (int jj = 0; jj < P; ++jj) load(jj, jj);
        store_load(0, 0, P);
        ring_barrier();
        for (int s0 = 0; s0 < nstp; s0 += UNR) {
#pragma unroll
            for (int i = 0; i < UNR; ++i) {
                // step s0 + i: stage s0 + i + 1 -> buffer (i + 1) % 2, and its
                // register slot takes stage s0 + i + 1 + P
                store_load((i + 1) % P, (i + 1) % 2, s0 + i + 1 + P);
                ring_barrier();
            }
        }
        return;
    }

    // ---------------- consumers ----------------
    const int wm = wave % WM, wn = wave / WM;
    acc_t acc[CB][TP];
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int p = 0; p < TP; ++p) acc[j][p] = acc_t{};
    const int ar = wm * 32 + lr;
    ring_barrier();
    for (int st = 0; st < nstp; ++st) {   // stages past nst hold zeros
        const int b = st & 1;
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
            const int q = sl * 2 + lh;
            frag aF[TP], aN[NNEG];
#pragma unroll
            for (int p = 0; p < TP; ++p)
                aF[p] = __builtin_bit_cast(frag, sbuf[b][p][ar * RUNS + (q ^ dw_swz<RUNS>(ar))]);
            if constexpr (!G3 && GRP == 0) make_neg<T, MM, true>(aF, aN);
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int bc = dw_row<CPC>((wn * CB + j) * 32 + lr);
                if constexpr (G3) {   // diagonal plane products, one column fragment at a time
#pragma unroll
                    for (int p = 0; p < TP; ++p)
                        acc[j][p] = MM::mma(
                            aF[p], __builtin_bit_cast(frag, sbuf[b][p][SR + bc * RUNS + (q ^ dw_swz<RUNS>(bc))]),
                            acc[j][p]);
                } else {
                    frag bF[T];
#pragma unroll
                    for (int p = 0; p < T; ++p)
                        bF[p] = __builtin_bit_cast(frag, sbuf[b][p][SR + bc * RUNS + (q ^ dw_swz<RUNS>(bc))]);
                    if constexpr (GRP != 0) oct_mma_dw<MM, SWAP>(acc[j], aF, bF);
                    else freq_mma<T, MM, true>(acc[j], aF, aN, bF);
                }
            }
        }
        ring_barrier();
    }
    dw_epilogue<T, IO, CB, SWAP, DIRECT, TP, GRP>(acc, r0 + wm * 32, c0 + wn * CB * 32, lh, lr, NR, NCc, CT, DT, split,
                                         ws, dw);
}

// ===========================================================================
// Weight-gradient kernel with an LDS copy ring (orders 2, 4, 8): the product
// of dw_kernel, but the raw tuples of each stage are copied HBM -> LDS by the
// buffer unit into an NS-deep ring (no VGPR staging), so NS - 1 stages of
// loads stay in flight while one is multiplied.  (dw_kernel stages one stage
// through registers, and its loads wait out the full memory latency every
// stage.)  Each wave reads the raw tuples of its own fragments from LDS --
// KL consecutive rows n of one channel per lane -- and applies the group DFT
// itself, so a tuple is transformed by each of the two waves that use it.
// LDS stage layout (bytes): row part [KSTG rows n][BR channels][T] followed by
// the column part [KSTG][BC][T]; each row n of a part is one contiguous run
// of the source row.  The stage offset (rows) rides in the scalar offset; the
// last stage checks each chunk's row against the chunk end, channel tails are
// out-of-range offsets.
// ===========================================================================
template <int T, typename IO, int WM, int WN, int CB, int KS, int NS, bool SWAP, bool DIRECT, int OCC>
__global__ __launch_bounds__(WM *WN * 64, OCC) void dwr_kernel(
    const IO *__restrict__ x, const IO *__restrict__ dy, float *__restrict__ ws,
    IO *__restrict__ dw, int N, int CT, int DT, int chunk) {
    typedef M32<IO> MM;
    typedef typename MM::frag frag;
    typedef typename MM::acc_t acc_t;
    constexpr int ES = sizeof(IO), KL = MM::KL, TB = T * ES;
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int BR = WM * 32, BC = WN * CB * 32;
    constexpr int KSTG = KS * 2 * KL;                       // rows n per stage
    constexpr int RROW = BR * TB / 16, CROW = BC * TB / 16;  // chunks per row n
    constexpr int ACH = KSTG * RROW, BCH = KSTG * CROW, SCH = ACH + BCH;
    constexpr int LPS = SCH / NT;
    constexpr int NNEG = (T - 1) / 2 > 0 ? (T - 1) / 2 : 1;
    typedef typename Raw<TB>::type rawt;
    static_assert(Pow2<T>::value && TB >= 4, "a tuple is one aligned LDS read");
    static_assert(ACH % 64 == 0 && SCH % NT == 0, "stage shape");
    static_assert((NS - 1) * LPS < 64 && NS >= 2, "vmcnt range");

    __shared__ __attribute__((aligned(16))) u32x4 ring[NS][SCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 31, lh = lane >> 5;

    const IO *src_r = SWAP ? x : dy;
    const IO *src_c = SWAP ? dy : x;
    const int NR = SWAP ? CT : DT, NCc = SWAP ? DT : CT;
    const int tiles_c = (NCc + BC - 1) / BC;
    const int tiles = ((NR + BR - 1) / BR) * tiles_c;
    const int t_all = xcd_tile(blockIdx.x, gridDim.x);
    const int split = t_all / tiles, tile = t_all % tiles;
    const int r0 = (tile / tiles_c) * BR, c0 = (tile % tiles_c) * BC;
    const int nbeg = split * chunk;
    const int nrows = min(N, nbeg + chunk) - nbeg;
    const int nst = (nrows + KSTG - 1) / KSTG;

    const rsrc_t rr = make_rsrc(src_r + (size_t)nbeg * NR * T, (uint32_t)nrows * NR * TB);
    const rsrc_t rc = make_rsrc(src_c + (size_t)nbeg * NCc * T, (uint32_t)nrows * NCc * TB);

    // ---- per-thread copy slots: chunk (li * NW + wave) * 64 + lane ----
    uint32_t l_off[LPS];
    int l_kk[LPS];
#pragma unroll
    for (int li = 0; li < LPS; ++li) {
        const int i = (li * NW + wave) * 64 + lane;
        if (i < ACH) {
            const int n = i / RROW, q = i % RROW;
            l_off[li] = r0 + q * 16 / TB < NR ? ((uint32_t)n * NR + r0) * TB + q * 16 : OOB;
            l_kk[li] = n;
        } else {
            const int n = (i - ACH) / CROW, q = (i - ACH) % CROW;
            l_off[li] = c0 + q * 16 / TB < NCc ? ((uint32_t)n * NCc + c0) * TB + q * 16 : OOB;
            l_kk[li] = n;
        }
    }
    auto issue = [&](int st) {
        if (st >= nst) return;
        const int k0 = st * KSTG;
        dma_stage<LPS, NW, ACH>(rr, rc, ring[st % NS], l_off, l_kk, wave, (uint32_t)k0 * NR * TB,
                                (uint32_t)k0 * NCc * TB, k0 + KSTG <= nrows, k0, nrows, nrows);
    };

    acc_t acc[CB][T];
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int p = 0; p < T; ++p) acc[j][p] = acc_t{};

    frag aF[KS][T], aN[KS][NNEG], bF[KS][CB][T];
    const int ach = wm * 32 + lr;
    auto load_frags = [&](const u32x4 *buf) {
        const char *b = reinterpret_cast<const char *>(buf);
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
            const int n0 = (sl * 2 + lh) * KL;
            rawt t[KL];
            IO io[KL * T];
#pragma unroll
            for (int v = 0; v < KL; ++v) t[v] = *reinterpret_cast<const rawt *>(b + ((n0 + v) * BR + ach) * TB);
            raw_to_io(t, io);
            tuples_to_frags<T, IO>(io, aF[sl]);
            make_neg<T, MM, true>(aF[sl], aN[sl]);
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int bch = (wn * CB + j) * 32 + lr;
#pragma unroll
                for (int v = 0; v < KL; ++v)
                    t[v] = *reinterpret_cast<const rawt *>(b + ACH * 16 + ((n0 + v) * BC + bch) * TB);
                raw_to_io(t, io);
                tuples_to_frags<T, IO>(io, bF[sl][j]);
            }
        }
    };

#pragma unroll
    for (int st = 0; st < NS; ++st) issue(st);
    if (NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * LPS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    ring_barrier();
    load_frags(ring[0]);
    for (int ks = 0; ks < nst; ++ks) {
#pragma unroll
        for (int sl = 0; sl < KS; ++sl)
#pragma unroll
            for (int j = 0; j < CB; ++j) freq_mma<T, MM, true>(acc[j], aF[sl], aN[sl], bF[sl][j]);
        if (ks + 1 < nst) {
            if (ks + NS - 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            ring_barrier();   // every wave is done reading stage ks
            issue(ks + NS);
            load_frags(ring[(ks + 1) % NS]);
        }
    }

    dw_epilogue<T, IO, CB, SWAP, DIRECT>(acc, r0 + wm * 32, c0 + wn * CB * 32, lh, lr, NR, NCc, CT, DT, split,
                                         ws, dw);
}

// dw[d, c, :] = IDFT( sum_{s < S} ws[s, ., ., :] ), s in increasing order.
// Thread idx walks the workspace order: (d, c) with c fastest, or (SWAP)
// (c, d) with d fastest.
template <int T, typename IO, bool SWAP, int GRP = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void dw_finalize(
    const float *__restrict__ ws, IO *__restrict__ dw, int CT, int DT, int S) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t plane = (size_t)DT * CT;
    if (idx >= plane) return;
    float f[T];
#pragma unroll
    for (int p = 0; p < T; ++p) f[p] = 0.0f;
    // FB independent loads in flight per batch (one thread per output
    // element leaves few threads per CU), added in split order
    constexpr int FB = 16;
    int s = 0;
    for (; s + FB - 1 < S; s += FB) {
        float v[FB][T];
#pragma unroll
        for (int u = 0; u < FB; ++u) {
            const float *src = ws + ((size_t)(s + u) * plane + idx) * T;
            if constexpr (Pow2<T>::value) {
                typedef float ftup __attribute__((ext_vector_type(T)));
                const ftup w = *reinterpret_cast<const ftup *>(src);
#pragma unroll
                for (int p = 0; p < T; ++p) v[u][p] = w[p];
            } else {
#pragma unroll
                for (int p = 0; p < T; ++p) v[u][p] = src[p];
            }
        }
#pragma unroll
        for (int u = 0; u < FB; ++u)
#pragma unroll
            for (int p = 0; p < T; ++p) f[p] += v[u][p];
    }
    for (; s + 3 < S; s += 4) {
        float v[4][T];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float *src = ws + ((size_t)(s + u) * plane + idx) * T;
#pragma unroll
            for (int p = 0; p < T; ++p) v[u][p] = src[p];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int p = 0; p < T; ++p) f[p] += v[u][p];
    }
    for (; s < S; ++s) {
        const float *src = ws + ((size_t)s * plane + idx) * T;
#pragma unroll
        for (int p = 0; p < T; ++p) f[p] += src[p];
    }
    const size_t d = SWAP ? idx % DT : idx / CT, c = SWAP ? idx / DT : idx % CT;
    if constexpr (Pow2<T>::value) {
        typedef typename Tuple<IO, T>::type tup;
        *reinterpret_cast<tup *>(dw + (d * CT + c) * T) = grp_out<T, IO, GRP>(f, 0.0f);
    } else {
        float y[T];
        Dft<T>::inv(f, y);
#pragma unroll
        for (int t = 0; t < T; ++t) dw[(d * CT + c) * T + t] = (IO)y[t];
    }
}

// Weight spectrum in both orientations, in the blocked layout the row kernel
// streams (see SpecLayout).  One thread per (column, run of KL consecutive k):
// it transforms those KL tuples of Wt and writes the T 16-byte chunks, one per
// plane, of that column and k-run.  Part 0 (columns d, k = c) is followed by
// part 1 (columns c, k = d); padding is zero.  Each value is the fp32 group
// DFT of one Wt tuple rounded once to the I/O type by the same code for both
// parts, so the two orientations hold identical values.
template <int T, typename IO, int GRP = 0>
__global__ __launch_bounds__(256) void spectrum_kernel(const IO *__restrict__ wt, IO *__restrict__ what,
                                                       int CT, int DT, int kb0, int kb1,
                                                       int64_t units0, int64_t units) {
    constexpr int KL = 16 / sizeof(IO), KC = 2 * KL;
    // stored planes: T, or with Gauss's products the weight-side planes of
    // gauss_b (part 1 in their conjugate form) plus any zero padding plane
    constexpr bool G3 = Gauss<T, IO>::V && GRP == 0;
    constexpr int TP = GRP ? T : math_planes<T, IO>(), TPS = GRP ? T : stored_planes<T, IO>();
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const bool second = u >= units0;
    const int64_t uu = second ? u - units0 : u;
    const int kbn = second ? kb1 : kb0;
    const int NC = second ? CT : DT, K = second ? DT : CT;
    const int h = (int)(uu % 2), c = (int)((uu / 2) % 32);
    const int64_t blk = uu / 64;           // (column block, k block) of the part
    const int kb = (int)(blk % kbn), cb = (int)(blk / kbn);
    const int col = cb * 32 + c, k0 = kb * KC + h * KL;
    IO v[TPS][KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = k0 + j;
        float f[T], g[TPS];
#pragma unroll
        for (int q = 0; q < T; ++q) f[q] = 0.0f;
        if (col < NC && k < K) {
            const int d = second ? k : col, cx = second ? col : k;
            const IO *wp = wt + ((size_t)d * CT + cx) * T;
            float xv[T];
            if constexpr (Pow2<T>::value) {
                typedef typename Tuple<IO, T>::type tup;
                const tup w = *reinterpret_cast<const tup *>(wp);
#pragma unroll
                for (int t = 0; t < T; ++t) xv[t] = (float)w[t];
            } else {
#pragma unroll
                for (int t = 0; t < T; ++t) xv[t] = (float)wp[t];
            }
            GrpT<T, GRP>::fwd(xv, f);
            if (GRP && second) {   // octic: part 1 holds the E blocks transposed
                const float t = f[5];
                f[5] = f[6];
                f[6] = t;
            }
        }
        if constexpr (G3) {
            gauss_b<T>(f, g, second);
        } else {
#pragma unroll
            for (int q = 0; q < T; ++q) g[q] = f[q];
        }
#pragma unroll
        for (int q = TP; q < TPS; ++q) g[q] = 0.0f;
#pragma unroll
        for (int q = 0; q < TPS; ++q) v[q][j] = (IO)g[q];
    }
    // chunk of plane q: block blk, plane q, column c, k-run half h
    IO *part = what + (second ? units0 * TPS * KL : 0);
#pragma unroll
    for (int q = 0; q < TPS; ++q) {
        u32x4 w;
        __builtin_memcpy(&w, v[q], 16);
        *reinterpret_cast<u32x4 *>(part + ((blk * TPS + q) * 64 + c * 2 + h) * KL) = w;
    }
}

// ===========================================================================
// Bias gradient: db[d] = sum_{n,g} dy[n, d, g].  dy is read as a flat
// [N][D_T*T] matrix in 16-byte chunks.  Block (x, y) covers BIAS_CL chunks of
// every row of split y; thread (chunk lane cl, row group rg < BIAS_RG) keeps
// a column sum per element of its chunk over rows nbeg + rg, + BIAS_RG, ...
// in increasing n (four independent loads in flight).  The row groups are
// then added in rg order through LDS and the T elements of each d in g order.
// Split partials go to the workspace as [split][D_T] and bias_finalize adds
// them in a fixed order (or the block writes db directly when there is one
// split).  A block covers CL 16-byte chunks of a row with CL a multiple of
// T (16 for T = 2, 4, 8; 15, 15, 12, 14 for T = 3, 5, 6, 7), so no tuple
// straddles two blocks; the block has CL * BIAS_RG threads.
// ===========================================================================
constexpr int BIAS_RG = 16;
__host__ __device__ constexpr int bias_cl(int T) { return (T & (T - 1)) == 0 ? 16 : T * (16 / T); }

template <typename IO, bool DIRECT, int CL, bool EL>
__global__ __launch_bounds__(256) void bias_partial(const IO *__restrict__ dy, float *__restrict__ ws,
                                                    IO *__restrict__ db, int N, int DT, int T, int chunk) {
    constexpr int EC = 16 / (int)sizeof(IO);   // elements per 16-byte chunk
    constexpr int BE = CL * EC;                // elements of a row per block
    __shared__ float red[BIAS_RG][BE];
    const int cl = threadIdx.x % CL, rg = threadIdx.x / CL;
    const int rowlen = DT * T;
    const int e0 = blockIdx.x * BE + cl * EC;
    const int nbeg = blockIdx.y * chunk, nend = min(N, nbeg + chunk);
    float acc[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) acc[e] = 0.0f;
    typedef IO vec_t __attribute__((ext_vector_type(EC)));
    if (EL && e0 < rowlen) {
        // rows that are not a whole number of 16-byte chunks: one element at
        // a time, elements past the row end skipped
        for (int n = nbeg + rg; n < nend; n += BIAS_RG) {
            const IO *p = dy + (size_t)n * rowlen + e0;
#pragma unroll
            for (int e = 0; e < EC; ++e)
                if (e0 + e < rowlen) acc[e] += (float)p[e];
        }
    } else if (e0 < rowlen) {
        const size_t step = (size_t)BIAS_RG * rowlen;
        const IO *p = dy + (size_t)(nbeg + rg) * rowlen + e0;
        int n = nbeg + rg;
        for (; n + 3 * BIAS_RG < nend; n += 4 * BIAS_RG, p += 4 * step) {
            vec_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const vec_t *>(p + u * step);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < EC; ++e) acc[e] += (float)v[u][e];
        }
        for (; n < nend; n += BIAS_RG, p += step) {
            const vec_t v = *reinterpret_cast<const vec_t *>(p);
#pragma unroll
            for (int e = 0; e < EC; ++e) acc[e] += (float)v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < EC; ++e) red[rg][cl * EC + e] = acc[e];
    __syncthreads();
    const int t = threadIdx.x;
    const int d = (blockIdx.x * BE) / T + t;
    if (t < BE / T && d < DT) {
        float tot = 0.0f;
        for (int g = 0; g < T; ++g) {
            const int j = t * T + g;
            float v = red[0][j];
#pragma unroll
            for (int r = 1; r < BIAS_RG; ++r) v += red[r][j];
            tot += v;
        }
        if (DIRECT) db[d] = (IO)tot;
        else ws[(size_t)blockIdx.y * DT + d] = tot;
    }
}

// db[d] = sum of the S split partials: thread (d lane, split group sg of 4)
// adds splits sg, sg + 4, ... in order, then the groups are added in sg order.
template <typename IO>
__global__ __launch_bounds__(256) void bias_finalize(const float *__restrict__ ws, IO *__restrict__ db,
                                                     int DT, int S) {
    __shared__ float red[4][64];
    const int dl = threadIdx.x & 63, sg = threadIdx.x >> 6;
    const int d = blockIdx.x * 64 + dl;
    float tot = 0.0f;
    if (d < DT) {
        int s = sg;
        for (; s + 12 < S; s += 16) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = ws[(size_t)(s + 4 * u) * DT + d];
#pragma unroll
            for (int u = 0; u < 4; ++u) tot += v[u];
        }
        for (; s < S; s += 4) tot += ws[(size_t)s * DT + d];
    }
    red[sg][dl] = tot;
    __syncthreads();
    if (sg == 0 && d < DT) db[d] = (IO)(((red[0][dl] + red[1][dl]) + red[2][dl]) + red[3][dl]);
}

// ===========================================================================
// Launch configurations (a fixed rule on T and dtype) and host launchers.
//
// The configurations come from sweeps on MI355X; the values below are the
// measured best.
//   RowCfg<4, f16>: 128 x 64 tiles (4 waves of 32 rows, 64 columns each): every
//   activation row is transformed by one wave only.  ViT-B fc1 fp16 forward /
//   input gradient 41.5 / 41.0 us with the 64 x 128 tiles of two column
//   waves, 40.9 / 40.0 us with these; 128 x 128 (8 waves), 64 x 256 and
//   3-deep copy rings were slower (44 - 50 us).
// ===========================================================================
template <int T, typename IO> struct RowCfg;      // forward / input gradient
template <> struct RowCfg<2, f16>   { enum { WM = 2, WN = 2, CB = 4, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<4, f16>   { enum { WM = 4, WN = 1, CB = 2, KS = 1, NS = 2, OCC = 2 }; };
// Pipelined main loop (row_kernel's PIPE): measured 1-1.5 us faster at the
// ViT-B fc1/fc2 shapes for order 4 in fp16, and at order 2 (steady-state
// training steps: fp16 N = 32768 at 1024 -> 1024 637 -> 620 us, at
// 2048 -> 2048 2384 -> 2330; fp32 N = 12608 at 512 -> 512 397 -> 378,
// N = 16384 at 1024 -> 1024 1644 -> 1571; small layers unchanged).  It needs
// a second set of A fragments, so the narrow tiles (4 workgroups per CU) and
// the orders whose registers do not fit (order 8 spills) or that measured
// slower (order 3) keep the plain loop.
template <int T, typename IO> struct RowPipe { enum { V = 0 }; };
template <> struct RowPipe<4, f16> { enum { V = 1 }; };
template <> struct RowPipe<2, f16> { enum { V = 1 }; };
template <> struct RowPipe<2, float> { enum { V = 1 }; };
// Narrow alternative (64 x 64 tiles, four workgroups per CU) for layers whose
// RowCfg tiles leave CUs idle or spill into a nearly empty extra round.
template <int T, typename IO> struct RowCfgN { enum { USE = 0 }; };
template <> struct RowCfgN<4, f16>  { enum { USE = 1, WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 4 }; };
template <> struct RowCfg<8, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<2, float> { enum { WM = 2, WN = 2, CB = 4, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<4, float> { enum { WM = 2, WN = 2, CB = 2, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<8, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 2 }; };
// Orders 3, 5, 6, 7: a stage is 128*KS*T*(1+CB) chunks, which must fill
// whole 256-thread rounds (KS*T*(1+CB) even).
template <> struct RowCfg<3, f16>   { enum { WM = 2, WN = 2, CB = 2, KS = 2, NS = 2, OCC = 2 }; };
template <> struct RowCfg<5, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 2 }; };
template <> struct RowCfg<6, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 2 }; };
template <> struct RowCfg<7, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<3, float> { enum { WM = 2, WN = 2, CB = 3, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<5, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<6, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 2 }; };
template <> struct RowCfg<7, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 2, OCC = 2 }; };
// Per group: the octic layer (GRP = 1) takes the order-8 tiles (64 x 64,
// measured best among 128 x 32, 32 x 128, 64 x 32, 128 x 64, 64 x 128,
// two-slice stages and 3-deep rings at the D8 layers N = 12608, 768 -> 3072
// and N = 16384, 1024 -> 4096, both dtypes).
template <int T, typename IO, int GRP> struct RowCfgG : RowCfg<T, IO> {};

template <int T, typename IO> struct DwCfg {     // weight gradient (tile BR x BC)
    enum { WM = 2, WN = 2, CB = 1, KS = 1, OCC = 2 };
};
template <> struct DwCfg<3, f16>   { enum { WM = 2, WN = 2, CB = 2, KS = 2, OCC = 2 }; };
template <> struct DwCfg<5, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 2, OCC = 2 }; };
template <> struct DwCfg<6, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 2, OCC = 2 }; };
template <> struct DwCfg<7, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 2, OCC = 1 }; };
template <> struct DwCfg<2, f16>   { enum { WM = 2, WN = 2, CB = 2, KS = 2, OCC = 2 }; };
template <> struct DwCfg<4, f16>   { enum { WM = 2, WN = 2, CB = 2, KS = 2, OCC = 2 }; };
// Narrow alternative (64 x 64 tiles) for layers that the DwCfg tiles cut into
// too few tiles to fill the GPU (dw_plan picks it when it launches at least
// 25% more workgroups; measured at 384 -> 1152 channels, N = 12608, fp16:
// 32.0 -> 27.2 us).
template <int T, typename IO> struct DwCfgN { enum { USE = 0, WM = 2, WN = 2, CB = 1, KS = 1, OCC = 2 }; };
template <> struct DwCfgN<4, f16>  { enum { USE = 1, WM = 2, WN = 2, CB = 1, KS = 2, OCC = 2 }; };
template <> struct DwCfg<8, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 2, OCC = 1 }; };
template <> struct DwCfg<2, float> { enum { WM = 2, WN = 2, CB = 2, KS = 2, OCC = 2 }; };
template <> struct DwCfg<4, float> { enum { WM = 2, WN = 2, CB = 1, KS = 2, OCC = 2 }; };
template <> struct DwCfg<8, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, OCC = 2 }; };

// Producer/consumer weight gradient (dwp_kernel): CB 32-column blocks per
// consumer wave (T * CB planes of accumulators <= 8 x 16 per lane), KS MFMA k
// slices per stage, producer register ring of P stages (its tuples must fit
// the registers a producer has beside the transform).
template <int T, typename IO> struct DwpCfg { enum { USE = 0, CB = 1, KS = 2, P = 2 }; };
template <typename IO> struct DwpCfg<8, IO> { enum { USE = 1, CB = 1, KS = 2, P = 2 }; };
// fp32 with Gauss's products stages 11 planes: 8-row stages, since two
// buffers of 16-row stages (176 KB) would not fit the LDS
template <> struct DwpCfg<8, float> { enum { USE = 1, CB = 1, KS = 1, P = 2 }; };
// Order 4 (dw_plan takes it unless the narrow or ring-staged plan runs): 64 x 128
// tiles, 32-row stages (the fp32 planes are Gauss's five).
template <> struct DwpCfg<4, f16> { enum { USE = 1, CB = 2, KS = 2, P = 2 }; };
template <> struct DwpCfg<4, float> { enum { USE = 1, CB = 2, KS = 2, P = 2 }; };
// Order 2 in fp16 (dw_plan takes it always): 64 x 256 tiles.
template <> struct DwpCfg<2, f16> { enum { USE = 1, CB = 4, KS = 2, P = 2 }; };
// The octic group: the order-8 configuration, but 16-row stages in fp32 too
// (its 8 planes fit two LDS stage buffers, where Gauss's 11 of the cyclic
// order 8 do not).
template <typename IO> struct DwpCfgOct : DwpCfg<8, IO> {};
template <> struct DwpCfgOct<float> { enum { USE = 1, CB = 1, KS = 2, P = 2 }; };

// Ring-staged weight gradient, used for fp32 layers of order 2 or 4 whose
// register-staged plan would not fill the GPU: 64 x 64 tiles, a stage of
// KS * 2 * KL rows n, NS stages of LDS per workgroup.  (Order 8 instances
// exist and are correct but are not dispatched.)
template <int T, typename IO> struct DwrCfg;
template <> struct DwrCfg<2, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 4 }; };
template <> struct DwrCfg<4, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 3 }; };
template <> struct DwrCfg<8, f16>   { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 1 }; };
template <> struct DwrCfg<2, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 4 }; };
template <> struct DwrCfg<4, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 3 }; };
template <> struct DwrCfg<8, float> { enum { WM = 2, WN = 2, CB = 1, KS = 1, NS = 3, OCC = 1 }; };

// Compute units of the current device (cached per device id); MI355X's count
// when the device or its attribute cannot be queried, so the launch plans
// never divide by zero.
static int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MI355X_CUS;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return MI355X_CUS;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int T, typename IO, int GRP = 0>
static uint32_t spectrum_part_bytes(int K, int NC) {
    constexpr int KC = 2 * M32<IO>::KL, TPS = GRP ? T : stored_planes<T, IO>();
    return (uint32_t)(((NC + 31) / 32) * (int64_t)((K + KC - 1) / KC) * TPS * 32 * KC * sizeof(IO));
}

// Activation rows of K tuples are a whole number of 16-byte chunks (the
// buffer unit copies them HBM -> LDS) unless the layout below says otherwise:
// then the element-granular copy path (EL) runs, with pieces of `gran` bytes.
template <int T, typename IO> constexpr bool can_be_ragged() { return (T * (int)sizeof(IO)) % 16 != 0; }
static int row_gran(int K, int TB) {
    const int64_t b = (int64_t)K * TB;
    return (b & 7) == 0 ? 8 : (b & 3) == 0 ? 4 : 2;
}

// The few-tile kernel with KW waves (k slices per stage): 8 for orders up to
// 4 when the contraction is long (N = 256, 4096 -> 4096 fp16: forward 16.5
// -> 14.8 us, input gradient 15.8 -> 15.0 us: half the stages and twice the
// waves to hide copy latency), else 4 (at K = 16 the larger workgroup only
// adds launch and reduction time: 7.4 -> 9.5 us; orders above 4 do not fit
// eight waves' stage in LDS).
template <int T, typename IO, bool CONJ, int KW, int GRP = 0>
static hipError_t launch_rowk_kw(const void *act, const void *bpl, const void *bias, void *out, int M, int K,
                                 int NC, hipStream_t st) {
    const int tk = ((M + 31) / 32) * ((NC + 31) / 32);
    const int col_major = NC > M;   // consecutive tiles share the larger operand
    constexpr int NSK = T > 4 || KW > 4 ? 2 : 3;
    constexpr int TB = T * (int)sizeof(IO);
    if constexpr (can_be_ragged<T, IO>()) {
        if (((int64_t)K * TB) % 16 != 0) {
            hipLaunchKernelGGL((rowk_kernel<T, IO, CONJ, NSK, true, KW, GRP>), dim3(tk), dim3(KW * 64), 0, st,
                               (const IO *)act, (const IO *)bpl, (IO *)out, M, K, NC,
                               spectrum_part_bytes<T, IO, GRP>(K, NC), (const IO *)bias, col_major, row_gran(K, TB));
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((rowk_kernel<T, IO, CONJ, NSK, false, KW, GRP>), dim3(tk), dim3(KW * 64), 0, st,
                       (const IO *)act, (const IO *)bpl, (IO *)out, M, K, NC, spectrum_part_bytes<T, IO, GRP>(K, NC),
                       (const IO *)bias, col_major, 16);
    return hipGetLastError();
}

template <int T, typename IO, bool CONJ, int GRP = 0>
static hipError_t launch_rowk(const void *act, const void *bpl, const void *bias, void *out, int M, int K,
                              int NC, hipStream_t st) {
    if constexpr (T <= 4) {
        if (K >= 256) return launch_rowk_kw<T, IO, CONJ, 8, GRP>(act, bpl, bias, out, M, K, NC, st);
    }
    return launch_rowk_kw<T, IO, CONJ, 4, GRP>(act, bpl, bias, out, M, K, NC, st);
}

// Whether a layer with `tiles` row-kernel tiles (contraction length K) runs
// on the few-tile kernel instead: 32 x 32 tiles with the k range of each
// stage split over the waves (rowk_kernel).  Below half the CUs in tiles it
// always does.  Below three quarters of them it does too when K >= 256, for
// fp32 (the octic group included) and for orders 5-7 in fp16, whose tiles
// do more matrix work per stage (whole training steps of small layers in
// the steady state: fp32 orders 2-8 at 126-189 tiles 2-30% faster, the
// octic group in fp32 at 128 tiles 20-25% (at 188 tiles 1.5% slower), fp16
// orders 5-7 at 128 tiles 4-17%; at K = 128, or at 197-250 tiles, the row
// tiles stayed ahead by up to 19%).  fp16 orders 2, 3 and 8 and the octic
// group in fp16 keep the half-CU rule (the wider one: order 3 5% slower,
// the others within 1%).  Order 4
// in fp16, whose pipelined 128 x 64 tiles are the fastest row tiles, keeps
// them down to a quarter of the CUs unless K >= 512 (64 tiles at K = 256,
// N = 2048, 256 -> 256: step 46.0 -> 43.0 us; at K = 512 the few-tile
// kernel stayed 4% ahead).
template <int T, typename IO, int GRP>
static bool rowk_first(int tiles, int K, int cus) {
    if constexpr (GRP == 0 && T == 4 && sizeof(IO) == 2) return 4 * tiles < cus || (2 * tiles < cus && K >= 512);
    if constexpr (sizeof(IO) == 4 || (GRP == 0 && T >= 5 && T <= 7))
        return 2 * tiles < cus || (4 * tiles < 3 * cus && K >= 256);
    return 2 * tiles < cus;
}

template <int T, typename IO, bool CONJ, int GRP = 0>
static hipError_t launch_row(const void *act, const void *bpl, const void *bias, void *out, int M, int K,
                             int NC, hipStream_t st) {
    if (M == 0) return hipSuccess;
    typedef RowCfgG<T, IO, GRP> C;
    constexpr int BM = C::WM * 32, BN = C::WN * C::CB * 32;
    const int tiles = ((M + BM - 1) / BM) * ((NC + BN - 1) / BN);
    const int cus = cu_count();
    if (rowk_first<T, IO, GRP>(tiles, K, cus)) return launch_rowk<T, IO, CONJ, GRP>(act, bpl, bias, out, M, K, NC, st);
    constexpr int TB = T * (int)sizeof(IO);
    if constexpr (can_be_ragged<T, IO>()) {
        if (((int64_t)K * TB) % 16 != 0) {
            // ragged rows: the wide tiles with the plain loop, every tile whole
            hipLaunchKernelGGL((row_kernel<T, IO, CONJ, C::WM, C::WN, C::CB, C::KS, C::NS, C::OCC, false, true, GRP>),
                               dim3(tiles), dim3(C::WM * C::WN * 64), 0, st, (const IO *)act, (const IO *)bpl,
                               (IO *)out, M, K, NC, spectrum_part_bytes<T, IO, GRP>(K, NC), (const IO *)bias,
                               C::CB % 2 == 0 ? ((M + BM - 1) / BM) * ((NC + BN / 2 - 1) / (BN / 2) / 2) : tiles,
                               row_gran(K, TB));
            return hipGetLastError();
        }
    }
    if constexpr ((int)RowCfgN<T, IO>::USE != 0 && !Gauss<T, IO>::V && GRP == 0) {
        // Narrow tiles when the wide ones leave CUs idle, or need more
        // rounds of resident workgroups than the narrow ones (measured at
        // 384 -> 1152 channels, N = 12608, fp16: forward 18.6 -> 15.5 us,
        // input gradient 18.4 -> 16.6 us; long layers stay on wide tiles).
        typedef RowCfgN<T, IO> Q;
        constexpr int BNq = Q::WN * Q::CB * 32;
        const int tq = ((M + Q::WM * 32 - 1) / (Q::WM * 32)) * ((NC + BNq - 1) / BNq);
        const int rounds = (tiles + C::OCC * cus - 1) / (C::OCC * cus);
        const int rounds_q = (tq + Q::OCC * cus - 1) / (Q::OCC * cus);
        if (tiles < cus || rounds_q < rounds) {
            hipLaunchKernelGGL((row_kernel<T, IO, CONJ, Q::WM, Q::WN, Q::CB, Q::KS, Q::NS, Q::OCC, false, false>),
                               dim3(tq), dim3(Q::WM * Q::WN * 64), 0, st, (const IO *)act, (const IO *)bpl,
                               (IO *)out, M, K, NC, spectrum_part_bytes<T, IO>(K, NC), (const IO *)bias, tq, 16);
            return hipGetLastError();
        }
    }
    // Work plan in half-width column units (row_kernel): pairs of units run
    // as whole tiles, an odd last unit per row block as a half-width
    // workgroup.  When the pairs take more than one round of resident
    // workgroups and the half-width workgroups left after the whole rounds
    // fit in one round, the pairs of that last round are split into halves
    // too (nbig = pairs run whole); when there are fewer pairs than CUs and
    // they fit one round as halves, all of them run as halves, so that no CU
    // idles (steady-state steps: fp16 order 3 at N = 8192, 128 -> 512
    // 67.5 -> 64.5 us, order 2 at N = 8192, 256 -> 256 44.9 -> 43.4, fp32
    // ViT-S proj 80.0 -> 78.0; no layer slower).
    int nbig = tiles, grid = tiles;
    if constexpr (C::CB % 2 == 0) {
        const int hn = (NC + BN / 2 - 1) / (BN / 2), fpr = hn / 2;
        const int rblocks = (M + BM - 1) / BM, npairs = rblocks * fpr, nodd = rblocks * (hn % 2);
        const int slots = C::OCC * cus;
        const int full = npairs / slots * slots, rem = npairs - full;
        nbig = npairs;
        if (rem > 0 && 2 * rem + nodd <= slots && (full > 0 || npairs < cus)) nbig = full;
        grid = nbig + 2 * (npairs - nbig) + nodd;
    }
    hipLaunchKernelGGL(
        (row_kernel<T, IO, CONJ, C::WM, C::WN, C::CB, C::KS, C::NS, C::OCC, (bool)RowPipe<T, IO>::V && GRP == 0,
                    false, GRP>),
        dim3(grid), dim3(C::WM * C::WN * 64), 0, st, (const IO *)act, (const IO *)bpl, (IO *)out, M, K, NC,
        spectrum_part_bytes<T, IO, GRP>(K, NC), (const IO *)bias, nbig, 16);
    return hipGetLastError();
}

template <int T, typename IO, int GRP = 0>
static hipError_t launch_spectrum(const void *wt, void *what, int CT, int DT, hipStream_t st) {
    const SpecLayout L = spec_layout(CT, DT, T, sizeof(IO), GRP);
    constexpr int KL = 16 / sizeof(IO);
    // one thread per (column, k-run): TPS chunks each; every part is whole
    // (column block, k block) blocks of TPS * 64 chunks
    constexpr int TPS = GRP ? T : stored_planes<T, IO>();
    const int64_t units0 = L.elems0 / KL / TPS, units = (L.elems0 + L.elems1) / KL / TPS;
    hipLaunchKernelGGL((spectrum_kernel<T, IO, GRP>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                       st, (const IO *)wt, (IO *)what, CT, DT, (int)L.kb0, (int)L.kb1, units0, units);
    return hipGetLastError();
}

template <int T, typename IO, bool SWAP, class C>
static hipError_t launch_dw_reg(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl, int N,
                                int CT, int DT, hipStream_t st);
// The producer/consumer weight gradient plus the finalize when rows are split.
template <int T, typename IO, bool SWAP, bool WIDE>
static hipError_t launch_dw_pc_w(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl, int N,
                               int CT, int DT, hipStream_t st) {
    typedef DwpCfg<T, IO> C;
    const size_t n = (size_t)CT * DT;
    const int grid = pl.tiles * pl.splits;
    if (pl.splits == 1) {
        hipLaunchKernelGGL((dwp_kernel<T, IO, C::CB, C::KS, C::P, SWAP, true, WIDE>), dim3(grid), dim3(512), 0, st,
                           (const IO *)x, (const IO *)dy, (float *)ws, (IO *)dw, N, CT, DT, pl.chunk);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((dwp_kernel<T, IO, C::CB, C::KS, C::P, SWAP, false, WIDE>), dim3(grid), dim3(512), 0, st,
                       (const IO *)x, (const IO *)dy, (float *)ws, (IO *)dw, N, CT, DT, pl.chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dw_finalize<T, IO, SWAP>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float *)ws, (IO *)dw, CT, DT, pl.splits);
    return hipGetLastError();
}

template <int T, typename IO, bool SWAP>
static hipError_t launch_dw_pc(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl, int N,
                               int CT, int DT, hipStream_t st) {
    typedef DwpCfg<T, IO> C;
    constexpr int CPC = dw_cpl(T * (int)sizeof(IO), 2 * C::CB * 32 * C::KS * 2, 256);
    const int NCc = SWAP ? DT : CT;
    if constexpr (CPC > 1) {
        if (NCc % CPC == 0) return launch_dw_pc_w<T, IO, SWAP, true>(x, dy, dw, ws, pl, N, CT, DT, st);
    }
    return launch_dw_pc_w<T, IO, SWAP, false>(x, dy, dw, ws, pl, N, CT, DT, st);
}

// Weight gradient of the octic-group layer: the producer/consumer kernel on
// the octic plan (dw_plan(.., 8, .., 1)), with the octic transform and
// products, and the finalize with the octic inverse transform.
template <typename IO, bool SWAP>
static hipError_t launch_dw_octic_t(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl, int N,
                                    int CT, int DT, hipStream_t st) {
    typedef DwpCfgOct<IO> C;
    const size_t n = (size_t)CT * DT;
    const int grid = pl.tiles * pl.splits;
    if (pl.splits == 1) {
        hipLaunchKernelGGL((dwp_kernel<8, IO, C::CB, C::KS, C::P, SWAP, true, false, 1>), dim3(grid), dim3(512), 0,
                           st, (const IO *)x, (const IO *)dy, (float *)ws, (IO *)dw, N, CT, DT, pl.chunk);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((dwp_kernel<8, IO, C::CB, C::KS, C::P, SWAP, false, false, 1>), dim3(grid), dim3(512), 0,
                       st, (const IO *)x, (const IO *)dy, (float *)ws, (IO *)dw, N, CT, DT, pl.chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dw_finalize<8, IO, SWAP, 1>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float *)ws, (IO *)dw, CT, DT, pl.splits);
    return hipGetLastError();
}

template <typename IO>
static hipError_t launch_dw_octic(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                                  hipStream_t st) {
    const DwPlan pl = dw_plan(N, CT, DT, 8, sizeof(IO), 1);
    if (pl.splits == 0) {  // N == 0: the gradient is zero
        const size_t n = (size_t)CT * DT;
        hipLaunchKernelGGL((dw_finalize<8, IO, false, 1>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           (const float *)ws, (IO *)dw, CT, DT, 0);
        return hipGetLastError();
    }
    return pl.swap ? launch_dw_octic_t<IO, true>(x, dy, dw, ws, pl, N, CT, DT, st)
                   : launch_dw_octic_t<IO, false>(x, dy, dw, ws, pl, N, CT, DT, st);
}


template <int T, typename IO, bool SWAP>
static hipError_t launch_dw_t(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl,
                              int N, int CT, int DT, hipStream_t st) {
    if constexpr ((int)DwpCfg<T, IO>::USE != 0) {
        if (pl.pc) return launch_dw_pc<T, IO, SWAP>(x, dy, dw, ws, pl, N, CT, DT, st);
    }
    const size_t n = (size_t)CT * DT;
    const int grid = pl.tiles * pl.splits;
    if constexpr (Pow2<T>::value) {
      if (pl.ring) {
        typedef DwrCfg<T, IO> R;
        if (pl.splits == 1) {
            hipLaunchKernelGGL((dwr_kernel<T, IO, R::WM, R::WN, R::CB, R::KS, R::NS, SWAP, true, R::OCC>),
                               dim3(grid), dim3(R::WM * R::WN * 64), 0, st, (const IO *)x, (const IO *)dy,
                               (float *)ws, (IO *)dw, N, CT, DT, pl.chunk);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((dwr_kernel<T, IO, R::WM, R::WN, R::CB, R::KS, R::NS, SWAP, false, R::OCC>),
                           dim3(grid), dim3(R::WM * R::WN * 64), 0, st, (const IO *)x, (const IO *)dy,
                           (float *)ws, (IO *)dw, N, CT, DT, pl.chunk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((dw_finalize<T, IO, SWAP>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           (const float *)ws, (IO *)dw, CT, DT, pl.splits);
        return hipGetLastError();
      }
    }
    if constexpr ((int)DwCfgN<T, IO>::USE != 0) {
        if (pl.narrow) return launch_dw_reg<T, IO, SWAP, DwCfgN<T, IO>>(x, dy, dw, ws, pl, N, CT, DT, st);
    }
    return launch_dw_reg<T, IO, SWAP, DwCfg<T, IO>>(x, dy, dw, ws, pl, N, CT, DT, st);
}

template <int T, typename IO, bool SWAP, class C, bool WIDE>
static hipError_t launch_dw_reg_w(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl, int N,
                                  int CT, int DT, hipStream_t st) {
    const size_t n = (size_t)CT * DT;
    const int grid = pl.tiles * pl.splits;
    if (pl.splits == 1) {
        hipLaunchKernelGGL((dw_kernel<T, IO, C::WM, C::WN, C::CB, C::KS, SWAP, true, C::OCC, WIDE>), dim3(grid),
                           dim3(C::WM * C::WN * 64), 0, st, (const IO *)x, (const IO *)dy, (float *)ws,
                           (IO *)dw, N, CT, DT, pl.chunk);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((dw_kernel<T, IO, C::WM, C::WN, C::CB, C::KS, SWAP, false, C::OCC, WIDE>), dim3(grid),
                       dim3(C::WM * C::WN * 64), 0, st, (const IO *)x, (const IO *)dy, (float *)ws,
                       (IO *)dw, N, CT, DT, pl.chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dw_finalize<T, IO, SWAP>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float *)ws, (IO *)dw, CT, DT, pl.splits);
    return hipGetLastError();
}

// The register-staged weight gradient (dw_kernel) with tile configuration C,
// plus the finalize when the rows are split.  The wide loads (several
// adjacent channels per access) need channel counts that are multiples of the
// channels per access.
template <int T, typename IO, bool SWAP, class C>
static hipError_t launch_dw_reg(const void *x, const void *dy, void *dw, void *ws, const DwPlan &pl, int N,
                                int CT, int DT, hipStream_t st) {
    constexpr int TB = T * (int)sizeof(IO), KS2 = C::KS * 2, NT = C::WM * C::WN * 64;
    constexpr int CPR = dw_cpl(TB, C::WM * 32 * KS2, NT), CPC = dw_cpl(TB, C::WN * C::CB * 32 * KS2, NT);
    const int NR = SWAP ? CT : DT, NCc = SWAP ? DT : CT;
    if constexpr (CPR > 1 || CPC > 1) {
        if (NR % CPR == 0 && NCc % CPC == 0)
            return launch_dw_reg_w<T, IO, SWAP, C, true>(x, dy, dw, ws, pl, N, CT, DT, st);
    }
    return launch_dw_reg_w<T, IO, SWAP, C, false>(x, dy, dw, ws, pl, N, CT, DT, st);
}

template <int T, typename IO>
static hipError_t launch_dw(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                            hipStream_t st) {
    const DwPlan pl = dw_plan(N, CT, DT, T, sizeof(IO));
    const size_t n = (size_t)CT * DT;
    if (pl.splits == 0) {  // N == 0: the gradient is zero
        hipLaunchKernelGGL((dw_finalize<T, IO, false>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           st, (const float *)ws, (IO *)dw, CT, DT, 0);
        return hipGetLastError();
    }
    return pl.swap ? launch_dw_t<T, IO, true>(x, dy, dw, ws, pl, N, CT, DT, st)
                   : launch_dw_t<T, IO, false>(x, dy, dw, ws, pl, N, CT, DT, st);
}

template <int T, typename IO>
static hipError_t launch_bias(const void *dy, void *db, void *ws, int N, int DT, hipStream_t st) {
    const BiasPlan pl = bias_plan(N, DT, T, (int)sizeof(IO));
    constexpr int CL = bias_cl(T);
    const int be = CL * (16 / (int)sizeof(IO));
    const dim3 grid((unsigned)((DT * T + be - 1) / be), (unsigned)pl.splits);
    const bool el = ((int64_t)DT * T * (int64_t)sizeof(IO)) % 16 != 0;
    if (pl.splits <= 1) {
        if (el)
            hipLaunchKernelGGL((bias_partial<IO, true, CL, true>), grid, dim3(CL * BIAS_RG), 0, st, (const IO *)dy,
                               (float *)ws, (IO *)db, N, DT, T, pl.chunk);
        else
            hipLaunchKernelGGL((bias_partial<IO, true, CL, false>), grid, dim3(CL * BIAS_RG), 0, st, (const IO *)dy,
                               (float *)ws, (IO *)db, N, DT, T, pl.chunk);
        return hipGetLastError();
    }
    if (el)
        hipLaunchKernelGGL((bias_partial<IO, false, CL, true>), grid, dim3(CL * BIAS_RG), 0, st, (const IO *)dy,
                           (float *)ws, (IO *)db, N, DT, T, pl.chunk);
    else
        hipLaunchKernelGGL((bias_partial<IO, false, CL, false>), grid, dim3(CL * BIAS_RG), 0, st, (const IO *)dy,
                           (float *)ws, (IO *)db, N, DT, T, pl.chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bias_finalize<IO>), dim3((unsigned)((DT + 63) / 64)), dim3(256), 0, st,
                       (const float *)ws, (IO *)db, DT, pl.splits);
    return hipGetLastError();
}

// Tile sizes of the weight-gradient kernel, for the split plan.
template <int T, typename IO>
static void dw_tile(bool ring, bool narrow, bool pc, int *br, int *bc, int *kc, int *occ, int grp = 0) {
    if (pc && grp) {
        typedef DwpCfgOct<IO> C;
        *br = 64;
        *bc = 2 * C::CB * 32;
        *kc = C::KS * 2 * M32<IO>::KL;
        *occ = 1;
        return;
    }
    if (pc) {
        typedef DwpCfg<T, IO> C;
        *br = 64;
        *bc = 2 * C::CB * 32;
        *kc = C::KS * 2 * M32<IO>::KL;
        *occ = 1;
        return;
    }
    if constexpr (Pow2<T>::value) {
        if (ring) {
            typedef DwrCfg<T, IO> C;
            *br = C::WM * 32;
            *bc = C::WN * C::CB * 32;
            *kc = C::KS * 2 * M32<IO>::KL;
            *occ = C::OCC;
            return;
        }
    }
    if (narrow) {
        typedef DwCfgN<T, IO> C;
        *br = C::WM * 32;
        *bc = C::WN * C::CB * 32;
        *kc = C::KS * 2 * M32<IO>::KL;
        *occ = C::OCC;
        return;
    }
    {
        typedef DwCfg<T, IO> C;
        *br = C::WM * 32;
        *bc = C::WN * C::CB * 32;
        *kc = C::KS * 2 * M32<IO>::KL;
        *occ = C::OCC;
    }
}

}  // namespace eqk

// ---------------------------------------------------------------------------
// Internal entry points (declared in eqlinear_internal.h).
// ---------------------------------------------------------------------------
#define EQK_DISPATCH(T_, DT_, CALL)                                        \
    do {                                                                   \
        if ((DT_) == 0) {                                                  \
            if ((T_) == 2) { typedef float IO; constexpr int T = 2; CALL; } \
            if ((T_) == 3) { typedef float IO; constexpr int T = 3; CALL; } \
            if ((T_) == 4) { typedef float IO; constexpr int T = 4; CALL; } \
            if ((T_) == 5) { typedef float IO; constexpr int T = 5; CALL; } \
            if ((T_) == 6) { typedef float IO; constexpr int T = 6; CALL; } \
            if ((T_) == 7) { typedef float IO; constexpr int T = 7; CALL; } \
            if ((T_) == 8) { typedef float IO; constexpr int T = 8; CALL; } \
        } else {                                                           \
            if ((T_) == 2) { typedef eqk::f16 IO; constexpr int T = 2; CALL; } \
            if ((T_) == 3) { typedef eqk::f16 IO; constexpr int T = 3; CALL; } \
            if ((T_) == 4) { typedef eqk::f16 IO; constexpr int T = 4; CALL; } \
            if ((T_) == 5) { typedef eqk::f16 IO; constexpr int T = 5; CALL; } \
            if ((T_) == 6) { typedef eqk::f16 IO; constexpr int T = 6; CALL; } \
            if ((T_) == 7) { typedef eqk::f16 IO; constexpr int T = 7; CALL; } \
            if ((T_) == 8) { typedef eqk::f16 IO; constexpr int T = 8; CALL; } \
        }                                                                  \
        return hipErrorInvalidValue;                                       \
    } while (0)

namespace {
// Split plan for one weight-gradient kernel with tile br x bc, kc rows per
// stage and occ resident workgroups per CU.
DwPlan plan_tiles(int64_t N, int64_t C_T, int64_t D_T, int T, int elem_bytes, int br, int bc, int kc,
                  int occ) {
    DwPlan p;
    p.ring = 0;
    p.narrow = 0;
    p.pc = 0;
    // Rows of the tile are d unless c rows and d columns waste fewer MFMA
    // blocks on tile padding.
    auto waste = [&](int64_t nr, int64_t nc) {
        return ((nr + br - 1) / br) * br * ((nc + bc - 1) / bc) * bc - nr * nc;
    };
    p.swap = waste(C_T, D_T) < waste(D_T, C_T) ? 1 : 0;
    const int64_t NR = p.swap ? C_T : D_T, NC = p.swap ? D_T : C_T;
    p.tiles = (int)(((NR + br - 1) / br) * ((NC + bc - 1) / bc));
    if (N <= 0) {
        p.splits = 0;
        p.chunk = 0;
        return p;
    }
    // As many splits as fit the MI355X in one wave of workgroups (256 CUs x
    // the kernel's resident workgroups per CU): one more workgroup than that
    // would start a second, nearly empty round that the whole launch waits
    // for.  But every split also writes (and the finalize reads) a whole fp32
    // tile of partial planes, so a split gets at least ROWS_MIN rows: below
    // that the partial traffic costs more than the parallelism gains
    // (measured on MI355X over 96x96 .. 1024x1024 channel shapes; fp32
    // products are slower, so there more splits pay).  Every chunk is a whole
    // number of stages.
    const int64_t slots = (int64_t)MI355X_CUS * occ, ROWS_MIN = elem_bytes == 2 ? 224 : 96;
    int64_t s = slots / p.tiles;
    if (s > N / ROWS_MIN) s = N / ROWS_MIN;
    // Shorter splits where a lone workgroup would run its stages at the
    // memory latency (never below two splits, whose partials would replace
    // the single split's direct store).  The orders whose transform and
    // products make a stage long (fp32, and orders 3 and 5-8 in fp16) take
    // splits of at least 128 (fp16) or 64 (fp32) rows up to the resident
    // slots; orders 2 and 4 in fp16 only fill a quarter of the CUs that way
    // (more partials cost them more than the parallelism gains).  Weight gradient
    // alone, warm, us: N = 1024, 128 -> 128, fp16 orders 4 / 5 / 7 / 8
    // 15.3 / 27.3 / 35.3 / 23.7 -> 11.4 / 17.9 / 22.5 / 17.6, fp32 order 6
    // 32.3 -> 24.4; N = 4096, 128 -> 128, fp16 orders 4 / 7 17.3 / 40.2 ->
    // 15.2 / 31.4; N = 16384, 64 -> 64, fp16 orders 3 / 5 / 7 21.6 / 36.4 /
    // 42.9 -> 18.9 / 33.0 / 35.0; N = 4096, 256 -> 256, fp16 order 5 38.4 ->
    // 34.9; filling every slot at orders 2 and 4 in fp16 instead: N = 32768,
    // 64 -> 64 20.7 -> 23.6, N = 2048, 512 -> 512 (order 2) 22.1 -> 24.6;
    // half the CUs: N = 16384, 64 -> 64 19.1 -> 19.4.
    if (s >= 2) {
        const bool light = elem_bytes == 2 && (T == 2 || T == 4);
        int64_t s_low = N / (elem_bytes == 2 ? 128 : 64);
        const int64_t cap = light ? MI355X_CUS / 4 / p.tiles : slots / p.tiles;
        if (s_low > cap) s_low = cap;
        if (s < s_low) s = s_low;
    }
    const int64_t stages = (N + kc - 1) / kc;
    if (s > stages) s = stages;
    if (s < 1) s = 1;
    int64_t chunk = ((N + s - 1) / s + kc - 1) / kc * kc;
    // A chunk is addressed through 32-bit buffer offsets: keep its rows of
    // both operands below 2^31 bytes.
    const int64_t row_bytes = (C_T > D_T ? C_T : D_T) * T * elem_bytes;
    const int64_t max_chunk = (((int64_t)1 << 31) - 1) / row_bytes / kc * kc;
    if (chunk > max_chunk) chunk = max_chunk;
    p.chunk = (int)chunk;
    p.splits = (int)((N + chunk - 1) / chunk);
    return p;
}
}  // namespace

// Which weight-gradient kernel runs, and its split plan.  The
// producer/consumer kernel (dwp_kernel) for order 8, the octic group and
// order 2 in fp16.  Otherwise the register-staged kernel (dw_kernel; narrow
// 64 x 64 tiles for order 4 in fp16 when they launch enough more
// workgroups) unless its plan launches fewer workgroups than the GPU has
// CUs: then each workgroup's stage latency is exposed, and for orders 2
// and 4 in fp32 the ring-staged kernel (dwr_kernel) with its deeper copy
// pipeline and smaller tiles is used instead; other order-4 plans take the
// producer/consumer kernel.  (At order 8 the ring
// kernel needs one workgroup per CU to hold its registers and was measured
// slower: 30.4 vs 25.3 us at N = 256, 1024 -> 4096 channels, fp16.)  A pure
// function of the shape (the CU count is MI355X's, not queried), so the
// workspace size never depends on the device.
DwPlan dw_plan(int64_t N, int64_t C_T, int64_t D_T, int T, int elem_bytes, int grp) {
    int br = 0, bc = 0, kc = 0, occ = 2;
    auto tile = [&](auto io, bool ring, bool narrow, bool pc) {
        typedef decltype(io) IO;
        switch (T) {
            case 2: eqk::dw_tile<2, IO>(ring, narrow, pc, &br, &bc, &kc, &occ); break;
            case 3: eqk::dw_tile<3, IO>(ring, narrow, pc, &br, &bc, &kc, &occ); break;
            case 4: eqk::dw_tile<4, IO>(ring, narrow, pc, &br, &bc, &kc, &occ); break;
            case 5: eqk::dw_tile<5, IO>(ring, narrow, pc, &br, &bc, &kc, &occ); break;
            case 6: eqk::dw_tile<6, IO>(ring, narrow, pc, &br, &bc, &kc, &occ); break;
            case 7: eqk::dw_tile<7, IO>(ring, narrow, pc, &br, &bc, &kc, &occ); break;
            default: eqk::dw_tile<8, IO>(ring, narrow, pc, &br, &bc, &kc, &occ, grp); break;
        }
    };
    auto plan = [&](bool ring, bool narrow, bool pc = false) {
        if (elem_bytes == 4) tile(float{}, ring, narrow, pc);
        else tile(eqk::f16{}, ring, narrow, pc);
        return plan_tiles(N, C_T, D_T, T, elem_bytes, br, bc, kc, occ);
    };
    // The producer/consumer kernel for order 8, where it measured faster
    // (C8 at N = 16384, 1024 -> 4096: fp16 113 -> 101 us, fp32 350 -> 328 us),
    // and for order 2 in fp16 on 64 x 256 tiles (weight gradient at
    // N = 32768, 4096 -> 4096: 1325 -> 1010 us; whole training step in the
    // steady state at N = 12608, 768 -> 3072 / 32768, 1024 -> 1024 /
    // 4096, 2048 -> 2048: 209 -> 191 / 212 -> 189 / 123 -> 117 us, small
    // layers within +-1%; fp32 was slower, up to 23%).
    // The octic group (grp = 1) always takes the producer/consumer kernel.
    if (grp || T == 8 || (T == 2 && elem_bytes == 2)) {   // DwpCfg<T>::USE
        DwPlan q = plan(false, false, true);
        q.pc = 1;
        return q;
    }
    DwPlan p = plan(false, false);
    if (T == 4 && elem_bytes == 2) {   // DwCfgN<4, f16>
        DwPlan q = plan(false, true);
        if (4 * (int64_t)q.tiles * q.splits > 5 * (int64_t)p.tiles * p.splits) {
            q.narrow = 1;
            p = q;
        }
    }
    // The ring kernel copies 16-byte chunks of channel rows: both channel
    // rows must be whole chunks.  fp32 only: in fp16 the producer/consumer
    // kernel runs these small grids faster (weight gradient alone, order 4:
    // N = 4096 at 128 -> 128 17.6 -> 15.6 us, N = 2048 at 256 -> 256
    // 19.7 -> 18.7, N = 512 at 512 -> 512 20.1 -> 19.0; in fp32 N = 1024 at
    // 128 -> 128 it was 14.9 against 20.0).
    const bool rows16 = (C_T * T * elem_bytes) % 16 == 0 && (D_T * T * elem_bytes) % 16 == 0;
    if (rows16 && elem_bytes == 4 && (T == 2 || T == 4) && (int64_t)p.tiles * p.splits < MI355X_CUS) {
        DwPlan q = plan(true, false);
        q.ring = 1;
        return q;
    }
    // Order 4: the producer/consumer kernel (64 x 128 tiles, one workgroup
    // per CU, half the splits) unless the narrow tiles run.  Measured on
    // MI355X over the whole training step in the steady state, fp16: ViT-B
    // FFN fc1 / fc2 (N = 12608, 768 <-> 3072) 151 -> 145 / 147 -> 143 us,
    // N = 12608, 1536 -> 1536 149 -> 144, N = 8192, 1024 -> 4096 156 -> 148;
    // since its producers interleave transform and loads also 4096 x 4096
    // 1675 -> 1628, N = 50000 at ViT-B fc1 width 473 -> 458, N = 16384 at
    // 1024 -> 4096 246 -> 242, N = 32768 at 2048 -> 2048 and N = 4096 at ViT-B
    // fc1 width unchanged; fp32: ViT-S qkv 166 -> 164, N = 32768 at
    // 1024 -> 1024 564 -> 557, N = 8192 at 1024 -> 4096 568 -> 562.
    if (T == 4 && !p.narrow) {
        DwPlan q = plan(false, false, true);
        q.pc = 1;
        return q;
    }
    return p;
}

BiasPlan bias_plan(int64_t N, int64_t D_T, int T, int elem_bytes) {
    // About 1024 workgroups (four per CU) so that enough loads are in flight
    // to cover HBM latency, and at least 64 rows per split.
    BiasPlan p;
    const int64_t be = eqk::bias_cl(T) * (16 / elem_bytes);
    const int64_t cols = (D_T * T + be - 1) / be;
    int64_t s = (1024 + cols - 1) / cols;
    const int64_t max_s = (N + 63) / 64;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    p.chunk = (int)((N + s - 1) / s);
    if (p.chunk < 1) p.chunk = 1;
    p.splits = (int)((N + p.chunk - 1) / p.chunk);
    if (p.splits < 1) p.splits = 1;
    return p;
}

int spectrum_planes(int T, int elem_bytes) {
    auto planes = [&](auto io) {
        typedef decltype(io) IO;
        switch (T) {
            case 2: return eqk::stored_planes<2, IO>();
            case 3: return eqk::stored_planes<3, IO>();
            case 4: return eqk::stored_planes<4, IO>();
            case 5: return eqk::stored_planes<5, IO>();
            case 6: return eqk::stored_planes<6, IO>();
            case 7: return eqk::stored_planes<7, IO>();
            default: return eqk::stored_planes<8, IO>();
        }
    };
    return elem_bytes == 4 ? planes(float{}) : planes(eqk::f16{});
}

hipError_t eqk_backward_bias(const void *dy, void *db, void *ws, int N, int DT, int T, int dt,
                             hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_bias<T, IO>(dy, db, ws, N, DT, st)));
}

hipError_t eqk_spectrum(const void *wt, void *what, int CT, int DT, int T, int dt, hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_spectrum<T, IO>(wt, what, CT, DT, st)));
}

hipError_t eqk_forward(const void *x, const void *what, const void *bias, void *y, int N, int CT, int DT,
                       int T, int dt, hipStream_t st) {
    // B planes: part 0 of the spectrum (columns d, k = c)
    EQK_DISPATCH(T, dt, return (eqk::launch_row<T, IO, false>(x, what, bias, y, N, CT, DT, st)));
}

hipError_t eqk_backward_input(const void *dy, const void *what, void *dx, int N, int CT, int DT, int T,
                              int dt, hipStream_t st) {
    // B planes: part 1 of the spectrum (columns c, k = d)
    const int esz = dt == 0 ? 4 : 2;
    const void *wtr = (const char *)what + (size_t)spec_layout(CT, DT, T, esz).elems0 * esz;
    EQK_DISPATCH(T, dt, return (eqk::launch_row<T, IO, true>(dy, wtr, nullptr, dx, N, DT, CT, st)));
}

hipError_t eqk_backward_weight(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                               int T, int dt, hipStream_t st) {
    EQK_DISPATCH(T, dt, return (eqk::launch_dw<T, IO>(x, dy, dw, ws, N, CT, DT, st)));
}

// The octic group (T = 8 components per tuple).
hipError_t eqk_octic_spectrum(const void *wt, void *what, int CT, int DT, int dt, hipStream_t st) {
    return dt == 0 ? eqk::launch_spectrum<8, float, 1>(wt, what, CT, DT, st)
                   : eqk::launch_spectrum<8, eqk::f16, 1>(wt, what, CT, DT, st);
}

hipError_t eqk_octic_forward(const void *x, const void *what, const void *bias, void *y, int N, int CT, int DT,
                             int dt, hipStream_t st) {
    return dt == 0 ? eqk::launch_row<8, float, false, 1>(x, what, bias, y, N, CT, DT, st)
                   : eqk::launch_row<8, eqk::f16, false, 1>(x, what, bias, y, N, CT, DT, st);
}

hipError_t eqk_octic_backward_input(const void *dy, const void *what, void *dx, int N, int CT, int DT, int dt,
                                    hipStream_t st) {
    // B planes: part 1 of the spectrum (columns c, k = d; E blocks transposed)
    const int esz = dt == 0 ? 4 : 2;
    const void *wtr = (const char *)what + (size_t)spec_layout(CT, DT, 8, esz, 1).elems0 * esz;
    return dt == 0 ? eqk::launch_row<8, float, true, 1>(dy, wtr, nullptr, dx, N, DT, CT, st)
                   : eqk::launch_row<8, eqk::f16, true, 1>(dy, wtr, nullptr, dx, N, DT, CT, st);
}

hipError_t eqk_octic_backward_weight(const void *x, const void *dy, void *dw, void *ws, int N, int CT, int DT,
                                     int dt, hipStream_t st) {
    return dt == 0 ? eqk::launch_dw_octic<float>(x, dy, dw, ws, N, CT, DT, st)
                   : eqk::launch_dw_octic<eqk::f16>(x, dy, dw, ws, N, CT, DT, st);
}
