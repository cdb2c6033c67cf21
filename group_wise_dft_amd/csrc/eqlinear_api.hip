// eqlinear_api.hip -- the C ABI of libeqlinear.so (declared in
// include/eqlinear.h): argument validation, then one launch sequence on the
// caller's stream.  Validation runs before any HIP call, so a rejected call
// touches neither the device nor the outputs.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/eqlinear.h"
#include "eqlinear_internal.h"

// Device scratch of eqlinear_backward_weight_noalloc: the weight gradient's
// fp32 split partials.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never passes this name to a kernel (on the host
// it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[EQL_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_addr[MAX_DEVICES];
std::mutex scratch_mu;

eql_status noalloc_scratch(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return EQL_ERR_HIP;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EQL_ERR_HIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return EQL_OK;
}

struct Span {
    const void *p;
    size_t bytes;
};

size_t elem_bytes(eql_dtype dt) { return dt == EQL_F16 ? 2 : 4; }

bool overlap(Span a, Span b) {
    if (a.bytes == 0 || b.bytes == 0 || !a.p || !b.p) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Sizes, dtype and group order.  Kernel indices are 32-bit for rows and
// channels and 64-bit for element offsets; the limits below keep both safe.
eql_status check_shape(int64_t N, int64_t C_T, int64_t D_T, int32_t T, eql_dtype dt) {
    if (N < 0 || C_T < 0 || D_T < 0) return EQL_ERR_SHAPE;
    if (dt != EQL_F32 && dt != EQL_F16) return EQL_ERR_UNSUPPORTED;
    if (T < 2 || T > 8) return EQL_ERR_UNSUPPORTED;
    if (C_T < 1 || D_T < 1) return EQL_ERR_UNSUPPORTED;
    // Kernels address each tile through 32-bit buffer offsets: a channel
    // count of at most 65536 keeps a row block below 2^31 bytes, and the
    // cached spectrum (both orientations, blocked) must stay below 2^31 bytes.
    if (N >= ((int64_t)1 << 30) || C_T > 65536 || D_T > 65536) return EQL_ERR_UNSUPPORTED;
    const SpecLayout L = spec_layout(C_T, D_T, T, (int)elem_bytes(dt));
    if ((L.elems0 + L.elems1) * (int64_t)elem_bytes(dt) >= ((int64_t)1 << 31)) return EQL_ERR_UNSUPPORTED;
    return EQL_OK;
}

eql_status check_ptr(const void *p, size_t bytes) {
    if (bytes == 0) return EQL_OK;  // an empty array may be NULL
    if (!p) return EQL_ERR_NULL;
    if (((uintptr_t)p & 15u) != 0) return EQL_ERR_ALIGN;
    return EQL_OK;
}

eql_status from_hip(hipError_t e) { return e == hipSuccess ? EQL_OK : EQL_ERR_HIP; }

}  // namespace

extern "C" {

const char *eqlinear_status_string(eql_status s) {
    switch (s) {
        case EQL_OK: return "ok";
        case EQL_ERR_NULL: return "a required pointer is NULL";
        case EQL_ERR_SHAPE: return "a size is negative";
        case EQL_ERR_UNSUPPORTED: return "unsupported group order, dtype or channel count";
        case EQL_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case EQL_ERR_WORKSPACE: return "workspace missing or too small";
        case EQL_ERR_ALIAS: return "an output overlaps an input";
        case EQL_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

size_t eqlinear_spectrum_size(int64_t C_T, int64_t D_T, int32_t T, eql_dtype dtype) {
    if (check_shape(0, C_T, D_T, T, dtype) != EQL_OK) return 0;
    const SpecLayout L = spec_layout(C_T, D_T, T, (int)elem_bytes(dtype));
    return (size_t)(L.elems0 + L.elems1) * elem_bytes(dtype);
}

size_t eqlinear_bias_workspace_size(int64_t N, int64_t D_T, int32_t T, eql_dtype dtype) {
    if (check_shape(N, 1, D_T, T, dtype) != EQL_OK) return 0;
    const BiasPlan p = bias_plan(N, D_T, T, (int)elem_bytes(dtype));
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)D_T * sizeof(float);
}

size_t eqlinear_workspace_size(int64_t N, int64_t C_T, int64_t D_T, int32_t T, eql_dtype dtype) {
    if (check_shape(N, C_T, D_T, T, dtype) != EQL_OK) return 0;
    const DwPlan p = dw_plan(N, C_T, D_T, T, (int)elem_bytes(dtype));
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)T * (size_t)D_T * (size_t)C_T * sizeof(float);
}

eql_status eqlinear_weight_spectrum(const void *w_tilde, void *w_hat, int64_t C_T, int64_t D_T,
                                    int32_t T, eql_dtype dtype, void *stream) {
    eql_status s = check_shape(0, C_T, D_T, T, dtype);
    if (s != EQL_OK) return s;
    const size_t bytes = (size_t)C_T * D_T * T * elem_bytes(dtype);
    const size_t hbytes = eqlinear_spectrum_size(C_T, D_T, T, dtype);
    if ((s = check_ptr(w_tilde, bytes)) != EQL_OK) return s;
    if ((s = check_ptr(w_hat, hbytes)) != EQL_OK) return s;
    if (overlap({w_hat, hbytes}, {w_tilde, bytes})) return EQL_ERR_ALIAS;
    return from_hip(eqk_spectrum(w_tilde, w_hat, (int)C_T, (int)D_T, T, dtype == EQL_F16,
                                 (hipStream_t)stream));
}

eql_status eqlinear_forward(const void *x, const void *w_hat, const void *bias, void *y, int64_t N,
                            int64_t C_T, int64_t D_T, int32_t T, eql_dtype dtype, void *stream) {
    eql_status s = check_shape(N, C_T, D_T, T, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bx = (size_t)N * C_T * T * e, bw = eqlinear_spectrum_size(C_T, D_T, T, dtype), by = (size_t)N * D_T * T * e;
    const size_t bb = (size_t)D_T * e;
    if ((s = check_ptr(x, bx)) != EQL_OK) return s;
    if ((s = check_ptr(w_hat, bw)) != EQL_OK) return s;
    if ((s = check_ptr(y, by)) != EQL_OK) return s;
    if (bias && ((uintptr_t)bias & 15u) != 0) return EQL_ERR_ALIGN;
    if (overlap({y, by}, {x, bx}) || overlap({y, by}, {w_hat, bw})) return EQL_ERR_ALIAS;
    if (overlap({y, by}, {bias, bb})) return EQL_ERR_ALIAS;
    if (N == 0) return EQL_OK;
    return from_hip(eqk_forward(x, w_hat, bias, y, (int)N, (int)C_T, (int)D_T, T, dtype == EQL_F16,
                                (hipStream_t)stream));
}

eql_status eqlinear_backward_input(const void *dy, const void *w_hat, void *dx, int64_t N, int64_t C_T,
                                   int64_t D_T, int32_t T, eql_dtype dtype, void *stream) {
    eql_status s = check_shape(N, C_T, D_T, T, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bdy = (size_t)N * D_T * T * e, bw = eqlinear_spectrum_size(C_T, D_T, T, dtype), bdx = (size_t)N * C_T * T * e;
    if ((s = check_ptr(dy, bdy)) != EQL_OK) return s;
    if ((s = check_ptr(w_hat, bw)) != EQL_OK) return s;
    if ((s = check_ptr(dx, bdx)) != EQL_OK) return s;
    if (overlap({dx, bdx}, {dy, bdy}) || overlap({dx, bdx}, {w_hat, bw})) return EQL_ERR_ALIAS;
    if (N == 0) return EQL_OK;
    return from_hip(eqk_backward_input(dy, w_hat, dx, (int)N, (int)C_T, (int)D_T, T, dtype == EQL_F16,
                                       (hipStream_t)stream));
}

eql_status eqlinear_backward_weight(const void *x, const void *dy, void *dw_tilde, void *workspace,
                                    size_t workspace_bytes, int64_t N, int64_t C_T, int64_t D_T,
                                    int32_t T, eql_dtype dtype, void *stream) {
    eql_status s = check_shape(N, C_T, D_T, T, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bx = (size_t)N * C_T * T * e, bdy = (size_t)N * D_T * T * e, bw = (size_t)D_T * C_T * T * e;
    if ((s = check_ptr(x, bx)) != EQL_OK) return s;
    if ((s = check_ptr(dy, bdy)) != EQL_OK) return s;
    if ((s = check_ptr(dw_tilde, bw)) != EQL_OK) return s;
    const size_t need = eqlinear_workspace_size(N, C_T, D_T, T, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return EQL_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 15u) != 0) return EQL_ERR_ALIGN;
    }
    const Span out{dw_tilde, bw}, ws{workspace, need};
    if (overlap(out, {x, bx}) || overlap(out, {dy, bdy})) return EQL_ERR_ALIAS;
    if (overlap(ws, {x, bx}) || overlap(ws, {dy, bdy}) || overlap(ws, out)) return EQL_ERR_ALIAS;
    return from_hip(eqk_backward_weight(x, dy, dw_tilde, workspace, (int)N, (int)C_T, (int)D_T, T,
                                        dtype == EQL_F16, (hipStream_t)stream));
}

eql_status eqlinear_backward_weight_noalloc(const void *x, const void *dy, void *dw_tilde, int64_t N,
                                            int64_t C_T, int64_t D_T, int32_t T, eql_dtype dtype,
                                            void *stream) {
    eql_status s = check_shape(N, C_T, D_T, T, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bx = (size_t)N * C_T * T * e, bdy = (size_t)N * D_T * T * e, bw = (size_t)D_T * C_T * T * e;
    if ((s = check_ptr(x, bx)) != EQL_OK) return s;
    if ((s = check_ptr(dy, bdy)) != EQL_OK) return s;
    if ((s = check_ptr(dw_tilde, bw)) != EQL_OK) return s;
    const Span out{dw_tilde, bw};
    if (overlap(out, {x, bx}) || overlap(out, {dy, bdy})) return EQL_ERR_ALIAS;
    // the same split plan (and summation order) as eqlinear_backward_weight
    const size_t need = eqlinear_workspace_size(N, C_T, D_T, T, dtype);
    if (need > EQL_NOALLOC_SCRATCH_BYTES) return EQL_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0 && (s = noalloc_scratch(&ws)) != EQL_OK) return s;
    return from_hip(eqk_backward_weight(x, dy, dw_tilde, ws, (int)N, (int)C_T, (int)D_T, T,
                                        dtype == EQL_F16, (hipStream_t)stream));
}

eql_status eqlinear_backward_bias(const void *dy, void *db, void *workspace, size_t workspace_bytes,
                                  int64_t N, int64_t D_T, int32_t T, eql_dtype dtype, void *stream) {
    // The bias gradient has no input channels; C_T = 1 stands in for the
    // shared shape checks.
    eql_status s = check_shape(N, 1, D_T, T, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bdy = (size_t)N * D_T * T * e, bb = (size_t)D_T * e;
    if ((s = check_ptr(dy, bdy)) != EQL_OK) return s;
    if ((s = check_ptr(db, bb)) != EQL_OK) return s;
    const size_t need = eqlinear_bias_workspace_size(N, D_T, T, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return EQL_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 15u) != 0) return EQL_ERR_ALIGN;
    }
    const Span out{db, bb}, ws{workspace, need};
    if (overlap(out, {dy, bdy}) || overlap(ws, {dy, bdy}) || overlap(ws, out)) return EQL_ERR_ALIAS;
    return from_hip(eqk_backward_bias(dy, db, workspace, (int)N, (int)D_T, T, dtype == EQL_F16,
                                      (hipStream_t)stream));
}

// ---- The octic group (T = 8 components per tuple) ----

size_t eqlinear_octic_spectrum_size(int64_t C_T, int64_t D_T, eql_dtype dtype) {
    if (check_shape(0, C_T, D_T, 8, dtype) != EQL_OK) return 0;
    const SpecLayout L = spec_layout(C_T, D_T, 8, (int)elem_bytes(dtype), 1);
    return (size_t)(L.elems0 + L.elems1) * elem_bytes(dtype);
}

size_t eqlinear_octic_workspace_size(int64_t N, int64_t C_T, int64_t D_T, eql_dtype dtype) {
    if (check_shape(N, C_T, D_T, 8, dtype) != EQL_OK) return 0;
    const DwPlan p = dw_plan(N, C_T, D_T, 8, (int)elem_bytes(dtype), 1);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)8 * (size_t)D_T * (size_t)C_T * sizeof(float);
}

eql_status eqlinear_octic_weight_spectrum(const void *w_tilde, void *w_hat, int64_t C_T, int64_t D_T,
                                          eql_dtype dtype, void *stream) {
    eql_status s = check_shape(0, C_T, D_T, 8, dtype);
    if (s != EQL_OK) return s;
    const size_t bytes = (size_t)C_T * D_T * 8 * elem_bytes(dtype);
    const size_t hbytes = eqlinear_octic_spectrum_size(C_T, D_T, dtype);
    if ((s = check_ptr(w_tilde, bytes)) != EQL_OK) return s;
    if ((s = check_ptr(w_hat, hbytes)) != EQL_OK) return s;
    if (overlap({w_hat, hbytes}, {w_tilde, bytes})) return EQL_ERR_ALIAS;
    return from_hip(eqk_octic_spectrum(w_tilde, w_hat, (int)C_T, (int)D_T, dtype == EQL_F16, (hipStream_t)stream));
}

eql_status eqlinear_octic_forward(const void *x, const void *w_hat, const void *bias, void *y, int64_t N,
                                  int64_t C_T, int64_t D_T, eql_dtype dtype, void *stream) {
    eql_status s = check_shape(N, C_T, D_T, 8, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bx = (size_t)N * C_T * 8 * e, bw = eqlinear_octic_spectrum_size(C_T, D_T, dtype), by = (size_t)N * D_T * 8 * e;
    const size_t bb = (size_t)D_T * e;
    if ((s = check_ptr(x, bx)) != EQL_OK) return s;
    if ((s = check_ptr(w_hat, bw)) != EQL_OK) return s;
    if ((s = check_ptr(y, by)) != EQL_OK) return s;
    if (bias && ((uintptr_t)bias & 15u) != 0) return EQL_ERR_ALIGN;
    if (overlap({y, by}, {x, bx}) || overlap({y, by}, {w_hat, bw})) return EQL_ERR_ALIAS;
    if (overlap({y, by}, {bias, bb})) return EQL_ERR_ALIAS;
    if (N == 0) return EQL_OK;
    return from_hip(eqk_octic_forward(x, w_hat, bias, y, (int)N, (int)C_T, (int)D_T, dtype == EQL_F16,
                                      (hipStream_t)stream));
}

eql_status eqlinear_octic_backward_input(const void *dy, const void *w_hat, void *dx, int64_t N, int64_t C_T,
                                         int64_t D_T, eql_dtype dtype, void *stream) {
    eql_status s = check_shape(N, C_T, D_T, 8, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bdy = (size_t)N * D_T * 8 * e, bw = eqlinear_octic_spectrum_size(C_T, D_T, dtype), bdx = (size_t)N * C_T * 8 * e;
    if ((s = check_ptr(dy, bdy)) != EQL_OK) return s;
    if ((s = check_ptr(w_hat, bw)) != EQL_OK) return s;
    if ((s = check_ptr(dx, bdx)) != EQL_OK) return s;
    if (overlap({dx, bdx}, {dy, bdy}) || overlap({dx, bdx}, {w_hat, bw})) return EQL_ERR_ALIAS;
    if (N == 0) return EQL_OK;
    return from_hip(eqk_octic_backward_input(dy, w_hat, dx, (int)N, (int)C_T, (int)D_T, dtype == EQL_F16,
                                             (hipStream_t)stream));
}

eql_status eqlinear_octic_backward_weight(const void *x, const void *dy, void *dw_tilde, void *workspace,
                                          size_t workspace_bytes, int64_t N, int64_t C_T, int64_t D_T,
                                          eql_dtype dtype, void *stream) {
    eql_status s = check_shape(N, C_T, D_T, 8, dtype);
    if (s != EQL_OK) return s;
    const size_t e = elem_bytes(dtype);
    const size_t bx = (size_t)N * C_T * 8 * e, bdy = (size_t)N * D_T * 8 * e, bw = (size_t)D_T * C_T * 8 * e;
    if ((s = check_ptr(x, bx)) != EQL_OK) return s;
    if ((s = check_ptr(dy, bdy)) != EQL_OK) return s;
    if ((s = check_ptr(dw_tilde, bw)) != EQL_OK) return s;
    const size_t need = eqlinear_octic_workspace_size(N, C_T, D_T, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return EQL_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 15u) != 0) return EQL_ERR_ALIGN;
    }
    const Span out{dw_tilde, bw}, ws{workspace, need};
    if (overlap(out, {x, bx}) || overlap(out, {dy, bdy})) return EQL_ERR_ALIAS;
    if (overlap(ws, {x, bx}) || overlap(ws, {dy, bdy}) || overlap(ws, out)) return EQL_ERR_ALIAS;
    return from_hip(eqk_octic_backward_weight(x, dy, dw_tilde, workspace, (int)N, (int)C_T, (int)D_T,
                                              dtype == EQL_F16, (hipStream_t)stream));
}

}  // extern "C"
