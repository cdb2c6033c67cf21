// peaks.hip -- microbenchmarks of the MI355X (gfx950) rates the EQ-Linear
// kernels are bound by: matrix-core throughput, HBM streaming, and the
// per-CU data paths (LDS reads and writes, buffer -> LDS copies, L2 -> VGPR
// loads).  Built into libeqlinear_peaks.so, separate from the layer's
// library; bench.py --peaks drives it and reports achievable peaks next to
// the published ones.
//
// Each kernel runs a fixed amount of work per workgroup; the host times the
// launch with HIP events and divides.  Every kernel also returns the wave
// clock (s_memtime) and the constant 100 MHz clock (s_memrealtime) around its
// loop, so the shader clock during the run is known.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void clocks(uint64_t *clk, int slot) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        clk[2 * slot] = __builtin_amdgcn_s_memtime();
        clk[2 * slot + 1] = __builtin_amdgcn_s_memrealtime();
    }
}

// MFMA throughput: each wave keeps 4 independent 32x32 accumulators and
// issues `iters` rounds of 4 MFMAs.
__global__ __launch_bounds__(256) void mfma_f16_loop(float *out, int iters, uint64_t *clk) {
    f16x8 a, b;
    for (int i = 0; i < 8; ++i) { a[i] = (_Float16)(threadIdx.x * 0.001f + i); b[i] = (_Float16)(i * 0.5f); }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    clocks(clk, 0);
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    clocks(clk, 1);
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_f32_loop(float *out, int iters, uint64_t *clk) {
    const float a = threadIdx.x * 0.001f, b = 0.5f;
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    clocks(clk, 0);
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c3, 0, 0, 0);
    }
    clocks(clk, 1);
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// HBM: dst = src over n 16-byte elements, grid-stride, 4 loads in flight.
__global__ __launch_bounds__(256) void copy16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        __builtin_nontemporal_store(v0, &dst[i]);
        __builtin_nontemporal_store(v1, &dst[i + stride]);
        __builtin_nontemporal_store(v2, &dst[i + 2 * stride]);
        __builtin_nontemporal_store(v3, &dst[i + 3 * stride]);
    }
    for (; i < n; i += stride) __builtin_nontemporal_store(src[i], &dst[i]);
}

// LDS reads: every lane reads 16 bytes per ds_read_b128 from a 64 KB
// buffer, lane-contiguous (no bank conflicts); iters x 8 reads per thread.
__global__ __launch_bounds__(256) void lds_read(float *out, int iters, uint64_t *clk) {
    __shared__ u32x4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    u32x4 acc = {};
    int idx = threadIdx.x;
    clocks(clk, 0);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= buf[(idx + j * 256 + i * 64) & 4095];
    }
    clocks(clk, 1);
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc[0] + acc[1] + acc[2] + acc[3]);
}

// LDS writes: ds_write_b128, lane-contiguous; iters x 8 writes per thread.
__global__ __launch_bounds__(256) void lds_write(float *out, int iters, uint64_t *clk) {
    __shared__ u32x4 buf[4096];
    u32x4 v = {(unsigned)threadIdx.x, 5u, 6u, 7u};
    clocks(clk, 0);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) buf[(threadIdx.x + j * 256 + i * 64) & 4095] = v + (unsigned)j;
        __asm__ volatile("" ::: "memory");
    }
    __syncthreads();
    clocks(clk, 1);
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)buf[(threadIdx.x * 7) & 4095][0];
}

// Buffer -> LDS copies (16 bytes per lane, no VGPR staging) from an
// L2-resident source of `bytes`; iters x 8 copies per thread, waited every
// 8 so at most 8 per thread are in flight.
__global__ __launch_bounds__(256) void lds_dma(const u32x4 *__restrict__ src, uint32_t bytes, float *out,
                                               int iters, uint64_t *clk) {
    __shared__ u32x4 buf[8][256];
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(src), (short)0, (int)bytes, 0x00020000);
    const uint32_t base = (uint32_t)((blockIdx.x * 4096u + threadIdx.x) * 16u) % bytes;
    clocks(clk, 0);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)&buf[j][(threadIdx.x & ~63)],
                                                     16, (base + (uint32_t)(j * 4096 + i * 1024)) % bytes, 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    }
    clocks(clk, 1);
    __syncthreads();
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)buf[threadIdx.x & 7][threadIdx.x][0];
}

// L2 -> VGPR loads: 16 bytes per lane per buffer load from an L2-resident
// source; iters x 8 loads per thread in flight together.
__global__ __launch_bounds__(256) void l2_load(const u32x4 *__restrict__ src, uint32_t bytes, float *out, int iters,
                                               uint64_t *clk) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(src), (short)0, (int)bytes, 0x00020000);
    const uint32_t base = (uint32_t)((blockIdx.x * 4096u + threadIdx.x) * 16u) % bytes;
    u32x4 acc = {};
    clocks(clk, 0);
    for (int i = 0; i < iters; ++i) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (base + (uint32_t)(j * 4096 + i * 1024)) % bytes, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j];
    }
    clocks(clk, 1);
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

}  // namespace

extern "C" {

// kind: 0 mfma fp16, 1 mfma fp32, 2 lds read, 3 lds write, 4 buffer->LDS
// copy, 5 L2 -> VGPR load.  grid workgroups of 256 threads; out holds
// grid * 256 floats; src (kinds 4, 5) `bytes` of device memory; clk 4
// uint64 device values.  Returns the hipError_t of the launch.
int peaks_run(int kind, int grid, int iters, float *out, const void *src, uint32_t bytes, uint64_t *clk,
              void *stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_f16_loop, dim3(grid), dim3(256), 0, st, out, iters, clk); break;
        case 1: hipLaunchKernelGGL(mfma_f32_loop, dim3(grid), dim3(256), 0, st, out, iters, clk); break;
        case 2: hipLaunchKernelGGL(lds_read, dim3(grid), dim3(256), 0, st, out, iters, clk); break;
        case 3: hipLaunchKernelGGL(lds_write, dim3(grid), dim3(256), 0, st, out, iters, clk); break;
        case 4:
            hipLaunchKernelGGL(lds_dma, dim3(grid), dim3(256), 0, st, (const u32x4 *)src, bytes, out, iters, clk);
            break;
        case 5:
            hipLaunchKernelGGL(l2_load, dim3(grid), dim3(256), 0, st, (const u32x4 *)src, bytes, out, iters, clk);
            break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// HBM copy of n 16-byte elements with grid workgroups.
int peaks_copy(const void *src, void *dst, size_t n, int grid, void *stream) {
    hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst, n);
    return (int)hipGetLastError();
}

}  // extern "C"
