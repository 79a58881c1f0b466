// peaks.hip — attainable peaks of the GPU the library runs on, for the
// measurement side: the rooflines divide by the spec-sheet peaks, and these
// loops give the rates this GPU actually reaches under the same clock and
// power limits, so that a kernel's fraction can be read against both.
//
//   * matrix cores: every wave runs 8 independent accumulator chains of the
//     16x16x32 bf16 (or 16x16x128 FP8) MFMA, the instructions of the
//     attention (or the indexer), for a fixed count of iterations;
//   * HBM: a streaming read (16-byte non-temporal loads, the result folded
//     into one word per thread) and a streaming copy (non-temporal loads and
//     stores) over a caller-provided buffer much larger than the caches.
//
// Timed with HIP events on the caller's stream; the call waits for it.
#include <hip/hip_runtime.h>

#include "dsa.h"
#include "dsa_device.h"

namespace dsa {

namespace {

constexpr int PK_CHAINS = 8;       // independent accumulators per wave (the drains name all 8)
constexpr int PK_THREADS = 256;    // 4 waves per workgroup
constexpr int PK_WG_PER_CU = 4;    // 16 waves per compute unit, 4 per SIMD

// The chains are inline asm with VGPR accumulators updated in place
// (dst == srcC: back-to-back MFMAs of one opcode need no wait states), as the
// attention writes its QK products: written with the builtin, the compiler
// rotated the loop-carried accumulators through the AGPRs with about 50 moves
// per 8 MFMAs, which halved the rate.  The first product takes an inline zero
// accumulator; before the VALU reads the results, more wait states than any
// 16x16 MFMA needs.
__global__ __launch_bounds__(PK_THREADS) void peak_bf16_kernel(int iters, float *out) {
    const int l = lane_id();
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(l + i));
        b[i] = (__bf16)(0.002f * (float)(l - i));
    }
    f32x4 acc[PK_CHAINS];
#pragma unroll
    for (int c = 0; c < PK_CHAINS; ++c)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc[c]) : "v"(a), "v"(b));
    for (int it = 1; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PK_CHAINS; ++c)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]),
                 "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]));
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < PK_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * PK_THREADS + threadIdx.x] = s;   // (keeps the loop)
}

__global__ __launch_bounds__(PK_THREADS) void peak_fp8_kernel(int iters, float *out) {
    const int l = lane_id();
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 + l + i;   // small E4M3 codes
        b[i] = 0x30303030 + l - i;
    }
    f32x4 acc[PK_CHAINS];   // (in-place inline asm chains, as above; E4M3 operands)
#pragma unroll
    for (int c = 0; c < PK_CHAINS; ++c)
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(acc[c]) : "v"(a), "v"(b));
    for (int it = 1; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PK_CHAINS; ++c)
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]),
                 "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]));
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < PK_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * PK_THREADS + threadIdx.x] = s;
}

// n16: 16-byte units; every thread takes 4 units per step, grid-strided.
__global__ __launch_bounds__(PK_THREADS) void peak_read_kernel(const i32x4 *src, int64_t n16, int32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * PK_THREADS;
    int32_t x = 0;
    int64_t i = (int64_t)blockIdx.x * PK_THREADS + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        i32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const i32x4 v = __builtin_nontemporal_load(src + i);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[blockIdx.x * PK_THREADS + threadIdx.x] = x;
}

__global__ __launch_bounds__(PK_THREADS) void peak_copy_kernel(const i32x4 *src, i32x4 *dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * PK_THREADS;
    int64_t i = (int64_t)blockIdx.x * PK_THREADS + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        i32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t measure_peaks(void *buf, size_t bytes, hipStream_t s, dsa_peaks *r) {
    int dev = 0, ncu = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int grid = PK_WG_PER_CU * ncu;
    // scratch for the per-thread results: the buffer's first grid * PK_THREADS
    // words (overwritten by the bandwidth loops' data afterwards, which is
    // never checked)
    float *fo = static_cast<float *>(buf);
    const int64_t half16 = (int64_t)(bytes / 2 / 16);
    const i32x4 *src = static_cast<const i32x4 *>(buf);
    i32x4 *dst = static_cast<i32x4 *>(buf) + half16;
    hipEvent_t ev[2];
    if ((e = hipEventCreate(&ev[0])) != hipSuccess) return e;
    if ((e = hipEventCreate(&ev[1])) != hipSuccess) {
        (void)hipEventDestroy(ev[0]);
        return e;
    }
    // best of 3 runs of each loop (the first run also warms the clocks)
    auto timed = [&](auto launch, float &best) -> hipError_t {
        best = 1e30f;
        for (int rep = 0; rep < 3; ++rep) {
            hipError_t x;
            if ((x = hipEventRecord(ev[0], s)) != hipSuccess) return x;
            launch();
            if ((x = hipGetLastError()) != hipSuccess) return x;
            if ((x = hipEventRecord(ev[1], s)) != hipSuccess) return x;
            if ((x = hipEventSynchronize(ev[1])) != hipSuccess) return x;
            float ms = 0.f;
            if ((x = hipEventElapsedTime(&ms, ev[0], ev[1])) != hipSuccess) return x;
            best = ms < best ? ms : best;
        }
        return hipSuccess;
    };
    const int bf16_iters = 20000, fp8_iters = 10000;
    const double waves = (double)grid * (PK_THREADS / kWave);
    float ms = 0.f;
    e = timed([&] { hipLaunchKernelGGL(peak_bf16_kernel, dim3(grid), dim3(PK_THREADS), 0, s, bf16_iters, fo); }, ms);
    if (e == hipSuccess) r->bf16_tflops = waves * bf16_iters * PK_CHAINS * (2.0 * 16 * 16 * 32) / (ms * 1e-3) / 1e12;
    if (e == hipSuccess)
        e = timed([&] { hipLaunchKernelGGL(peak_fp8_kernel, dim3(grid), dim3(PK_THREADS), 0, s, fp8_iters, fo); }, ms);
    if (e == hipSuccess) r->fp8_tflops = waves * fp8_iters * PK_CHAINS * (2.0 * 16 * 16 * 128) / (ms * 1e-3) / 1e12;
    const int bgrid = 8 * ncu;
    int32_t *xo = static_cast<int32_t *>(buf);   // (the read loop's words land at the buffer's start)
    if (e == hipSuccess)
        e = timed([&] { hipLaunchKernelGGL(peak_read_kernel, dim3(bgrid), dim3(PK_THREADS), 0, s, src + 1024 * 1024 / 16 * 4,
                                           2 * half16 - 1024 * 1024 / 16 * 4, xo); }, ms);
    if (e == hipSuccess) r->hbm_read_gbs = (double)(2 * half16 - 1024 * 1024 / 16 * 4) * 16 / (ms * 1e-3) / 1e9;
    if (e == hipSuccess)
        e = timed([&] { hipLaunchKernelGGL(peak_copy_kernel, dim3(bgrid), dim3(PK_THREADS), 0, s, src, dst, half16); }, ms);
    if (e == hipSuccess) r->hbm_copy_gbs = (double)half16 * 16 * 2 / (ms * 1e-3) / 1e9;
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    return e;
}

}  // namespace dsa
