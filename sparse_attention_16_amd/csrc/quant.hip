// quant.hip — FP8 quantisation of the indexer inputs and the cache append on
// gfx950.
//
// The index score of the page "Техотчёт DeepSeek-V3.2 (2025): разреженное
// внимание DSA и масштабирование RL", section "Молниеносный индексатор", runs
// on FP8 values.  Each group of values (one token's 64 x 128 indexer query, or
// one cached 128-value indexer key) is quantised with its own scale:
//   s    = absmax / 448 (binary32; 1 for an all-zero group),
//   code = E4M3FN(x / s): the nearest code to the binary32 quotient, ties to
//          the even mantissa, magnitudes above 448 saturate to 448, the sign
//          bit follows the quotient.
// The code only depends on which side of an E4M3FN rounding midpoint the
// quotient lies, so it is taken from y = x * RN(1/s), within 2 ulp of the
// correctly rounded quotient, by the hardware conversion (round to nearest
// even; it gives the same code as e4m3_rne below for every binary32 of
// magnitude under 460, and |y| stays below 449, so its saturation mode never
// matters).  When y - 4 ulp and y + 4 ulp round to different codes (a
// midpoint within a few ulps: about one value in 10^5), the correctly rounded
// division is rounded in software instead.
//
// HBM-bound: 4 bytes read and 1 byte written per value, one group per 32 (key)
// or 256 (query) threads, 16-byte loads.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

// E4M3FN code of a binary32 value (round to nearest even, saturating):
// exact power-of-two scaling, then rounding to an integer number of steps.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t code;
    if (a >= 448.f) {
        code = 0x7Eu;                                    // largest finite value
    } else if (a < 0.015625f) {                          // below 2^-6: steps of 2^-9
        code = (uint32_t)rintf(a * 512.f);               // 0..8; 8 is 2^-6, code 0x08
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6 .. 8
        uint32_t m = (uint32_t)rintf(ldexpf(a, 3 - e));            // 8 .. 16
        if (m == 16u) {
            m = 8u;
            e += 1;
        }
        code = ((uint32_t)(e + 7) << 3) | (m - 8u);
        code = code > 0x7Eu ? 0x7Eu : code;
    }
    return code | sign;
}

template <int COLS, int NT>
__global__ __launch_bounds__(256) void quant_groups_kernel(const float *__restrict__ x, int64_t rows,
                                                          uint8_t *__restrict__ codes,
                                                          float *__restrict__ scale, int rep,
                                                          const int64_t *__restrict__ dst, int64_t nout) {
    constexpr int VPT = COLS / NT;
    constexpr int GPB = 256 / NT;     // groups per workgroup
    static_assert(VPT % 4 == 0 && COLS % NT == 0 && 256 % NT == 0, "group layout");
    __shared__ float red[GPB][(NT + 63) / 64];
    const int g = threadIdx.x / NT, i = threadIdx.x % NT;
    const int64_t r = (int64_t)blockIdx.x * GPB + g;
    const bool live = r < rows;
    const int64_t orow = live ? (dst ? dst[r] : r) : -1;

    // values i*4 + 4*NT*u .. +3: consecutive threads read consecutive 16 bytes
    float v[VPT];
    const float *xr = x + (live ? r : 0) * COLS;
#pragma unroll
    for (int u = 0; u < VPT / 4; ++u) {
        const float4 f = live ? *reinterpret_cast<const float4 *>(xr + 4 * (i + NT * u)) : float4{0.f, 0.f, 0.f, 0.f};
        v[4 * u] = f.x;
        v[4 * u + 1] = f.y;
        v[4 * u + 2] = f.z;
        v[4 * u + 3] = f.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) amax = fmaxf(amax, fabsf(v[j]));
    // maximum over the group's threads (lanes of one wave, then the waves)
#pragma unroll
    for (int d = 1; d < (NT < 64 ? NT : 64); d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if (NT > 64) {
        if ((i & 63) == 0) red[g][i >> 6] = amax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < (NT + 63) / 64; ++w) amax = fmaxf(amax, red[g][w]);
    }
    const float s = amax == 0.f ? 1.f : amax / 448.f;
    const float rs = 1.f / s;    // correctly rounded reciprocal

    if (orow < 0 || orow >= nout) return;
    uint8_t *cr = codes + orow * COLS;
#pragma unroll
    for (int u = 0; u < VPT / 4; ++u) {
        // y = v * (1/s) is within 2 ulps of the exact quotient v / s.  The
        // hardware conversion rounds to nearest even exactly like e4m3_rne
        // (checked on every fp32 of magnitude below 460) and is monotone, so
        // when y +- 4 ulps give the same code, so does v / s; otherwise (a
        // rounding boundary within a few ulps, rare) the exact quotient is
        // rounded in software.
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = v[4 * u + j] * rs;
        uint32_t packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)packed, true);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = __float_as_uint(y[j]) & 0x7FFFFFFFu;
            const uint32_t lh = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                __uint_as_float(a - (a < 4u ? a : 4u)), __uint_as_float(a + 4u), 0, false);
            if (((lh ^ (lh >> 8)) & 0xFFu) != 0u) {
                const uint32_t c = e4m3_rne(v[4 * u + j] / s);
                packed = (packed & ~(0xFFu << (8 * j))) | (c << (8 * j));
            }
        }
        *reinterpret_cast<uint32_t *>(cr + 4 * (i + NT * u)) = packed;
    }
    for (int j = i; j < rep; j += NT) scale[orow * rep + j] = s;
}

// Copies rows of `bytes16` 16-byte chunks: row r of src to row dst[r] of out
// (rows outside [0, nout) skipped).  One 16-byte chunk per thread.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4 *__restrict__ src, int64_t rows, int bytes16,
                                                        const int64_t *__restrict__ dst, int64_t nout,
                                                        uint4 *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= rows * bytes16) return;
    const int64_t r = t / bytes16;
    const int c = (int)(t - r * bytes16);
    const int64_t o = dst[r];
    if (o < 0 || o >= nout) return;
    out[o * bytes16 + c] = src[r * bytes16 + c];
}

}  // namespace

hipError_t launch_quant_queries(const float *q, int64_t T, uint8_t *q_fp8, float *q_scale, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    // one token = 64 heads x 128 values, one scale (repeated in its 64 head entries)
    hipLaunchKernelGGL((quant_groups_kernel<64 * 128, 256>), dim3((unsigned)T), dim3(256), 0, s, q, T, q_fp8,
                       q_scale, 64, (const int64_t *)nullptr, T);
    return hipGetLastError();
}

hipError_t launch_append_cache(const float *k_new, const uint16_t *kv_new, int64_t R, const int64_t *dst,
                               uint8_t *k_fp8, float *k_scale, uint16_t *kv, int64_t N, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    // one key = 128 values, 32 threads per key, 8 keys per workgroup
    hipLaunchKernelGGL((quant_groups_kernel<128, 32>), dim3((unsigned)((R + 7) / 8)), dim3(256), 0, s, k_new, R,
                       k_fp8, k_scale, 1, dst, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !kv_new) return e;
    constexpr int B16 = 576 * 2 / 16;   // 72 chunks per latent row
    const int64_t n = R * B16;
    hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint4 *>(kv_new), R, B16, dst, N, reinterpret_cast<uint4 *>(kv));
    return hipGetLastError();
}

}  // namespace dsa
