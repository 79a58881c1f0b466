// dsa_device.h — device helpers shared by the gfx950 kernels of the DSA hot
// path: vector types for the MFMA operands, lane/wave helpers, cross-lane
// reductions, bf16 conversion and the order-preserving float key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;

#define DSA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16x16x128 FP8 (OCP E4M3FN) x FP8 -> fp32 matrix-core product, unscaled.
// Operand layout (checked on gfx950): A lane l holds row l%16 and 32
// consecutive k bytes starting at 32*(l/16); B lane l holds column l%16 and
// the same k bytes; C lane l holds column l%16, rows 4*(l/16)+i, i < 4.
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 matrix-core product.  A lane l: row l%16, k = 8*(l/16)+i;
// B lane l: column l%16, k = 8*(l/16)+i; C lane l: column l%16, rows
// 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read: within each 16-lane group, lanes 4r..4r+3 address row r
// (4 consecutive 16-bit values each, so a row is 16 values); lane i of the
// group receives column i: {row0[i], row1[i], row2[i], row3[i]}.
__device__ __forceinline__ i16x4 lds_read_tr16(const DSA_LDS void *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS i16x4 *)p);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// Value of lane (l ^ 16): ds_swizzle in bit-mask mode (and 0x1F, xor 0x10),
// which needs no address register.
__device__ __forceinline__ float xor16_f(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt 0) but not for outstanding global or direct-to-LDS loads
// (vmcnt), so a gather in flight keeps flying across it.  The wavefront-scope
// fences emit no wait; they only stop the compiler from moving LDS accesses
// across the barrier.  (A workgroup-scope LDS fence would also wait for the
// in-flight direct-to-LDS loads, and an asm memory clobber hides the LDS
// buffers' alias scopes from the compiler's wait insertion.)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// One 16-byte-per-lane direct-to-LDS load from sbase + voff (a scalar base
// and a 32-bit per-lane offset) to LDS lds + 16 * lane.  Issued from asm, so
// the compiler's wait insertion does not track it (it cannot tell which LDS
// buffer the load writes and would fence later LDS reads of unrelated buffers
// with a wait for it); a kernel using it waits for these loads explicitly
// with vmcnt before the barrier that publishes the buffer.  M0 must be
// written one instruction ahead of the load.
__device__ __forceinline__ void dma16s(uint64_t sbase, uint32_t voff, const DSA_LDS void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "m0");
}

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Order-preserving key of a fp32 score: a > b  <=>  key(a) > key(b) for
// non-NaN values, with -0 mapped to the key of +0 so that they tie.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sequence of a query row: the b with cu_q[b] <= t < cu_q[b+1] (binary search).
__device__ __forceinline__ int find_seq(const int32_t *cu_q, int B, int t) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Per-row view of the batch: cache offset, context length and visible count
// (clamped so that every cache access stays inside [0, total_kv)).
struct RowInfo {
    int64_t kv0;
    int ctx;
    int pos;
    int nvis;
};

__device__ __forceinline__ RowInfo row_info(const int32_t *cu_q, const int64_t *cu_kv,
                                            const int32_t *pos0, int B, int64_t total_kv,
                                            int max_kv, int t) {
    int b = find_seq(cu_q, B, t);
    RowInfo r;
    int64_t a = cu_kv[b], e = cu_kv[b + 1];
    a = a < 0 ? 0 : (a > total_kv ? total_kv : a);
    e = e < a ? a : (e > total_kv ? total_kv : e);
    int64_t c = e - a;
    r.kv0 = a;
    r.ctx = (int)(c > max_kv ? max_kv : c);
    r.pos = pos0[b] + (t - cu_q[b]);
    int nv = r.pos + 1;
    r.nvis = nv < 0 ? 0 : (nv > r.ctx ? r.ctx : nv);
    return r;
}

}  // namespace dsa
