// sparse_mla_bwd.hip — backward of the sparse MQA-mode attention on gfx950.
//
// Page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
// масштабирование RL": the attention of section "Отбор и основное внимание"
// (one selected set and one latent row per key, shared by all 128 heads; the
// value is the row's first 512 dims) is trained in the sparse stage of
// section "Как учили индексатор", where all parameters learn.  For query row
// t, head h and selected slot j (position s_j):
//   P[h,j]   = exp(scale <q[t,h,:], kv[s_j,:]> - lse[t,h])
//   dP[h,j]  = <dout[t,h,:], kv[s_j,:512]>,   delta[h] = <dout[t,h,:], out[t,h,:]>
//   dZs[h,j] = scale P[h,j] (dP[h,j] - delta[h])      (the softmax's backward, scaled)
//   dq[t,h,:]    = sum_j dZs[h,j] kv[s_j,:]
//   dkv[s_j,:]  += sum_h dZs[h,j] q[t,h,:]   +   [sum_h P[h,j] dout[t,h,:], 0 .. 0]
// In chunks of query rows (the workspace holds one chunk), each kernel one
// workgroup per row (the longest rows first):
//   bwd_zero: dkv zeroed (once);
//   bwd_dz:   delta per head, then the logits and dP on the bf16 MFMA (each
//             32-slot block of rows gathered into LDS with direct-to-LDS
//             loads, the forward's layout; q and dout rows in VGPRs), P and
//             dZs rounded to bf16 into a workspace [row][slot][head] (bf16 is
//             also what the products below take as MFMA operands);
//   bwd_dq:   dq^T = K^T dZs^T: both operands through LDS transpose reads,
//             the accumulators (a wave's dims x all heads) in registers;
//   bwd_g:    per block [dZs^T | P^T] [q | dout] over the 128 heads, with the
//             row's q and dout resident in VGPRs in head-contraction layout:
//             each slot's 576 sums, rounded to bf16 into a workspace;
//   bwd_count, bwd_scan_*, bwd_scatter: the chunk's usable slots sorted by
//             cache row (counting sort);
//   bwd_reduce: per cache row, its listed sums added in fp32 into dkv in
//             ascending slot order (the list sorted first), so dkv is the
//             same bit for bit on every run.
// (fp32 atomic adds of every slot's sums into dkv were bound by the atomic
// rate: 3.75e10 adds at 32K take 113 ms; this route moves 2 x 1152 bytes
// per slot through memory instead.)
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int H = 128, D = 576, DV = 512;
constexpr int BK = 32;                    // slots per block
constexpr int NW = 8;                     // waves per workgroup
constexpr int NT = NW * kWave;
constexpr int KS = D / 32;                // 18 k-steps over the dims (16 latent + 2 rope)
constexpr int KSV = DV / 32;              // 16 k-steps over the value dims
constexpr int ROWB = D * 2;               // 1152 bytes per latent row
constexpr int PA = 1056;                  // LDS pitch of a row's first 1024 bytes
constexpr int RB = BK * PA;               // rope slabs: 4 x (8 rows x 128 B)
constexpr int BUF = RB + BK * 128;        // 37888 bytes per gathered block
constexpr int ZP = H * 2;                 // 256 bytes per slot row of a P / dZs block
constexpr int ZBUF = BK * ZP;             // 8 KB per P / dZs block
constexpr int MAX_SEL = 2048;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int AHEAD = 3;                  // k-steps of K operands read ahead in bwd_dz
constexpr int GTP = D + 8;                // pitch (in bf16) of a slot row of bwd_g's LDS tile

typedef DSA_LDS uint8_t lds_u8;
typedef __attribute__((ext_vector_type(8))) short i16x8;

// The row's selected positions in LDS (-1 for an unusable slot: -1 entry,
// outside the context, past k), and the number of 32-slot blocks up to the
// last usable one.  maskv: lane b holds block b's 32-bit usable-slot mask.
struct Slots {
    int nblk;
    uint32_t maskv;
};
__device__ __forceinline__ Slots stage_slots(const BwdParams &p, int t, const RowInfo &ri, int32_t *sel) {
    const int nsel = ri.ctx > 0 ? p.k : 0;
    const int32_t *__restrict__ idx_row = p.idx + (int64_t)t * p.k;
    Slots s;
    s.nblk = (nsel + BK - 1) / BK;
    for (int j = threadIdx.x; j < s.nblk * BK; j += NT) {
        const int v = j < nsel ? idx_row[j] : -1;
        sel[j] = (v >= 0 && v < ri.ctx) ? v : -1;
    }
    const int l = lane_id();
    s.maskv = 0;
    for (int it = 0; it * kWave < nsel; ++it) {
        const int j = it * kWave + l;
        const bool ok = j < nsel && (uint32_t)idx_row[j] < (uint32_t)ri.ctx;
        const uint64_t m = __ballot(ok);
        s.maskv = l == 2 * it ? (uint32_t)m : (l == 2 * it + 1 ? (uint32_t)(m >> 32) : s.maskv);
    }
    const uint64_t live = __ballot(s.maskv != 0u);
    const int nlive = live ? 64 - (int)__builtin_clzll(live) : 0;
    s.nblk = s.nblk < nlive ? s.nblk : nlive;
    return s;
}

__device__ __forceinline__ uint64_t seq_base(const uint16_t *kv, int64_t kv0) {
    const uint64_t b = (uint64_t)(uintptr_t)kv + (uint64_t)kv0 * ROWB;
    // (readfirstlane returns int: widen through uint32_t, or the low word is sign-extended)
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
}

// Loads block blk's 32 rows into buf: wave w the latent parts of rows
// 4w .. 4w+3 (1 KB each), waves 0..3 the rope slab of rows 8w .. 8w+7 (lane
// l: row 8w + l/8, its 16-byte chunk (l%8) ^ (l/8)).  Unusable slots load
// the sequence's row 0 (the row must have a context).
__device__ __forceinline__ void gather8(const DSA_LDS int32_t *sel, int blk, int wave, int l, uint64_t kvb,
                                        lds_u8 *buf) {
    const i32x4 a = *reinterpret_cast<const DSA_LDS i32x4 *>(sel + blk * BK + 4 * wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pos = __builtin_amdgcn_readfirstlane(a[i]);
        const uint32_t row = pos < 0 ? 0u : (uint32_t)pos;
        dma16s(kvb + (uint64_t)row * ROWB, 16u * (uint32_t)l, buf + (4 * wave + i) * PA);
    }
    if (wave < 4) {
        const int ps = sel[blk * BK + 8 * wave + (l >> 3)];
        const uint32_t row = ps < 0 ? 0u : (uint32_t)ps;
        dma16s(kvb, row * ROWB + 1024u + 16u * (uint32_t)((l & 7) ^ (l >> 3)), buf + RB + wave * 1024);
    }
}

// A device address made wave-uniform (scalar) for dma16s.
__device__ __forceinline__ uint64_t uniform_base(const void *ptr) {
    const uint64_t v = (uint64_t)(uintptr_t)ptr;
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}

// LDS layout of a [32 slots][128 heads] bf16 block: slot rows of 256 bytes
// (the 64 banks exactly), the 16-byte chunk c of row r stored at chunk
// c ^ zsw(r).  The swizzle spreads the rows a read touches over distinct
// banks: the 16 rows of a 16-byte A-operand read (zsw is a permutation of
// 0..15 over r mod 16), and the 4 rows x 32 bytes of a transpose read
// (zsw(r) differs above bit 0 between the 4 rows 4g .. 4g+3).
__device__ __forceinline__ int zsw(int r) { return ((r << 1) | ((r >> 3) & 1)) & 15; }
__device__ __forceinline__ int zoff(int r, int byte) {
    return r * ZP + 16 * ((byte >> 4) ^ zsw(r)) + (byte & 15);
}

// One 8 KB block [32 slots][128 heads] of a workspace array into LDS in that
// layout (wave w: slots 4w .. 4w+3, one 1 KB load; lane l fills LDS chunk
// l%16 of slot row 4w + l/16 with the chunk of the row that belongs there).
__device__ __forceinline__ void load_zblock(const uint16_t *src, int wave, int l, lds_u8 *buf) {
    uint64_t base = (uint64_t)(uintptr_t)src + (uint64_t)wave * 1024;
    base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
    const int r = 4 * wave + (l >> 4);
    const uint32_t voff = 256u * (uint32_t)(l >> 4) + 16u * (uint32_t)((l & 15) ^ zsw(r));
    dma16s(base, voff, buf + wave * 1024);
}

__device__ __forceinline__ bf16x8 tr_pair(const lds_u8 *lo, const lds_u8 *hi) {
    const i16x4 a = lds_read_tr16(lo), b = lds_read_tr16(hi);
    const i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Byte offset (in a gathered block) of the 8 bytes a lane addresses for a
// transpose read of K^T: key row kr, dims d0 .. d0+3 (d0 a multiple of 4).
__device__ __forceinline__ int kt_off(int kr, int d0) {
    if (d0 < 512) return kr * PA + 2 * d0;
    const int c = (d0 - 512) >> 3, half = ((d0 - 512) >> 2) & 1, rr = kr & 7;
    return RB + (kr >> 3) * 1024 + rr * 128 + 16 * (c ^ rr) + 8 * half;
}

}  // namespace

__global__ __launch_bounds__(256) void bwd_zero_kernel(float4 *x, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
        x[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// P and dZs of every usable block of a row.  Wave w owns heads 16w .. 16w+15:
// its q (18 k-steps) and dout (16 k-steps) operands stay in VGPRs.
__global__ __launch_bounds__(NT) void bwd_dz_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t kb[2][BUF];
    __shared__ __attribute__((aligned(16))) int32_t sel[MAX_SEL];
    __shared__ __attribute__((aligned(16))) uint16_t tz[NW][2][BK * 16];   // per wave: P, dZs of a block

    const int t = p.t0 + p.tc - 1 - (int)blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const Slots sl = stage_slots(p, t, ri, sel);
    const int nblk = sl.nblk;

    const int h = 16 * wave + row16;
    bf16x8 qb[KS], gb[KSV];
    {
        const uint16_t *qrow = p.q + ((int64_t)t * H + h) * D + 8 * grp;
        const uint16_t *grow = p.dout + ((int64_t)t * H + h) * DV + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) gb[ks] = *reinterpret_cast<const bf16x8 *>(grow + 32 * ks);
    }
    const float ls = p.lse[(int64_t)t * H + h];
    const float lse2 = ls > -INFINITY && ls < INFINITY ? ls * LOG2E : INFINITY;   // no finite lse: P = 0
    // delta = <dout, out> of the lane's head: its 128 of the 512 dims (the
    // same chunks as its dout operands), then the sum over the 4 lane groups
    float dl = 0.f;
    {
        const uint16_t *orow = p.out + ((int64_t)t * H + h) * DV + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
            const bf16x8 o8 = *reinterpret_cast<const bf16x8 *>(orow + 32 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) dl = fmaf((float)gb[ks][e], (float)o8[e], dl);
        }
        dl += shfl_xor_f(dl, 16);
        dl += shfl_xor_f(dl, 32);
    }
    const uint64_t kvb = seq_base(p.kv, ri.kv0);

    const int rr = row16 & 7;
    const int kA = row16 * PA + 16 * grp;
    const int kR = RB + (row16 >> 3) * 1024 + rr * 128;
    const int kR16 = kR + 16 * (grp ^ rr);
    const int kR17 = kR + 16 * ((4 + grp) ^ rr);
    auto koff = [&](int ks, int mt) {
        return ks < 16 ? kA + mt * 16 * PA + 64 * ks : (ks == 16 ? kR16 : kR17) + mt * 2048;
    };
    DSA_LDS uint16_t *tp = (DSA_LDS uint16_t *)tz[wave][0];
    DSA_LDS uint16_t *tzd = (DSA_LDS uint16_t *)tz[wave][1];
    uint16_t *ps_row = p.ps + (int64_t)(t - p.t0) * p.kpad * H;
    uint16_t *dz_row = p.dzs + (int64_t)(t - p.t0) * p.kpad * H;

    __syncthreads();   // the slot positions
    if (nblk > 0) gather8((const DSA_LDS int32_t *)sel, 0, wave, l, kvb, (lds_u8 *)kb[0]);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    lds_barrier();

    for (int b = 0; b < nblk; ++b) {
        const int cur = b & 1;
        const lds_u8 *buf = (const lds_u8 *)kb[cur];
        if (b + 1 < nblk) gather8((const DSA_LDS int32_t *)sel, b + 1, wave, l, kvb, (lds_u8 *)kb[cur ^ 1]);

        // S^T = K q^T and dP^T = V dout^T: lane = head row16, keys 16*mt + 4*grp + r
        f32x4 s[2], g[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            g[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        bf16x8 kr[AHEAD + 1][2];
#pragma unroll
        for (int ks = 0; ks < AHEAD; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) kr[ks][mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(buf + koff(ks, mt));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + AHEAD < KS) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    kr[(ks + AHEAD) % (AHEAD + 1)][mt] =
                        *reinterpret_cast<const DSA_LDS bf16x8 *>(buf + koff(ks + AHEAD, mt));
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                s[mt] = mfma_bf16_16x16x32(kr[ks % (AHEAD + 1)][mt], qb[ks], s[mt]);
                if (ks < KSV) g[mt] = mfma_bf16_16x16x32(kr[ks % (AHEAD + 1)][mt], gb[ks], g[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // P and dZs of the block's slots (0 for unusable ones), transposed
        // through the wave's LDS tiles to [slot][16 heads] rows
        const uint32_t vmask = __builtin_amdgcn_readlane(sl.maskv, b);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = 16 * mt + 4 * grp + r;
                const bool ok = (vmask >> slot) & 1u;
                const float pe = ok ? __builtin_amdgcn_exp2f(fmaf(s[mt][r], p.scale_log2, -lse2)) : 0.f;
                const float dz = p.scale * pe * (g[mt][r] - dl);
                tp[slot * 16 + row16] = __builtin_bit_cast(uint16_t, (__bf16)pe);
                tzd[slot * 16 + row16] = __builtin_bit_cast(uint16_t, (__bf16)dz);
            }
        {
            // lane l: slot l/2, heads 8*(l%2) .. +7 of the wave's 16
            const int slot = l >> 1, hh = 8 * (l & 1);
            const int64_t o = (int64_t)(b * BK + slot) * H + 16 * wave + hh;
            *reinterpret_cast<bf16x8 *>(ps_row + o) = *reinterpret_cast<const DSA_LDS bf16x8 *>(tp + slot * 16 + hh);
            *reinterpret_cast<bf16x8 *>(dz_row + o) = *reinterpret_cast<const DSA_LDS bf16x8 *>(tzd + slot * 16 + hh);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of block b+1
        lds_barrier();
    }
}

// dq^T[dims x heads] = sum over blocks of K^T[dims x 32] dZs^T[32 x heads].
// Wave w owns latent dim tiles 4w .. 4w+3 and, for w < 4, rope tile w.
__global__ __launch_bounds__(NT) void bwd_dq_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t kb[2][BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t zb[2][ZBUF];
    __shared__ __attribute__((aligned(16))) int32_t sel[MAX_SEL];

    const int t = p.t0 + p.tc - 1 - (int)blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const Slots sl = stage_slots(p, t, ri, sel);
    const int nblk = sl.nblk;
    const int nct = wave < 4 ? 5 : 4;
    const uint64_t kvb = seq_base(p.kv, ri.kv0);
    const uint16_t *dz_row = p.dzs + (int64_t)(t - p.t0) * p.kpad * H;

    // transpose-read addressing: lane row16 of a 16-lane group points at row
    // (4*grp + row16/4) [+16 for the second half], 4 columns 4*(row16%4) ..
    const int trow = 4 * grp + (row16 >> 2), tcol = 4 * (row16 & 3);
    auto dim_tile = [&](int i) { return i < 4 ? 4 * wave + i : 32 + wave; };

    f32x4 acc[5][8];
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int T = 0; T < 8; ++T) acc[i][T] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();
    if (nblk > 0) {
        gather8((const DSA_LDS int32_t *)sel, 0, wave, l, kvb, (lds_u8 *)kb[0]);
        load_zblock(dz_row, wave, l, (lds_u8 *)zb[0]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();

    for (int b = 0; b < nblk; ++b) {
        const int cur = b & 1;
        const lds_u8 *buf = (const lds_u8 *)kb[cur];
        const lds_u8 *zbuf = (const lds_u8 *)zb[cur];
        if (b + 1 < nblk) {
            gather8((const DSA_LDS int32_t *)sel, b + 1, wave, l, kvb, (lds_u8 *)kb[cur ^ 1]);
            load_zblock(dz_row + (int64_t)(b + 1) * BK * H, wave, l, (lds_u8 *)zb[cur ^ 1]);
        }
        bf16x8 a[5];
#pragma unroll
        for (int i = 0; i < 5; ++i)
            if (i < nct) {
                const int d0 = 16 * dim_tile(i) + tcol;
                a[i] = tr_pair(buf + kt_off(trow, d0), buf + kt_off(16 + trow, d0));
            }
#pragma unroll
        for (int T = 0; T < 8; ++T) {
            const int c0 = 2 * (16 * T + tcol);
            const bf16x8 bz = tr_pair(zbuf + zoff(trow, c0), zbuf + zoff(16 + trow, c0));
#pragma unroll
            for (int i = 0; i < 5; ++i)
                if (i < nct) acc[i][T] = mfma_bf16_16x16x32(a[i], bz, acc[i][T]);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();
    }

    // lane holds dims 16*tile + 4*grp + r of head 16*T + row16
#pragma unroll
    for (int i = 0; i < 5; ++i)
        if (i < nct)
#pragma unroll
            for (int T = 0; T < 8; ++T) {
                float *o = p.dq + ((int64_t)t * H + 16 * T + row16) * D + 16 * dim_tile(i) + 4 * grp;
                *reinterpret_cast<f32x4 *>(o) = acc[i][T];
            }
}

// Each usable slot's dkv contribution, summed over the heads: per block,
// D[32 slots x dims] = dZs^T[32 x 128 heads] q[128 x dims] (+ P^T dout on the
// value dims), rounded to bf16 into g[(t - t0) * kpad + slot][576].  Wave w
// owns latent dim tiles 4w .. 4w+3 and, for w < 4, rope tile w; the row's q
// and dout for those dims stay in VGPRs as MFMA B operands.
__global__ __launch_bounds__(NT) void bwd_g_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t zb[2][ZBUF];
    __shared__ __attribute__((aligned(1024))) uint8_t pb[2][ZBUF];
    __shared__ __attribute__((aligned(16))) int32_t sel[MAX_SEL];
    // two blocks' sums, [32 slots][576 dims] at a 1168-byte pitch (the 4 slots
    // a wave writes at once then fall in distinct banks)
    __shared__ __attribute__((aligned(16))) uint16_t gt[2][BK * GTP];

    const int t = p.t0 + p.tc - 1 - (int)blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const Slots sl = stage_slots(p, t, ri, sel);
    const int nblk = sl.nblk;
    const int nct = wave < 4 ? 5 : 4;
    auto dim_tile = [&](int i) { return i < 4 ? 4 * wave + i : 32 + wave; };
    const int64_t lrow = (int64_t)(t - p.t0) * p.kpad;
    const uint16_t *dz_row = p.dzs + lrow * H;
    const uint16_t *ps_row = p.ps + lrow * H;

    // B operands: lane (dim row16 of a tile, group grp) holds heads
    // 32*ks + 8*grp .. +7 at that dim.  Per k-step, the 32 q rows (36 KB) and
    // 32 dout rows (32 KB) of those heads are copied contiguously into the
    // (not yet used) tile buffers with 1 KB direct-to-LDS loads, and the
    // operands read back with transpose reads (rows = heads, columns = dims:
    // lane row16 gets 4 heads of its dim per read).
    bf16x8 qb[4][5], gb[4][4];
    {
        lds_u8 *stage = (lds_u8 *)gt;
        constexpr int QB = 32 * D * 2, GB = 32 * DV * 2;   // 36864, 32768 bytes
        static_assert(QB + GB <= (int)sizeof(gt), "staging fits the tile buffers");
        const uint64_t qbase = uniform_base(p.q + (int64_t)t * H * D);
        const uint64_t gbase = uniform_base(p.dout + (int64_t)t * H * DV);
        const int hr = 8 * grp + (row16 >> 2), dc = 4 * (row16 & 3);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {   // (unrolled: qb[ks] and gb[ks] must stay registers)
            for (int c = wave; c < QB / 1024; c += NW)
                dma16s(qbase + (uint64_t)ks * QB + 1024u * c, 16u * (uint32_t)l, stage + 1024 * c);
            for (int c = wave; c < GB / 1024; c += NW)
                dma16s(gbase + (uint64_t)ks * GB + 1024u * c, 16u * (uint32_t)l, stage + QB + 1024 * c);
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            lds_barrier();
#pragma unroll
            for (int i = 0; i < 5; ++i)
                if (i < nct) {
                    const lds_u8 *a = stage + hr * (2 * D) + 2 * (16 * dim_tile(i) + dc);
                    qb[ks][i] = tr_pair(a, a + 4 * (2 * D));
                }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const lds_u8 *a = stage + QB + hr * (2 * DV) + 2 * (16 * dim_tile(i) + dc);
                gb[ks][i] = tr_pair(a, a + 4 * (2 * DV));
            }
            lds_barrier();   // (the next k-step's loads overwrite the stage)
        }
    }

    // block b's 32 g rows (contiguous in g) from the LDS tile, 16-byte pieces
    auto copy_out = [&](int b) {
        const DSA_LDS uint16_t *tile = (const DSA_LDS uint16_t *)gt[b & 1];
        uint16_t *grow = p.g + (lrow + (int64_t)b * BK) * D;
        for (int c = threadIdx.x; c < BK * D / 8; c += NT) {
            const int r = c / (D / 8), o = c % (D / 8);
            *reinterpret_cast<bf16x8 *>(grow + 8 * c) = *reinterpret_cast<const DSA_LDS bf16x8 *>(tile + r * GTP + 8 * o);
        }
    };

    // Operand blocks are loaded one block ahead into two buffers.
    auto load_ops = [&](int blk) {
        load_zblock(dz_row + (int64_t)blk * BK * H, wave, l, (lds_u8 *)zb[blk & 1]);
        load_zblock(ps_row + (int64_t)blk * BK * H, wave, l, (lds_u8 *)pb[blk & 1]);
    };
    __syncthreads();
    if (nblk > 0) load_ops(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();

    for (int b = 0; b < nblk; ++b) {
        const int cur = b & 1;
        if (b + 1 < nblk) load_ops(b + 1);
        const lds_u8 *zbuf = (const lds_u8 *)zb[cur];
        const lds_u8 *pbuf = (const lds_u8 *)pb[cur];
        f32x4 acc[2][5];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 5; ++i) acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                // A: slot 16*mt + row16, heads 32*ks + 8*grp .. +7
                const int off = zoff(16 * mt + row16, 2 * (32 * ks + 8 * grp));
                const bf16x8 az = *reinterpret_cast<const DSA_LDS bf16x8 *>(zbuf + off);
                const bf16x8 ap = *reinterpret_cast<const DSA_LDS bf16x8 *>(pbuf + off);
#pragma unroll
                for (int i = 0; i < 5; ++i)
                    if (i < nct) acc[mt][i] = mfma_bf16_16x16x32(az, qb[ks][i], acc[mt][i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][i] = mfma_bf16_16x16x32(ap, gb[ks][i], acc[mt][i]);
            }
            __builtin_amdgcn_sched_barrier(0);   // (keeps the operand reads from all moving up front)
        }
        // lane holds slots 16*mt + 4*grp + r of dim 16*tile + row16: into the tile
        DSA_LDS uint16_t *tile = (DSA_LDS uint16_t *)gt[b & 1];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 5; ++i)
                    if (i < nct)
                        tile[(16 * mt + 4 * grp + r) * GTP + 16 * dim_tile(i) + row16] =
                            __builtin_bit_cast(uint16_t, (__bf16)acc[mt][i][r]);
        // block b+1's loads, and the previous block's copy-out stores (issued a
        // whole block ago, so normally done)
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        lds_barrier();   // publishes block b's tile and block b+1's operands
        copy_out(b);     // (its stores complete under the next block's products)
    }
}

// Slots per cache row over the chunk's usable slots (one workgroup per row).
__global__ __launch_bounds__(256) void bwd_count_kernel(BwdParams p) {
    const int t = p.t0 + (int)blockIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int32_t *idx_row = p.idx + (int64_t)t * p.k;
    for (int j = threadIdx.x; j < p.k; j += 256) {
        const int v = idx_row[j];
        if (v >= 0 && v < ri.ctx) atomicAdd(p.cnt + ri.kv0 + v, 1);
    }
}

// Exclusive prefix of cnt[0 .. n) in place, in three launches: per 1024
// elements (256 threads x 4), the block totals, then their prefixes added.
__global__ __launch_bounds__(256) void bwd_scan_blocks_kernel(int32_t *x, int64_t n, int32_t *bsum) {
    __shared__ int32_t wsum[4];
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    int32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = i0 + e < n ? x[i0 + e] : 0;
    const int32_t s = v[0] + v[1] + v[2] + v[3];
    int32_t inc = s;
    const int l = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(inc, d, kWave);
        if (l >= d) inc += o;
    }
    if (l == kWave - 1) wsum[w] = inc;
    __syncthreads();
    int32_t base = 0;
    for (int u = 0; u < w; ++u) base += wsum[u];
    int32_t e = base + inc - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (i0 + k < n) x[i0 + k] = e;
        e += v[k];
    }
    if (threadIdx.x == 255) bsum[blockIdx.x] = base + inc;
}

__global__ __launch_bounds__(1024) void bwd_scan_totals_kernel(int32_t *bsum, int nb) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    const int l = lane_id(), w = threadIdx.x >> 6;
    for (int c0 = 0; c0 < nb; c0 += 1024) {
        const int i = c0 + (int)threadIdx.x;
        const int32_t s = i < nb ? bsum[i] : 0;
        int32_t inc = s;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t o = __shfl_up(inc, d, kWave);
            if (l >= d) inc += o;
        }
        if (l == kWave - 1) wsum[w] = inc;
        __syncthreads();
        int32_t base = carry;
        for (int u = 0; u < w; ++u) base += wsum[u];
        if (i < nb) bsum[i] = base + inc - s;
        __syncthreads();
        if (threadIdx.x == 1023) carry = base + inc;
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void bwd_scan_add_kernel(int32_t *x, int64_t n, const int32_t *bsum, int32_t *cur,
                                                          int64_t ncur) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int32_t add = bsum[blockIdx.x];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (i0 + e < n) {
            const int32_t v = x[i0 + e] + add;
            x[i0 + e] = v;
            if (i0 + e < ncur) cur[i0 + e] = v;
        }
}

// The chunk's usable slots listed by cache row (order within a row is the
// order the atomics land in; the reduce sorts each row's list first).
__global__ __launch_bounds__(256) void bwd_scatter_kernel(BwdParams p) {
    const int t = p.t0 + (int)blockIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int32_t *idx_row = p.idx + (int64_t)t * p.k;
    for (int j = threadIdx.x; j < p.k; j += 256) {
        const int v = idx_row[j];
        if (v >= 0 && v < ri.ctx) {
            const int32_t at = atomicAdd(p.cur + ri.kv0 + v, 1);
            p.list[at] = (int32_t)blockIdx.x * p.kpad + j;
        }
    }
}

constexpr int RED_T = 128;        // threads of the reduce workgroup
constexpr int SORT_CAP = 4096;    // longest list sorted in LDS (16 KB)

// Ascending sort of a[0 .. m) by the workgroup (bitonic network over the next
// power of two P >= m, with every comparator putting the smaller value at the
// lower index: the first step of each merge pairs i with its mirror i ^ (kk-1),
// the later ones i with i + jj).  The positions m .. P are taken as +inf and
// never touched: a comparator whose upper element lies there already holds
// the smaller value below.  sync() orders each step's accesses before the next.
template <typename Ptr, typename Sync>
__device__ __forceinline__ void sort_ascending(Ptr a, int m, Sync sync) {
    int P = 1;
    while (P < m) P <<= 1;
    for (int kk = 2; kk <= P; kk <<= 1) {
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            const int lg = 31 - __builtin_clz(jj);
            for (int c = (int)threadIdx.x; c < (P >> 1); c += RED_T) {
                const int i = ((c >> lg) << (lg + 1)) + (c & (jj - 1));
                const int u = jj == (kk >> 1) ? (i ^ (kk - 1)) : i + jj;
                if (u < m) {
                    const int32_t x = a[i], y = a[u];
                    if (y < x) {
                        a[i] = y;
                        a[u] = x;
                    }
                }
            }
            sync();
        }
    }
}

// dkv[s, :] += the chunk's listed contributions to cache row s, summed in
// fp32 in ascending slot order (the list is sorted first, so the sums and
// their rounding do not depend on the order the scatter's atomics landed in):
// one workgroup per cache row, threads 0..71 own 8 dims each.  Lists up to
// SORT_CAP entries are sorted in LDS, longer ones (only rows selected by
// more than 4096 slots of the chunk, i.e. repeated positions) in place.
__global__ __launch_bounds__(RED_T) void bwd_reduce_kernel(BwdParams p) {
    __shared__ int32_t srt[SORT_CAP];
    const int64_t s = blockIdx.x;
    const int32_t beg = p.cnt[s], end = p.cnt[s + 1];
    const int m = end - beg;
    if (m <= 0) return;
    const int32_t *lst;
    if (m <= SORT_CAP) {
        for (int i = (int)threadIdx.x; i < m; i += RED_T) srt[i] = p.list[beg + i];
        lds_barrier();
        if (m > 1) sort_ascending(srt, m, [] { lds_barrier(); });
        lst = srt;
    } else {
        sort_ascending(p.list + beg, m, [] { __syncthreads(); });
        lst = p.list + beg;
    }
    if (threadIdx.x >= D / 8) return;
    const int d0 = 8 * (int)threadIdx.x;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int i = 0;
    for (; i + 4 <= m; i += 4) {
        bf16x8 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = *reinterpret_cast<const bf16x8 *>(p.g + (int64_t)lst[i + u] * D + d0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
    }
    for (; i < m; ++i) {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p.g + (int64_t)lst[i] * D + d0);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
    }
    f32x4 *o = reinterpret_cast<f32x4 *>(p.dkv + s * D + d0);
    o[0] += f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] += f32x4{acc[4], acc[5], acc[6], acc[7]};
}

__global__ __launch_bounds__(256) void bwd_zero_i32_kernel(int32_t *x, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0;
}

hipError_t launch_sparse_mla_bwd(const BwdParams &p0, int T, hipStream_t s) {
    const int64_t N = p0.total_kv;
    const int64_t n4 = N * D / 4;
    auto grid_for = [](int64_t n) { const int64_t g = (n + 255) / 256; return (unsigned)(g < 4096 ? g : 4096); };
    if (n4 > 0) {
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(grid_for(n4)), dim3(256), 0, s, reinterpret_cast<float4 *>(p0.dkv),
                           n4);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t nscan = N + 1;                          // the last entry becomes the total
    const unsigned nb = (unsigned)((nscan + 1023) / 1024);
    for (int t0 = 0; t0 < T; t0 += BWD_CHUNK) {
        BwdParams p = p0;
        p.t0 = t0;
        p.tc = T - t0 < BWD_CHUNK ? T - t0 : BWD_CHUNK;
        hipLaunchKernelGGL(bwd_zero_i32_kernel, dim3(grid_for(nscan)), dim3(256), 0, s, p.cnt, nscan);
        hipLaunchKernelGGL(bwd_dz_kernel, dim3(p.tc), dim3(NT), 0, s, p);
        hipLaunchKernelGGL(bwd_dq_kernel, dim3(p.tc), dim3(NT), 0, s, p);
        hipLaunchKernelGGL(bwd_g_kernel, dim3(p.tc), dim3(NT), 0, s, p);
        if (N > 0) {
            hipLaunchKernelGGL(bwd_count_kernel, dim3(p.tc), dim3(256), 0, s, p);
            hipLaunchKernelGGL(bwd_scan_blocks_kernel, dim3(nb), dim3(256), 0, s, p.cnt, nscan, p.bsum);
            hipLaunchKernelGGL(bwd_scan_totals_kernel, dim3(1), dim3(1024), 0, s, p.bsum, (int)nb);
            hipLaunchKernelGGL(bwd_scan_add_kernel, dim3(nb), dim3(256), 0, s, p.cnt, nscan, p.bsum, p.cur, N);
            hipLaunchKernelGGL(bwd_scatter_kernel, dim3(p.tc), dim3(256), 0, s, p);
            hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)N), dim3(RED_T), 0, s, p);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsa
