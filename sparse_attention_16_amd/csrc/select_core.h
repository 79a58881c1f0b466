// select_core.h — exact top-k selects by one 1024-thread workgroup: of
// register-held uint32 keys (select_regs: the top-k merge, the fused path's
// workgroup select and recompute, and the top-k kernel's tie fallback), and of
// candidate keys staged in LDS (lds_cand_select: the top-k kernel).  Selection rule (page "Техотчёт
// DeepSeek-V3.2 (2025): разреженное внимание DSA и масштабирование RL",
// section "Отбор и основное внимание", Top-k(I_{t,:})): the k largest keys,
// ties to the lower array position; keys are order-preserving images of fp32
// scores (score_key), 0 = no key.
#pragma once

#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int TPB = 1024;                                  // threads per workgroup (16 waves, 4 per SIMD)
constexpr int NWAVE = TPB / kWave;                         // 16
constexpr int NBIN = 2048;                                 // histogram bins
constexpr int BPT = NBIN / TPB;                            // bins scanned per thread
constexpr int CCAP = 512;                                  // candidates ranked directly (one per thread)
constexpr int CH_V4 = TOPK_CHUNK / (4 * TPB);              // 4-key groups per thread, chunk kernel
constexpr int MG_V4 = TOPK_MAX_CHUNKS * 2048 / (4 * TPB);  // 4-key groups per thread, merge kernel
static_assert(NBIN % TPB == 0 && CH_V4 * 4 * TPB == TOPK_CHUNK && MG_V4 * 4 * TPB == TOPK_MAX_CHUNKS * 2048,
              "register layout");

struct SelectShared {
    union {
        uint32_t hist[NBIN + kWave];  // histogram, one spare entry per lane after it
        uint32_t okey[2048];          // selected keys by slot (written once the histogram is done)
    };
    uint32_t ckey[CCAP];             // uncertain keys ...
    uint32_t cpos[CCAP];             // ... and their positions (thread << 6 | register index)
    uint32_t tbits[TPB][2];          // uncertain keys taken, as bits of their owner's key mask
    int32_t ocol[2048];              // selected columns by slot
    uint32_t wtot[NWAVE];            // scan and reduction scratch
    uint32_t wmin[NWAVE], wmax[NWAVE];
    uint32_t ncand;
    uint32_t prefix;                 // bin b1, or radix key bits fixed so far
    uint32_t rem;                    // keys still needed inside the prefix
    uint32_t kappa, need_eq;
};

// Marks the register keys as changed (no instruction): values derived from
// them in an earlier phase (validity masks, bins) are recomputed instead of
// being kept live across the phases, which would not fit in the registers.
template <int N>
__device__ __forceinline__ void launder(uint32_t (&kr)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(kr[i]));
}

// Score of a key (inverse of score_key; key != 0).
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Inclusive scan over the 64 lanes of a wave with DPP lane moves (VALU only,
// no LDS round trip): row shifts by 1, 2, 4, 8 scan each 16-lane row, then
// the last lane of row 0 is added to row 1 and 3 and that of rows 0-1 to
// rows 2-3.  Lanes a move has no source for take the identity `id`.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t x) {
    return wave_scan(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Block-wide exclusive scan of one value per thread (in thread order).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wtot) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    const uint32_t x = wave_scan_add(v);
    if (l == 63) wtot[w] = x;
    lds_barrier();
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) off += (i < w) ? wtot[i] : 0u;
    lds_barrier();
    return off + x - v;
}

// From the counts in sh.hist (bin i = digit i, larger digits = larger keys),
// picks the bin holding the sh.rem-th largest key: sh.prefix = (prefix <<
// width) | bin, sh.rem = rank inside that bin.
__device__ __forceinline__ void pick_bin(int width, SelectShared &sh) {
    const int top = NBIN - 1 - BPT * (int)threadIdx.x;   // this thread's bins: top, top-1, ...
    uint32_t c[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        c[i] = sh.hist[top - i];
        sum += c[i];
    }
    const uint32_t above = block_excl_scan(sum, sh.wtot);
    const uint32_t rem = sh.rem, prefix = sh.prefix;
    lds_barrier();
    uint32_t acc = above;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        if (acc < rem && rem <= acc + c[i]) {
            sh.prefix = (prefix << width) | (uint32_t)(top - i);
            sh.rem = rem - acc;
        }
        acc += c[i];
    }
    lds_barrier();
}

__device__ __forceinline__ void clear_hist(SelectShared &sh) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) sh.hist[threadIdx.x + i * TPB] = 0u;
}

// Exact kappa by three radix passes over the register keys (key 0 = no key).
template <int NV4>
__device__ __forceinline__ void radix_kappa(uint32_t (&kr)[4 * NV4], int ngroups, int k, SelectShared &sh) {
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
    }
    constexpr int SHIFT[3] = {21, 10, 0}, WIDTH[3] = {11, 11, 10};
    static_assert(NBIN >= (1 << 11), "the radix digits index the histogram");
#pragma unroll
    for (int ps = 0; ps < 3; ++ps) {
        clear_hist(sh);
        lds_barrier();
        const uint32_t prefix = sh.prefix;
        const int hi = SHIFT[ps] + WIDTH[ps];
        launder(kr);
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < ngroups) {
                const uint32_t key = kr[i];
                const bool match = key != 0u && (hi == 32 || (key >> (hi & 31)) == prefix);
                atomicAdd(&sh.hist[match ? (key >> SHIFT[ps]) & ((1u << WIDTH[ps]) - 1u) : NBIN + lane_id()], 1u);
            }
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // one 4-key group at a time
        }
        lds_barrier();
        pick_bin(WIDTH[ps], sh);
    }
    if (threadIdx.x == 0) {
        sh.kappa = sh.prefix;
        sh.need_eq = sh.rem;
    }
    lds_barrier();
}

// Steps 1-4 over the register keys kr (key 0 = no key).  Thread tz holds the
// G * 4 consecutive columns 4 * G * tz + j in kr[j], j < 4 * G (G <= NV4), at
// least k + 1 of all keys real; lmin / lmax are the thread's smallest nonzero
// and largest key (0xFFFFFFFF / 0 when it has none).  tz is the thread index,
// passed in so that a caller's loop can keep the column arithmetic from being
// hoisted out of it and held in registers.  On return (after a barrier)
// sh.ocol[slot], slot < k, holds the columns of the k selected keys, slot =
// rank in column order, and sh.okey[slot] their keys when want_keys.
//
// Every thread ends with a mask of its selected keys (bit j = kr[j]):
//   * keys at or above khi, a key whose value bin is known to lie above the
//     bin b1 of the k-th largest key, are selected outright;
//   * keys in [klo, khi), a few bins' worth around b1, are collected in LDS
//     and ranked (key descending, then column): the first k - #outright are
//     selected and set their bits in their owner's mask;
//   * keys below klo are not selected.
// The masks' popcounts give each thread its first slot (one block scan), and
// each thread writes only its selected columns.
template <int NV4, class Hook>
__device__ __forceinline__ void select_regs(uint32_t (&kr)[4 * NV4], int G, uint32_t lmin, uint32_t lmax, int k,
                                            SelectShared &sh, int tz, bool want_keys, Hook &&hook) {
    static_assert(4 * NV4 <= 64, "key masks hold 64 bits");
    const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;

    // 1. range (keys order like scores: min/max over keys)
    uint32_t kmin = wave_scan(lmin, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    uint32_t kmax = wave_scan(lmax, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    if (l == 63) {   // the inclusive scan's last lane holds the wave's result
        sh.wmin[w] = kmin;
        sh.wmax[w] = kmax;
    }
    clear_hist(sh);
    sh.tbits[tid][0] = 0u;
    sh.tbits[tid][1] = 0u;
    if (tid == 0) {
        sh.ncand = 0;
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
    }
    lds_barrier();
    hook(2);
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) {
        kmin = sh.wmin[x] < kmin ? sh.wmin[x] : kmin;
        kmax = sh.wmax[x] > kmax ? sh.wmax[x] : kmax;
    }
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const float range = vmax - vmin;
    const float inv = (float)NBIN / range;
    // value bins need a finite, positive range with a finite scale
    const bool binned = range > 0.f && range < INFINITY && inv < INFINITY;

    uint32_t m0 = 0u, m1 = 0u;   // selected keys: bit j of (m1:m0) = kr[j]
    bool done = false;
    if (binned) {
        // 2. value histogram, bin b1
        auto bin_of = [&](uint32_t key) {
            const float t = (key_value(key) - vmin) * inv;
            return (uint32_t)fminf(t, (float)(NBIN - 1));
        };
        launder(kr);
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < G) atomicAdd(&sh.hist[kr[i] != 0u ? bin_of(kr[i]) : NBIN + l], 1u);
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // one 4-key group at a time
        }
        lds_barrier();
        hook(3);
        pick_bin(0, sh);   // prefix = b1
        const uint32_t b1 = sh.prefix;
        // 3. key thresholds around b1, each checked with the histogram's own
        // bin arithmetic (bins are non-decreasing in the key): keys >= khi lie
        // in bins above b1, keys < klo in bins below it.  A quarter bin of
        // margin; when a check fails the threshold falls back to the range's end.
        const float bw = range / (float)NBIN;
        uint32_t klo = kmin, khi = kmax + 1u;
        if (b1 > 0u) {
            const uint32_t c = score_key(vmin + ((float)b1 - 0.25f) * bw);
            if (c > kmin && c <= kmax && bin_of(c - 1u) < b1) klo = c;
        }
        if (b1 < (uint32_t)(NBIN - 1)) {
            const uint32_t c = score_key(vmin + ((float)b1 + 1.25f) * bw);
            if (c > kmin && c <= kmax && bin_of(c) > b1) khi = c;
        }
        const uint32_t span = khi - klo;
        hook(4);
        launder(kr);
        uint32_t nunc = 0;
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < G) {
                const uint32_t key = kr[i];
                const uint32_t bit = key >= khi ? 1u << (i & 31) : 0u;
                if (i < 32) m0 |= bit; else m1 |= bit;
                nunc += key - klo < span ? 1u : 0u;   // (key 0 wraps past span: klo >= 1)
            }
        }
        hook(5);
        // outright count per wave (summed after the barrier below)
        const uint32_t ns = wave_scan_add((uint32_t)(__builtin_popcount(m0) + __builtin_popcount(m1)));
        if (l == 63) sh.wtot[w] = ns;
        if (__ballot(nunc != 0u) != 0ull) {   // a wave holding uncertain keys: one atomic per wave
            const uint32_t x = wave_scan_add(nunc);
            uint32_t base = 0;
            if (l == 63) base = atomicAdd(&sh.ncand, x);
            uint32_t p = (uint32_t)__builtin_amdgcn_readlane((int)base, 63) + x - nunc;
            if (nunc != 0u) {
#pragma unroll
                for (int i = 0; i < 4 * NV4; ++i) {
                    if (i / 4 < G) {
                        const uint32_t key = kr[i];
                        if (key - klo < span) {
                            if (p < (uint32_t)CCAP) {
                                sh.ckey[p] = key;
                                sh.cpos[p] = ((uint32_t)tz << 6) | (uint32_t)i;
                            }
                            ++p;
                        }
                    }
                }
            }
        }
        lds_barrier();
        hook(6);
        const uint32_t nc = sh.ncand;
        uint32_t sure = 0;
#pragma unroll
        for (int i = 0; i < NWAVE; ++i) sure += sh.wtot[i];
        if (nc <= (uint32_t)CCAP) {
            // sure < k <= sure + nc: the outright keys are all in bins above
            // b1, and the uncertain ones include every key of b1.  Uncertain
            // key c is selected when fewer than k - sure uncertain keys come
            // before it (larger, or equal at a lower column).
            const uint32_t need = (uint32_t)k - sure;
            if (nc <= (uint32_t)kWave) {
                if (w == 0) {   // one wave, the keys in its lanes
                    const uint32_t key = (uint32_t)l < nc ? sh.ckey[l] : 0u;
                    const uint32_t pos = (uint32_t)l < nc ? sh.cpos[l] : 0u;
                    uint32_t before = 0;
                    for (uint32_t j = 0; j < nc; ++j) {
                        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)key, (int)j);
                        const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)pos, (int)j);
                        before += (o > key || (o == key && op < pos)) ? 1u : 0u;
                    }
                    if ((uint32_t)l < nc && before < need)
                        atomicOr(&sh.tbits[pos >> 6][(pos >> 5) & 1u], 1u << (pos & 31u));
                }
            } else if ((uint32_t)tid < nc) {
                const uint32_t key = sh.ckey[tid], pos = sh.cpos[tid];
                uint32_t before = 0;
                for (uint32_t j = 0; j < nc; ++j) {
                    const uint32_t o = sh.ckey[j];
                    before += (o > key || (o == key && sh.cpos[j] < pos)) ? 1u : 0u;
                }
                if (before < need) atomicOr(&sh.tbits[pos >> 6][(pos >> 5) & 1u], 1u << (pos & 31u));
            }
            lds_barrier();
            m0 |= sh.tbits[tid][0];
            m1 |= sh.tbits[tid][1];
            done = true;
        }
    }
    if (!done) {
        // exact kappa by radix passes; then keys > kappa, and the first
        // need_eq keys == kappa in column order
        radix_kappa<NV4>(kr, G, k, sh);
        const uint32_t kappa = sh.kappa, need_eq = sh.need_eq;
        launder(kr);
        m0 = m1 = 0u;
        uint32_t eqc = 0;
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < G) {
                const uint32_t bit = kr[i] > kappa ? 1u << (i & 31) : 0u;
                if (i < 32) m0 |= bit; else m1 |= bit;
                eqc += kr[i] == kappa ? 1u : 0u;
            }
        }
        const uint32_t eqb = block_excl_scan(eqc, sh.wtot);
        uint32_t quota = need_eq > eqb ? need_eq - eqb : 0u;
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < G && kr[i] == kappa && quota != 0u) {
                if (i < 32) m0 |= 1u << (i & 31); else m1 |= 1u << (i & 31);
                --quota;
            }
        }
    }

    // 4. emit: each thread's selected keys take consecutive slots from the
    // count of selected keys in the threads before it (column order)
    uint32_t slot = block_excl_scan((uint32_t)(__builtin_popcount(m0) + __builtin_popcount(m1)), sh.wtot);
    const int colbase = 4 * G * tz;
    if (want_keys) {
        launder(kr);
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < G && (((i < 32 ? m0 : m1) >> (i & 31)) & 1u)) {
                if (slot < (uint32_t)k) {   // (exactly k keys are selected)
                    sh.ocol[slot] = colbase + i;
                    sh.okey[slot] = kr[i];
                }
                ++slot;
            }
        }
    } else {
        while (m0 != 0u) {
            if (slot < (uint32_t)k) sh.ocol[slot] = colbase + __builtin_ctz(m0);   // (exactly k keys are selected)
            ++slot;
            m0 &= m0 - 1u;
        }
        while (m1 != 0u) {
            if (slot < (uint32_t)k) sh.ocol[slot] = colbase + 32 + __builtin_ctz(m1);
            ++slot;
            m1 &= m1 - 1u;
        }
    }
    lds_barrier();   // selection in sh.ocol / sh.okey
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t m) {   // set bits of m below this lane
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The bin holding the rank-th largest of the values counted in hist[0, NB)
// (bins ordered like the values; 1 <= rank <= the total): b, with rem = its
// rank inside the bin and above = the count in the bins above it.  Wave w
// sums the group of bins [GB w, GB w + GB) into gsum[w]; after one barrier
// every wave finds the group from the 16 sums and then the bin inside it on
// its own (the same answer in every wave, no barrier after).  Each lane reads
// a handful of words.
template <int NB>
__device__ __forceinline__ void block_pick_bin(const uint32_t *hist, uint32_t *gsum, uint32_t rank, uint32_t &b,
                                               uint32_t &rem, uint32_t &above) {
    constexpr int GB = NB / NWAVE;   // bins per group
    constexpr int PL = GB / kWave;   // bins per lane
    static_assert(PL * kWave * NWAVE == NB && NWAVE <= kWave, "bin groups");
    const int l = lane_id(), w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < PL; ++q) sum += hist[GB * w + PL * l + q];
    sum = wave_scan_add(sum);
    if (l == 63) gsum[w] = sum;   // (the inclusive scan's last lane: the wave's total)
    lds_barrier();
    // the group: lane g holds group NWAVE - 1 - g (from the top)
    const uint32_t gv = l < NWAVE ? gsum[NWAVE - 1 - l] : 0u;
    const uint32_t gx = wave_scan_add(gv) - gv;
    const uint64_t gown = __ballot(l < NWAVE && gx < rank && rank <= gx + gv);   // exactly one lane
    const int gl = (int)__builtin_ctzll(gown);
    const int grp = NWAVE - 1 - gl;
    const uint32_t gabove = (uint32_t)__builtin_amdgcn_readlane((int)gx, gl);
    const uint32_t grank = rank - gabove;
    // the bin inside the group: lane l holds bins top - PL l - q, q < PL
    const int top = GB * grp + GB - 1;
    uint32_t c[PL], lsum = 0;
#pragma unroll
    for (int q = 0; q < PL; ++q) {
        c[q] = hist[top - PL * l - q];
        lsum += c[q];
    }
    uint32_t acc = wave_scan_add(lsum) - lsum;
    int mine = -1;
    uint32_t mrem = 0, mabove = 0;
#pragma unroll
    for (int q = 0; q < PL; ++q) {
        if (acc < grank && grank <= acc + c[q]) {
            mine = top - PL * l - q;
            mrem = grank - acc;
            mabove = acc;
        }
        acc += c[q];
    }
    const uint64_t own = __ballot(mine >= 0);   // exactly one lane
    const int src = (int)__builtin_ctzll(own);
    b = (uint32_t)__builtin_amdgcn_readlane(mine, src);
    rem = (uint32_t)__builtin_amdgcn_readlane((int)mrem, src);
    above = gabove + (uint32_t)__builtin_amdgcn_readlane((int)mabove, src);
}

// Exact k largest of nc candidate keys held in LDS in column order (ckey[j],
// order-preserving keys, j < nc, k < nc <= CAP), ties to the lower index:
//   * a 2048-bin value histogram over [vlo, vhi] (clamped at both ends, so
//     non-decreasing in the key; vlo / vhi bound the keys' values), and the
//     bin b1 of the k-th largest (block_pick_bin: per-wave group sums, one
//     barrier, then every wave on its own);
//   * every key of a bin above b1 is taken; b1's keys (a few on spread-out
//     scores) are listed and ranked by every wave on its own (key descending,
//     then index), and the first rem = k - #above are taken;
//   * wave w owns the slots [S w, S w + S), S = the candidates per wave
//     rounded up to 64, and calls emit(r, j) for each taken candidate j with
//     its output slot r (its rank in index order).
// Returns false, having emitted nothing, when [vlo, vhi] cannot be binned or
// b1 holds more than 64 keys (many equal scores): the caller then selects
// another way (sh free again: the call ends with a barrier, or has not
// touched it).  Uses sh.hist, sh.ncand, sh.ckey/cpos[0, 64), sh.tbits as a
// CAP-bit map, gsum and wcnt [NWAVE].
template <int CAP, class Emit>
__device__ __forceinline__ bool lds_cand_select(const uint32_t *ckey, int nc, int k, float vlo, float vhi,
                                                SelectShared &sh, uint32_t *gsum, uint32_t *wcnt, Emit &&emit) {
    constexpr int NB = NBIN;
    constexpr int SPW_MAX = CAP / NWAVE;
    static_assert(CAP % (NWAVE * kWave) == 0 && CAP / 32 <= 2 * TPB && CCAP >= kWave, "candidate select tables");
    const float crange = vhi - vlo;
    const float cinv = (float)NB / crange;
    if (!(crange > 0.f && crange < INFINITY && cinv < INFINITY)) return false;
    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nu = (nc + NWAVE * kWave - 1) / (NWAVE * kWave);   // slots per lane
    const int S = kWave * nu;
    uint32_t *chist = sh.hist;
    uint32_t *selb = reinterpret_cast<uint32_t *>(sh.tbits);
    for (int i = tid; i < NB; i += TPB) chist[i] = 0u;
    if (tid == 0) sh.ncand = 0u;
    auto kbin = [&](uint32_t key) {
        return (uint32_t)fminf(fmaxf((key_value(key) - vlo) * cinv, 0.f), (float)(NB - 1));
    };
    lds_barrier();
#pragma unroll
    for (int u = 0; u < SPW_MAX / kWave; ++u) {
        const int j = S * w + kWave * u + l;
        if (u < nu && j < nc) atomicAdd(&chist[kbin(ckey[j])], 1u);
    }
    lds_barrier();
    uint32_t b1, rem, above;
    block_pick_bin<NB>(chist, gsum, (uint32_t)k, b1, rem, above);
    uint32_t gtw = 0;
#pragma unroll
    for (int u = 0; u < SPW_MAX / kWave; ++u) {
        const int j = S * w + kWave * u + l;
        const bool ok = u < nu && j < nc;
        const uint32_t bj = ok ? kbin(ckey[j]) : 0u;
        gtw += (uint32_t)__popcll(__ballot(ok && bj > b1));
        if (ok && bj == b1) {
            const uint32_t q = atomicAdd(&sh.ncand, 1u);
            if (q < (uint32_t)kWave) {
                sh.ckey[q] = ckey[j];
                sh.cpos[q] = (uint32_t)j;
            }
        }
    }
    if (l == 0) wcnt[w] = gtw;
    lds_barrier();
    const uint32_t nb1 = sh.ncand;
    if (nb1 > (uint32_t)kWave) {
        lds_barrier();   // every thread has read nb1
        return false;
    }
    // lane e holds b1's entry e
    const uint32_t key = (uint32_t)l < nb1 ? sh.ckey[l] : 0u;
    const uint32_t pos = (uint32_t)l < nb1 ? sh.cpos[l] : 0u;
    uint32_t before = 0;
    for (uint32_t e = 0; e < nb1; ++e) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)key, (int)e);
        const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)pos, (int)e);
        before += (o > key || (o == key && op < pos)) ? 1u : 0u;
    }
    const bool sel = (uint32_t)l < nb1 && before < rem;
    // this wave's first output slot: the keys above b1 in the waves before
    // it, and the taken b1 keys at lower indices
    uint32_t slot = (uint32_t)__popcll(__ballot(sel && pos < (uint32_t)(S * w)));
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) slot += x < w ? wcnt[x] : 0u;
    // the taken b1 keys of this wave's slots, as bits of its own words of
    // selb (written and read by this wave only: LDS keeps a wave's operations
    // in order)
    if (l < S / 32) selb[(S / 32) * w + l] = 0u;
    if (sel && pos / (uint32_t)S == (uint32_t)w) atomicOr(&selb[pos >> 5], 1u << (pos & 31u));
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
#pragma unroll
    for (int u = 0; u < SPW_MAX / kWave; ++u) {
        if (u >= nu) break;
        const int j = S * w + kWave * u + l;
        bool tk = false;
        if (j < nc) {
            const uint32_t bj = kbin(ckey[j]);
            tk = bj > b1 || (bj == b1 && ((selb[j >> 5] >> (j & 31)) & 1u));
        }
        const uint64_t mt = __ballot(tk);
        const uint32_t r = slot + lane_rank(mt);
        if (tk && r < (uint32_t)k) emit(r, j);   // (exactly k are taken)
        slot += (uint32_t)__popcll(mt);
    }
    return true;
}

}  // namespace

}  // namespace dsa
