// Phases shared by the two construction kernels of libdtree (the streaming kernel in
// build_kernels.hip, the W-resident kernel in build_resident.hip): workgroup barriers and
// scans, bounded waits and work tickets, the expansion epilogue on MFMA accumulators,
// the merge of a parent row's split records, the per-request select and the emit.
// Functions that depend on the workgroup size take it as the template parameter NT.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {

// Phase timestamps (DT_TRACE builds only): thread 0 of a workgroup records the wall clock
// for (level, slot), 16 slots per level.  Slots: 0 woke for the level, 1 first expansion item set up, 2
// expansion items done, 3 merge loop done, 4 a select done, 5 a merge published, 6 first
// merge task started, 7 a select's candidates loaded, 8 tile-mode parent rows read.  Level 0 slot 0 = kernel start; the last level's slots 0/1 = emit start/end.
#ifdef DT_TRACE
#define DT_STAMP(lv, sl)                                                                    \
    do {                                                                                    \
        if (threadIdx.x == 0)                                                               \
            a.trace[((size_t)blockIdx.x * kTraceLevels + (lv)) * 16 + (sl)] = wall_clock64(); \
    } while (0)
#else
#define DT_STAMP(lv, sl) \
    do {                 \
    } while (0)
#endif

// ---------------------------------------------------------------------------------------
// Workgroup helpers.
// ---------------------------------------------------------------------------------------
// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every global load,
// store and atomic this wavefront has in flight (one memory round trip after a store);
// exchanges of global data between workgroups use publish_wg() instead.
__device__ __forceinline__ void lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Exclusive prefix sum over a workgroup of NW wavefronts: a shuffle scan inside each
// wavefront, then the wavefront totals through LDS (two barriers).  sh needs NW ints.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) sh[w] = x;
    lds_sync();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int si = sh[i];
        base += i < w ? si : 0;
        tot += si;
    }
    if (total) *total = tot;
    lds_sync();  // sh is free for the caller again
    return base + x - v;
}

template <int NW>
__device__ __forceinline__ int block_sum(int v, int* sh) {
    int total;
    block_exclusive_scan<NW>(v, sh, &total);
    return total;
}

// Bounded waits poll at most BuildArgs::spin_limit times (each poll sleeps ~128 cycles; the
// default, kSpinLimit, is about two seconds, far above any level's work).

// Thread 0 waits until *p >= target (or the error flag is set); the result is broadcast to
// the workgroup.  Returns false on error or time-out.
__device__ __forceinline__ bool wait_at_least(unsigned* sync, const unsigned* p, unsigned target,
                                              int* bcast, uint32_t limit) {
    if (threadIdx.x == 0) {
        int ok = 1;
        uint32_t it = 0;
        while ((int)(cld32(p) - target) < 0) {
            __builtin_amdgcn_s_sleep(2);
            if (++it > limit) {
                cst32(sync + kSyncErr, 1u);
                ok = 0;
                break;
            }
            if ((it & 63u) == 0u && cld32(sync + kSyncErr) != 0u) {
                ok = 0;
                break;
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        bcast[0] = ok;
    }
    lds_sync();
    const bool ok = bcast[0] != 0;
    lds_sync();
    return ok;
}

// Thread 0 waits until the generation word's level reaches `level` (or the error flag is
// set); the word is broadcast to the workgroup.  Returns false on error or time-out.
__device__ __forceinline__ bool wait_gen(unsigned* sync, int level, int* bcast, uint64_t* gen,
                                         uint32_t limit) {
    if (threadIdx.x == 0) {
        int ok = 1;
        uint32_t it = 0;
        uint64_t g;
        while ((int)((g = cld64(sync + kSyncGen)) & 0xFFu) < level) {
            __builtin_amdgcn_s_sleep(2);
            if (++it > limit) {
                cst32(sync + kSyncErr, 1u);
                ok = 0;
                break;
            }
            if ((it & 63u) == 0u && cld32(sync + kSyncErr) != 0u) {
                ok = 0;
                break;
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        bcast[0] = ok;
        bcast[1] = (int)(uint32_t)g;
        bcast[2] = (int)(uint32_t)(g >> 32);
    }
    lds_sync();
    const bool ok = bcast[0] != 0;
    *gen = (uint64_t)(uint32_t)bcast[1] | ((uint64_t)(uint32_t)bcast[2] << 32);
    lds_sync();
    return ok;
}

// Work tickets of a level: thread 0 takes the next index of the level's counter and the
// workgroup gets it through LDS.  Indices below T*S are expansion items, the next M are
// merge rows, larger ones mean the level has no work left for this workgroup.  Tickets are
// handed out in increasing order, so by the time any merge row is claimed every expansion
// item has been claimed by a running workgroup: a workgroup only ever waits for work that
// running workgroups hold, and a round completes with any number of resident workgroups.
__device__ __forceinline__ int claim_ticket(unsigned* sync, int level, int* bcast) {
    if (threadIdx.x == 0) bcast[0] = (int)cadd32(sync + kSyncClaim + level, 1u);
    lds_sync();
    const int c = bcast[0];
    lds_sync();
    return c;
}

// Vocabulary splits for T tiles on a grid of G workgroups: about one item per workgroup,
// at most kMaxSplits (so that one workgroup can merge a row's records in one pass), and a
// multiple of 8 when >= 8 so that all tiles of one split run on the same XCD (blocks are
// dealt round-robin to the 8 XCDs) and share that split's W rows in its L2.
__device__ __forceinline__ int splits_for(int T, int G, int NB) {
    int s = T > 0 ? G / T : 1;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s >= 8) s &= ~7;
    if (s > NB) s = NB;
    if (s < 1) s = 1;
    return s;
}

// Parent rows of a level (two buffers: a level's selects write the next level's rows while
// other requests' merges still read the current ones).
__device__ __forceinline__ RowRec* level_rows(const BuildArgs& a, int level) {
    return a.rows + (size_t)(level & 1) * a.R * a.Ncap;
}

// Staging of one request's emit (see emit_request).
struct EmitSmem {
    uint64_t keys[kMaxNcap];
    uint32_t lowc[kMaxNcap];  // canonical order (zero-padded to a multiple of 8)
    int parc[kMaxNcap];
    int fcnt[kMaxB + 1];
    int n;
    uint32_t fself[kMaxB * kMaxNcap + 8];  // front[d][m].self for d = 1..B-1 (0 = no node)
};

// ---------------------------------------------------------------------------------------
// Shared memory of the persistent kernel (one workgroup; phases reuse the first region).
// ---------------------------------------------------------------------------------------
// Staging of one request's select (see select_request).
struct SelSmem {
    uint64_t keys[kSelectSlots];
    uint64_t sorted[kMaxNcap];
    int ctok[kMaxNcap * kMaxK];
    uint64_t chash[kMaxNcap * kMaxK];
};

// vmcnt(N) with expcnt and lgkmcnt unconstrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait for this wavefront's outstanding global loads (including global->LDS copies).
__device__ __forceinline__ void wait_vm() { wait_vmcnt<0>(); }

// LDS reads of the staging ring, written as asm that waits for its own results: the compiler
// would otherwise drain every global->LDS copy in flight before each read (it cannot tell
// the slot being read from the slots still being filled).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void lds_read4_b128(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                               u32x4_t& r0, u32x4_t& r1, u32x4_t& r2, u32x4_t& r3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}
__device__ __forceinline__ void lds_read4_b64(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                              u32x2_t& r0, u32x2_t& r1, u32x2_t& r2, u32x2_t& r3) {
    asm volatile(
        "ds_read_b64 %0, %4\n\t"
        "ds_read_b64 %1, %5\n\t"
        "ds_read_b64 %2, %6\n\t"
        "ds_read_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads(), which would also wait for
// every global load in flight; the callers order LDS themselves.
__device__ __forceinline__ void bare_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------------------
// Expansion epilogue on the accumulators.  Lane half h holds columns c0 + 8j + 4h + i
// (j, i = 0..3) of its parent row; lw[j] holds the raw block logits of group j (4 bf16 in
// .x/.y, or 4 floats).
// ---------------------------------------------------------------------------------------
constexpr float kGumbelMax = 17.35f;  // -log(-log u) < 17.33 for u <= 1 - 2^-25

// Raw block logits of the four column groups of a lane: 4 bf16 per group in a uint2, or 4
// floats in a uint4.
template <bool L_BF16>
struct LGroups {
    typename std::conditional<L_BF16, uint2, uint4>::type g[4];
};

template <bool L_BF16>
__device__ __forceinline__ void load_lgroups(const BuildArgs& a, size_t lbase, int c0, int h,
                                             bool lvec, LGroups<L_BF16>& lw) {
    if (lvec) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int c = c0 + 8 * j + 4 * h;
            c = c < a.V ? c : a.V - 4;  // V is a multiple of 4 here; masked in the epilogue
            if constexpr (L_BF16)
                lw.g[j] = *(const uint2*)((const uint16_t*)a.L + lbase + c);
            else
                lw.g[j] = *(const uint4*)((const float*)a.L + lbase + c);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int c = c0 + 8 * j + 4 * h + i;
                c = c < a.V ? c : a.V - 1;
                if constexpr (L_BF16)
                    w[i] = (uint32_t)((const uint16_t*)a.L)[lbase + c];
                else
                    w[i] = __float_as_uint(((const float*)a.L)[lbase + c]);
            }
            if constexpr (L_BF16)
                lw.g[j] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
            else
                lw.g[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// Descending bitonic sort of n = 1, 2, 4 or 8 floats (compile-time indices).
template <int N>
__device__ __forceinline__ void sort_desc(float* v) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool desc = (i & size) == 0;
                    const float hi = fmaxf(v[i], v[j]), lo = fminf(v[i], v[j]);
                    v[i] = desc ? hi : lo;
                    v[j] = desc ? lo : hi;
                }
            }
        }
    }
}

// The KT-th largest of 16 values (a lower bound for pruning candidates): sort groups of KT,
// then merge sorted groups pairwise keeping the KT largest (the elementwise maxima of one
// list and the reversed other list are exactly the KT largest of both, as a bitonic
// sequence); the last merge only needs the minimum of that set.
template <int KT>
__device__ __forceinline__ float kth_largest16(const float (&z)[16]) {
    constexpr int NG = 16 / KT;
    float g[NG][KT];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
#pragma unroll
        for (int i = 0; i < KT; ++i) g[q][i] = z[q * KT + i];
        sort_desc<KT>(g[q]);
    }
#pragma unroll
    for (int n = NG; n > 2; n >>= 1) {
#pragma unroll
        for (int q = 0; q < n / 2; ++q) {
            float c[KT];
#pragma unroll
            for (int i = 0; i < KT; ++i) c[i] = fmaxf(g[2 * q][i], g[2 * q + 1][KT - 1 - i]);
            // bitonic -> descending: half-cleaners
#pragma unroll
            for (int half = KT / 2; half >= 1; half >>= 1) {
#pragma unroll
                for (int i = 0; i < KT; ++i) {
                    if ((i & half) == 0) {
                        const float hi = fmaxf(c[i], c[i + half]), lo = fminf(c[i], c[i + half]);
                        c[i] = hi;
                        c[i + half] = lo;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < KT; ++i) g[q][i] = c[i];
        }
    }
    float m = INFINITY;
#pragma unroll
    for (int i = 0; i < KT; ++i) m = fminf(m, fmaxf(g[0][i], g[1][KT - 1 - i]));
    return m;
}

// Block logits of a lane's 16 columns as float32, laid out like the accumulator, so that the
// MFMA chain adds the Markov bias onto them: z = L + U.W comes out of the MFMA directly.
template <bool L_BF16>
__device__ __forceinline__ void lgroups_to_acc(const LGroups<L_BF16>& lw, f32x16& acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (L_BF16) {
            acc[4 * j + 0] = bf16_lo(lw.g[j].x);
            acc[4 * j + 1] = bf16_hi(lw.g[j].x);
            acc[4 * j + 2] = bf16_lo(lw.g[j].y);
            acc[4 * j + 3] = bf16_hi(lw.g[j].y);
        } else {
            acc[4 * j + 0] = __uint_as_float(lw.g[j].x);
            acc[4 * j + 1] = __uint_as_float(lw.g[j].y);
            acc[4 * j + 2] = __uint_as_float(lw.g[j].z);
            acc[4 * j + 3] = __uint_as_float(lw.g[j].w);
        }
    }
}

// Per-lane select through an all-ones / all-zero bit mask.  The mask passes an empty asm
// statement so that the compiler cannot see it is a boolean: written as plain selects, a
// tree keyed on the bits of a per-lane index is folded back into a dynamic vector index,
// which is lowered through a private (scratch) copy of the vector.
__device__ __forceinline__ uint32_t lane_bit_mask(int e, int bit) {
    uint32_t m = 0u - (((uint32_t)e >> bit) & 1u);
    asm volatile("" : "+v"(m));
    return m;
}
__device__ __forceinline__ float sel_bits(uint32_t m, float if_clear, float if_set) {
    return __uint_as_float((__float_as_uint(if_set) & m) | (__float_as_uint(if_clear) & ~m));
}

// z[e] for a per-lane index e (0..15): a 4-level select tree in registers.
__device__ __forceinline__ float select16(const f32x16& z, int e) {
    const uint32_t m0 = lane_bit_mask(e, 0), m1 = lane_bit_mask(e, 1), m2 = lane_bit_mask(e, 2),
                   m3 = lane_bit_mask(e, 3);
    float v8[8], v4[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) v8[i] = sel_bits(m0, z[2 * i], z[2 * i + 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = sel_bits(m1, v8[2 * i], v8[2 * i + 1]);
    const float v0 = sel_bits(m2, v4[0], v4[1]), v1 = sel_bits(m2, v4[2], v4[3]);
    return sel_bits(m3, v0, v1);
}

// Epilogue of one 32-column block for one parent row: z holds the row's 16 values of this
// lane (columns c0 + 8(e/4) + 4h + e%4).  Updates the online log-sum-exp, then offers the
// values that can still rank among the KT best to the ranked list.  Any lane's KT-th list
// entry is a lower bound for the row's final KT-th entry (its list holds KT entries of other
// columns that rank above it), so the candidate test uses the best such bound known: the
// lane's own and `row_kth` (LDS, shared by the workgroup's lanes of the row; may be null).
template <int KT, bool SAMPLE>
__device__ __forceinline__ void expand_epilogue(const BuildArgs& a, f32x16& z, int c0, int h,
                                                uint64_t hh, bool live, uint64_t* row_kth,
                                                TopK<KT>& top, Lse2& st) {
    if (c0 + kBlockCols > a.V) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (c0 + 8 * (e >> 2) + 4 * h + (e & 3) >= a.V) z[e] = -INFINITY;
    }
    float zmax = z[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) zmax = fmaxf(zmax, z[e]);
    if (zmax != -INFINITY) {
        const float cm = zmax * a.y2scale;
        if (cm > st.m) {
            st.s = (st.m == -INFINITY) ? 0.0f : st.s * exp2f(st.m - cm);
            st.m = cm;
        }
        // terms below 2^-126 of the running maximum flush to zero: far below float32
        // resolution of the sum
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) ps += __builtin_amdgcn_exp2f(z[e] * a.y2scale - st.m);
        st.s += ps;
    }
    // lanes l and l ^ 32 hold the same row: each takes the better of the two KT-th entries.
    // A swap of the wavefront's halves leaves the entries of lanes l % 32 and l % 32 + 32 in
    // the two results (a VALU exchange, no LDS round trip).
    uint64_t kth = top.k[KT - 1];
    {
        const uint32_t lo = (uint32_t)kth, hi = (uint32_t)(kth >> 32);
        const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        const uint64_t e0 = ((uint64_t)sh[0] << 32) | sl[0], e1 = ((uint64_t)sh[1] << 32) | sl[1];
        kth = e0 > kth ? e0 : kth;
        kth = e1 > kth ? e1 : kth;
    }
    if (!live) return;
    if (row_kth) kth = kth > *row_kth ? kth : *row_kth;
    const float tk = kth ? entry_key(kth) : -INFINITY;
    // Candidates are values z with z >= thr, a superset of those that can enter the list
    // (ties and the Gumbel noise are settled by push(), which compares exact entries).
    // Sample keys are z / T + G with G < kGumbelMax, so z < (tk - kGumbelMax) T cannot
    // qualify.  thr never drops below the lowest finite float, so masked columns (-inf)
    // never qualify.
    float thr = SAMPLE ? (tk - kGumbelMax) / a.invT : tk;
    if (zmax < thr) return;
    if constexpr (!SAMPLE) {
        if (top.k[KT - 1] == 0) thr = fmaxf(thr, kth_largest16<KT>(*(const float(*)[16]) & z));
    }
    thr = fmaxf(thr, -3.402823466e38f);
    // Candidates are offered one at a time per lane, lowest index first: the wavefront loops
    // while any of its lanes has one left, which is one or two rounds once the lists are
    // warm (instead of 16 predicated insertions whenever any lane has a candidate).
    // Insertion order does not change the list (push keeps the KT largest entries).
    if constexpr (SAMPLE) {
        uint32_t gm = 0;  // 4-column groups with a candidate
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool any = z[4 * j] >= thr || z[4 * j + 1] >= thr || z[4 * j + 2] >= thr ||
                             z[4 * j + 3] >= thr;
            gm |= any ? (1u << j) : 0u;
        }
        if (gm == 0u) return;
        while (gm != 0u) {
            const int j = __builtin_ctz(gm);
            gm &= gm - 1u;
            float zg[4];
            {
                const uint32_t m0 = lane_bit_mask(j, 0), m1 = lane_bit_mask(j, 1);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    zg[i] = sel_bits(m1, sel_bits(m0, z[i], z[4 + i]), sel_bits(m0, z[8 + i], z[12 + i]));
            }
            const int cg = c0 + 8 * j + 4 * h;
            const uint4 w = rand4((uint32_t)(cg >> 2), STREAM_GUMBEL, hh, a.seed_lo, a.seed_hi);
            const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (zg[i] >= thr) {
                    // Exact pre-test before the key is formed: y + G(u) >= tk, with
                    // G(u) = -log(-log u) increasing in u, holds iff u >= exp(-e^(y - tk)).
                    // The 2^-16 margin in u (worth > 4e-5 in key units, since G' >= e) covers
                    // the float error of both sides, so no column whose key could reach the
                    // list is skipped; push() still compares the exact keys.  An empty list
                    // (tk = -inf) gives a bound of 0.
                    const float ustar = __expf(-__expf(zg[i] * a.invT - tk));
                    if (u01(wv[i]) >= ustar - 1.52587890625e-05f)
                        top.push(pack_entry(zg[i] * a.invT + gumbel(wv[i]), cg + i), zg[i] * a.y2scale);
                }
            }
        }
    } else {
        uint32_t mask = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) mask |= (z[e] >= thr) ? (1u << e) : 0u;
        if (mask == 0u) return;
        while (mask != 0u) {
            const int e = __builtin_ctz(mask);
            mask &= mask - 1u;
            const float v = select16(z, e);
            top.push(pack_entry(v, c0 + 8 * (e >> 2) + 4 * h + (e & 3)), v * a.y2scale);
        }
    }
    if (row_kth && top.k[KT - 1] != 0)
        atomicMax((unsigned long long*)row_kth, (unsigned long long)top.k[KT - 1]);
}

// Record of a list: (m, s) of the log-sum-exp, then KT packed entries as (lo, hi) words,
// then the KT tempered logits.
template <int KT>
__device__ __forceinline__ void put_list(float* v, const TopK<KT>& t, const Lse2& s) {
    v[0] = s.m;
    v[1] = s.s;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
        v[2 + 2 * i] = __uint_as_float((uint32_t)t.k[i]);
        v[3 + 2 * i] = __uint_as_float((uint32_t)(t.k[i] >> 32));
        v[2 + 2 * KT + i] = t.y[i];
    }
}

template <int KT>
__device__ __forceinline__ void get_list(const float* v, TopK<KT>& t, Lse2& s) {
    s.m = v[0];
    s.s = v[1];
#pragma unroll
    for (int i = 0; i < KT; ++i) {
        t.k[i] = (uint64_t)__float_as_uint(v[2 + 2 * i]) |
                 ((uint64_t)__float_as_uint(v[3 + 2 * i]) << 32);
        t.y[i] = v[2 + 2 * KT + i];
    }
}

// ---------------------------------------------------------------------------------------
// Merge of one parent row (whole workgroup): combine its S split records; child j gets
// q = 2^(y2 - lse2), bin = min(15, floor(16 q)), s = fl32(s_parent * cal[bin]),
// logq = (y2 - lse2) ln 2, and its selection key.  Returns the row's request.
// ---------------------------------------------------------------------------------------
template <int KT>
__device__ __forceinline__ void fetch_record(const float* rec, uint64_t (&w)[rec_floats(KT) / 2]) {
#pragma unroll
    for (int q = 0; q < rec_floats(KT) / 2; ++q) w[q] = cld64((const char*)rec + 8 * q);
}

template <int KT>
__device__ __forceinline__ void merge_fetched(const uint64_t (&w)[rec_floats(KT) / 2], TopK<KT>& top,
                                              Lse2& acc) {
    constexpr int RS = rec_floats(KT);
    float v[RS];
#pragma unroll
    for (int q = 0; q < RS / 2; ++q) {
        v[2 * q] = __uint_as_float((uint32_t)w[q]);
        v[2 * q + 1] = __uint_as_float((uint32_t)(w[q] >> 32));
    }
    TopK<KT> o;
    Lse2 os;
    get_list<KT>(v, o, os);
    acc.merge(os.m, os.s);
    top.merge(o.k, o.y);
}

// Returns the row's request and its rows at this level (F) through *req / *F.  NT threads
// (S <= NT split records, one per thread); mrec holds one list per wavefront, mchild
// receives the row's children as (token | survival << 32, hash) pairs.
template <int KT, int NT>
__device__ __forceinline__ void merge_row(const BuildArgs& a, int level, int S, int m,
                                          float (*mrec)[rec_floats(KT)],
                                          uint64_t (*mchild)[kMaxK], int* req_out, int* F_out) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x + opaque_zero(), lane = tid & 63, wave = threadIdx.x >> 6;
    constexpr int RS = rec_floats(KT);
    TopK<KT> top;
    top.init();
    Lse2 acc;
    acc.init();
    const float* base = a.partials + (size_t)m * S * RS;
    const int s0 = tid < S ? tid : S - 1;
    // the parent row is loaded with the split records (one round trip)
    const RowRec* rr = level_rows(a, level) + m;
    const uint64_t r0 = cld64(rr), r1 = cld64((const char*)rr + 8), r2 = cld64((const char*)rr + 16),
                   r3 = cld64((const char*)rr + 24);
    uint64_t w0[RS / 2];
    fetch_record<KT>(base + (size_t)s0 * RS, w0);
    const int req = (int)(uint32_t)r0, fi = (int)(uint32_t)(r0 >> 32);
    const float par_s = __uint_as_float((uint32_t)(r1 >> 32));
    const uint64_t par_hash = r2;
    *req_out = req;
    *F_out = (int)(uint32_t)r3;
    const int lvl = level - 1;
    if (tid < S) merge_fetched<KT>(w0, top, acc);
    DT_STAMP(level, 9);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        acc.merge_xor(off);
        top.merge_xor(off);
    }
    if (lane == 0) put_list<KT>(mrec[wave], top, acc);
    lds_sync();
    DT_STAMP(level, 10);
    if (wave == 0) {
        get_list<KT>(mrec[lane % NW], top, acc);
#pragma unroll
        for (int off = 1; off < NW; off <<= 1) {
            acc.merge_xor(off);
            top.merge_xor(off);
        }
        const float lse2 = acc.m + log2f(acc.s);
        // lane j < k computes child j (every lane holds the whole merged list; each picks
        // its own entry with selects, so the k children are computed side by side)
        uint64_t kj = top.k[0];
        float yj = top.y[0];
#pragma unroll
        for (int j = 1; j < KT; ++j) {
            kj = lane == j ? top.k[j] : kj;
            yj = lane == j ? top.y[j] : yj;
        }
        if (lane < a.k) {
            const int j = lane;
            const float l2 = yj - lse2;
            const float q = exp2f(l2);
            int bin = (int)floorf(16.0f * q);
            bin = bin > 15 ? 15 : (bin < 0 ? 0 : bin);
            float cv = a.cal[0];
#pragma unroll
            for (int ii = 1; ii < 16; ++ii) cv = (bin == ii) ? a.cal[ii] : cv;
            ChildRec c;
            // a list shorter than k (possible only with non-finite logits) leaves the
            // missing children token -1: never selected
            c.token = kj != 0 ? entry_tok(kj) : -1;
            c.s = par_s * cv;
            c.logq = l2 * 0.69314718055994530942f;
            c.pad = 0;
            c.hash = child_hash(par_hash, c.token);
            st_child(a.arena + (((size_t)req * a.B + lvl) * a.Ncap + fi) * a.k + j, c);
            mchild[0][j] = (uint64_t)(uint32_t)c.token | ((uint64_t)__float_as_uint(c.s) << 32);
            mchild[1][j] = c.hash;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Select, one workgroup per request, run by the workgroup that merged the request's last
// row: candidates = the kept set + this level's children (read as child records, with the
// kept count, budget and threshold, in one round of loads); drop survival < tau; bitonic
// sort (descending key) in LDS; keep min(n_budget, #left).  The kept nodes of depth `level`
// become the next frontier in canonical order: their frontier entries (for the emit) and
// their parent rows of the next level, at rows allocated with one atomic that also counts
// the requests.  The last request to finish publishes the next level's sizes in the
// generation word.
// ---------------------------------------------------------------------------------------

// `mine` (or null): the children of a single-row request, just merged by this workgroup and
// still in LDS as (token | survival << 32, hash) pairs.
template <int NT>
__device__ __forceinline__ void select_request(const BuildArgs& a, int level, int req, int F,
                                               unsigned nreq, SelSmem& ss, int* sh, int* bcast,
                                               const uint64_t (*mine)[kMaxK]) {
    // per-thread values below are recomputed at every call: hoisted out of the persistent
    // loop they were spilled and reloaded one round trip at a time
    const int tid = threadIdx.x + opaque_zero();
    const int lvl = level - 1;
    const int Ncap = a.Ncap, k = a.k;
    const int nchild = F * k;
    const int nprev = cldi(a.scount + req);
    const int nbudget = cldi(a.nbeff + req);
    const float tau = a.tau[req];
    // slot i < Ncap: kept node i (valid if i < nprev); slot Ncap + c: child c of this level
    const ChildRec* crow = a.arena + ((size_t)req * a.B + lvl) * Ncap * k;
    constexpr int Q = (kMaxNcap + kMaxNcap * kMaxK + NT - 1) / NT;  // slots per thread
    uint64_t kk[Q], cw0[Q], cw2[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int i = tid + q * NT;
        kk[q] = 0;
        cw0[q] = 0;
        cw2[q] = 0;
        if (i < Ncap) kk[q] = cld64(a.skeys + (size_t)req * Ncap + i);
        else if (i < Ncap + nchild) {
            if (mine) {
                cw0[q] = mine[0][i - Ncap];
                cw2[q] = mine[1][i - Ncap];
            } else {
                cw0[q] = cld64(crow + (i - Ncap));
                cw2[q] = cld64((const char*)(crow + (i - Ncap)) + 16);
            }
        }
    }
    const int ncand = nprev + nchild;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int i = tid + q * NT;
        if (i < Ncap) {
            if (i < nprev) ss.keys[i] = (key_surv(kk[q]) < tau) ? 0 : kk[q];
        } else if (i < Ncap + nchild) {
            const int c = i - Ncap;
            const int tok = (int)(uint32_t)cw0[q];
            const float sv = __uint_as_float((uint32_t)(cw0[q] >> 32));
            uint64_t key = tok >= 0 ? make_key(sv, level, c / k, c % k) : 0;
            if (key != 0 && sv < tau) key = 0;
            ss.keys[nprev + c] = key;
            ss.ctok[c] = tok;
            ss.chash[c] = cw2[q];
        }
    }
    const int ncand8 = (ncand + 7) & ~7;  // zero padding (zero keys never count)
    for (int i = ncand + tid; i < ncand8; i += blockDim.x) ss.keys[i] = 0;
    lds_sync();
    DT_STAMP(level, 7);
    // Nonzero keys are distinct (the low word names the node), so a key's position in the
    // descending order is the number of larger keys: one pass, no sorting network.  The
    // count reads eight keys per step so that their LDS latencies overlap.
    // A candidate is kept iff its rank is below the budget; one workgroup sum counts the kept
    // nodes (low half) and the kept nodes of this level's depth, the next frontier (high half).
    int cnt = 0;
    for (int i = tid; i < ncand; i += blockDim.x) {
        const uint64_t key = ss.keys[i];
        if (key == 0) continue;
        int rank = 0;
        for (int m = 0; m < ncand8; m += 8) {
            uint64_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = ss.keys[m + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) rank += v[q] > key ? 1 : 0;
        }
        if (rank < nbudget) {
            ss.sorted[rank] = key;
            cnt += 1 + ((level < a.B && low_depth((uint32_t)key) == level) ? (1 << 16) : 0);
        }
    }
    cnt = block_sum<NT / 64>(cnt, sh);  // includes barriers: ss.sorted is complete
    const int nkept = cnt & 0xFFFF;
    const int fnext = cnt >> 16;
    const int nk8 = (nkept + 7) & ~7;
    for (int i = nkept + tid; i < nk8; i += blockDim.x) ss.sorted[i] = 0;  // depth 63: never counted
    lds_sync();
    // rows of the next level, allocated with one atomic
    if (tid == 0) {
        unsigned base = 0;
        if (fnext > 0 && a.R > 1) {  // a single request's rows always start at 0
            uint64_t* alloc = (uint64_t*)(a.sync + kSyncAlloc) + level + 1;
            base = (unsigned)__hip_atomic_fetch_add(alloc, (uint64_t)fnext, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        }
        bcast[0] = (int)base;
    }
    for (int i = tid; i < nkept; i += blockDim.x) cst64(a.skeys + (size_t)req * Ncap + i, ss.sorted[i]);
    if (tid == 0) {
        csti(a.scount + req, nkept);
        csti(a.fcount + req * (a.B + 1) + level, fnext);
    }
    lds_sync();
    const int base = bcast[0];
    if (fnext > 0) {
        RowRec* nrows = level_rows(a, level + 1) + base;
        // head token of a next-level row: the node's own token (parent-conditioned), the
        // chain token of this depth (every row of this level shares one distribution, so
        // the rank-0 child of the first row is the greedy chain's next token), or none
        const int chain_tok = ss.ctok[0];
        auto htok_of = [&](int t) {
            return a.cond == DT_COND_CHAIN ? chain_tok : (a.cond == DT_COND_NONE ? -1 : t);
        };
        for (int i = tid; i < nkept; i += blockDim.x) {
            const uint32_t low = (uint32_t)ss.sorted[i];
            if (low_depth(low) != level) continue;
            int rank = 0;
            for (int m = 0; m < nk8; m += 8) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t lm = (uint32_t)ss.sorted[m + q];
                    rank += (low_depth(lm) == level && lm > low) ? 1 : 0;
                }
            }
            const int c = low_fi(low) * k + low_rank(low);
            const int tok = ss.ctok[c];
            const float sv = key_surv(ss.sorted[i]);
            const uint64_t hh = ss.chash[c];
            FrontEntry e;
            e.self = low;
            e.token = tok;
            e.s = sv;
            e.pad = 0;
            e.hash = hh;
            st_front(a.front + ((size_t)req * (a.B + 1) + level) * Ncap + rank, e);
            RowRec* rr = nrows + rank;
            cst64(rr, (uint64_t)(uint32_t)req | ((uint64_t)(uint32_t)rank << 32));
            cst64((char*)rr + 8, (uint64_t)(uint32_t)tok | ((uint64_t)__float_as_uint(sv) << 32));
            cst64((char*)rr + 16, hh);
            cst64((char*)rr + 24, (uint64_t)(uint32_t)fnext | ((uint64_t)(uint32_t)htok_of(tok) << 32));
        }
    }
    publish_wg();
    if (tid == 0 && a.R == 1) {
        // a single request's select is the level's last
        cst64(a.sync + kSyncGen, pack_gen(level, fnext > 0 ? 1 : 0, fnext));
    } else if (tid == 0) {
        // (selects done << 48) | (requests with rows at the next level << 32) | rows: the
        // select that completes the level learns the next level's sizes from the same atomic
        const uint64_t inc = (1ull << 48) | ((uint64_t)(fnext > 0) << 32) | (uint64_t)fnext;
        const uint64_t old = __hip_atomic_fetch_add((uint64_t*)(a.sync + kSyncDone) + level, inc,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t now = old + inc;
        if ((unsigned)(now >> 48) == nreq)
            cst64(a.sync + kSyncGen, pack_gen(level, (int)((now >> 32) & 0xFFFFu), (int)(uint32_t)now));
    }
}

// ---------------------------------------------------------------------------------------
// Emit, one request per workgroup.  The request's selected keys, frontier sizes and
// frontier identities are staged in LDS first (one round of parallel loads), then node i
// (thread i) finds its canonical index = number of kept nodes whose key low word is larger
// (depth asc, parent index asc, rank asc), its parent and its expansion slot from LDS.
// ---------------------------------------------------------------------------------------

template <int NT>
__device__ __forceinline__ void emit_request(const BuildArgs& a, int req, bool failed,
                                             EmitSmem& e) {
    const int tid = threadIdx.x + opaque_zero();
    const int B = a.B, k = a.k, Ncap = a.Ncap;
    // One round of loads: the error flag, the kept keys and their count, the frontier sizes
    // and every frontier identity (invalid slots are zeroed once the sizes are in LDS).  A
    // failed round (this workgroup's or another's wait gave up) emits empty trees.
    const uint32_t err = cld32(a.sync + kSyncErr);
    const int rst = cldi(a.rstat + req);
    int n = cldi(a.scount + req);
    uint64_t key = 0;
    if (tid < Ncap) key = cld64(a.skeys + (size_t)req * Ncap + tid);
    int fc = 0;
    if (tid <= B) fc = cldi(a.fcount + req * (B + 1) + tid);
    constexpr int kFs = (kMaxB * kMaxNcap + NT - 1) / NT;
    uint32_t fs[kFs];
#pragma unroll
    for (int q = 0; q < kFs; ++q) {
        const int i = tid + q * NT;
        fs[q] = i < (B - 1) * Ncap
                    ? (uint32_t)cld64(a.front + ((size_t)req * (B + 1) + 1 + i / Ncap) * Ncap + i % Ncap)
                    : 0u;
    }
    failed = failed || err != 0u;
    n = failed ? 0 : n;
    if (tid < kMaxNcap) e.keys[tid] = tid < n ? key : 0;  // zero padding: never counted
    if (tid <= B) e.fcnt[tid] = failed ? 0 : fc;
    lds_sync();
    DT_STAMP(kTraceLevels - 2, 0);
#pragma unroll
    for (int q = 0; q < kFs; ++q) {
        const int i = tid + q * NT;
        if (i < (B - 1) * Ncap) e.fself[i] = (i % Ncap) < e.fcnt[1 + i / Ncap] ? fs[q] : 0u;
    }
    // The LDS scans below read eight entries per step so that their latencies overlap; the
    // arrays are zero-padded to a multiple of eight (a node's low word is never zero).
    const int n8 = (n + 7) & ~7;
    if (tid < n) {
        const uint32_t mylow = (uint32_t)e.keys[tid];
        int canon = 0;
        for (int m = 0; m < n8; m += 8) {
#pragma unroll
            for (int q = 0; q < 8; ++q) canon += ((uint32_t)e.keys[m + q] > mylow) ? 1 : 0;
        }
        e.lowc[canon] = mylow;
    } else if (tid < n8) {
        e.lowc[tid] = 0u;
    }
    lds_sync();
    DT_STAMP(kTraceLevels - 2, 1);
    const size_t ob = (size_t)req * Ncap;
    int par = -2;
    if (tid < n) {
        const uint32_t low = e.lowc[tid];
        const int depth = low_depth(low);
        const int fi = low_fi(low), j = low_rank(low);
        par = -1;
        if (depth > 1) {
            const uint32_t pid = e.fself[(depth - 2) * Ncap + fi];
            for (int m = 0; m < n8; m += 8) {
#pragma unroll
                for (int q = 0; q < 8; ++q) par = (e.lowc[m + q] == pid) ? m + q : par;
            }
        }
        int slot = -1;
        if (depth < B) {
            const int F = e.fcnt[depth];
            const uint32_t* row = e.fself + (depth - 1) * Ncap;
            for (int m = 0; m < F; m += 8) {
                uint32_t v[8];  // read unconditionally (padded row), then compared
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = row[m + q];
#pragma unroll
                for (int q = 0; q < 8; ++q) slot = (v[q] == low && m + q < F) ? m + q : slot;
            }
        }
        // The candidate row and the node's record are loaded together, unconditionally (from
        // clamped addresses inside the arena), before any store.
        const ChildRec* crow = a.arena + (((size_t)req * B + (slot >= 0 ? depth : 0)) * Ncap + (slot >= 0 ? slot : 0)) * k;
        uint64_t cw[kMaxK];
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj) cw[jj] = cld64(crow + (jj < k ? jj : k - 1));
        const ChildRec c = ld_child(a.arena + (((size_t)req * B + (depth - 1)) * Ncap + fi) * k + j);
        int cv[kMaxK];
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj) cv[jj] = slot >= 0 ? (int)(uint32_t)cw[jj] : -1;
        a.out.token[ob + tid] = c.token;
        a.out.depth[ob + tid] = (uint8_t)depth;
        a.out.surv[ob + tid] = c.s;
        a.out.logq[ob + tid] = c.logq;
        const size_t cb = ((size_t)req * (Ncap + 1) + tid + 1) * k;
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj)
            if (jj < k) a.out.cand[cb + jj] = cv[jj];
    }
    if (tid < kMaxNcap) e.parc[tid] = par;
    lds_sync();
    DT_STAMP(kTraceLevels - 2, 2);
    if (tid < n) {
        uint64_t m = 0;
        int x = tid;
        while (x >= 0) {
            m |= 1ull << x;
            x = e.parc[x];
        }
        a.out.anc_mask[ob + tid] = m;
        a.out.parent[ob + tid] = (int16_t)par;
    } else if (tid < Ncap) {
        a.out.token[ob + tid] = -1;
        a.out.parent[ob + tid] = -2;
        a.out.depth[ob + tid] = 0;
        a.out.anc_mask[ob + tid] = 0;
        a.out.surv[ob + tid] = 0.0f;
        a.out.logq[ob + tid] = 0.0f;
        const size_t cb = ((size_t)req * (Ncap + 1) + tid + 1) * k;
        for (int jj = 0; jj < k; ++jj) a.out.cand[cb + jj] = -1;
    }
    if (tid < k) {
        const bool rooted = e.fcnt[0] == 1;
        a.out.cand[(size_t)req * (Ncap + 1) * k + tid] =
            rooted ? (int)(uint32_t)cld64(a.arena + ((size_t)req * B * Ncap) * k + tid) : -1;
    }
    if (tid == 0) {
        a.out.n_nodes[req] = n;
        a.out.status[req] = rst | (failed ? DT_REQ_SYNC_TIMEOUT : 0);
        if (a.out.n_expand) {
            int ex = 0;
            for (int l = 0; l < B; ++l) ex += e.fcnt[l];
            a.out.n_expand[req] = ex;
        }
    }
    lds_sync();
}

}  // namespace dt
