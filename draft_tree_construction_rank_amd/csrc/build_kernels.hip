// Tree construction on gfx950: a set-up kernel and one persistent kernel per round.
//
// The round walks block positions d = 1..B (PCTree summary: every position's logits come
// from one backbone forward, so a level needs no new drafter pass).  Per level, inside the
// persistent kernel k_build:
//   expand  - every workgroup takes (row tile or group, vocabulary split) items: the Markov
//             bias of the parents over the split (bf16 MFMA 32x32x16, fp32 accumulate, W as
//             the A operand so that each lane holds one parent row) is added to the block
//             logits, tempered, and folded into that row's online log-sum-exp and top-k (or
//             Gumbel-top-k) in registers; z never reaches memory;
//   merge   - once all splits of a tile are in, parent row m is merged by workgroup m mod G:
//             the split records are combined, each child's probability is calibrated to an
//             edge estimate and multiplied into the path survival (TreeSpark core idea);
//   select  - the workgroup that merges a request's last row keeps the best n_budget nodes
//             with survival >= tau (best-first with per-round stopping equals this
//             expand-then-select because survival never increases along a path), writes the
//             next frontier and its parent-row records, and the select that completes the
//             level publishes the next level's sizes in the generation word every workgroup
//             waits on.
// A level with no parent rows ends the loop at once (per-round stopping), and the kernel
// emits the trees.  Workgroups hand data to each other only through agent-coherent accesses
// (dt_device.h), counters and the generation word; every wait is bounded and raises an
// error flag on time-out.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {

// The persistent construction kernel runs one workgroup of kWaves wavefronts per CU.
constexpr int kWaves = kBuildWaves;
constexpr int kThreads = 64 * kWaves;

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
template <int NW = kWaves>
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

__device__ __forceinline__ int block_sum(int v, int* sh) {
    int total;
    block_exclusive_scan(v, sh, &total);
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

// Group-mode staging ring: kStages slots, each one 32-column block of W (32 rows of Wt, 16 KB
// at r = 256) and the matching 64-byte segments of the block logits of the group's 256 rows
// (16 KB).
constexpr int kStages = 4;

template <int KT>
struct BuildSmem {
    union {
        uint16_t sA[kTileRows * kAStride];  // bf16 parent rows of U (tile-mode expand)
        float sAf[kTileRows * kAfStride];   // f32 parent rows of U (tile-mode expand)
        struct {
            uint4 w[kStages][kBlockCols * 32];
            uint4 l[kStages][kGroupRows * 4];
        } g;                                            // group-mode staging ring
        float xrec[kWaves][kTileRows][rec_floats(KT)];  // per-wavefront lists of a tile item
        SelSmem sel;                                    // select
        EmitSmem em;                                    // emit
    } u;
    float mrec[kWaves][rec_floats(KT)];  // per-wavefront lists of a merged row
    size_t lbase[kTileRows];
    size_t glbase[kGroupRows];  // group mode: block-logit row offset of each row of the group
    uint64_t hash[kTileRows];
    uint64_t rkth[128];  // per parent row of an item: the largest KT-th list entry seen so far
    int tok[kTileRows];
    int sh[256];
    int bcast[4];
    int lrows[kMaxB + 2];  // parent rows of each level (as read from the generation word)
    uint64_t mchild[2][kMaxK];  // children of the row just merged (see select_request)
};

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

// One item: tile `tile` of the level's parent rows x vocabulary split `split`.  Wavefront w
// takes the split's 32-column blocks w, w+kWaves, ...; the wavefronts' lists are combined in
// LDS and one record per parent row is published.
template <int KT, bool SAMPLE, bool HEAD_BF16, bool L_BF16>
__device__ __forceinline__ void expand_item(const BuildArgs& a, int level, int M, int S, int tile,
                                            int split, BuildSmem<KT>& sm) {
    constexpr int RS = rec_floats(KT);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int lvl = level - 1;
    const int m0 = tile * kTileRows;
    const int nrows = min(kTileRows, M - m0);
    const int NB = (a.V + kBlockCols - 1) / kBlockCols;
    const int b_beg = (int)((long long)split * NB / S);
    const int b_end = (int)((long long)(split + 1) * NB / S);
    bf16x8 wf[16];
    if (tid < kTileRows) {
        int tok = 0;
        size_t lb = 0;
        uint64_t hh = 0;
        if (tid < nrows) {
            const RowRec* rr = level_rows(a, level) + m0 + tid + opaque_zero();
            const uint64_t w0 = cld64(rr), w1 = cld64((const char*)rr + 8);
            hh = cld64((const char*)rr + 16);
            const int req = (int)(uint32_t)w0;
            tok = (int)(uint32_t)w1;
            tok = (uint32_t)tok < (uint32_t)a.V ? tok : 0;  // never index U out of range
            lb = ((size_t)req * a.B + lvl) * (size_t)a.V;
        }
        sm.tok[tid] = tok;
        sm.lbase[tid] = lb;
        sm.hash[tid] = hh;
        sm.rkth[tid] = 0;
    }
    lds_sync();
    DT_STAMP(level, 8);
    if constexpr (HEAD_BF16)
        load_a_tile<true, kThreads>(a.U, a.r, nrows, [&](int row) { return sm.tok[row]; }, sm.u.sA, nullptr);
    else
        load_a_tile<false, kThreads>(a.U, a.r, nrows, [&](int row) { return sm.tok[row]; }, nullptr, sm.u.sAf);
    lds_sync();
    // The first W block is loaded only once the parent rows are staged: issued earlier, the
    // whole grid's first blocks (32 MB) queue ahead of the set-up loads.
    if constexpr (HEAD_BF16) {
        if (b_beg + wave < b_end) load_wfrag(a.Wt, a.V, a.r, (b_beg + wave) * kBlockCols, wf);
    }

    DT_STAMP(level, 1);
    const bool two = nrows > 32;
    const int p0 = lane & 31;
    const size_t lb0 = sm.lbase[p0], lb1 = sm.lbase[32 + p0];
    const uint64_t hh0 = sm.hash[p0], hh1 = sm.hash[32 + p0];
    const bool lvec = (a.V & 3) == 0;
    const bool live0 = p0 < nrows, live1 = 32 + p0 < nrows;  // rows past nrows only pad the tile
    TopK<KT> t0, t1;
    Lse2 s0, s1;
    t0.init();
    t1.init();
    s0.init();
    s1.init();
    if constexpr (HEAD_BF16) {
        // Software pipeline: the W fragments and block logits of block b + 4 are in flight
        // while block b's epilogue runs.
        int blk = b_beg + wave;
        LGroups<L_BF16> n0, n1;
        if (blk < b_end) {
            load_lgroups<L_BF16>(a, lb0, blk * kBlockCols, h, lvec, n0);
            if (two) load_lgroups<L_BF16>(a, lb1, blk * kBlockCols, h, lvec, n1);
        }
        for (; blk < b_end; blk += kWaves) {
            const int c0 = blk * kBlockCols;
            f32x16 acc0, acc1;
            lgroups_to_acc<L_BF16>(n0, acc0);
            if (two) lgroups_to_acc<L_BF16>(n1, acc1);
            mma_wfrag(wf, two, sm.u.sA, acc0, acc1);
            if (blk + kWaves < b_end) {
                load_wfrag(a.Wt, a.V, a.r, c0 + kWaves * kBlockCols, wf);
                load_lgroups<L_BF16>(a, lb0, c0 + kWaves * kBlockCols, h, lvec, n0);
                if (two) load_lgroups<L_BF16>(a, lb1, c0 + kWaves * kBlockCols, h, lvec, n1);
            }
            expand_epilogue<KT, SAMPLE>(a, acc0, c0, h, hh0, live0, sm.rkth + p0, t0, s0);
            if (two) expand_epilogue<KT, SAMPLE>(a, acc1, c0, h, hh1, live1, sm.rkth + 32 + p0, t1, s1);
        }
    } else {
        for (int blk = b_beg + wave; blk < b_end; blk += kWaves) {
            const int c0 = blk * kBlockCols;
            LGroups<L_BF16> l0, l1;
            load_lgroups<L_BF16>(a, lb0, c0, h, lvec, l0);
            if (two) load_lgroups<L_BF16>(a, lb1, c0, h, lvec, l1);
            f32x16 acc0, acc1;
            lgroups_to_acc<L_BF16>(l0, acc0);
            if (two) lgroups_to_acc<L_BF16>(l1, acc1);
            xblock_mma_f32(a.Wt, a.V, a.r, c0, two, sm.u.sAf, acc0, acc1);
            expand_epilogue<KT, SAMPLE>(a, acc0, c0, h, hh0, live0, sm.rkth + p0, t0, s0);
            if (two) expand_epilogue<KT, SAMPLE>(a, acc1, c0, h, hh1, live1, sm.rkth + 32 + p0, t1, s1);
        }
    }
    // lanes l and l ^ 32 hold the same parent row
    s0.merge_xor(32);
    t0.merge_xor(32);
    if (two) {
        s1.merge_xor(32);
        t1.merge_xor(32);
    }
    lds_sync();  // the lists below overwrite the U tile
    if (h == 0) {
        put_list<KT>(sm.u.xrec[wave][p0], t0, s0);
        if (two) put_list<KT>(sm.u.xrec[wave][32 + p0], t1, s1);
    }
    lds_sync();
    {
        // kWaves consecutive threads per parent row combine the wavefronts' lists
        const int row = tid / kWaves, w = tid % kWaves;
        TopK<KT> t;
        Lse2 s;
        get_list<KT>(sm.u.xrec[w][row], t, s);
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            s.merge_xor(off);
            t.merge_xor(off);
        }
        if (row < nrows) {
            // the row's kWaves lanes write one 16-byte piece of its record each
            float v[RS];
#pragma unroll
            for (int i = 0; i < RS; ++i) v[i] = 0.0f;
            put_list<KT>(v, t, s);
            uint4* rec = (uint4*)(a.partials + ((size_t)(m0 + row) * S + split) * RS);
#pragma unroll
            for (int c = 0; c < RS / 4; ++c)
                if (c % kWaves == w)
                    cst128(rec + c, make_uint4(__float_as_uint(v[4 * c]), __float_as_uint(v[4 * c + 1]),
                                               __float_as_uint(v[4 * c + 2]), __float_as_uint(v[4 * c + 3])));
        }
    }
    lds_sync();
}

// ---------------------------------------------------------------------------------------
// Group-mode expansion (levels with more than kTileRows parent rows, bf16 heads and logits,
// V a multiple of 8): an item is a group of kGroupRows = 256 parent rows x a vocabulary split.
// Wavefront w owns rows 32w .. 32w+31 of the group and keeps their U rows as MFMA B fragments
// in registers for the whole item.  Each 32-column block of W (32 rows of Wt, 16 KB at
// r = 256) and the rows' 64-byte segments of block logits (16 KB) are copied once per
// workgroup into an LDS ring of kStages slots with global->LDS loads, so that three blocks
// are in flight while one is multiplied: with a single block in flight the copies' latency,
// not HBM bandwidth, bounded the loop.  Every wavefront issues exactly four 1 KB copies per
// block (two of W, two of logits) and nothing else in the loop, so "this wavefront's copies
// of block b are done" is a vmcnt wait with the count of copies issued after them.
//
// LDS layouts (16-byte slots): W row j's chunk c sits at slot 32j + (c ^ (j & 31)), so the
// fragment reads of 16 consecutive lanes hit distinct banks; the logits piece p (8 columns) of
// group row i sits at slot 4i + (p ^ ((i >> 2) & 3)).
// ---------------------------------------------------------------------------------------

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

// Per-item source addresses of this wavefront's copies: its two W chunks (as an offset
// within a block of Wt rows) and its two logit pieces (row offset into L, piece column).
struct GroupCopy {
    size_t wofs[16 / kWaves];
    size_t lofs[(kGroupRows * 4 / 64) / kWaves];
    int lcol[(kGroupRows * 4 / 64) / kWaves];
};
constexpr int kCopiesPerBlock = 16 / kWaves + (kGroupRows * 4 / 64) / kWaves;

template <int KT>
__device__ __forceinline__ GroupCopy group_copy_setup(const BuildArgs& a, const BuildSmem<KT>& sm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = a.r >> 3;  // 16-byte chunks per row of Wt
    GroupCopy gc;
#pragma unroll
    for (int q = 0; q < 16 / kWaves; ++q) {
        const int j = (16 / kWaves) * wave + q;  // 1 KB piece j = LDS slots 64j .. 64j+63
        const int row = 2 * j + (lane >> 5);     // W row within the block
        int c = (lane & 31) ^ (row & 31);        // chunk that belongs in this slot
        c = c < chunks ? c : 0;                  // past r: any finite data (U is zero there)
        gc.wofs[q] = (size_t)row * a.r + c * 8;
    }
#pragma unroll
    for (int q = 0; q < (kGroupRows * 4 / 64) / kWaves; ++q) {
        const int j = ((kGroupRows * 4 / 64) / kWaves) * wave + q;
        const int sl = 64 * j + lane;
        const int row = sl >> 2, piece = (sl & 3) ^ ((row >> 2) & 3);
        gc.lofs[q] = sm.glbase[row];
        gc.lcol[q] = 8 * piece;
    }
    return gc;
}

// Issue this wavefront's copies of block `blk` into ring slot `slot` (kCopiesPerBlock
// global->LDS loads of 16 bytes per lane; every address clamped into its array).
template <int KT>
__device__ __forceinline__ void stage_block(const BuildArgs& a, const GroupCopy& gc, int blk, int slot,
                                            BuildSmem<KT>& sm) {
    const int wave = threadIdx.x >> 6;
    const int c0 = blk * kBlockCols;
    // rows of the block past V read the last row of Wt (their columns are masked)
    const int wlast = a.V - kBlockCols;
#pragma unroll
    for (int q = 0; q < 16 / kWaves; ++q) {
        const int j = (16 / kWaves) * wave + q;
        size_t off = (size_t)c0 * a.r + gc.wofs[q];
        if (c0 > wlast) {
            const int row = (int)(gc.wofs[q] / a.r);
            const int col = c0 + row < a.V ? c0 + row : a.V - 1;
            off = (size_t)col * a.r + (gc.wofs[q] - (size_t)row * a.r);
        }
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)((const uint16_t*)a.Wt + off),
            (__attribute__((address_space(3))) void*)(sm.u.g.w[slot] + 64 * j), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < (kGroupRows * 4 / 64) / kWaves; ++q) {
        const int j = ((kGroupRows * 4 / 64) / kWaves) * wave + q;
        int col = c0 + gc.lcol[q];
        col = col <= a.V - 8 ? col : a.V - 8;  // past V: any data (masked in the epilogue)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)((const uint16_t*)a.L + gc.lofs[q] + col),
            (__attribute__((address_space(3))) void*)(sm.u.g.l[slot] + 64 * j), 16, 0, 0);
    }
}

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

template <int KT, bool SAMPLE>
__device__ __forceinline__ void expand_group(const BuildArgs& a, int level, int M, int S, int grp,
                                             int split, BuildSmem<KT>& sm) {
    constexpr int RS = rec_floats(KT);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, p0 = lane & 31;
    const int lvl = level - 1;
    const int rl = 32 * wave + p0;  // row within the group
    const int row = grp * kGroupRows + rl;
    const bool live = row < M;
    const int NB = (a.V + kBlockCols - 1) / kBlockCols;
    const int b_beg = (int)((long long)split * NB / S);
    const int b_end = (int)((long long)(split + 1) * NB / S);

    int tok = 0;
    size_t lb = 0;
    uint64_t hh = 0;
    if (live) {
        const RowRec* rr = level_rows(a, level) + row;
        const uint64_t w0 = cld64(rr), w1 = cld64((const char*)rr + 8);
        hh = cld64((const char*)rr + 16);
        const int req = (int)(uint32_t)w0;
        tok = (int)(uint32_t)w1;
        tok = (uint32_t)tok < (uint32_t)a.V ? tok : 0;  // never index U out of range
        lb = ((size_t)req * a.B + lvl) * (size_t)a.V;
    }
    // B fragments: U[tok][16 s + 8 h .. +8], zero past r
    bf16x8 uf[16];
    {
        const uint16_t* urow = (const uint16_t*)a.U + (size_t)tok * a.r;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int kk = 16 * s + 8 * h;
            const uint4 v = *(const uint4*)(urow + (kk < a.r ? kk : 0));
            uf[s] = __builtin_bit_cast(bf16x8, kk < a.r ? v : make_uint4(0, 0, 0, 0));
        }
    }
    if (h == 0) sm.glbase[rl] = lb;
    DT_STAMP(level, 1);
    lds_sync();
    const GroupCopy gc = group_copy_setup<KT>(a, sm);
    // prologue: blocks b_beg .. b_beg + kStages - 2 in flight
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
        if (b_beg + i < b_end) stage_block<KT>(a, gc, b_beg + i, (b_beg + i) % kStages, sm);
    TopK<KT> top;
    Lse2 st;
    top.init();
    st.init();
    const int swz = (rl >> 2) & 3;
    static_assert(kStages - 2 <= 2, "the wait counts below cover two blocks in flight");
    for (int blk = b_beg; blk < b_end; ++blk) {
        // this wavefront's copies of block blk are done once at most the copies of the
        // blocks issued after it are outstanding
        const int after = min(kStages - 2, b_end - 1 - blk);
        if (after >= 2) wait_vmcnt<2 * kCopiesPerBlock>();
        else if (after == 1) wait_vmcnt<kCopiesPerBlock>();
        else wait_vmcnt<0>();
        bare_barrier();  // block blk staged by every wavefront; slot (blk - 1) read by all
        if (blk + kStages - 1 < b_end)
            stage_block<KT>(a, gc, blk + kStages - 1, (blk + kStages - 1) % kStages, sm);
        const int slot = blk % kStages;
        const uint32_t wb = lds_addr(sm.u.g.w[slot] + p0 * 32);
        const uint32_t lb0 = lds_addr(sm.u.g.l[slot] + 4 * rl) + 8 * h;
        f32x16 acc;
        {
            u32x2_t l0, l1, l2, l3;
            lds_read4_b64(lb0 + 16 * (0 ^ swz), lb0 + 16 * (1 ^ swz), lb0 + 16 * (2 ^ swz),
                          lb0 + 16 * (3 ^ swz), l0, l1, l2, l3);
            const u32x2_t lv[4] = {l0, l1, l2, l3};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[4 * j + 0] = bf16_lo(lv[j].x);
                acc[4 * j + 1] = bf16_hi(lv[j].x);
                acc[4 * j + 2] = bf16_lo(lv[j].y);
                acc[4 * j + 3] = bf16_hi(lv[j].y);
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x4_t w0, w1, w2, w3;
            lds_read4_b128(wb + 16 * ((8 * g + 0 + h) ^ p0), wb + 16 * ((8 * g + 2 + h) ^ p0),
                           wb + 16 * ((8 * g + 4 + h) ^ p0), wb + 16 * ((8 * g + 6 + h) ^ p0),
                           w0, w1, w2, w3);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w0), uf[4 * g + 0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w1), uf[4 * g + 1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w2), uf[4 * g + 2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w3), uf[4 * g + 3], acc, 0, 0, 0);
        }
        // each row lives in two lanes of one wavefront: no workgroup-shared bound
        expand_epilogue<KT, SAMPLE>(a, acc, blk * kBlockCols, h, hh, live, nullptr, top, st);
    }
    st.merge_xor(32);
    top.merge_xor(32);
    if (live) {
        // lanes l and l ^ 32 split the row's record into alternate 16-byte pieces
        float v[RS];
#pragma unroll
        for (int i = 0; i < RS; ++i) v[i] = 0.0f;
        put_list<KT>(v, top, st);
        uint4* rec = (uint4*)(a.partials + ((size_t)row * S + split) * RS);
#pragma unroll
        for (int c = 0; c < RS / 4; ++c)
            if ((c & 1) == h)
                cst128(rec + c, make_uint4(__float_as_uint(v[4 * c]), __float_as_uint(v[4 * c + 1]),
                                           __float_as_uint(v[4 * c + 2]), __float_as_uint(v[4 * c + 3])));
    }
    wait_vm();
    lds_sync();  // no copy into the staging ring is left in flight
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

// Returns the row's request and its rows at this level (F) through *req / *F.
template <int KT>
__device__ __forceinline__ void merge_row(const BuildArgs& a, int level, int S, int m,
                                          BuildSmem<KT>& sm, int* req_out, int* F_out) {
    const int tid = threadIdx.x + opaque_zero(), lane = tid & 63, wave = threadIdx.x >> 6;
    constexpr int RS = rec_floats(KT);
    TopK<KT> top;
    top.init();
    Lse2 acc;
    acc.init();
    const float* base = a.partials + (size_t)m * S * RS;
    static_assert(kThreads >= kMaxSplits, "one split record per thread");
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
    if (lane == 0) put_list<KT>(sm.mrec[wave], top, acc);
    lds_sync();
    DT_STAMP(level, 10);
    if (wave == 0) {
        get_list<KT>(sm.mrec[lane % kWaves], top, acc);
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
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
            sm.mchild[0][j] = (uint64_t)(uint32_t)c.token | ((uint64_t)__float_as_uint(c.s) << 32);
            sm.mchild[1][j] = c.hash;
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
    uint64_t kk[2], cw0[2], cw2[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = tid + q * kThreads;
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
    for (int q = 0; q < 2; ++q) {
        const int i = tid + q * kThreads;
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
    cnt = block_sum(cnt, sh);  // includes barriers: ss.sorted is complete
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
            cst64((char*)rr + 24, (uint64_t)(uint32_t)fnext);
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
    constexpr int kFs = (kMaxB * kMaxNcap + kThreads - 1) / kThreads;
    uint32_t fs[kFs];
#pragma unroll
    for (int q = 0; q < kFs; ++q) {
        const int i = tid + q * kThreads;
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
        const int i = tid + q * kThreads;
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

// ---------------------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------------------
// Round set-up: control words and per-level counters (all workgroups), then roots, budgets,
// status bits and the level-1 parent rows, one per request with a valid root (workgroup 0).
__global__ __launch_bounds__(256) void k_build_init(const BuildArgs a) {
    __shared__ int sh[256];
    const int tid = threadIdx.x;
    {
        const size_t nt = (size_t)(a.B + 2) * a.Tmax, nr = (size_t)(a.B + 2) * a.R;
        for (size_t i = (size_t)blockIdx.x * blockDim.x + tid; i < nt + nr; i += (size_t)gridDim.x * blockDim.x) {
            if (i < nt) a.tdone[i] = 0u;
            else a.rdone[i - nt] = 0u;
        }
    }
    if (blockIdx.x != 0) return;
    for (int i = tid; i < kSyncWords; i += blockDim.x) a.sync[i] = 0u;
    const int R = a.R;
    const int per = (R + blockDim.x - 1) / blockDim.x;
    const int r0 = tid * per;
    int cnt = 0;
    for (int r = r0; r < r0 + per && r < R; ++r) {
        const int32_t root = a.root_token[r];
        int nb = a.n_budget[r];
        int st = 0;
        if (nb < 0 || nb > a.Ncap) {
            st |= DT_REQ_BUDGET_CLAMPED;
            nb = nb < 0 ? 0 : a.Ncap;
        }
        const bool ok = root >= 0 && root < a.V;
        if (!ok) st |= DT_REQ_BAD_ROOT;
        FrontEntry e;
        e.self = 0xFFFFFFFFu;
        e.token = ok ? root : 0;
        e.s = 1.0f;
        e.pad = 0;
        e.hash = root_hash(a.round, r, root);
        a.front[(size_t)r * (a.B + 1) * a.Ncap] = e;
        for (int l = 0; l <= a.B; ++l) a.fcount[r * (a.B + 1) + l] = 0;
        a.fcount[r * (a.B + 1)] = ok ? 1 : 0;
        a.scount[r] = 0;
        a.nbeff[r] = nb;
        a.rstat[r] = st;
        cnt += ok ? 1 : 0;
    }
    int total;
    int off = block_exclusive_scan<4>(cnt, sh, &total);
    RowRec* rows = level_rows(a, 1);
    for (int r = r0; r < r0 + per && r < R; ++r) {
        const int32_t root = a.root_token[r];
        if (root >= 0 && root < a.V) {
            RowRec rr;
            rr.req = r;
            rr.fi = 0;
            rr.token = root;
            rr.s = 1.0f;
            rr.hash = root_hash(a.round, r, root);
            rr.F = 1;
            rr.pad = 0;
            rows[off++] = rr;
        }
    }
    __syncthreads();  // sync[] is cleared before the generation word is written
    if (tid == 0) *(uint64_t*)(a.sync + kSyncGen) = pack_gen(0, total, total);
}

// The level loop.  The grid is the kernel's resident capacity, launched plainly.  Work is
// handed out by per-level tickets (claim_ticket), so a workgroup only waits for work that
// running workgroups hold: a round completes with any number of resident workgroups (a
// workgroup dispatched late finds its level's tickets used up and goes on to the next level
// or the emit).  Every wait is still bounded and reports DT_REQ_SYNC_TIMEOUT if it gives up.
template <int KT, bool SAMPLE, bool HEAD_BF16, bool L_BF16>
__global__ __launch_bounds__(kThreads, 1) void k_build(const BuildArgs a) {
    __shared__ __attribute__((aligned(16))) BuildSmem<KT> sm;
    const int tid = threadIdx.x;
    const int NB = (a.V + kBlockCols - 1) / kBlockCols;
    bool failed = false;
    DT_STAMP(0, 0);
    if (tid < kMaxB + 2) sm.lrows[tid] = 0;  // levels never reached expand no rows
    // the first ticket of a level is taken while the workgroup waits for the level to open
    int ticket = claim_ticket(a.sync, 1, sm.bcast);
    for (int level = 1;; ++level) {
        // the previous level's selects are complete once the generation reaches level - 1;
        // the generation word also carries this level's row and request counts
        uint64_t gen;
        if (!wait_gen(a.sync, level - 1, sm.bcast, &gen, a.spin_limit)) {
            failed = true;
            break;
        }
        if (level > a.B) break;
        DT_STAMP(level, 0);
        const int M = (int)(gen >> 32);
        const unsigned nreq = ((uint32_t)gen) >> 8;
        if (tid == 0) sm.lrows[level] = M;
        if (M == 0) break;
        // tile mode (<= kTileRows rows, or float32 heads) or group mode (kGroupRows-row groups)
        const bool grp_mode = HEAD_BF16 && L_BF16 && (a.V & 7) == 0 && M > kTileRows;
        const int GR = grp_mode ? kGroupRows : kTileRows;
        const int T = (M + GR - 1) / GR;
        const int S = splits_for(T, (int)gridDim.x, NB);
        const int NI = T * S;
        unsigned* tdone = a.tdone + (size_t)level * a.Tmax;
        // expansion items: ticket c is vocabulary split c % S of row tile (or group) c / S
        for (; ticket < NI; ticket = claim_ticket(a.sync, level, sm.bcast)) {
            const int item = ticket;
            if constexpr (HEAD_BF16 && L_BF16) {
                if (grp_mode) expand_group<KT, SAMPLE>(a, level, M, S, item / S, item % S, sm);
                else expand_item<KT, SAMPLE, HEAD_BF16, L_BF16>(a, level, M, S, item / S, item % S, sm);
            } else {
                expand_item<KT, SAMPLE, HEAD_BF16, L_BF16>(a, level, M, S, item / S, item % S, sm);
            }
            publish_wg();
            if (tid == 0) cadd32(tdone + item / S, 1u);
        }
        DT_STAMP(level, 2);
        bool first_task = true;
        // merges: ticket NI + m is parent row m, merged once all splits of its tile are in
        for (; ticket < NI + M; ticket = claim_ticket(a.sync, level, sm.bcast)) {
            const int m = ticket - NI;
            if (!wait_at_least(a.sync, tdone + m / GR, (unsigned)S, sm.bcast, a.spin_limit)) {
                failed = true;
                break;
            }
            if (first_task) DT_STAMP(level, 6);
            first_task = false;
            int req, F;
            merge_row<KT>(a, level, S, m, sm, &req, &F);
            if (F == 1) {
                // the request's only row: its select follows at once, with the children from
                // LDS (its closing publish also covers the child records)
                lds_sync();
                DT_STAMP(level, 5);
                select_request(a, level, req, F, nreq, sm.u.sel, sm.sh, sm.bcast + 3, sm.mchild);
                DT_STAMP(level, 4);
            } else {
                publish_wg();
                DT_STAMP(level, 5);
                if (tid == 0)
                    sm.bcast[2] = (cadd32(a.rdone + (size_t)level * a.R + req, 1u) + 1u == (unsigned)F) ? 1 : 0;
                lds_sync();
                if (sm.bcast[2]) {
                    select_request(a, level, req, F, nreq, sm.u.sel, sm.sh, sm.bcast + 3, nullptr);
                    DT_STAMP(level, 4);
                }
            }
            lds_sync();
        }
        DT_STAMP(level, 3);
        if (failed) break;
        ticket = claim_ticket(a.sync, level + 1, sm.bcast);
    }
    DT_STAMP(kTraceLevels - 1, 0);
    if (failed) cst32(a.sync + kSyncErr, 1u);
    for (int req = blockIdx.x; req < a.R; req += gridDim.x)
        emit_request(a, req, failed, sm.u.em);
    if (blockIdx.x == 0 && a.out.level_rows) {
        lds_sync();
        for (int l = tid; l < a.B; l += blockDim.x) a.out.level_rows[l] = sm.lrows[l + 1];
    }
    DT_STAMP(kTraceLevels - 1, 1);
}

// ---------------------------------------------------------------------------------------
// Launch sequence of one round.
// ---------------------------------------------------------------------------------------
// Resident workgroups of a kernel on the current device (cached per kernel and device).
static int resident_grid(const void* f) {
    static std::mutex mu;
    static const void* keys[64];
    static int devs[64], vals[64], n = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < n; ++i)
        if (keys[i] == f && devs[i] == dev) return vals[i];
    int per = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, f, kThreads, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    int g = per * cus;
    if (g > kMaxGrid) g = kMaxGrid;
    if (n < 64) {
        keys[n] = f;
        devs[n] = dev;
        vals[n] = g;
        ++n;
    }
    return g;
}

template <int KT, bool SAMPLE, bool HEAD_BF16, bool L_BF16>
static hipError_t launch_build_t(const BuildArgs& a, hipStream_t st) {
    const void* f = (const void*)k_build<KT, SAMPLE, HEAD_BF16, L_BF16>;
    const int G = resident_grid(f);
    if (G < 1) return hipErrorLaunchFailure;
    {
        // enough workgroups to clear the per-level counters in a few stores per thread
        const size_t words = (size_t)(a.B + 2) * (a.Tmax + a.R);
        int g = (int)((words + 256 * 16 - 1) / (256 * 16));
        g = g < 1 ? 1 : (g > 256 ? 256 : g);
        hipLaunchKernelGGL(k_build_init, dim3(g), dim3(256), 0, st, a);
    }
    if (a.timing_hook) a.timing_hook(st, 0);
    // a plain launch: the loop needs no co-residency guarantee (see k_build), and a
    // cooperative launch costs about 18 us more per round on this stack
    hipLaunchKernelGGL((k_build<KT, SAMPLE, HEAD_BF16, L_BF16>), dim3(G), dim3(kThreads), 0, st, a);
    if (a.timing_hook) a.timing_hook(st, 1);
    return hipGetLastError();
}

template <int KT, bool SAMPLE>
static hipError_t launch_build_ks(const dt_params* p, const BuildArgs& a, hipStream_t st) {
    const bool hb = p->head_dtype == DT_BF16, lb = p->logits_dtype == DT_BF16;
    if (hb) return lb ? launch_build_t<KT, SAMPLE, true, true>(a, st)
                      : launch_build_t<KT, SAMPLE, true, false>(a, st);
    return lb ? launch_build_t<KT, SAMPLE, false, true>(a, st)
              : launch_build_t<KT, SAMPLE, false, false>(a, st);
}

template <int KT>
static hipError_t launch_build_kt(const dt_params* p, const BuildArgs& a, hipStream_t st) {
    return p->mode == DT_SAMPLE ? launch_build_ks<KT, true>(p, a, st)
                                : launch_build_ks<KT, false>(p, a, st);
}

hipError_t launch_build(const dt_params* p, const Layout& lay, const BuildArgs& a,
                        hipStream_t st) {
    switch (lay.KT) {
        case 1: return launch_build_kt<1>(p, a, st);
        case 2: return launch_build_kt<2>(p, a, st);
        case 4: return launch_build_kt<4>(p, a, st);
        default: return launch_build_kt<8>(p, a, st);
    }
}

}  // namespace dt
