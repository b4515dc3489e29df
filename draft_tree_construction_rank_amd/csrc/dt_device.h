// Device-side helpers of libdtree: counter-based randomness, selection keys, bf16 loads and
// the top-k register lists used by the fused expansion kernel.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dt_internal.h"

namespace dt {

// ---------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): ten rounds; each multiplies counter words 0 and 2 by the two Philox constants,
// mixes the high halves with words 1, 3 and the key, and advances the key by the Weyl
// constants.  Written here from that definition; checked against the published
// known-answer vectors by the test suite.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        // each 32 x 32 -> 64-bit product is one v_mad_u64_u32 (separate low and high
        // multiplies ran at 0.72x the rate on this part, measured)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// SplitMix64 output function applied to x + golden gamma (Steele, Lea, Flood 2014).
__device__ __host__ __forceinline__ uint64_t mix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Random stream of a node = hash of its token path; the root's also folds in the round and
// the request index.
__device__ __host__ __forceinline__ uint64_t root_hash(uint32_t round, int32_t req, int32_t tok) {
    const uint64_t a = mix64(((uint64_t)round << 32) | (uint64_t)(uint32_t)req);
    return mix64(a ^ (uint64_t)(uint32_t)tok);
}
__device__ __host__ __forceinline__ uint64_t child_hash(uint64_t h, int32_t tok) {
    return mix64(h ^ (uint64_t)(uint32_t)tok);
}

enum : uint32_t { STREAM_GUMBEL = 1, STREAM_ACCEPT = 2, STREAM_RESID = 3 };

// Four words for indices 4*g .. 4*g+3 of one (stream, node) pair.
__device__ __forceinline__ uint4 rand4(uint32_t g, uint32_t stream, uint64_t h, uint32_t k0,
                                       uint32_t k1) {
    return philox10(make_uint4(g, stream, (uint32_t)h, (uint32_t)(h >> 32)), k0, k1);
}

// Uniform in (0, 1): u = (m + 1/2) 2^-24 with m = the top 24 bits of a word.  In float32,
// m + 1/2 is exact only for m < 2^23; above that the sum would round, so callers that need
// 1 - u use one_minus_u01(), which is exact for m >= 2^23.
__device__ __forceinline__ float u01(uint32_t w) {
    return ((float)(w >> 8) + 0.5f) * (1.0f / 16777216.0f);
}
__device__ __forceinline__ float one_minus_u01(uint32_t w) {
    return ((float)(16777216u - (w >> 8)) - 0.5f) * (1.0f / 16777216.0f);
}

// Gumbel(0, 1) = -log(-log u).  For u > 1/2, -log u = -log1p(-(1 - u)) with 1 - u exact, so
// it keeps full relative precision near u = 1, where the largest Gumbel values, the ones
// that decide the top-k, come from.
__device__ __forceinline__ float gumbel(uint32_t w) {
    const uint32_t m = w >> 8;
    const float t = (m >= (1u << 23)) ? -log1pf(-one_minus_u01(w))
                                      : -logf(((float)m + 0.5f) * (1.0f / 16777216.0f));
    return -logf(t);
}

// ---------------------------------------------------------------------------------------
// Selection keys: one u64, larger = better.  High word = survival bits (survival >= 0, so
// the IEEE bit pattern orders like the value); low word = (63 - depth, 127 - frontier index
// of the parent, 15 - sibling rank), so ties go to the shallower node, then to the earlier
// parent in canonical order, then to the lower sibling rank: the (survival desc, depth asc,
// rank-path asc) order.  The low word alone orders nodes canonically (depth, path).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t node_low(int depth, int fi, int j) {
    return ((uint32_t)(63 - depth) << 11) | ((uint32_t)(127 - fi) << 4) | (uint32_t)(15 - j);
}
__device__ __forceinline__ uint64_t make_key(float s, int depth, int fi, int j) {
    return ((uint64_t)__float_as_uint(s) << 32) | node_low(depth, fi, j);
}
__device__ __forceinline__ float key_surv(uint64_t key) { return __uint_as_float((uint32_t)(key >> 32)); }
__device__ __forceinline__ int low_depth(uint32_t low) { return 63 - (int)((low >> 11) & 63u); }
__device__ __forceinline__ int low_fi(uint32_t low) { return 127 - (int)((low >> 4) & 127u); }
__device__ __forceinline__ int low_rank(uint32_t low) { return 15 - (int)(low & 15u); }

// ---------------------------------------------------------------------------------------
// Coherent accesses for data that workgroups of one persistent kernel hand to each other.
// Each XCD has its own L2, so a plain load can return a line another XCD has since
// rewritten.  Agent-scope relaxed atomics are issued with the agent-coherence bit: stores
// write through to the coherent level and loads read from it, so no L2 writeback or
// invalidate is needed.  publish() waits until this wavefront's earlier stores have been
// acknowledged; a workgroup publishes (every wavefront, then a barrier) before one thread
// announces the data with a counter or flag.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t cld32(const void* p) {
    return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cld64(const void* p) {
    return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst32(void* p, uint32_t v) {
    __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst64(void* p, uint64_t v) {
    __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-coherent store (the same write-through cache policy as cst64, which the
// compiler emits for agent-scope relaxed atomic stores; there is no 16-byte atomic).  Its
// completion is covered by publish(): vector memory counters drain in issue order.
__device__ __forceinline__ void cst128(void* p, uint4 v) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 d = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(d) : "memory");
}
__device__ __forceinline__ uint32_t cadd32(void* p, uint32_t v) {
    return __hip_atomic_fetch_add((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int cldi(const int* p) { return (int)cld32(p); }
__device__ __forceinline__ void csti(int* p, int v) { cst32(p, (uint32_t)v); }
__device__ __forceinline__ void publish() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void publish_wg() {
    publish();
    __syncthreads();
}

__device__ __forceinline__ FrontEntry ld_front(const FrontEntry* p) {
    const uint64_t w0 = cld64(p), w1 = cld64((const char*)p + 8), w2 = cld64((const char*)p + 16);
    FrontEntry e;
    e.self = (uint32_t)w0;
    e.token = (int32_t)(uint32_t)(w0 >> 32);
    e.s = __uint_as_float((uint32_t)w1);
    e.pad = (uint32_t)(w1 >> 32);
    e.hash = w2;
    return e;
}
__device__ __forceinline__ void st_front(FrontEntry* p, const FrontEntry& e) {
    cst64(p, (uint64_t)e.self | ((uint64_t)(uint32_t)e.token << 32));
    cst64((char*)p + 8, (uint64_t)__float_as_uint(e.s) | ((uint64_t)e.pad << 32));
    cst64((char*)p + 16, e.hash);
}
__device__ __forceinline__ ChildRec ld_child(const ChildRec* p) {
    const uint64_t w0 = cld64(p), w1 = cld64((const char*)p + 8), w2 = cld64((const char*)p + 16);
    ChildRec c;
    c.token = (int32_t)(uint32_t)w0;
    c.s = __uint_as_float((uint32_t)(w0 >> 32));
    c.logq = __uint_as_float((uint32_t)w1);
    c.pad = (uint32_t)(w1 >> 32);
    c.hash = w2;
    return c;
}
__device__ __forceinline__ void st_child(ChildRec* p, const ChildRec& c) {
    cst64(p, (uint64_t)(uint32_t)c.token | ((uint64_t)__float_as_uint(c.s) << 32));
    cst64((char*)p + 8, (uint64_t)__float_as_uint(c.logq) | ((uint64_t)c.pad << 32));
    cst64((char*)p + 16, c.hash);
}

// ---------------------------------------------------------------------------------------
// bf16 / f32 element access
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float load_logit(const void* base, size_t idx, bool bf16) {
    return bf16 ? bf16_to_f32(((const uint16_t*)base)[idx]) : ((const float*)base)[idx];
}

// ---------------------------------------------------------------------------------------
// Ranked lists held in registers.  An entry is one u64 whose unsigned order is the ranking
// order (key desc, token asc): high word = the key's float bits mapped to an order-preserving
// unsigned (ord32), low word = ~token.  0 marks an empty slot (below every real entry).  The
// tempered logit y (log2 units) travels with each entry.  Lists are sorted descending and
// use compile-time indices only (no scratch).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord32(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t pack_entry(float key, int tok) {
    return ((uint64_t)ord32(key) << 32) | (uint64_t)(~(uint32_t)tok);
}
__device__ __forceinline__ int entry_tok(uint64_t e) { return (int)~(uint32_t)e; }
__device__ __forceinline__ float entry_key(uint64_t e) { return unord32((uint32_t)(e >> 32)); }

template <int KT>
struct TopK {
    uint64_t k[KT];
    float y[KT];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            k[i] = 0;
            y[i] = -INFINITY;
        }
    }
    // Insert one entry: a branch-free pass of compare-exchanges down the sorted list.
    __device__ __forceinline__ void push(uint64_t c, float yc) {
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            const bool gt = c > k[i];
            const uint64_t tk = k[i];
            const float ty = y[i];
            k[i] = gt ? c : tk;
            y[i] = gt ? yc : ty;
            c = gt ? tk : c;
            yc = gt ? ty : yc;
        }
    }
    // Keep the KT best of this list and another sorted list (bitonic merge: the pairwise
    // maxima of this list and the reversed other list form a bitonic sequence holding the KT
    // best, which half-cleaners then sort).
    __device__ __forceinline__ void merge(const uint64_t (&ok)[KT], const float (&oy)[KT]) {
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            const bool gt = ok[KT - 1 - i] > k[i];
            k[i] = gt ? ok[KT - 1 - i] : k[i];
            y[i] = gt ? oy[KT - 1 - i] : y[i];
        }
#pragma unroll
        for (int half = KT / 2; half >= 1; half >>= 1) {
#pragma unroll
            for (int i = 0; i < KT; ++i) {
                if ((i & half) == 0) {
                    const int j = i + half;
                    const bool sw = k[j] > k[i];
                    const uint64_t ki = k[i], kj = k[j];
                    const float yi = y[i], yj = y[j];
                    k[i] = sw ? kj : ki;
                    k[j] = sw ? ki : kj;
                    y[i] = sw ? yj : yi;
                    y[j] = sw ? yi : yj;
                }
            }
        }
    }
    // Merge with the list held by lane (lane ^ off) of the same wavefront.
    __device__ __forceinline__ void merge_xor(int off) {
        uint64_t ok[KT];
        float oy[KT];
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            const uint32_t lo = __shfl_xor((uint32_t)k[i], off);
            const uint32_t hi = __shfl_xor((uint32_t)(k[i] >> 32), off);
            ok[i] = ((uint64_t)hi << 32) | lo;
            oy[i] = __shfl_xor(y[i], off);
        }
        merge(ok, oy);
    }
};

// Online log-sum-exp in log2 units: value = m + log2(s).
struct Lse2 {
    float m, s;
    __device__ __forceinline__ void init() { m = -INFINITY; s = 0.0f; }
    __device__ __forceinline__ void merge(float om, float os) {
        if (om == -INFINITY) return;
        if (m == -INFINITY) { m = om; s = os; return; }
        const float nm = fmaxf(m, om);
        s = s * exp2f(m - nm) + os * exp2f(om - nm);
        m = nm;
    }
    __device__ __forceinline__ void merge_xor(int off) {
        const float om = __shfl_xor(m, off), os = __shfl_xor(s, off);
        merge(om, os);
    }
};

}  // namespace dt
