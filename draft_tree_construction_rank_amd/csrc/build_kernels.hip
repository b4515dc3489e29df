// Tree construction on gfx950: a level-synchronous loop of two kernels per level.
//
// The round walks block positions d = 1..B (PCTree summary: every position's logits come
// from one backbone forward, so a level needs no new drafter pass):
//   k_expand        - fused Markov bias (bf16 MFMA 32x32x16, fp32 accumulate) + bias-add +
//                     temperature + online log-sum-exp + per-row top-k (or Gumbel-top-k)
//                     over a vocabulary split, for every frontier parent of every request;
//   k_merge_select  - one workgroup per request: combine the splits of each of its parents,
//                     calibrate each child's probability to an edge estimate and multiply
//                     survivals (TreeSpark core idea), then keep the best n_budget nodes with
//                     survival >= tau (best-first with per-round stopping equals this
//                     expand-then-select because survival never increases along a path) and
//                     define the next frontier; the last workgroup compacts the next level's
//                     parent rows across requests.
// Kernels of a level with no parent rows return at once.  k_build_init and k_emit open and
// close the round (emit: canonical order and ancestor masks).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {

// ---------------------------------------------------------------------------------------
// Workgroup helpers (256 threads).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int t = threadIdx.x, n = blockDim.x;
    sh[t] = v;
    __syncthreads();
    for (int off = 1; off < n; off <<= 1) {
        const int add = (t >= off) ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    const int incl = sh[t];
    if (total) *total = sh[n - 1];
    __syncthreads();
    return incl - v;
}

__device__ __forceinline__ int block_sum(int v, int* sh) {
    int total;
    block_exclusive_scan(v, sh, &total);
    return total;
}

__device__ __forceinline__ int load_int(const unsigned* p) {
    return (int)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Vocabulary splits for T tiles on a grid of G workgroups: about one item per workgroup,
// at most kMaxSplits (so that one workgroup can merge a request's records), and a multiple
// of 8 when >= 8 so that all tiles of one split run on the same XCD (blocks are dealt
// round-robin to the 8 XCDs) and share that split's W columns in its L2.
__device__ __forceinline__ int splits_for(int T, int G, int NC) {
    int s = T > 0 ? G / T : 1;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s >= 8) s &= ~7;
    if (s > NC) s = NC;
    if (s < 1) s = 1;
    return s;
}

// Writes the parent-row list (request, frontier index) for front level `level` from fcount,
// in request order, and the row count.  One workgroup.
__device__ __forceinline__ void compact_rows(const BuildArgs& a, int level, int* sh) {
    const int R = a.R, B = a.B;
    const int per = (R + blockDim.x - 1) / blockDim.x;
    const int r0 = threadIdx.x * per;
    int cnt = 0;
    for (int r = r0; r < r0 + per && r < R; ++r) cnt += a.fcount[r * (B + 1) + level];
    int total;
    int off = block_exclusive_scan(cnt, sh, &total);
    for (int r = r0; r < r0 + per && r < R; ++r) {
        const int f = a.fcount[r * (B + 1) + level];
        a.roff[r] = off;
        for (int i = 0; i < f; ++i) a.rows[off + i] = make_int2(r, i);
        off += f;
    }
    if (threadIdx.x == 0) a.sync[kSyncRows] = (unsigned)total;
}

// ---------------------------------------------------------------------------------------
// Phase A, one item: a tile of 64 parent rows x one vocabulary split.
// C[64 x 128 chunk] = A[64 x r] . Wt[chunk x r]^T on MFMA into LDS, then the epilogue:
// thread t owns row t/4 and columns (t%4)*32 .. +32 of every chunk; its running (max, sum)
// and top-KT list persist across the split's chunks.  The block-logit values of the next
// chunk are loaded right after the current chunk's epilogue so that their latency overlaps
// the next MFMA.
// ---------------------------------------------------------------------------------------
struct ExpandSmem {
    uint16_t sA[kTileRows * kAStride];
    float sZ[kTileRows * kZStride];
    int sTok[kTileRows];
    int sReq[kTileRows];
    uint64_t sHash[kTileRows];
};
struct ExpandSmemF {
    float sAf[kTileRows * kAfStride];
    float sZ[kTileRows * kZStride];
    int sTok[kTileRows];
    int sReq[kTileRows];
    uint64_t sHash[kTileRows];
};

// Largest value the Gumbel transform can return: u <= 1 - 2^-25, so -log(-log u) < 17.33;
// the bound below leaves room for float32 rounding.
constexpr float kGumbelMax = 17.35f;

// One chunk of one row for one thread: 32 columns cb .. cb+31 whose bias is in zr (LDS, this
// thread's own slots) and whose block logits are in l.  Updates the online log-sum-exp and
// the ranked list.  Candidates for the list are found with a mask against the current k-th
// key, then inserted one at a time from LDS, so the insertion code exists once.
template <int KT, bool SAMPLE>
__device__ __forceinline__ void epilogue_chunk(const BuildArgs& a, float* zr, int cb,
                                               const float (&l)[32], uint64_t ehash,
                                               TopK<KT>& top, Lse2& acc2) {
    const int nvalid = min(32, a.V - cb);
    float z[32];
    float cm = -INFINITY;
    // columns past V hold -inf in zr (see expand_item), so no per-column conditions here
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        z[j] = zr[j] + l[j];
        cm = fmaxf(cm, z[j]);
    }
    cm *= a.y2scale;
    if (cm > acc2.m) {
        acc2.s = (acc2.m == -INFINITY) ? 0.0f : acc2.s * exp2f(acc2.m - cm);
        acc2.m = cm;
    }
    float ps = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) ps += exp2f(z[j] * a.y2scale - acc2.m);  // exp2(-inf) = 0
    acc2.s += ps;
    // Candidates: a superset test against the current k-th key (ties and the Gumbel noise are
    // settled by push(), which re-checks the exact order).
    const float tk = top.key[KT - 1];
    // sample keys are z / T + G with G < kGumbelMax, so z < (tk - kGumbelMax) T cannot qualify
    const float thr = SAMPLE ? (tk - kGumbelMax) / a.invT : tk;
    uint32_t mask = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) mask |= (z[j] >= thr ? 1u : 0u) << j;
    if (nvalid < 32) mask &= nvalid > 0 ? (1u << nvalid) - 1u : 0u;
    if (mask == 0u) return;
#pragma unroll
    for (int j = 0; j < 32; ++j) zr[j] = z[j];
    if constexpr (SAMPLE) {
        for (int g = 0; g < 8; ++g) {
            uint32_t gm = (mask >> (4 * g)) & 15u;
            if (gm == 0u) continue;
            const uint4 w = rand4((uint32_t)((cb >> 2) + g), STREAM_GUMBEL, ehash, a.seed_lo,
                                  a.seed_hi);
            while (gm) {
                const int e = __builtin_ctz(gm);
                gm &= gm - 1u;
                const uint32_t we = e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
                const float zj = zr[4 * g + e];
                top.push(zj * a.invT + gumbel(we), zj * a.y2scale, cb + 4 * g + e);
            }
        }
    } else {
        while (mask) {
            const int j = __builtin_ctz(mask);
            mask &= mask - 1u;
            const float zj = zr[j];
            top.push(zj, zj * a.y2scale, cb + j);
        }
    }
}

// Raw block-logit words of 32 consecutive columns: 4 x 16 bytes for bf16 rows (the common
// case), else nothing (float32 or unaligned rows are read in the epilogue itself).
struct LWords {
    uint4 w[4];
};

__device__ __forceinline__ void load_lwords(const BuildArgs& a, size_t lbase, int cb, bool lvec,
                                            LWords& lw) {
    if (lvec && a.logits_bf16 && cb + 32 <= a.V) {
        const uint4* lp = (const uint4*)((const uint16_t*)a.L + lbase + cb);
#pragma unroll
        for (int q = 0; q < 4; ++q) lw.w[q] = lp[q];
    }
}

// Block-logit values of 32 consecutive columns.  The common case (bf16 rows, 16-byte
// aligned, a full chunk) unpacks the prefetched words; otherwise the values are added into
// the thread's LDS slots here, with -inf past V, and l is zero.
__device__ __forceinline__ void block_logits32(const BuildArgs& a, size_t lbase, int cb, bool lvec,
                                               const LWords& lw, float* zr, float (&l)[32]) {
    if (lvec && a.logits_bf16 && cb + 32 <= a.V) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = lw.w[q];
            l[q * 8 + 0] = bf16_lo(v.x); l[q * 8 + 1] = bf16_hi(v.x);
            l[q * 8 + 2] = bf16_lo(v.y); l[q * 8 + 3] = bf16_hi(v.y);
            l[q * 8 + 4] = bf16_lo(v.z); l[q * 8 + 5] = bf16_hi(v.z);
            l[q * 8 + 6] = bf16_lo(v.w); l[q * 8 + 7] = bf16_hi(v.w);
        }
        return;
    }
#pragma unroll 1
    for (int j = 0; j < 32; ++j)
        zr[j] = (cb + j < a.V) ? zr[j] + load_logit(a.L, lbase + cb + j, a.logits_bf16) : -INFINITY;
#pragma unroll
    for (int j = 0; j < 32; ++j) l[j] = 0.0f;
}

template <int KT, bool SAMPLE, bool HEAD_BF16, typename Sm>
__device__ __forceinline__ void expand_item(const BuildArgs& a, int level, int M, int S, int tile,
                                            int split, Sm& sm) {
    const int tid = threadIdx.x;
    const int lvl = level - 1;
    const int m0 = tile * kTileRows;
    const int nrows = min(kTileRows, M - m0);
    const int c_beg = (int)((long long)split * a.NC / S);
    const int c_end = (int)((long long)(split + 1) * a.NC / S);

    if (tid < kTileRows) {
        int tok = 0, req = 0;
        uint64_t h = 0;
        if (tid < nrows) {
            const int2 rq = a.rows[m0 + tid];
            const FrontEntry& fe = a.front[((size_t)rq.x * (a.B + 1) + lvl) * a.Ncap + rq.y];
            tok = fe.token;
            req = rq.x;
            h = fe.hash;
        }
        sm.sTok[tid] = tok;
        sm.sReq[tid] = req;
        sm.sHash[tid] = h;
    }
    __syncthreads();
    if constexpr (HEAD_BF16)
        load_a_tile<true>(a.U, a.r, nrows, [&](int row) { return sm.sTok[row]; }, sm.sA, nullptr);
    else
        load_a_tile<false>(a.U, a.r, nrows, [&](int row) { return sm.sTok[row]; }, nullptr, sm.sAf);
    __syncthreads();

    const int erow = tid >> 2, epart = tid & 3;
    const bool eactive = erow < nrows;
    const uint64_t ehash = sm.sHash[erow];
    const size_t lbase = ((size_t)sm.sReq[erow] * a.B + lvl) * (size_t)a.V;
    const bool lvec = a.logits_bf16 ? ((a.V & 7) == 0) : ((a.V & 3) == 0);
    TopK<KT> top;
    top.init();
    Lse2 acc2;
    acc2.init();
    const bool two = nrows > 32;

    LWords lw;
    if (eactive && c_beg < c_end) load_lwords(a, lbase, c_beg * kChunkCols + epart * 32, lvec, lw);
    for (int c = c_beg; c < c_end; ++c) {
        const int col0 = c * kChunkCols;
        if constexpr (HEAD_BF16)
            mma_chunk<true>(a.Wt, a.V, a.r, col0, two, sm.sA, nullptr, sm.sZ);
        else
            mma_chunk<false>(a.Wt, a.V, a.r, col0, two, nullptr, sm.sAf, sm.sZ);
        if (eactive) {
            float lv[32];
            float* zr = sm.sZ + erow * kZStride + epart * 32;
            block_logits32(a, lbase, col0 + epart * 32, lvec, lw, zr, lv);
            if (c + 1 < c_end) load_lwords(a, lbase, col0 + kChunkCols + epart * 32, lvec, lw);
            epilogue_chunk<KT, SAMPLE>(a, zr, col0 + epart * 32, lv, ehash, top, acc2);
        }
        __syncthreads();
    }
    acc2.merge_xor(1);
    acc2.merge_xor(2);
    top.merge_xor(1);
    top.merge_xor(2);
    if (eactive && epart == 0) {
        constexpr int RS = rec_floats(KT);
        float v[RS];
#pragma unroll
        for (int i = 0; i < RS; ++i) v[i] = 0.0f;
        v[0] = acc2.m;
        v[1] = acc2.s;
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            v[2 + i] = top.key[i];
            v[2 + KT + i] = top.y[i];
            v[2 + 2 * KT + i] = __int_as_float(top.tok[i]);
        }
        float4* rec = (float4*)(a.partials + ((size_t)(m0 + erow) * S + split) * RS);
#pragma unroll
        for (int q = 0; q < RS / 4; ++q)
            rec[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------------------
// Phase B, one wavefront per parent row: combine the S split records; child j gets
// q = 2^(y2 - lse2), bin = min(15, floor(16 q)), s = fl32(s_parent * cal[bin]),
// logq = (y2 - lse2) ln 2, and its selection key.
// ---------------------------------------------------------------------------------------
template <int KT>
__device__ __forceinline__ void merge_record(const float4 (&q)[rec_floats(KT) / 4], TopK<KT>& top,
                                             Lse2& acc) {
    float v[rec_floats(KT)];
#pragma unroll
    for (int i = 0; i < rec_floats(KT) / 4; ++i) {
        v[4 * i] = q[i].x;
        v[4 * i + 1] = q[i].y;
        v[4 * i + 2] = q[i].z;
        v[4 * i + 3] = q[i].w;
    }
    acc.merge(v[0], v[1]);
#pragma unroll
    for (int i = 0; i < KT; ++i) top.push(v[2 + i], v[2 + KT + i], __float_as_int(v[2 + 2 * KT + i]));
}

template <int KT>
__device__ __forceinline__ void merge_row(const BuildArgs& a, int level, int S, int row) {
    constexpr int RS = rec_floats(KT), NQ = RS / 4;
    const int lane = threadIdx.x & 63;
    TopK<KT> top;
    top.init();
    Lse2 acc;
    acc.init();
    const float4* base = (const float4*)(a.partials + (size_t)row * S * RS);
    // two records per lane per round, both loaded before either is merged
    for (int s0 = lane; s0 < S; s0 += 128) {
        const int s1 = s0 + 64 < S ? s0 + 64 : s0;
        float4 q0[NQ], q1[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            q0[i] = base[(size_t)s0 * NQ + i];
            q1[i] = base[(size_t)s1 * NQ + i];
        }
        merge_record<KT>(q0, top, acc);
        if (s0 + 64 < S) merge_record<KT>(q1, top, acc);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        acc.merge_xor(off);
        top.merge_xor(off);
    }
    const float lse2 = acc.m + log2f(acc.s);
    const int2 rq = a.rows[row];
    const int lvl = level - 1;
    const FrontEntry par = a.front[((size_t)rq.x * (a.B + 1) + lvl) * a.Ncap + rq.y];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
        if (j < a.k && lane == j) {
            const float l2 = top.y[j] - lse2;
            const float q = exp2f(l2);
            int bin = (int)floorf(16.0f * q);
            bin = bin > 15 ? 15 : (bin < 0 ? 0 : bin);
            ChildRec c;
            c.token = top.tok[j];
            float cv = a.cal[0];
#pragma unroll
            for (int ii = 1; ii < 16; ++ii) cv = (bin == ii) ? a.cal[ii] : cv;
            c.s = par.s * cv;
            c.logq = l2 * 0.69314718055994530942f;
            c.pad = 0;
            c.hash = child_hash(par.hash, c.token);
            a.arena[(((size_t)rq.x * a.B + lvl) * a.Ncap + rq.y) * a.k + j] = c;
            a.ckeys[(size_t)rq.x * a.Ncap * a.k + rq.y * a.k + j] = make_key(c.s, level, rq.y, j);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Phase C, one workgroup per request: candidates = the kept set + this level's children;
// drop survival < tau; bitonic sort (descending key) in LDS; keep min(n_budget, #left).
// The kept nodes of depth `level` become the next frontier in canonical order.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void select_request(const BuildArgs& a, int level, int req,
                                               uint64_t* keys, int* sh) {
    const int tid = threadIdx.x;
    const int lvl = level - 1;
    const int F = a.fcount[req * (a.B + 1) + lvl];
    const int nprev = a.scount[req];
    const int ncand = nprev + F * a.k;
    const float tau = a.tau[req];
    int P = 2;
    while (P < ncand) P <<= 1;
    for (int i = tid; i < P; i += blockDim.x) {
        uint64_t key = 0;
        if (i < nprev) key = a.skeys[(size_t)req * a.Ncap + i];
        else if (i < ncand) key = a.ckeys[(size_t)req * a.Ncap * a.k + (i - nprev)];
        if (key != 0 && key_surv(key) < tau) key = 0;
        keys[i] = key;
    }
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += blockDim.x) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = ((lo & size) == 0);
                const uint64_t x = keys[lo], y = keys[hi];
                if ((x < y) == desc) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    int nz = 0;
    for (int i = tid; i < P; i += blockDim.x) nz += keys[i] != 0 ? 1 : 0;
    nz = block_sum(nz, sh);
    const int nkept = min(a.nbeff[req], nz);
    for (int i = tid; i < nkept; i += blockDim.x) a.skeys[(size_t)req * a.Ncap + i] = keys[i];
    if (tid == 0) a.scount[req] = nkept;
    int fnext = 0;
    if (level < a.B) {
        for (int i = tid; i < nkept; i += blockDim.x) {
            const uint32_t low = (uint32_t)keys[i];
            if (low_depth(low) != level) continue;
            int rank = 0;
            for (int m = 0; m < nkept; ++m) {
                const uint32_t lm = (uint32_t)keys[m];
                if (low_depth(lm) == level && lm > low) ++rank;
            }
            const int fi = low_fi(low), j = low_rank(low);
            const ChildRec& c = a.arena[(((size_t)req * a.B + lvl) * a.Ncap + fi) * a.k + j];
            FrontEntry e;
            e.self = low;
            e.token = c.token;
            e.s = c.s;
            e.pad = 0;
            e.hash = c.hash;
            a.front[((size_t)req * (a.B + 1) + level) * a.Ncap + rank] = e;
        }
        int cnt = 0;
        for (int i = tid; i < nkept; i += blockDim.x)
            cnt += (low_depth((uint32_t)keys[i]) == level) ? 1 : 0;
        fnext = block_sum(cnt, sh);
    }
    if (tid == 0) a.fcount[req * (a.B + 1) + level] = fnext;
    __syncthreads();
}

// ---------------------------------------------------------------------------------------
// Emit, one request (threads 0..63 of the workgroup).  Canonical index of a kept node =
// number of kept nodes whose key low word is larger (depth asc, parent index asc, rank asc).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void emit_request(const BuildArgs& a, int req, uint32_t* lowc,
                                             int* parc) {
    const int lane = threadIdx.x;
    const int B = a.B, k = a.k, Ncap = a.Ncap;
    const int n = a.scount[req];
    if (lane < n) {
        const uint32_t mylow = (uint32_t)a.skeys[(size_t)req * Ncap + lane];
        int canon = 0;
        for (int m = 0; m < n; ++m)
            if ((uint32_t)a.skeys[(size_t)req * Ncap + m] > mylow) ++canon;
        lowc[canon] = mylow;
    }
    __syncthreads();
    const size_t ob = (size_t)req * Ncap;
    int par = -2;
    if (lane < n) {
        const uint32_t low = lowc[lane];
        const int depth = low_depth(low);
        const int fi = low_fi(low), j = low_rank(low);
        const ChildRec& c = a.arena[(((size_t)req * B + (depth - 1)) * Ncap + fi) * k + j];
        if (depth == 1) {
            par = -1;
        } else {
            const uint32_t pid = a.front[((size_t)req * (B + 1) + (depth - 1)) * Ncap + fi].self;
            par = -1;
            for (int m = 0; m < n; ++m)
                if (lowc[m] == pid) par = m;
        }
        a.out.token[ob + lane] = c.token;
        a.out.depth[ob + lane] = (uint8_t)depth;
        a.out.surv[ob + lane] = c.s;
        a.out.logq[ob + lane] = c.logq;
        const size_t cb = ((size_t)req * (Ncap + 1) + lane + 1) * k;
        int slot = -1;
        if (depth < B) {
            const int F = a.fcount[req * (B + 1) + depth];
            for (int m = 0; m < F; ++m)
                if (a.front[((size_t)req * (B + 1) + depth) * Ncap + m].self == low) slot = m;
        }
        for (int jj = 0; jj < k; ++jj)
            a.out.cand[cb + jj] =
                slot >= 0 ? a.arena[(((size_t)req * B + depth) * Ncap + slot) * k + jj].token : -1;
    }
    if (lane < kMaxNcap) parc[lane] = par;
    __syncthreads();
    if (lane < n) {
        uint64_t m = 0;
        int x = lane;
        while (x >= 0) {
            m |= 1ull << x;
            x = parc[x];
        }
        a.out.anc_mask[ob + lane] = m;
        a.out.parent[ob + lane] = (int16_t)par;
    } else if (lane < Ncap) {
        a.out.token[ob + lane] = -1;
        a.out.parent[ob + lane] = -2;
        a.out.depth[ob + lane] = 0;
        a.out.anc_mask[ob + lane] = 0;
        a.out.surv[ob + lane] = 0.0f;
        a.out.logq[ob + lane] = 0.0f;
        const size_t cb = ((size_t)req * (Ncap + 1) + lane + 1) * k;
        for (int jj = 0; jj < k; ++jj) a.out.cand[cb + jj] = -1;
    }
    if (lane < k) {
        const bool rooted = a.fcount[req * (B + 1)] == 1;
        a.out.cand[(size_t)req * (Ncap + 1) * k + lane] =
            rooted ? a.arena[((size_t)req * B * Ncap) * k + lane].token : -1;
    }
    if (lane == 0) {
        a.out.n_nodes[req] = n;
        a.out.status[req] = a.rstat[req];
        if (a.out.n_expand) {
            int e = 0;
            for (int l = 0; l < B; ++l) e += a.fcount[req * (B + 1) + l];
            a.out.n_expand[req] = e;
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------------------
// Round set-up (one workgroup): roots, budgets, status bits, the level-1 parent rows.
__global__ __launch_bounds__(256) void k_build_init(const BuildArgs a) {
    __shared__ int sh[256];
    const int tid = threadIdx.x;
    for (int r = tid; r < a.R; r += blockDim.x) {
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
        a.pdone[r] = 0;
    }
    if (a.out.level_rows)
        for (int l = tid; l < a.B; l += blockDim.x) a.out.level_rows[l] = 0;
    if (tid < kSyncWords) a.sync[tid] = 0u;
    __syncthreads();
    compact_rows(a, 0, sh);
}

template <int KT, bool SAMPLE, bool HEAD_BF16>
__global__ __launch_bounds__(256, 2) void k_expand(const BuildArgs a, int level) {
    using Sm = typename std::conditional<HEAD_BF16, ExpandSmem, ExpandSmemF>::type;
    __shared__ __attribute__((aligned(16))) Sm sm;
    const int M = load_int(a.sync + kSyncRows);
    if (M == 0) return;
    const int T = (M + kTileRows - 1) / kTileRows;
    const int S = splits_for(T, gridDim.x, a.NC);
    for (int item = blockIdx.x; item < T * S; item += gridDim.x)
        expand_item<KT, SAMPLE, HEAD_BF16>(a, level, M, S, item / S, item % S, sm);
}

// P workgroups per request: part p merges parent rows p, p+P, .. (one wavefront per row);
// the last part to finish runs the request's select; the last request to finish compacts
// the next level's rows.
template <int KT>
__global__ __launch_bounds__(256) void k_merge_select(const BuildArgs a, int level, int G, int P) {
    __shared__ uint64_t keys[kSelectSlots];
    __shared__ int sh[256];
    __shared__ int s_flag;
    const int M = load_int(a.sync + kSyncRows);
    if (M == 0) return;
    const int tid = threadIdx.x, req = blockIdx.x / P, part = blockIdx.x % P;
    const int S = splits_for((M + kTileRows - 1) / kTileRows, G, a.NC);
    const int F = a.fcount[req * (a.B + 1) + level - 1];
    const int row0 = a.roff[req];
    for (int fi = part + P * (tid >> 6); fi < F; fi += 4 * P) merge_row<KT>(a, level, S, row0 + fi);
    __threadfence();
    __syncthreads();
    if (tid == 0) s_flag = (atomicAdd(a.pdone + req, 1) == P - 1) ? 1 : 0;
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    if (tid == 0) a.pdone[req] = 0;
    select_request(a, level, req, keys, sh);
    __threadfence();
    __syncthreads();
    if (tid == 0) s_flag = (atomicAdd(a.sync + kSyncFinish, 1u) == (unsigned)a.R - 1u) ? 1 : 0;
    __syncthreads();
    if (s_flag) {
        __threadfence();
        if (tid == 0) {
            a.sync[kSyncFinish] = 0u;
            if (a.out.level_rows) a.out.level_rows[level - 1] = M;
        }
        if (level < a.B) compact_rows(a, level, sh);
        else if (tid == 0) a.sync[kSyncRows] = 0u;
    }
}

__global__ __launch_bounds__(256) void k_emit(const BuildArgs a) {
    __shared__ uint32_t lowc[kMaxNcap];
    __shared__ int parc[kMaxNcap];
    emit_request(a, blockIdx.x, lowc, parc);
}

// ---------------------------------------------------------------------------------------
// Launch sequence of one round.
// ---------------------------------------------------------------------------------------
template <int KT, bool SAMPLE, bool HEAD_BF16>
static hipError_t launch_build_t(const BuildArgs& a, int G, hipStream_t st) {
    // merge parts per request: enough workgroups to give every parent row of a small batch
    // its own wavefront
    const int P = a.R >= 64 ? 1 : (64 / a.R > 16 ? 16 : 64 / a.R);
    hipLaunchKernelGGL(k_build_init, dim3(1), dim3(256), 0, st, a);
    for (int level = 1; level <= a.B; ++level) {
        if (a.timing_hook) a.timing_hook(st, 0);
        hipLaunchKernelGGL((k_expand<KT, SAMPLE, HEAD_BF16>), dim3(G), dim3(256), 0, st, a, level);
        if (a.timing_hook) a.timing_hook(st, 1);
        hipLaunchKernelGGL(k_merge_select<KT>, dim3(a.R * P), dim3(256), 0, st, a, level, G, P);
    }
    hipLaunchKernelGGL(k_emit, dim3(a.R), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int KT>
static hipError_t launch_build_kt(const dt_params* p, const BuildArgs& a, int G, hipStream_t st) {
    const bool sample = p->mode == DT_SAMPLE, hb = p->head_dtype == DT_BF16;
    if (sample) return hb ? launch_build_t<KT, true, true>(a, G, st)
                          : launch_build_t<KT, true, false>(a, G, st);
    return hb ? launch_build_t<KT, false, true>(a, G, st)
              : launch_build_t<KT, false, false>(a, G, st);
}

hipError_t launch_build(const dt_params* p, const Layout& lay, const BuildArgs& a,
                        hipStream_t st) {
    switch (lay.KT) {
        case 1: return launch_build_kt<1>(p, a, lay.G, st);
        case 2: return launch_build_kt<2>(p, a, lay.G, st);
        case 4: return launch_build_kt<4>(p, a, lay.G, st);
        default: return launch_build_kt<8>(p, a, lay.G, st);
    }
}

}  // namespace dt
