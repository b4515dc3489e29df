// Tree construction kernels for gfx950.
//
// One round is a level-synchronous loop over block positions d = 1..B (PCTree summary:
// every position's logits come from one backbone forward, so a level needs no new drafter
// pass).  Per level:
//   expand  - fused Markov bias (bf16 MFMA, fp32 accumulate) + bias-add + temperature +
//             online log-sum-exp + per-row top-k over a vocabulary split, for every
//             frontier parent of every request at once;
//   merge   - per parent: combine the vocabulary splits, calibrate each child's probability
//             to an edge estimate and multiply survivals (TreeSpark core idea);
//   select  - per request: keep the best n_budget nodes with survival >= tau (best-first
//             with per-round stopping, which equals this expand-then-select because
//             survival never increases along a path), define the next frontier, and (last
//             workgroup) compact the next level's parent rows across requests.
// After the loop, emit writes the trees in canonical order with ancestor masks.
#include <hip/hip_runtime.h>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {


// ---------------------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024).
// ---------------------------------------------------------------------------------------
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
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

// Block-wide sum; every thread gets the total.
__device__ int block_sum(int v, int* sh) {
    int total;
    block_exclusive_scan(v, sh, &total);
    return total;
}

// Writes the parent-row list (request, frontier index) for `level` (0-based front level)
// from fcount, in request order.  Called by a single workgroup.
__device__ void compact_rows(int R, int B, int level, const int* fcount, int2* rows, int* ctl,
                             int* level_rows_out, int* sh) {
    const int per = (R + blockDim.x - 1) / blockDim.x;
    const int r0 = threadIdx.x * per;
    int cnt = 0;
    for (int r = r0; r < r0 + per && r < R; ++r) cnt += fcount[r * (B + 1) + level];
    int total;
    int off = block_exclusive_scan(cnt, sh, &total);
    for (int r = r0; r < r0 + per && r < R; ++r) {
        const int f = fcount[r * (B + 1) + level];
        for (int i = 0; i < f; ++i) rows[off + i] = make_int2(r, i);
        off += f;
    }
    if (threadIdx.x == 0) {
        ctl[0] = total;
        ctl[1] = 0;
        if (level_rows_out) *level_rows_out = total;
    }
}

// ---------------------------------------------------------------------------------------
// init: root frontier entries, budgets, status bits, level-1 rows.  One workgroup.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_build_init(int R, int B, int V, int Ncap, uint32_t round,
                                                    const int32_t* __restrict__ root_token,
                                                    const int32_t* __restrict__ n_budget,
                                                    FrontEntry* front, int* fcount, int* scount,
                                                    int* nbeff, int* rstat, int2* rows, int* ctl,
                                                    int32_t* level_rows) {
    __shared__ int sh[256];
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
        const int32_t root = root_token[r];
        int nb = n_budget[r];
        int st = 0;
        if (nb < 0 || nb > Ncap) {
            st |= DT_REQ_BUDGET_CLAMPED;
            nb = nb < 0 ? 0 : Ncap;
        }
        const bool ok = root >= 0 && root < V;
        if (!ok) st |= DT_REQ_BAD_ROOT;
        FrontEntry e;
        e.self = 0xFFFFFFFFu;
        e.token = ok ? root : 0;
        e.s = 1.0f;
        e.pad = 0;
        e.hash = root_hash(round, r, root);
        front[(size_t)r * (B + 1) * Ncap] = e;
        for (int l = 0; l <= B; ++l) fcount[r * (B + 1) + l] = 0;
        fcount[r * (B + 1)] = ok ? 1 : 0;
        scount[r] = 0;
        nbeff[r] = nb;
        rstat[r] = st;
    }
    if (level_rows)
        for (int l = threadIdx.x; l < B; l += blockDim.x) level_rows[l] = 0;
    __syncthreads();
    compact_rows(R, B, 0, fcount, rows, ctl, nullptr, sh);
}

// ---------------------------------------------------------------------------------------
// expand: C[64 parents x 128 columns] = A[64 x r] * Wt[cols x r]^T per step on MFMA
// 32x32x16 bf16, then the epilogue over the tile.
//
// Grid: G workgroups, re-partitioned at run time from the number of parent rows M:
// T = ceil(M/64) tiles x S vocabulary splits (S a multiple of 8 when >= 8, so all tiles of
// one split fall on the same XCD and share that split's W columns in its L2).
// LDS: A tile (64 rows x r, bf16) and the 64 x 128 fp32 result tile.
// Epilogue mapping: thread t owns row t/4 and 32 consecutive columns (t%4)*32.. of every
// chunk; its running (max, sum) and top-KT list persist across chunks.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ void split_grid(int M, int G, int NC, int* T, int* S) {
    const int t = (M + kTileRows - 1) / kTileRows;
    int s = t > 0 ? G / t : 1;
    if (s >= 8) s &= ~7;
    if (s > NC) s = NC;
    if (s < 1) s = 1;
    *T = t;
    *S = s;
}

template <int KT, bool SAMPLE, bool HEAD_BF16>
__global__ __launch_bounds__(256) void k_expand(const ExpandArgs a) {
    const int M = a.ctl[0];
    if (M == 0) return;
    int T, S;
    split_grid(M, a.G, a.NC, &T, &S);
    const int tile = blockIdx.x / S, split = blockIdx.x % S;
    if (tile >= T) return;
    const int m0 = tile * kTileRows;
    const int nrows = min(kTileRows, M - m0);
    const int c_beg = (int)((long long)split * a.NC / S);
    const int c_end = (int)((long long)(split + 1) * a.NC / S);

    __shared__ __attribute__((aligned(16))) uint16_t sA[HEAD_BF16 ? kTileRows * kAStride : 1];
    __shared__ __attribute__((aligned(16))) float sAf[HEAD_BF16 ? 1 : kTileRows * kAfStride];
    __shared__ float sZ[kTileRows * kZStride];
    __shared__ int sReq[kTileRows];
    __shared__ uint64_t sHash[kTileRows];

    const int tid = threadIdx.x;
    const int r = a.r;
    const int lvl = a.level - 1;  // front level of the parents = block row used

    // ---- parent rows -> A tile in LDS
    load_a_tile<HEAD_BF16>(a.U, r, nrows, [&](int row) {
        const int2 rq = a.rows[m0 + row];
        return a.front[((size_t)rq.x * (a.B + 1) + lvl) * a.Ncap + rq.y].token;
    }, sA, sAf);
    if (tid < kTileRows) {
        int req = 0;
        uint64_t h = 0;
        if (tid < nrows) {
            const int2 rq = a.rows[m0 + tid];
            req = rq.x;
            h = a.front[((size_t)rq.x * (a.B + 1) + lvl) * a.Ncap + rq.y].hash;
        }
        sReq[tid] = req;
        sHash[tid] = h;
    }
    __syncthreads();

    // ---- epilogue ownership
    const int erow = tid >> 2, epart = tid & 3;
    const bool eactive = erow < nrows;
    const int ereq = sReq[erow];
    const uint64_t ehash = sHash[erow];
    const size_t lbase = ((size_t)ereq * a.B + lvl) * (size_t)a.V;
    const bool lvec = a.logits_bf16 ? ((a.V & 7) == 0) : ((a.V & 3) == 0);
    TopK<KT> top;
    top.init();
    Lse2 acc2;
    acc2.init();

    const bool two = nrows > 32;

    for (int c = c_beg; c < c_end; ++c) {
        const int col0 = c * kChunkCols;
        mma_chunk<HEAD_BF16>(a.Wt, a.V, r, col0, two, sA, sAf, sZ);

        if (eactive) {
            const int cb = col0 + epart * 32;
            float z[32];
            if (lvec && cb + 32 <= a.V) {
                if (a.logits_bf16) {
                    const uint4* lp = (const uint4*)((const uint16_t*)a.L + lbase + cb);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 v = lp[q];
                        z[q * 8 + 0] = bf16_lo(v.x); z[q * 8 + 1] = bf16_hi(v.x);
                        z[q * 8 + 2] = bf16_lo(v.y); z[q * 8 + 3] = bf16_hi(v.y);
                        z[q * 8 + 4] = bf16_lo(v.z); z[q * 8 + 5] = bf16_hi(v.z);
                        z[q * 8 + 6] = bf16_lo(v.w); z[q * 8 + 7] = bf16_hi(v.w);
                    }
                } else {
                    const float4* lp = (const float4*)((const float*)a.L + lbase + cb);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float4 v = lp[q];
                        z[q * 4 + 0] = v.x; z[q * 4 + 1] = v.y; z[q * 4 + 2] = v.z; z[q * 4 + 3] = v.w;
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    z[j] = (cb + j < a.V) ? load_logit(a.L, lbase + cb + j, a.logits_bf16) : 0.0f;
            }
            const float* zr = sZ + erow * kZStride + epart * 32;
            float cm = -INFINITY;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                z[j] += zr[j];
                if (cb + j < a.V) cm = fmaxf(cm, z[j] * a.y2scale);
            }
            if (cm > acc2.m) {
                acc2.s = (acc2.m == -INFINITY) ? 0.0f : acc2.s * exp2f(acc2.m - cm);
                acc2.m = cm;
            }
            float ps = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j)
                if (cb + j < a.V) ps += exp2f(z[j] * a.y2scale - acc2.m);
            acc2.s += ps;
            if constexpr (SAMPLE) {
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const uint4 w = rand4((uint32_t)((cb >> 2) + g), STREAM_GUMBEL, ehash,
                                          a.seed_lo, a.seed_hi);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = g * 4 + e;
                        if (cb + j < a.V) {
                            const float key = z[j] * a.invT + gumbel(ws[e]);
                            top.push(key, z[j] * a.y2scale, cb + j);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    if (cb + j < a.V) top.push(z[j], z[j] * a.y2scale, cb + j);
            }
        }
        __syncthreads();
    }

    // ---- combine the four column owners of each row, write the split's partial record
    acc2.merge_xor(1);
    acc2.merge_xor(2);
    top.merge_xor(1);
    top.merge_xor(2);
    if (eactive && epart == 0) {
        float* rec = a.partials + ((size_t)(m0 + erow) * S + split) * (2 + 3 * KT);
        rec[0] = acc2.m;
        rec[1] = acc2.s;
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            rec[2 + i] = top.key[i];
            rec[2 + KT + i] = top.y[i];
            rec[2 + 2 * KT + i] = __int_as_float(top.tok[i]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// merge: one wavefront per parent row.  Combines the S split records, then writes the k
// children: q = 2^(y2 - lse2), bin = min(15, floor(16 q)), s = fl32(s_parent * cal[bin]),
// logq = (y2 - lse2) ln 2, and each child's selection key.
// ---------------------------------------------------------------------------------------
template <int KT>
__global__ __launch_bounds__(256) void k_merge(const MergeArgs a) {
    const int M = a.ctl[0];
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;
    int T, S;
    split_grid(M, a.G, a.NC, &T, &S);
    TopK<KT> top;
    top.init();
    Lse2 acc;
    acc.init();
    for (int s = lane; s < S; s += 64) {
        const float* rec = a.partials + ((size_t)row * S + s) * (2 + 3 * KT);
        acc.merge(rec[0], rec[1]);
#pragma unroll
        for (int i = 0; i < KT; ++i)
            top.push(rec[2 + i], rec[2 + KT + i], __float_as_int(rec[2 + 2 * KT + i]));
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        acc.merge_xor(off);
        top.merge_xor(off);
    }
    const float lse2 = acc.m + log2f(acc.s);
    const int2 rq = a.rows[row];
    const int lvl = a.level - 1;
    const FrontEntry& par = a.front[((size_t)rq.x * (a.B + 1) + lvl) * a.Ncap + rq.y];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
        if (j < a.k && lane == j) {
            const float l2 = top.y[j] - lse2;
            const float q = exp2f(l2);
            int bin = (int)floorf(16.0f * q);
            bin = bin > 15 ? 15 : (bin < 0 ? 0 : bin);
            ChildRec c;
            c.token = top.tok[j];
            c.s = par.s * a.cal[bin];
            c.logq = l2 * 0.69314718055994530942f;
            c.pad = 0;
            c.hash = child_hash(par.hash, c.token);
            a.arena[(((size_t)rq.x * a.B + lvl) * a.Ncap + rq.y) * a.k + j] = c;
            a.ckeys[(size_t)rq.x * a.Ncap * a.k + rq.y * a.k + j] = make_key(c.s, a.level, rq.y, j);
        }
    }
}

// ---------------------------------------------------------------------------------------
// select: one workgroup per request.  Candidates = the kept set + this level's children;
// drop survival < tau; bitonic sort (descending key) in LDS; keep min(n_budget, #kept).
// The kept nodes of depth `level` become the next frontier in canonical order.  The last
// workgroup to finish compacts the next level's rows over all requests.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_select(const SelectArgs a) {
    const int M = a.ctl[0];
    if (M == 0) return;
    __shared__ uint64_t keys[kSelectSlots];
    __shared__ int sh[256];
    __shared__ int s_last;
    const int req = blockIdx.x, tid = threadIdx.x;
    const int lvl = a.level - 1;
    const int F = a.fcount[req * (a.B + 1) + lvl];
    const int nprev = a.scount[req];
    const int ncand = nprev + F * a.k;
    const float tau = a.tau[req];
    int P = 2;
    while (P < ncand) P <<= 1;
    for (int i = tid; i < P; i += 256) {
        uint64_t key = 0;
        if (i < nprev) key = a.skeys[(size_t)req * a.Ncap + i];
        else if (i < ncand) key = a.ckeys[(size_t)req * a.Ncap * a.k + (i - nprev)];
        if (key != 0 && key_surv(key) < tau) key = 0;
        keys[i] = key;
    }
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += 256) {
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
    for (int i = tid; i < P; i += 256) nz += keys[i] != 0 ? 1 : 0;
    nz = block_sum(nz, sh);
    const int nkept = min(a.nbeff[req], nz);
    for (int i = tid; i < nkept; i += 256) a.skeys[(size_t)req * a.Ncap + i] = keys[i];
    if (tid == 0) a.scount[req] = nkept;

    // next frontier: kept nodes of depth == level, in canonical order
    int fnext = 0;
    if (a.level < a.B) {
        const uint32_t want_depth = (uint32_t)a.level;
        for (int i = tid; i < nkept; i += 256) {
            const uint32_t low = (uint32_t)keys[i];
            if ((uint32_t)low_depth(low) != want_depth) continue;
            int rank = 0;
            for (int m = 0; m < nkept; ++m) {
                const uint32_t lm = (uint32_t)keys[m];
                if ((uint32_t)low_depth(lm) == want_depth && lm > low) ++rank;
            }
            const int fi = low_fi(low), j = low_rank(low);
            const ChildRec& c = a.arena[(((size_t)req * a.B + lvl) * a.Ncap + fi) * a.k + j];
            FrontEntry e;
            e.self = low;
            e.token = c.token;
            e.s = c.s;
            e.pad = 0;
            e.hash = c.hash;
            a.front[((size_t)req * (a.B + 1) + a.level) * a.Ncap + rank] = e;
        }
        int cnt = 0;
        for (int i = tid; i < nkept; i += 256)
            cnt += (low_depth((uint32_t)keys[i]) == a.level) ? 1 : 0;
        fnext = block_sum(cnt, sh);
    }
    if (tid == 0) a.fcount[req * (a.B + 1) + a.level] = fnext;

    // last workgroup compacts the next level's rows
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&a.ctl[1], 1) == a.R - 1) ? 1 : 0;
    __syncthreads();
    if (s_last) {
        __threadfence();
        if (tid == 0 && a.level_rows) a.level_rows[lvl] = M;
        __syncthreads();
        if (a.level < a.B) {
            compact_rows(a.R, a.B, a.level, a.fcount, a.rows, a.ctl, nullptr, sh);
        } else if (tid == 0) {
            a.ctl[0] = 0;
            a.ctl[1] = 0;
        }
    }
}

// ---------------------------------------------------------------------------------------
// emit: one wavefront per request.  Canonical index of a kept node = number of kept nodes
// whose key low word is larger (depth asc, parent frontier index asc, rank asc).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_emit(int R, int B, int k, int Ncap, const uint64_t* skeys,
                                             const int* scount, const FrontEntry* front,
                                             const int* fcount, const ChildRec* arena,
                                             const int* rstat, dt_tree out) {
    __shared__ uint32_t lowc[kMaxNcap];
    __shared__ int parc[kMaxNcap];
    const int req = blockIdx.x, lane = threadIdx.x;
    const int n = scount[req];
    uint32_t mylow = 0;
    int canon = -1;
    if (lane < n) {
        mylow = (uint32_t)skeys[(size_t)req * Ncap + lane];
        canon = 0;
        for (int m = 0; m < n; ++m)
            if ((uint32_t)skeys[(size_t)req * Ncap + m] > mylow) ++canon;
        lowc[canon] = mylow;
    }
    __syncthreads();
    // lane i now handles canonical node i
    const size_t ob = (size_t)req * Ncap;
    int par = -2, depth = 0;
    if (lane < n) {
        const uint32_t low = lowc[lane];
        depth = low_depth(low);
        const int fi = low_fi(low), j = low_rank(low);
        const ChildRec& c = arena[(((size_t)req * B + (depth - 1)) * Ncap + fi) * k + j];
        if (depth == 1) {
            par = -1;
        } else {
            const uint32_t pid = front[((size_t)req * (B + 1) + (depth - 1)) * Ncap + fi].self;
            par = -1;
            for (int m = 0; m < n; ++m)
                if (lowc[m] == pid) par = m;
        }
        out.token[ob + lane] = c.token;
        out.depth[ob + lane] = (uint8_t)depth;
        out.surv[ob + lane] = c.s;
        out.logq[ob + lane] = c.logq;
        // expanded? find its slot in the next level's frontier
        const int cb = ((req * (Ncap + 1)) + lane + 1) * k;
        int slot = -1;
        if (depth < B) {
            const int F = fcount[req * (B + 1) + depth];
            for (int m = 0; m < F; ++m)
                if (front[((size_t)req * (B + 1) + depth) * Ncap + m].self == low) slot = m;
        }
        for (int jj = 0; jj < k; ++jj)
            out.cand[cb + jj] =
                slot >= 0 ? arena[(((size_t)req * B + depth) * Ncap + slot) * k + jj].token : -1;
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
        out.anc_mask[ob + lane] = m;
        out.parent[ob + lane] = (int16_t)par;
    } else if (lane < Ncap) {
        out.token[ob + lane] = -1;
        out.parent[ob + lane] = -2;
        out.depth[ob + lane] = 0;
        out.anc_mask[ob + lane] = 0;
        out.surv[ob + lane] = 0.0f;
        out.logq[ob + lane] = 0.0f;
        const int cb = ((req * (Ncap + 1)) + lane + 1) * k;
        for (int jj = 0; jj < k; ++jj) out.cand[cb + jj] = -1;
    }
    if (lane < k) {
        const bool rooted = fcount[req * (B + 1)] == 1;
        out.cand[(size_t)req * (Ncap + 1) * k + lane] =
            rooted ? arena[((size_t)req * B * Ncap) * k + lane].token : -1;
    }
    if (lane == 0) {
        out.n_nodes[req] = n;
        out.status[req] = rstat[req];
        if (out.n_expand) {
            int e = 0;
            for (int l = 0; l < B; ++l) e += fcount[req * (B + 1) + l];
            out.n_expand[req] = e;
        }
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_build_init(const dt_params* p, const Layout& lay, char* ws,
                             const int32_t* root_token, const int32_t* n_budget,
                             int32_t* level_rows, hipStream_t st) {
    hipLaunchKernelGGL(k_build_init, dim3(1), dim3(256), 0, st, p->R, p->B, p->V, p->Ncap,
                       p->round, root_token, n_budget, (FrontEntry*)(ws + lay.front),
                       (int*)(ws + lay.fcount), (int*)(ws + lay.scount), (int*)(ws + lay.nbeff),
                       (int*)(ws + lay.rstat), (int2*)(ws + lay.rows), (int*)(ws + lay.ctl),
                       level_rows);
    return hipGetLastError();
}

template <int KT>
static void launch_expand_kt(const dt_params* p, const Layout& lay, const ExpandArgs& a,
                             hipStream_t st) {
    const bool sample = p->mode == DT_SAMPLE, hb = p->head_dtype == DT_BF16;
    if (sample) {
        if (hb) hipLaunchKernelGGL((k_expand<KT, true, true>), dim3(lay.G), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_expand<KT, true, false>), dim3(lay.G), dim3(256), 0, st, a);
    } else {
        if (hb) hipLaunchKernelGGL((k_expand<KT, false, true>), dim3(lay.G), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_expand<KT, false, false>), dim3(lay.G), dim3(256), 0, st, a);
    }
}

hipError_t launch_expand(const dt_params* p, const Layout& lay, const ExpandArgs& a,
                         hipStream_t st) {
    switch (lay.KT) {
        case 1: launch_expand_kt<1>(p, lay, a, st); break;
        case 2: launch_expand_kt<2>(p, lay, a, st); break;
        case 4: launch_expand_kt<4>(p, lay, a, st); break;
        default: launch_expand_kt<8>(p, lay, a, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const dt_params* p, const Layout& lay, const MergeArgs& a,
                        hipStream_t st) {
    const int rows = p->R * p->Ncap;
    const dim3 grid((rows + 3) / 4);
    switch (lay.KT) {
        case 1: hipLaunchKernelGGL(k_merge<1>, grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_merge<2>, grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL(k_merge<4>, grid, dim3(256), 0, st, a); break;
        default: hipLaunchKernelGGL(k_merge<8>, grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_select(const dt_params* p, const SelectArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_select, dim3(p->R), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_emit(const dt_params* p, const Layout& lay, char* ws, const dt_tree* out,
                       hipStream_t st) {
    hipLaunchKernelGGL(k_emit, dim3(p->R), dim3(64), 0, st, p->R, p->B, p->k, p->Ncap,
                       (const uint64_t*)(ws + lay.skeys), (const int*)(ws + lay.scount),
                       (const FrontEntry*)(ws + lay.front), (const int*)(ws + lay.fcount),
                       (const ChildRec*)(ws + lay.arena), (const int*)(ws + lay.rstat), *out);
    return hipGetLastError();
}

}  // namespace dt
