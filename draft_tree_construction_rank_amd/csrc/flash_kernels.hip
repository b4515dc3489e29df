// Two-stage M-ary draft tree (TreeFlash explainer, technical summary, methodology: two-stage
// inference construction) on this library's parent-conditioned Markov head.
//
// Stage 1 takes, for every block row j, the M tokens with the largest unconditioned block
// logits (ties: lower id); they are the tree's only tokens at depth j + 1.  Stage 2 evaluates
// the parent-conditioned law of every state (row j, token t) -- t = the root for j = 0 and
// t in S_{j-1} for j >= 1, 1 + M (B - 1) states a request -- as z = L[j] + U[t] . W over the
// whole vocabulary; the states do not depend on each other, so they are one MFMA pass (the
// expansion's 64 x 128 tiles) instead of one pass per level.  The final selection is the
// best-first top-N with per-round stopping of the parent-conditioned tree (same calibration,
// survival, order and emission) over the lattice in which a node of depth j with token t has
// the children S_j, with q from state (j, t) and siblings ranked by their conditional logit.
//
// Kernels: k_flash_sets (top-M of every block row: one 1024-thread workgroup a row),
// k_flash_lse (log-sum-exp of every state over vocabulary splits: a (64-state tile,
// split) workgroup streams the split's W columns through MFMA, adds the block logits and
// keeps an online log2-sum-exp per state), k_flash_select (one workgroup a request: the
// conditional logits of the lattice children as dot products, the split log-sum-exps
// combined, then the level-synchronous select and the emission, all in LDS).
#include <hip/hip_runtime.h>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {

constexpr int kFlashSetThreads = 256;
constexpr int kFlashSelThreads = 256;
constexpr int kFlashMaxStates = 1 + (kMaxB - 1) * kMaxK;  // 249
constexpr int kFlashPool = kMaxNcap + kMaxNcap * kMaxK;   // kept + one level's children

struct FlashArgs {
    const void* L;
    const void* U;
    const void* Wt;
    const int32_t* root_token;
    const int32_t* n_budget;
    const float* tau;
    int32_t* sets;  // [R][B][M]
    float2* lsep;   // [R * NS][SP] (max, sum) in log2 units
    float* zc;      // [R * NS][M] conditional logits of every state's children (set order)
    uint64_t* setp; // [R * B][P][8] stage-1 part lists
    dt_tree out;
    int R, B, M, V, r, Ncap, NS, SP, T, P;
    int logits_bf16;
    float cal[16];
};

__device__ __forceinline__ float flash_logit(const FlashArgs& a, size_t idx) {
    return a.logits_bf16 ? bf16_to_f32(((const uint16_t*)a.L)[idx]) : ((const float*)a.L)[idx];
}

// State s of a request: block row j and head token t (-1 for a bad root).
__device__ __forceinline__ void flash_state(const FlashArgs& a, int req, int s, int* j, int* t) {
    if (s == 0) {
        *j = 0;
        const int rt = a.root_token[req];
        *t = (rt >= 0 && rt < a.V) ? rt : -1;
    } else {
        *j = 1 + (s - 1) / a.M;
        *t = a.sets[((size_t)req * a.B + (*j - 1)) * a.M + (s - 1) % a.M];
    }
}

// ---- stage 1: top-M of every block row ----------------------------------------------------
// Each row is scanned by P workgroups (P parts of its columns); each part's ranked list of
// 8 packed (logit, token) entries goes to the workspace and a second kernel merges a row's P
// lists.  An entry enters a thread's list only if it beats the list's last entry (one
// compare for almost every element once the list is warm).
__device__ __forceinline__ void flash_offer(TopK<kMaxK>& top, float v, int c) {
    const uint64_t e = pack_entry(v, c);
    if (e > top.k[kMaxK - 1]) top.push(e, 0.0f);
}

__global__ __launch_bounds__(kFlashSetThreads) void k_flash_sets(FlashArgs a) {
    __shared__ uint64_t sk[kFlashSetThreads / 64][kMaxK];
    const int row = blockIdx.x / a.P, part = blockIdx.x % a.P;  // row = req * B + j
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t base = (size_t)row * a.V;
    TopK<kMaxK> top;
    top.init();
    if (a.logits_bf16 && (a.V & 7) == 0) {
        const uint4* p = (const uint4*)((const uint16_t*)a.L + base);
        const int ng = a.V / 8;
        const int g_beg = (int)((long)part * ng / a.P), g_end = (int)((long)(part + 1) * ng / a.P);
        for (int g0 = g_beg + tid; g0 < g_end; g0 += 2 * kFlashSetThreads) {
            const int g1 = g0 + kFlashSetThreads;
            const uint4 w0 = p[g0], w1 = p[g1 < g_end ? g1 : g0];
            const uint32_t x0[4] = {w0.x, w0.y, w0.z, w0.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                flash_offer(top, bf16_lo(x0[i]), 8 * g0 + 2 * i);
                flash_offer(top, bf16_hi(x0[i]), 8 * g0 + 2 * i + 1);
            }
            if (g1 < g_end) {
                const uint32_t x1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    flash_offer(top, bf16_lo(x1[i]), 8 * g1 + 2 * i);
                    flash_offer(top, bf16_hi(x1[i]), 8 * g1 + 2 * i + 1);
                }
            }
        }
    } else {
        const int c_beg = (int)((long)part * a.V / a.P), c_end = (int)((long)(part + 1) * a.V / a.P);
        for (int c = c_beg + tid; c < c_end; c += kFlashSetThreads) flash_offer(top, flash_logit(a, base + c), c);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) top.merge_xor(off);
    if (lane == 0)
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) sk[wave][i] = top.k[i];
    __syncthreads();
    if (wave == 0) {
        TopK<kMaxK> t;
        t.init();
        if (lane < kFlashSetThreads / 64)
#pragma unroll
            for (int i = 0; i < kMaxK; ++i) t.k[i] = sk[lane][i];
#pragma unroll
        for (int off = 1; off < kFlashSetThreads / 64; off <<= 1) t.merge_xor(off);
        if (lane < kMaxK) {
            uint64_t v = 0;
#pragma unroll
            for (int i = 0; i < kMaxK; ++i) v = lane == i ? t.k[i] : v;
            a.setp[((size_t)row * a.P + part) * kMaxK + lane] = v;
        }
    }
}

// One wavefront per row merges the row's P part lists into its set S_j (M tokens).
__global__ __launch_bounds__(64) void k_flash_sets_merge(FlashArgs a) {
    const int row = blockIdx.x, lane = threadIdx.x;
    TopK<kMaxK> t;
    t.init();
    if (lane < a.P)
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) t.k[i] = a.setp[((size_t)row * a.P + lane) * kMaxK + i];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) t.merge_xor(off);
    if (lane == 0)
#pragma unroll
        for (int i = 0; i < kMaxK; ++i)
            if (i < a.M) a.sets[(size_t)row * a.M + i] = entry_tok(t.k[i]);
}

// ---- stage 2: log-sum-exp of every state over vocabulary splits ---------------------------
// Workgroup b: XCD x = b % 8 takes splits x, x + 8, ...; the T tiles of one split are adjacent
// in that XCD's queue, so they run together and read the split's W columns from its L2.
template <bool HEAD_BF16>
__global__ __launch_bounds__(256) void k_flash_lse(FlashArgs a) {
    __shared__ __align__(16) uint16_t sA[kTileRows * kAStride];
    __shared__ __align__(16) float sAf[HEAD_BF16 ? 1 : kTileRows * kAfStride];
    __shared__ __align__(16) float sZ[kTileRows * kZStride];
    __shared__ int sTok[kTileRows];
    __shared__ size_t sLb[kTileRows];
    __shared__ int sTgt[kTileRows][kMaxK];
    const int b = blockIdx.x;
    const int idx = b >> 3;
    const int tile = idx % a.T;
    const int split = (idx / a.T) * 8 + (b & 7);
    if (split >= a.SP) return;
    const int tid = threadIdx.x;
    const int rows_total = a.R * a.NS;
    const int g0 = tile * kTileRows;
    const int nrows = min(kTileRows, rows_total - g0);
    if (tid < kTileRows) {
        int t = -1;
        size_t lb = 0;
        if (tid < nrows) {
            const int g = g0 + tid, req = g / a.NS;
            int j;
            flash_state(a, req, g % a.NS, &j, &t);
            lb = ((size_t)req * a.B + j) * a.V;
            for (int i = 0; i < a.M; ++i) sTgt[tid][i] = a.sets[((size_t)req * a.B + j) * a.M + i];
        }
        sTok[tid] = t;
        sLb[tid] = lb;
    }
    __syncthreads();
    load_a_tile<HEAD_BF16>(a.U, a.r, nrows, [&](int row) { return sTok[row]; }, sA, sAf);
    __syncthreads();
    const int chunks = (a.V + kChunkCols - 1) / kChunkCols;
    const int c_beg = (int)((long)split * chunks / a.SP), c_end = (int)((long)(split + 1) * chunks / a.SP);
    // thread: row tid / 4, columns 32 (tid % 4) .. +32 of each chunk
    const int row = tid >> 2, q = tid & 3;
    const bool live = row < nrows;
    const size_t lb = sLb[row];
    constexpr float kLog2e = 1.4426950408889634f;
    Lse2 st;
    st.init();
    for (int ch = c_beg; ch < c_end; ++ch) {
        const int col0 = ch * kChunkCols;
        mma_chunk<HEAD_BF16>(a.Wt, a.V, a.r, col0, nrows > 32, sA, sAf, sZ);
        if (live) {
            // the state's children that fall in this thread's 32 columns: their conditional
            // logits, the same fp32 values that enter the log-sum-exp
            const int cb = col0 + 32 * q;
            for (int i = 0; i < a.M; ++i) {
                const int off = sTgt[row][i] - cb;
                if (off >= 0 && off < 32)
                    a.zc[(size_t)(g0 + row) * a.M + i] = sZ[row * kZStride + 32 * q + off] + flash_logit(a, lb + cb + off);
            }
            float m = -INFINITY;
            float zv[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int c = col0 + 32 * q + i;
                const float z = c < a.V ? (sZ[row * kZStride + 32 * q + i] + flash_logit(a, lb + c)) * kLog2e
                                        : -INFINITY;
                zv[i] = z;
                m = fmaxf(m, z);
            }
            float s = 0.0f;
            if (m != -INFINITY)
#pragma unroll
                for (int i = 0; i < 32; ++i) s += exp2f(zv[i] - m);
            st.merge(m, s);
        }
        __syncthreads();  // sZ is rewritten by the next chunk
    }
    st.merge_xor(1);
    st.merge_xor(2);
    if (live && q == 0) a.lsep[(size_t)(g0 + row) * a.SP + split] = make_float2(st.m, st.s);
}

// ---- final selection and emission ------------------------------------------------------------
struct FlashSel {
    int32_t set[kMaxB][kMaxK];
    float lse2[kFlashMaxStates];
    uint8_t rslot[kFlashMaxStates][kMaxK];  // children of a state in sibling order: slots of S_j
    float cy2[kFlashMaxStates][kMaxK];      // their conditional logits (log2 units)
    // the select pool: kept nodes first, then one level's candidates
    uint64_t pkey[kFlashPool];
    int32_t ptok[kFlashPool];
    int16_t pstate[kFlashPool];  // the node's own state (-1 at depth B)
    int16_t pfi[kFlashPool];     // its index in the frontier of the level after its own
    float plogq[kFlashPool];
    // kept nodes, sorted by key descending
    uint64_t kkey[kMaxNcap];
    int32_t ktok[kMaxNcap];
    int16_t kstate[kMaxNcap];
    int16_t kfi[kMaxNcap];
    float klogq[kMaxNcap];
    int16_t front[kMaxNcap];  // frontier index -> kept index
    int16_t canon[kMaxNcap];  // kept index -> canonical position
    int16_t korder[kMaxNcap]; // canonical position -> kept index
    int16_t cpar[kMaxNcap];   // canonical position -> parent's canonical position
    uint64_t mask[kMaxNcap];  // canonical position -> ancestor mask
    int nkept, nfront, nvalid;
};

// One workgroup per request.  Reading of the final selection: the parent-conditioned tree's
// rule (survival from the calibration table, s < tau dropped, global order survival desc,
// depth asc, sibling-rank path asc, budget N) applied level by level; because survival
// never increases along a path this equals best-first over the lattice.
__global__ __launch_bounds__(kFlashSelThreads) void k_flash_select(FlashArgs a) {
    __shared__ FlashSel sm;
    const int req = blockIdx.x, tid = threadIdx.x;
    const int M = a.M, B = a.B, NS = a.NS, Ncap = a.Ncap;
    const int root = a.root_token[req];
    const bool bad_root = root < 0 || root >= a.V;
    int nb = a.n_budget[req];
    int status = bad_root ? DT_REQ_BAD_ROOT : 0;
    if (nb < 0 || nb > Ncap) {
        status |= DT_REQ_BUDGET_CLAMPED;
        nb = nb < 0 ? 0 : Ncap;
    }
    const float tau = a.tau[req];
    constexpr float kLn2 = 0.6931471805599453f, kLog2e = 1.4426950408889634f;
    for (int i = tid; i < B * M; i += kFlashSelThreads)
        sm.set[i / M][i % M] = a.sets[((size_t)req * B + i / M) * M + i % M];
    if (tid == 0) sm.nkept = 0;
    __syncthreads();
    if (!bad_root) {
        // log-sum-exp of every state: its splits' records combined, P threads a state
        const int P = NS <= kFlashSelThreads / 4 ? 4 : 1;
        for (int w = tid; w < ((NS * P + kFlashSelThreads - 1) / kFlashSelThreads) * kFlashSelThreads; w += kFlashSelThreads) {
            const int s = w / P, part = w % P;
            Lse2 st;
            st.init();
            if (s < NS) {
                const float2* rec = a.lsep + (size_t)(req * NS + s) * a.SP;
                for (int p = part * 16; p < a.SP; p += 16 * P) {
                    float2 v[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) v[u] = p + u < a.SP ? rec[p + u] : make_float2(-INFINITY, 0.0f);
#pragma unroll
                    for (int u = 0; u < 16; ++u) st.merge(v[u].x, v[u].y);
                }
            }
            if (P == 4) {
                st.merge_xor(1);
                st.merge_xor(2);
            }
            if (s < NS && part == 0) sm.lse2[s] = st.m + log2f(st.s);
        }
        // conditional logits of every state's children (written by the state pass)
        for (int w = tid; w < NS * M; w += kFlashSelThreads)
            sm.cy2[w / M][w % M] = a.zc[(size_t)(req * NS) * M + w] * kLog2e;
        __syncthreads();
        // sibling order of every state: conditional logit desc, token asc
        for (int s = tid; s < NS; s += kFlashSelThreads) {
            const int j = s == 0 ? 0 : 1 + (s - 1) / M;
            float y[kMaxK];
            int sl[kMaxK];
            for (int i = 0; i < M; ++i) {
                y[i] = sm.cy2[s][i];
                sl[i] = i;
            }
            for (int i = 1; i < M; ++i) {
                const float xy = y[i];
                const int xs = sl[i];
                int b = i - 1;
                while (b >= 0 && (y[b] < xy || (y[b] == xy && sm.set[j][sl[b]] > sm.set[j][xs]))) {
                    y[b + 1] = y[b];
                    sl[b + 1] = sl[b];
                    --b;
                }
                y[b + 1] = xy;
                sl[b + 1] = xs;
            }
            for (int i = 0; i < M; ++i) {
                sm.cy2[s][i] = y[i];
                sm.rslot[s][i] = (uint8_t)sl[i];
            }
        }
        __syncthreads();
        // level loop
        for (int d = 1; d <= B; ++d) {
            // frontier: the kept nodes of depth d - 1 (the root at d = 1), canonical order
            if (d == 1) {
                if (tid == 0) {
                    sm.nfront = 1;
                    sm.front[0] = -1;
                }
            } else {
                const bool fr = tid < sm.nkept && low_depth((uint32_t)sm.kkey[tid]) == d - 1;
                if (fr) {
                    const uint32_t lo = (uint32_t)sm.kkey[tid];
                    int fi = 0;
                    for (int e = 0; e < sm.nkept; ++e) {
                        const uint32_t le = (uint32_t)sm.kkey[e];
                        fi += (low_depth(le) == d - 1) & (le > lo);
                    }
                    sm.kfi[tid] = (int16_t)fi;
                    sm.front[fi] = (int16_t)tid;
                }
                const int nf = __syncthreads_count(fr);
                if (tid == 0) sm.nfront = nf;
            }
            if (tid == 0) sm.nvalid = 0;
            __syncthreads();
            const int nf = sm.nfront, nk = sm.nkept;
            if (nf == 0) break;
            // pool: the kept nodes, then every frontier node's M children
            for (int e = tid; e < nk; e += kFlashSelThreads) {
                sm.pkey[e] = sm.kkey[e];
                sm.ptok[e] = sm.ktok[e];
                sm.pstate[e] = sm.kstate[e];
                sm.pfi[e] = sm.kfi[e];
                sm.plogq[e] = sm.klogq[e];
            }
            for (int w = tid; w < nf * M; w += kFlashSelThreads) {
                const int fi = w / M, i = w % M;
                const int ke = sm.front[fi];
                const int ps = ke < 0 ? 0 : sm.kstate[ke];
                const float psurv = ke < 0 ? 1.0f : key_surv(sm.kkey[ke]);
                const float l2 = sm.cy2[ps][i] - sm.lse2[ps];
                const float q = exp2f(l2);
                const int bin = min(15, max(0, (int)floorf(16.0f * q)));
                const float sv = psurv * a.cal[bin];
                const int slot = sm.rslot[ps][i];
                const int e = nk + w;
                sm.pkey[e] = sv < tau ? 0ull : make_key(sv, d, fi, i);
                sm.ptok[e] = sm.set[d - 1][slot];
                sm.pstate[e] = (int16_t)(d < B ? 1 + (d - 1) * M + slot : -1);
                sm.pfi[e] = 0;
                sm.plogq[e] = l2 * kLn2;
            }
            __syncthreads();
            // keep the nb best: rank = number of larger keys (valid keys are distinct)
            const int np = nk + nf * M;
            int nv = 0;
            for (int e = tid; e < np; e += kFlashSelThreads) {
                const uint64_t ke = sm.pkey[e];
                if (ke == 0) continue;
                ++nv;
                int rank = 0;
                for (int f = 0; f < np; ++f) rank += sm.pkey[f] > ke;
                if (rank < nb) {
                    sm.kkey[rank] = ke;
                    sm.ktok[rank] = sm.ptok[e];
                    sm.kstate[rank] = sm.pstate[e];
                    sm.kfi[rank] = sm.pfi[e];
                    sm.klogq[rank] = sm.plogq[e];
                }
            }
            if (nv) atomicAdd(&sm.nvalid, nv);
            __syncthreads();
            if (tid == 0) sm.nkept = min(nb, sm.nvalid);
            __syncthreads();
        }
    }
    // emission in canonical order: depth asc, then (parent's frontier index, sibling rank)
    const int n = sm.nkept;
    if (tid < n) {
        const uint32_t lo = (uint32_t)sm.kkey[tid];
        const int dd = low_depth(lo);
        int pos = 0;
        for (int e = 0; e < n; ++e) {
            const uint32_t le = (uint32_t)sm.kkey[e];
            const int de = low_depth(le);
            pos += (de < dd) | ((de == dd) & (le > lo));
        }
        sm.canon[tid] = (int16_t)pos;
        sm.korder[pos] = (int16_t)tid;
    }
    __syncthreads();
    if (tid < n) {
        const int pos = sm.canon[tid];
        const uint32_t lo = (uint32_t)sm.kkey[tid];
        const int dd = low_depth(lo), pfi = low_fi(lo);
        int par = -1;
        if (dd > 1)
            for (int e = 0; e < n; ++e)
                if (low_depth((uint32_t)sm.kkey[e]) == dd - 1 && sm.kfi[e] == pfi) par = sm.canon[e];
        sm.cpar[pos] = (int16_t)par;
    }
    __syncthreads();
    // ancestor mask: the node's own bit and its ancestors' (each node walks its own path)
    if (tid < n) {
        uint64_t m = 0;
        for (int p = tid; p >= 0; p = sm.cpar[p]) m |= 1ull << p;
        sm.mask[tid] = m;
    }
    __syncthreads();
    const size_t base = (size_t)req * Ncap;
    for (int i = tid; i < Ncap; i += kFlashSelThreads) {
        if (i < n) {
            const int e = sm.korder[i];
            a.out.token[base + i] = sm.ktok[e];
            a.out.parent[base + i] = sm.cpar[i];
            a.out.depth[base + i] = (uint8_t)low_depth((uint32_t)sm.kkey[e]);
            a.out.anc_mask[base + i] = sm.mask[i];
            a.out.surv[base + i] = key_surv(sm.kkey[e]);
            a.out.logq[base + i] = sm.klogq[e];
        } else {
            a.out.token[base + i] = -1;
            a.out.parent[base + i] = -2;
            a.out.depth[base + i] = 0;
            a.out.anc_mask[base + i] = 0ull;
            a.out.surv[base + i] = 0.0f;
            a.out.logq[base + i] = 0.0f;
        }
    }
    // candidate rows: row 0 the root's children, row i + 1 node i's (none at depth B)
    const size_t cb = (size_t)req * (Ncap + 1) * M;
    for (int w = tid; w < (Ncap + 1) * M; w += kFlashSelThreads) {
        const int row = w / M, i = w % M;
        int v = -1;
        if (!bad_root) {
            if (row == 0) {
                v = sm.set[0][sm.rslot[0][i]];
            } else if (row - 1 < n) {
                const int e = sm.korder[row - 1];
                const int st = sm.kstate[e];
                const int dd = low_depth((uint32_t)sm.kkey[e]);
                if (st >= 0) v = sm.set[dd][sm.rslot[st][i]];
            }
        }
        a.out.cand[cb + w] = v;
    }
    if (tid == 0) {
        a.out.n_nodes[req] = n;
        a.out.status[req] = status;
        if (a.out.n_expand) {
            int ne = bad_root ? 0 : 1;
            for (int e = 0; e < n; ++e) ne += sm.kstate[e] >= 0;
            a.out.n_expand[req] = ne;
        }
    }
}

// ---- host side ------------------------------------------------------------------------------
FlashPlan flash_plan(const dt_params* p) {
    FlashPlan pl{};
    pl.M = p->k;
    pl.NS = 1 + (p->B - 1) * p->k;
    pl.T = (p->R * pl.NS + kTileRows - 1) / kTileRows;
    const int chunks = (p->V + kChunkCols - 1) / kChunkCols;
    int sp = (512 + pl.T - 1) / pl.T;
    sp = sp < 1 ? 1 : (sp > 256 ? 256 : sp);
    pl.SP = sp > chunks ? chunks : sp;
    const size_t sets = (size_t)p->R * p->B * p->k * sizeof(int32_t);
    pl.sets_bytes = (sets + 255) & ~(size_t)255;
    const size_t lsep = (size_t)p->R * pl.NS * pl.SP * sizeof(float2);
    pl.zc_off = pl.sets_bytes + ((lsep + 255) & ~(size_t)255);
    const size_t zc = (size_t)p->R * pl.NS * p->k * sizeof(float);
    pl.setp_off = pl.zc_off + ((zc + 255) & ~(size_t)255);
    const int rows = p->R * p->B;
    int parts = (512 + rows - 1) / rows;
    pl.P = parts < 1 ? 1 : (parts > 32 ? 32 : parts);
    pl.total = pl.setp_off + (((size_t)rows * pl.P * kMaxK * sizeof(uint64_t) + 255) & ~(size_t)255);
    return pl;
}

hipError_t launch_build_flash(const dt_params* p, const FlashPlan& pl, const void* L,
                              const void* U, const void* Wt, const int32_t* root_token,
                              const int32_t* n_budget, const float* tau, const dt_tree* out,
                              char* ws, hipStream_t st) {
    FlashArgs a{};
    a.L = L;
    a.U = U;
    a.Wt = Wt;
    a.root_token = root_token;
    a.n_budget = n_budget;
    a.tau = tau;
    a.sets = (int32_t*)ws;
    a.lsep = (float2*)(ws + pl.sets_bytes);
    a.zc = (float*)(ws + pl.zc_off);
    a.setp = (uint64_t*)(ws + pl.setp_off);
    a.P = pl.P;
    a.out = *out;
    a.R = p->R;
    a.B = p->B;
    a.M = pl.M;
    a.V = p->V;
    a.r = p->r;
    a.Ncap = p->Ncap;
    a.NS = pl.NS;
    a.SP = pl.SP;
    a.T = pl.T;
    a.logits_bf16 = p->logits_dtype == DT_BF16;
    for (int i = 0; i < 16; ++i) a.cal[i] = p->cal[i];
    k_flash_sets<<<p->R * p->B * pl.P, kFlashSetThreads, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_flash_sets_merge<<<p->R * p->B, 64, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = a.T * ((a.SP + 7) / 8) * 8;
    if (p->head_dtype == DT_BF16)
        k_flash_lse<true><<<grid, 256, 0, st>>>(a);
    else
        k_flash_lse<false><<<grid, 256, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_flash_select<<<p->R, kFlashSelThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace dt
