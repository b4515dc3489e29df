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
    int lvec;  // bf16 logits, V a multiple of 8, 16-byte aligned L: 16-byte loads of L rows
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
__device__ __forceinline__ void flash_offer(TopK<kMaxK>& top, float v, int c, uint64_t bound = 0) {
    const uint64_t e = pack_entry(v, c);
    const uint64_t kth = top.k[kMaxK - 1];
    if (e > (kth > bound ? kth : bound)) top.push(e, 0.0f);
}

// The largest last entry of the wavefront's lists: a lane whose list ends there holds
// kMaxK entries at least as large, so no element below it can reach the part's top kMaxK
// (entries are unique: each packs its own token).  Offering against it keeps the lanes of a
// wavefront from taking the insertion branch in turn once their lists are warm.
__device__ __forceinline__ uint64_t flash_wave_bound(const TopK<kMaxK>& top) {
    uint64_t k = top.k[kMaxK - 1];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, off), hi = __shfl_xor((uint32_t)(k >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    return k;
}

__global__ __launch_bounds__(kFlashSetThreads) void k_flash_sets(FlashArgs a) {
    __shared__ uint64_t sk[kFlashSetThreads / 64][kMaxK];
    const int row = blockIdx.x / a.P, part = blockIdx.x % a.P;  // row = req * B + j
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t base = (size_t)row * a.V;
    TopK<kMaxK> top;
    top.init();
    if (a.lvec) {
        const uint4* p = (const uint4*)((const uint16_t*)a.L + base);
        const int ng = a.V / 8;
        const int g_beg = (int)((long)part * ng / a.P), g_end = (int)((long)(part + 1) * ng / a.P);
        // four 16-byte loads in flight per thread (groups past the part reload its first);
        // the trip count is the same for every lane (the bound is a wavefront reduction)
        constexpr int kU = 4;
        uint64_t bound = 0;
        for (int gb = g_beg; gb < g_end; gb += kU * kFlashSetThreads) {
            const int g0 = gb + tid;
            uint4 w[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int g = g0 + u * kFlashSetThreads;
                w[u] = p[g < g_end ? g : g_beg];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int g = g0 + u * kFlashSetThreads;
                // the group's eight entries, a mask of those above the bound, then one
                // insertion per candidate (rare once the lists are warm)
                const uint32_t x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
                uint64_t e[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[2 * i] = pack_entry(bf16_lo(x[i]), 8 * g + 2 * i);
                    e[2 * i + 1] = pack_entry(bf16_hi(x[i]), 8 * g + 2 * i + 1);
                }
                const uint64_t kth = top.k[kMaxK - 1];
                const uint64_t thr = kth > bound ? kth : bound;
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) m |= (e[i] > thr) ? (1u << i) : 0u;
                m = g < g_end ? m : 0u;
                while (m != 0u) {
                    const int i = __builtin_ctz(m);
                    m &= m - 1u;
                    uint64_t v = e[0];
#pragma unroll
                    for (int q = 1; q < 8; ++q) v = q == i ? e[q] : v;
                    if (v > top.k[kMaxK - 1]) top.push(v, 0.0f);
                }
            }
            bound = flash_wave_bound(top);
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

// bf16 heads: the transposed block of the expansion (W as the MFMA A operand, the tile's U
// rows from LDS as B), so lane l holds state l % 32 (and 32 + l % 32) at 16 columns of each
// 32-column block and the online log-sum-exp runs on the accumulators; the block logits are
// the accumulators' initial values, so z = L + U.W leaves the MFMA directly.  Wavefront w
// takes the split's blocks w, w + 4, ...; the next block's W fragments and logits are loaded
// while the current block's epilogue runs.
constexpr int kFlashLseWaves = 4;
constexpr int kFlashTile = 128;  // states per workgroup of the bf16 state pass (4 MFMA row blocks)
static_assert(kFlashLseWaves * 64 == 256, "k_flash_lse runs 256 threads");

// Raw bf16 block logits of a lane's 16 columns (c0 + 8j + 4h + i), 16-byte-aligned rows only.
__device__ __forceinline__ void flash_lgroups(const FlashArgs& a, size_t lb, int c0, int h,
                                              uint2 (&g)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = c0 + 8 * j + 4 * h;
        g[j] = *(const uint2*)((const uint16_t*)a.L + lb + (c < a.V ? c : a.V - 4));
    }
}

// The accumulators' initial values: the block logits of the lane's columns (clamped into the
// row past V; those columns are masked in the epilogue).
__device__ __forceinline__ void flash_to_acc(const FlashArgs& a, const uint2 (&g)[4], size_t lb,
                                             int c0, int h, f32x16& acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (a.lvec) {
            acc[4 * j + 0] = bf16_lo(g[j].x);
            acc[4 * j + 1] = bf16_hi(g[j].x);
            acc[4 * j + 2] = bf16_lo(g[j].y);
            acc[4 * j + 3] = bf16_hi(g[j].y);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + 8 * j + 4 * h + i;
                acc[4 * j + i] = flash_logit(a, lb + (c < a.V ? c : a.V - 1));
            }
        }
    }
}

// One state's 16 values of a block: the conditional logits of its children that fall in
// these columns (the same fp32 values that enter the log-sum-exp), then the online
// log-sum-exp (log2 units).
__device__ __forceinline__ void flash_epi(const FlashArgs& a, f32x16& z, int c0, int h,
                                          const int* tgt, size_t zrow, Lse2& st) {
    if (c0 + kBlockCols > a.V) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (c0 + 8 * (e >> 2) + 4 * h + (e & 3) >= a.V) z[e] = -INFINITY;
    }
    for (int i = 0; i < a.M; ++i) {
        const int off = tgt[i] - c0;
        if (off >= 0 && off < kBlockCols && ((off >> 2) & 1) == h) {
            const int e = 4 * (off >> 3) + (off & 3);
            float v = z[0];
#pragma unroll
            for (int q = 1; q < 16; ++q) v = q == e ? z[q] : v;
            a.zc[zrow + i] = v;
        }
    }
    constexpr float kLog2e = 1.4426950408889634f;
    float zmax = z[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) zmax = fmaxf(zmax, z[e]);
    if (zmax == -INFINITY) return;
    const float cm = zmax * kLog2e;
    if (cm > st.m) {
        st.s = (st.m == -INFINITY) ? 0.0f : st.s * exp2f(st.m - cm);
        st.m = cm;
    }
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += exp2f(z[e] * kLog2e - st.m);
    st.s += ps;
}

__device__ __forceinline__ void flash_lse_blocks(const FlashArgs& a) {
    __shared__ __align__(16) uint16_t sA[kFlashTile * kAStride];
    __shared__ int sTok[kFlashTile];
    __shared__ size_t sLb[kFlashTile];
    __shared__ int sTgt[kFlashTile][kMaxK];
    __shared__ Lse2 sW[kFlashLseWaves][kFlashTile];
    const int b = blockIdx.x;
    const int idx = b >> 3;
    const int tile = idx % a.T;
    const int split = (idx / a.T) * 8 + (b & 7);
    if (split >= a.SP) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, p0 = lane & 31;
    const int rows_total = a.R * a.NS;
    const int g0 = tile * kFlashTile;
    const int nrows = min(kFlashTile, rows_total - g0);
    if (tid < kFlashTile) {
        int t = -1;
        size_t lb = 0;
        for (int i = 0; i < kMaxK; ++i) sTgt[tid][i] = -1;
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
    // the U rows of the tile's states, in two 64-row halves
    load_a_tile<true>(a.U, a.r, min(nrows, kTileRows), [&](int row) { return sTok[row]; }, sA, nullptr);
    load_a_tile<true>(a.U, a.r, max(nrows - kTileRows, 0), [&](int row) { return sTok[kTileRows + row]; },
                      sA + kTileRows * kAStride, nullptr);
    __syncthreads();
    const int NB = (a.V + kBlockCols - 1) / kBlockCols;
    const int b_beg = (int)((long)split * NB / a.SP), b_end = (int)((long)(split + 1) * NB / a.SP);
    // row block q (32 states: q * 32 + lane % 32) is live when the tile reaches it
    const int nq = (nrows + 31) >> 5;
    size_t lbq[4], zrq[4];
    bool liveq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = 32 * q + p0;
        lbq[q] = sLb[row];
        zrq[q] = (size_t)(g0 + row) * a.M;
        liveq[q] = row < nrows;
    }
    Lse2 st[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) st[q].init();
    // per block: row blocks 0-1, then 2-3 on the same W fragments (one accumulator pair
    // live at a time); the logits of the next pair and the next block are in flight while
    // the current pair's epilogue runs
    bf16x8 wf[16];
    uint2 la[2][4], lc[2][4];  // logits of row blocks 0-1 (this block), of 2-3
    int blk = b_beg + wave;
    if (blk < b_end) {
        load_wfrag(a.Wt, a.V, a.r, blk * kBlockCols, wf);
        if (a.lvec) {
            flash_lgroups(a, lbq[0], blk * kBlockCols, h, la[0]);
            if (nq > 1) flash_lgroups(a, lbq[1], blk * kBlockCols, h, la[1]);
        }
    }
    for (; blk < b_end; blk += kFlashLseWaves) {
        const int c0 = blk * kBlockCols;
        f32x16 acc0, acc1;
        flash_to_acc(a, la[0], lbq[0], c0, h, acc0);
        if (nq > 1) flash_to_acc(a, la[1], lbq[1], c0, h, acc1);
        mma_wfrag(wf, nq > 1, sA, acc0, acc1);
        if (nq > 2 && a.lvec) {
            flash_lgroups(a, lbq[2], c0, h, lc[0]);
            if (nq > 3) flash_lgroups(a, lbq[3], c0, h, lc[1]);
        }
        const bool more = blk + kFlashLseWaves < b_end;
        const int cn = c0 + kFlashLseWaves * kBlockCols;
        if (nq <= 2 && more) {
            load_wfrag(a.Wt, a.V, a.r, cn, wf);
            if (a.lvec) {
                flash_lgroups(a, lbq[0], cn, h, la[0]);
                if (nq > 1) flash_lgroups(a, lbq[1], cn, h, la[1]);
            }
        }
        if (liveq[0]) flash_epi(a, acc0, c0, h, sTgt[p0], zrq[0], st[0]);
        if (nq > 1 && liveq[1]) flash_epi(a, acc1, c0, h, sTgt[32 + p0], zrq[1], st[1]);
        if (nq > 2) {
            flash_to_acc(a, lc[0], lbq[2], c0, h, acc0);
            if (nq > 3) flash_to_acc(a, lc[1], lbq[3], c0, h, acc1);
            mma_wfrag(wf, nq > 3, sA + kTileRows * kAStride, acc0, acc1);
            if (more) {
                load_wfrag(a.Wt, a.V, a.r, cn, wf);
                if (a.lvec) {
                    flash_lgroups(a, lbq[0], cn, h, la[0]);
                    flash_lgroups(a, lbq[1], cn, h, la[1]);
                }
            }
            if (liveq[2]) flash_epi(a, acc0, c0, h, sTgt[64 + p0], zrq[2], st[2]);
            if (nq > 3 && liveq[3]) flash_epi(a, acc1, c0, h, sTgt[96 + p0], zrq[3], st[3]);
        }
    }
    // lanes l and l ^ 32 hold the same state; then the wavefronts' blocks
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        st[q].merge_xor(32);
        if (h == 0) sW[wave][32 * q + p0] = st[q];
    }
    __syncthreads();
    if (tid < nrows) {
        Lse2 t;
        t.init();
#pragma unroll
        for (int w = 0; w < kFlashLseWaves; ++w) t.merge(sW[w][tid].m, sW[w][tid].s);
        a.lsep[(size_t)(g0 + tid) * a.SP + split] = make_float2(t.m, t.s);
    }
}

// float32 heads: 64 x 128 chunks through an LDS tile (thread: state tid / 4, 32 columns of
// each chunk).
template <bool HEAD_BF16>
__device__ __forceinline__ void flash_lse_chunks(const FlashArgs& a) {
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
            if (a.lvec && cb + 32 <= a.V) {
                // the 32 block logits in four 16-byte loads
                const uint4* lp = (const uint4*)((const uint16_t*)a.L + lb + cb);
                uint4 lw[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) lw[g] = lp[g];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t w4[4] = {lw[g].x, lw[g].y, lw[g].z, lw[g].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 8 * g + 2 * e;
                        zv[i] = (sZ[row * kZStride + 32 * q + i] + bf16_lo(w4[e])) * kLog2e;
                        zv[i + 1] = (sZ[row * kZStride + 32 * q + i + 1] + bf16_hi(w4[e])) * kLog2e;
                    }
                }
#pragma unroll
                for (int i = 0; i < 32; ++i) m = fmaxf(m, zv[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const int c = cb + i;
                    const float z = c < a.V ? (sZ[row * kZStride + 32 * q + i] + flash_logit(a, lb + c)) * kLog2e
                                            : -INFINITY;
                    zv[i] = z;
                    m = fmaxf(m, z);
                }
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

template <bool HEAD_BF16>
__global__ __launch_bounds__(256) void k_flash_lse(FlashArgs a) {
    if constexpr (HEAD_BF16)
        flash_lse_blocks(a);
    else
        flash_lse_chunks<false>(a);
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
    // state tiles: 128 states for bf16 heads (k_flash_lse's transposed blocks), 64 for float32
    const int tile = p->head_dtype == DT_BF16 ? kFlashTile : kTileRows;
    pl.T = (p->R * pl.NS + tile - 1) / tile;
    const int chunks = (p->V + kChunkCols - 1) / kChunkCols;
    // about 512 workgroups, and a multiple of 8 splits so that every XCD takes the same
    // number (workgroup b runs on XCD b % 8; with 9 splits one XCD did twice the work)
    int sp = (512 + pl.T - 1) / pl.T;
    sp = sp < 8 ? 8 : (sp > 256 ? 256 : sp & ~7);
    pl.SP = sp > chunks ? chunks : sp;
    const size_t sets = (size_t)p->R * p->B * p->k * sizeof(int32_t);
    pl.sets_bytes = (sets + 255) & ~(size_t)255;
    const size_t lsep = (size_t)p->R * pl.NS * pl.SP * sizeof(float2);
    pl.zc_off = pl.sets_bytes + ((lsep + 255) & ~(size_t)255);
    const size_t zc = (size_t)p->R * pl.NS * p->k * sizeof(float);
    pl.setp_off = pl.zc_off + ((zc + 255) & ~(size_t)255);
    const int rows = p->R * p->B;
    // about 2048 workgroups for stage 1 (a 1024-row batch scanned whole rows per workgroup
    // at a quarter of the chip's bandwidth)
    int parts = (2048 + rows - 1) / rows;
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
    a.lvec = a.logits_bf16 && (p->V & 7) == 0 && ((uintptr_t)L & 15) == 0;
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
