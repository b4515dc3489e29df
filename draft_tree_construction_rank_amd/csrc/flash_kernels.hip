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
// Kernels: k_flash_sets (top-M of every block row: P workgroups a row, one list per part)
// and k_flash_sets_merge (a row's P lists), k_flash_lse (log-sum-exp of every state over
// vocabulary splits: a (state tile, split) workgroup streams the split's W columns through
// MFMA with the block logits as the accumulators' initial values, keeps an online
// log2-sum-exp per state and takes the children's conditional logits from the same
// accumulators), k_flash_select (one workgroup a request: the split log-sum-exps combined,
// sibling order, then the level-synchronous select over pruned pools and the emission, all
// in LDS).
#include <hip/hip_runtime.h>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {

constexpr int kFlashSetThreads = 256;
constexpr int kFlashSelThreads = 512;
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
// packed (logit, token) entries (the smallest of 1, 2, 4, 8 that holds M) goes to the
// workspace and a second kernel merges a row's P lists.  An entry enters a thread's list only if it beats the list's last entry.  For bf16
// logits read 8 at a time, each wavefront first takes a bound from its first loads (the
// M-th largest of its lanes' maxima), and a group of 8 whose largest value is below the
// bound or below a full list's last value is passed over with one float compare.
template <int KT>
__device__ __forceinline__ void flash_offer(TopK<KT>& top, float v, int c) {
    const uint64_t e = pack_entry(v, c);
    if (e > top.k[KT - 1]) top.push(e, 0.0f);
}

// A value b such that at least m lanes of the wavefront hold v >= b (-inf if fewer than m
// lanes hold a value): every one of those m lanes has an element of the row at least b, so
// the row's m-th largest value is too, and no element below b can be among its top m.
__device__ __forceinline__ float wave_mth_largest(float v, int m) {
    float b = -INFINITY;
    // each round takes the largest remaining value and the lanes holding it (at most 64)
    for (int r = 0; r < 64 && m > 0; ++r) {
        float t = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) t = fmaxf(t, __shfl_xor(t, off));
        const int c = __popcll(__ballot(v >= t));
        if (c == 0) {  // no ordered value left
            b = -INFINITY;
            break;
        }
        b = t;
        m -= c;
        if (t == -INFINITY) break;
        v = v >= t ? -INFINITY : v;
    }
    return m > 0 ? -INFINITY : b;
}

// KT = the list length for M (kt_for(M) <= kMaxK); a part's list goes out as kMaxK entries,
// zero-padded (zero is below every real entry).
template <int KT>
__global__ __launch_bounds__(kFlashSetThreads) void k_flash_sets(FlashArgs a) {
    __shared__ uint64_t sk[kFlashSetThreads / 64][KT];
    const int row = blockIdx.x / a.P, part = blockIdx.x % a.P;  // row = req * B + j
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t base = (size_t)row * a.V;
    TopK<KT> top;
    top.init();
    if (a.lvec) {
        const uint4* p = (const uint4*)((const uint16_t*)a.L + base);
        const int ng = a.V / 8;
        const int g_beg = (int)((long)part * ng / a.P), g_end = (int)((long)(part + 1) * ng / a.P);
        // four 16-byte loads in flight per thread (groups past the part reload its first);
        // the trip count is the same for every lane (the bound is a wavefront reduction)
        constexpr int kU = 4;
        float bound = -INFINITY;
        for (int gb = g_beg; gb < g_end; gb += kU * kFlashSetThreads) {
            const int g0 = gb + tid;
            uint4 w[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int g = g0 + u * kFlashSetThreads;
                w[u] = p[g < g_end ? g : g_beg];
            }
            float f[kU][8], gmax[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const uint32_t x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f[u][2 * i] = bf16_lo(x[i]);
                    f[u][2 * i + 1] = bf16_hi(x[i]);
                }
                const bool in = g0 + u * kFlashSetThreads < g_end;
                gmax[u] = in ? fmaxf(fmaxf(fmaxf(f[u][0], f[u][1]), fmaxf(f[u][2], f[u][3])),
                                     fmaxf(fmaxf(f[u][4], f[u][5]), fmaxf(f[u][6], f[u][7])))
                             : -INFINITY;
            }
            // first step: the bound from the M-th largest lane maximum, so that the lists
            // start near the row's top values instead of taking every early element
            if (gb == g_beg)
                bound = wave_mth_largest(fmaxf(fmaxf(gmax[0], gmax[1]), fmaxf(gmax[2], gmax[3])), a.M);
            // the threshold's value: a group whose largest value is below it holds no entry
            // above the threshold (a tie in value may still win on its token: exact test)
            const uint64_t kth = top.k[KT - 1];
            const float thrv = kth == 0 ? bound : fmaxf(bound, entry_key(kth));
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int g = g0 + u * kFlashSetThreads;
                if (g < g_end && gmax[u] >= thrv) {
                    // the group's entries at or above the threshold's value, one insertion
                    // each (an entry enters only if it beats the list's last)
                    uint32_t m = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) m |= (f[u][i] >= thrv) ? (1u << i) : 0u;
                    while (m != 0u) {
                        const int i = __builtin_ctz(m);
                        m &= m - 1u;
                        float v = f[u][0];
#pragma unroll
                        for (int q = 1; q < 8; ++q) v = q == i ? f[u][q] : v;
                        const uint64_t e = pack_entry(v, 8 * g + i);
                        if (e > top.k[KT - 1]) top.push(e, 0.0f);
                    }
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
        for (int i = 0; i < KT; ++i) sk[wave][i] = top.k[i];
    __syncthreads();
    if (wave == 0) {
        TopK<KT> t;
        t.init();
        if (lane < kFlashSetThreads / 64)
#pragma unroll
            for (int i = 0; i < KT; ++i) t.k[i] = sk[lane][i];
#pragma unroll
        for (int off = 1; off < kFlashSetThreads / 64; off <<= 1) t.merge_xor(off);
        if (lane < kMaxK) {
            uint64_t v = 0;
#pragma unroll
            for (int i = 0; i < KT; ++i) v = lane == i ? t.k[i] : v;
            a.setp[((size_t)row * a.P + part) * kMaxK + lane] = v;
        }
    }
}

// One wavefront per row merges the row's P part lists into its set S_j (M tokens); a part
// list's entries past KT are its zero padding.
template <int KT>
__global__ __launch_bounds__(64) void k_flash_sets_merge(FlashArgs a) {
    const int row = blockIdx.x, lane = threadIdx.x;
    TopK<KT> t;
    t.init();
    if (lane < a.P)
#pragma unroll
        for (int i = 0; i < KT; ++i) t.k[i] = a.setp[((size_t)row * a.P + lane) * kMaxK + i];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) t.merge_xor(off);
    if (lane == 0)
#pragma unroll
        for (int i = 0; i < KT; ++i)
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

// Raw bf16 block logits for a lane (16-byte-aligned rows only): lane half h loads the 16
// columns c0 + 16h .. as two 16-byte pieces, g = (piece 0, piece 1); a piece past V (pieces
// are whole: V is a multiple of 8) reloads the row's last one, masked in the epilogue.  The
// lane needs columns c0 + 8j + 4h + i instead: flash_to_acc swaps halves with lane l ^ 32 at
// use, so that the loads stay in flight until then.  (Two 16-byte loads per lane instead of
// four 8-byte ones: each load instruction touches every state's row once.)
__device__ __forceinline__ void flash_lgroups(const FlashArgs& a, size_t lb, int c0, int h,
                                              uint2 (&g)[4]) {
    const uint16_t* row = (const uint16_t*)a.L + lb;
    const int s0 = c0 + 16 * h, s1 = s0 + 8;
    const uint4 x0 = *(const uint4*)(row + (s0 < a.V ? s0 : a.V - 8));
    const uint4 x1 = *(const uint4*)(row + (s1 < a.V ? s1 : a.V - 8));
    g[0] = make_uint2(x0.x, x0.y);
    g[1] = make_uint2(x0.z, x0.w);
    g[2] = make_uint2(x1.x, x1.y);
    g[3] = make_uint2(x1.z, x1.w);
}

// The W fragments of a block; for r = 256 one row address per lane and the sixteen k-steps
// at immediate offsets (the general loader clamps and addresses every step).
__device__ __forceinline__ void flash_wfrag(const FlashArgs& a, int c0, bf16x8 (&wf)[16]) {
    if (a.r != 256) {
        load_wfrag(a.Wt, a.V, a.r, c0, wf);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int col = c0 + (lane & 31);
    const uint4* p = (const uint4*)((const uint16_t*)a.Wt + (size_t)(col < a.V ? col : a.V - 1) * 256) +
                     (lane >> 5);
#pragma unroll
    for (int s = 0; s < 16; ++s) wf[s] = __builtin_bit_cast(bf16x8, p[2 * s]);
}

// The accumulators' initial values: the block logits of the lane's columns (clamped into the
// row past V; those columns are masked in the epilogue).
template <bool LVEC>
__device__ __forceinline__ void flash_to_acc(const FlashArgs& a, const uint2 (&g)[4], size_t lb,
                                             int c0, int h, f32x16& acc) {
    if constexpr (LVEC) {
        // g holds groups 2h and 2h + 1 whole (flash_lgroups: g[2pc + e] is half e, columns
        // 4e .. 4e + 3, of piece pc): keep this lane's half h of each piece, send the other
        // half, and take the partner's half h of groups 2(1 - h) and 2(1 - h) + 1
        const uint32_t keep[4] = {h ? g[1].x : g[0].x, h ? g[1].y : g[0].y, h ? g[3].x : g[2].x,
                                  h ? g[3].y : g[2].y};
        const uint32_t send[4] = {h ? g[0].x : g[1].x, h ? g[0].y : g[1].y, h ? g[2].x : g[3].x,
                                  h ? g[2].y : g[3].y};
        uint32_t recv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // results: [0] lane l % 32's value, [1] lane l % 32 + 32's
            const auto sw = __builtin_amdgcn_permlane32_swap(send[i], send[i], false, false);
            recv[i] = h ? sw[0] : sw[1];
        }
        // group j's two dwords: from the piece of group j held by half j / 2
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool mine = (j >> 1) == h;
            const int pc = j & 1;  // which piece of the holder
            w[2 * j] = mine ? keep[2 * pc] : recv[2 * pc];
            w[2 * j + 1] = mine ? keep[2 * pc + 1] : recv[2 * pc + 1];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[4 * j + 0] = bf16_lo(w[2 * j]);
            acc[4 * j + 1] = bf16_hi(w[2 * j]);
            acc[4 * j + 2] = bf16_lo(w[2 * j + 1]);
            acc[4 * j + 3] = bf16_hi(w[2 * j + 1]);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        {
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
// log-sum-exp (log2 units).  ntgt is the state's smallest child column not yet passed by
// this wavefront's blocks (they come in increasing order), so most blocks test it alone.
__device__ __forceinline__ void flash_epi(const FlashArgs& a, f32x16& z, int c0, int h,
                                          const int* tgt, size_t zrow, int& ntgt, Lse2& st) {
    if (c0 + kBlockCols > a.V) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (c0 + 8 * (e >> 2) + 4 * h + (e & 3) >= a.V) z[e] = -INFINITY;
    }
    if (ntgt < c0 + kBlockCols) {
        int nx = 0x7FFFFFFF;
        for (int i = 0; i < a.M; ++i) {
            const int t = tgt[i], off = t - c0;
            if (off >= 0 && off < kBlockCols && ((off >> 2) & 1) == h) {
                const int e = 4 * (off >> 3) + (off & 3);
                float v = z[0];
#pragma unroll
                for (int q = 1; q < 16; ++q) v = q == e ? z[q] : v;
                a.zc[zrow + i] = v;
            }
            if (off >= kBlockCols) nx = min(nx, t);
        }
        ntgt = nx;
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
    // the hardware exp2 without exp2f's rescaling of tiny results: terms below 2^-126 of the
    // running maximum flush to zero, far below float32 resolution of the sum
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += __builtin_amdgcn_exp2f(z[e] * kLog2e - st.m);
    st.s += ps;
}

// LVEC: bf16 logits read 16 bytes at a time (a.lvec), fixed at compile time so that no
// per-group branch makes the compiler wait for every load in flight (the next block's
// fragments included) before it converts a group.
template <bool LVEC>
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
    int ntgt[4];  // per row block: the state's smallest child column not yet passed
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        st[q].init();
        int n = 0x7FFFFFFF;
        for (int i = 0; i < a.M; ++i) n = min(n, sTgt[32 * q + p0][i] < 0 ? n : sTgt[32 * q + p0][i]);
        ntgt[q] = n;
    }
    // per block: row blocks 0-1, then 2-3 on the same W fragments (one accumulator pair
    // live at a time); the logits of the next pair and the next block are in flight while
    // the current pair's epilogue runs
    bf16x8 wf[16];
    uint2 la[2][4], lc[2][4];  // logits of row blocks 0-1 (this block), of 2-3
    int blk = b_beg + wave;
    if (blk < b_end) {
        flash_wfrag(a, blk * kBlockCols, wf);
        if constexpr (LVEC) {
            flash_lgroups(a, lbq[0], blk * kBlockCols, h, la[0]);
            if (nq > 1) flash_lgroups(a, lbq[1], blk * kBlockCols, h, la[1]);
        }
    }
    for (; blk < b_end; blk += kFlashLseWaves) {
        const int c0 = blk * kBlockCols;
        f32x16 acc0, acc1;
        flash_to_acc<LVEC>(a, la[0], lbq[0], c0, h, acc0);
        if (nq > 1) flash_to_acc<LVEC>(a, la[1], lbq[1], c0, h, acc1);
        mma_wfrag(wf, nq > 1, sA, acc0, acc1);
        if (nq > 2 && LVEC) {
            flash_lgroups(a, lbq[2], c0, h, lc[0]);
            if (nq > 3) flash_lgroups(a, lbq[3], c0, h, lc[1]);
        }
        const bool more = blk + kFlashLseWaves < b_end;
        const int cn = c0 + kFlashLseWaves * kBlockCols;
        if (nq <= 2 && more) {
            flash_wfrag(a, cn, wf);
            if constexpr (LVEC) {
                flash_lgroups(a, lbq[0], cn, h, la[0]);
                if (nq > 1) flash_lgroups(a, lbq[1], cn, h, la[1]);
            }
        }
        if (liveq[0]) flash_epi(a, acc0, c0, h, sTgt[p0], zrq[0], ntgt[0], st[0]);
        if (nq > 1 && liveq[1]) flash_epi(a, acc1, c0, h, sTgt[32 + p0], zrq[1], ntgt[1], st[1]);
        if (nq > 2) {
            flash_to_acc<LVEC>(a, lc[0], lbq[2], c0, h, acc0);
            if (nq > 3) flash_to_acc<LVEC>(a, lc[1], lbq[3], c0, h, acc1);
            mma_wfrag(wf, nq > 3, sA + kTileRows * kAStride, acc0, acc1);
            if (more) {
                flash_wfrag(a, cn, wf);
                if constexpr (LVEC) {
                    flash_lgroups(a, lbq[0], cn, h, la[0]);
                    flash_lgroups(a, lbq[1], cn, h, la[1]);
                }
            }
            if (liveq[2]) flash_epi(a, acc0, c0, h, sTgt[64 + p0], zrq[2], ntgt[2], st[2]);
            if (nq > 3 && liveq[3]) flash_epi(a, acc1, c0, h, sTgt[96 + p0], zrq[3], ntgt[3], st[3]);
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
                for (int i = 0; i < 32; ++i) s += __builtin_amdgcn_exp2f(zv[i] - m);  // (as above)
            st.merge(m, s);
        }
        __syncthreads();  // sZ is rewritten by the next chunk
    }
    st.merge_xor(1);
    st.merge_xor(2);
    if (live && q == 0) a.lsep[(size_t)(g0 + row) * a.SP + split] = make_float2(st.m, st.s);
}

// LVEC (16-byte logit loads) is a separate kernel: one kernel with both paths needs more
// registers than two waves per SIMD allow.
template <bool HEAD_BF16, bool LVEC>
__global__ __launch_bounds__(256, 2) void k_flash_lse(FlashArgs a) {  // two workgroups per CU
    if constexpr (HEAD_BF16)
        flash_lse_blocks<LVEC>(a);
    else
        flash_lse_chunks<false>(a);
}

// ---- final selection and emission ------------------------------------------------------------
struct FlashSel {
    // the select pool's keys: kept nodes, then the level's surviving candidates (room for a
    // masked read of eight keys past the end)
    alignas(16) uint64_t pkey[kFlashPool + 8];
    alignas(16) uint64_t kkey[2][kMaxNcap];  // kept nodes by key desc (two buffers: one level's
                                             // input and output)
    // the candidates of a level kept at its end, as bits over their index w = (parent's
    // frontier index) M + sibling rank, which is their canonical order (by level parity)
    alignas(16) uint64_t cbits[2][kMaxNcap * kMaxK / 64];
    int16_t wpos[kMaxNcap * kMaxK];  // candidate index -> kept index at the end of its level
    int32_t ktok[2][kMaxNcap];
    int16_t kstate[2][kMaxNcap];  // the node's own state (-1 at depth B)
    int16_t kfi[2][kMaxNcap];     // its index in the frontier of the level after its own
    float klogq[2][kMaxNcap];
    // the level's surviving candidates, in pool order after the kept nodes
    int32_t ctok[kMaxNcap * kMaxK];
    int16_t cstate[kMaxNcap * kMaxK];
    float clogq[kMaxNcap * kMaxK];
    int32_t set[kMaxB][kMaxK];
    float cal[16];
    float lse2[kFlashMaxStates];
    uint8_t rslot[kFlashMaxStates][kMaxK];  // children of a state in sibling order: slots of S_j
    float cy2[kFlashMaxStates][kMaxK];      // their conditional logits (log2 units)
    float zraw[kFlashMaxStates * kMaxK];    // the same in set order, as the state pass wrote them
    int16_t pmap[kMaxB + 1][kMaxNcap];  // (depth, frontier index) -> canonical position
    int16_t korder[kMaxNcap];           // canonical position -> kept index
    int16_t cpar[kMaxNcap];             // canonical position -> parent's canonical position
    uint64_t mask[kMaxNcap];            // canonical position -> ancestor mask
    int ncand[2];                       // surviving candidates of a level (by level parity)
};

constexpr int kFlashBitWords = kMaxNcap * kMaxK / 64;
constexpr int kFlashZPer = (kFlashMaxStates * kMaxK + kFlashSelThreads - 1) / kFlashSelThreads;

// Set bits of the candidate bitmap below index w.
__device__ __forceinline__ int bits_below(const uint64_t (&bm)[kFlashBitWords], int w) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < kFlashBitWords; ++q) {
        const uint64_t m = q < (w >> 6) ? bm[q] : q == (w >> 6) ? bm[q] & ((1ull << (w & 63)) - 1ull) : 0ull;
        c += __popcll(m);
    }
    return c;
}

// Position of the n-th (from 0) set bit of m; m has more than n set bits.
__device__ __forceinline__ int nth_bit(uint64_t m, int n) {
    int pos = 0;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const int c = __popcll(m & ((1ull << s) - 1ull));
        if (n >= c) {
            n -= c;
            m >>= s;
            pos += s;
        }
    }
    return pos;
}

// Ranks of NO keys of this thread in the pool (number of larger pool keys): eight keys per
// step as four 16-byte LDS reads in flight, then the last fewer than eight masked by index.
template <int NO>
__device__ __forceinline__ void flash_rank(const uint64_t* pkey, int np, const uint64_t (&k)[NO],
                                           int (&r)[NO]) {
    const ulonglong2* p2 = (const ulonglong2*)pkey;
    const int n8 = np & ~7;
    for (int f = 0; f < n8 / 2; f += 4) {
        ulonglong2 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = p2[f + u];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int o = 0; o < NO; ++o) r[o] += (int)(x[u].x > k[o]) + (int)(x[u].y > k[o]);
    }
    ulonglong2 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = p2[n8 / 2 + u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int o = 0; o < NO; ++o)
            r[o] += (int)(n8 + 2 * u < np && x[u].x > k[o]) + (int)(n8 + 2 * u + 1 < np && x[u].y > k[o]);
}

// Position of the n-th (from 0) set bit of the candidate bitmap; it has more than n.
__device__ __forceinline__ int nth_bit_map(const uint64_t (&bm)[kFlashBitWords], int n) {
    int word = -1;
    uint64_t sel = 0;
#pragma unroll
    for (int q = 0; q < kFlashBitWords; ++q) {
        const int c = __popcll(bm[q]);
        if (word < 0) {
            if (n < c) {
                word = q;
                sel = bm[q];
            } else {
                n -= c;
            }
        }
    }
    return 64 * word + nth_bit(sel, n);
}

// Scatter of this thread's pool entries e = tid + kFlashSelThreads o that rank inside the
// budget into the output buffer of kept nodes.  A kept node of depth d - 1 takes its frontier index (its
// position in the level's frontier, which is in candidate-index order); a kept candidate
// starts with none and marks its index in the level's bitmap.
template <int NO>
__device__ __forceinline__ void flash_keep(FlashSel& sm, int cur, int nk, int np, int nb, int d,
                                           int M, const uint64_t (&bm)[kFlashBitWords], int tid) {
    uint64_t k[NO];
    int r[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) {
        const int e = tid + o * kFlashSelThreads;
        k[o] = e < np ? sm.pkey[e] : ~0ull;
        r[o] = 0;
    }
    flash_rank<NO>(sm.pkey, np, k, r);
    const int nxt = cur ^ 1;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
        const int e = tid + o * kFlashSelThreads;
        if (e >= np || r[o] >= nb) continue;
        const int rk = r[o];
        sm.kkey[nxt][rk] = k[o];
        const uint32_t lo = (uint32_t)k[o];
        const int w = low_fi(lo) * M + low_rank(lo);  // the node's index among its level's candidates
        if (e < nk) {
            const bool fr = low_depth(lo) == d - 1;
            sm.ktok[nxt][rk] = sm.ktok[cur][e];
            sm.kstate[nxt][rk] = sm.kstate[cur][e];
            sm.kfi[nxt][rk] = fr ? (int16_t)bits_below(bm, w) : sm.kfi[cur][e];
            sm.klogq[nxt][rk] = sm.klogq[cur][e];
        } else {
            const int c = e - nk;
            sm.ktok[nxt][rk] = sm.ctok[c];
            sm.kstate[nxt][rk] = sm.cstate[c];
            sm.kfi[nxt][rk] = 0;
            sm.klogq[nxt][rk] = sm.clogq[c];
            atomicOr((unsigned long long*)&sm.cbits[d & 1][w >> 6], 1ull << (w & 63));
            sm.wpos[w] = (int16_t)rk;
        }
    }
}

// One workgroup per request.  Reading of the final selection: the parent-conditioned tree's
// rule (survival from the calibration table, s < tau dropped, global order survival desc,
// depth asc, sibling-rank path asc, budget N) applied level by level; because survival
// never increases along a path this equals best-first over the lattice.  A candidate below
// the last of N kept keys cannot enter (N larger keys exist), so only the others join the
// level's pool.
__global__ __launch_bounds__(kFlashSelThreads) void k_flash_select(FlashArgs a) {
    __shared__ FlashSel sm;
    const int req = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
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
    // (every load of the set-up issued before the first is used: the token sets, the raw
    // child logits, the split records)
    const int nzc = NS * M;
    int sv = 0;
    if (tid < B * M) sv = a.sets[(size_t)req * B * M + tid];
    float zr[kFlashZPer];
#pragma unroll
    for (int u = 0; u < kFlashZPer; ++u) {
        const int w = tid + u * kFlashSelThreads;
        zr[u] = w < nzc ? a.zc[(size_t)req * nzc + w] : 0.0f;
    }
    if (tid < 16) sm.cal[tid] = a.cal[tid];
    if (tid < 2) sm.ncand[tid] = 0;
    if (tid < 2 * kFlashBitWords) sm.cbits[tid / kFlashBitWords][tid % kFlashBitWords] = 0ull;
    int cur = 0, nk = 0;
    if (!bad_root) {
        // every state's splits' log-sum-exp records combined: P threads a state, eight record
        // pairs a step with the next step's in flight
        int lp = 0;
        while (lp < 4 && (NS << (lp + 1)) <= kFlashSelThreads) ++lp;
        const int P = 1 << lp;
        for (int w0 = 0; w0 < NS * P; w0 += kFlashSelThreads) {
            const int w = w0 + tid, s = w >> lp, part = w & (P - 1);
            Lse2 st;
            st.init();
            if (s < NS) {
                const float2* rec = a.lsep + (size_t)(req * NS + s) * a.SP;
                if ((a.SP & 1) == 0) {
                    const float4* r4 = (const float4*)rec;
                    const int n2 = a.SP >> 1;
                    float4 v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int p = part + u * P;
                        v[u] = p < n2 ? r4[p] : make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
                    }
                    for (int p0 = part; p0 < n2; p0 += 8 * P) {
                        float4 nv[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int p = p0 + (8 + u) * P;
                            nv[u] = p < n2 ? r4[p] : make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
                        }
                        float mx = -INFINITY;
#pragma unroll
                        for (int u = 0; u < 8; ++u) mx = fmaxf(mx, fmaxf(v[u].x, v[u].z));
                        if (mx != -INFINITY) {
                            float sum = 0.0f;
#pragma unroll
                            for (int u = 0; u < 8; ++u)
                                sum += v[u].y * exp2f(v[u].x - mx) + v[u].w * exp2f(v[u].z - mx);
                            st.merge(mx, sum);
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u) v[u] = nv[u];
                    }
                } else {
                    for (int p = part; p < a.SP; p += P) st.merge(rec[p].x, rec[p].y);
                }
            }
            for (int off = 1; off < P; off <<= 1) st.merge_xor(off);
            if (s < NS && part == 0) sm.lse2[s] = st.m + log2f(st.s);
        }
        if (tid < B * M) sm.set[tid / M][tid % M] = sv;
#pragma unroll
        for (int u = 0; u < kFlashZPer; ++u) {
            const int w = tid + u * kFlashSelThreads;
            if (w < nzc) sm.zraw[w] = zr[u] == zr[u] ? zr[u] * kLog2e : -INFINITY;  // (a total order)
        }
        __syncthreads();
        // sibling order of every state's children: conditional logit desc, token asc (each
        // child counts the siblings ahead of it)
        for (int w = tid; w < nzc; w += kFlashSelThreads) {
            const int s = w / M, i = w - s * M;
            const int j = s == 0 ? 0 : 1 + (s - 1) / M;
            const float y = sm.zraw[w];
            const int t = sm.set[j][i];
            int rank = 0;
            for (int q = 0; q < M; ++q) {
                const float yq = sm.zraw[s * M + q];
                rank += (int)(yq > y || (yq == y && sm.set[j][q] < t));
            }
            sm.cy2[s][rank] = y;
            sm.rslot[s][rank] = (uint8_t)i;
        }
        __syncthreads();
        // level loop: the frontier (kept nodes of depth d - 1, the root at d = 1) in
        // canonical order, its children scored, the survivors compacted behind the kept
        // nodes, every pool entry ranked and the best nb kept
        for (int d = 1; nb > 0 && d <= B; ++d) {
            uint64_t bm[kFlashBitWords];
            int nf = 1;
#pragma unroll
            for (int q = 0; q < kFlashBitWords; ++q) bm[q] = d > 1 ? sm.cbits[(d - 1) & 1][q] : 0ull;
            if (d > 1) {
                nf = 0;
#pragma unroll
                for (int q = 0; q < kFlashBitWords; ++q) nf += __popcll(bm[q]);
            }
            if (nf == 0) break;
            // the bitmap this level's keep fills (last read by the level before)
            if (tid < kFlashBitWords) sm.cbits[d & 1][tid] = 0ull;
            const uint64_t thr = nk == nb ? sm.kkey[cur][nb - 1] : 0ull;
            const int nc = nf * M;
            int* ncand = &sm.ncand[d & 1];
            for (int e = tid; e < nk; e += kFlashSelThreads) sm.pkey[e] = sm.kkey[cur][e];
            for (int w0 = 0; w0 < nc; w0 += kFlashSelThreads) {
                const int w = w0 + tid;
                uint64_t key = 0;
                int tok = 0, cst = -1;
                float lq = 0.0f;
                if (w < nc) {
                    const int fi = w / M, i = w - fi * M;
                    const int ke = d == 1 ? -1 : sm.wpos[nth_bit_map(bm, fi)];
                    const int ps = ke < 0 ? 0 : sm.kstate[cur][ke];
                    const float psurv = ke < 0 ? 1.0f : key_surv(sm.kkey[cur][ke]);
                    const float l2 = sm.cy2[ps][i] - sm.lse2[ps];
                    const float q = exp2f(l2);
                    const int bin = min(15, max(0, (int)floorf(16.0f * q)));
                    const float sv = psurv * sm.cal[bin];
                    const int slot = sm.rslot[ps][i];
                    key = sv < tau ? 0ull : make_key(sv, d, fi, i);
                    tok = sm.set[d - 1][slot];
                    cst = d < B ? 1 + (d - 1) * M + slot : -1;
                    lq = l2 * kLn2;
                }
                const bool keep = key > thr;
                const uint64_t bal = __ballot(keep);
                int base = 0;
                if (lane == 0 && bal) base = atomicAdd(ncand, __popcll(bal));
                base = __shfl(base, 0);
                if (keep) {
                    const int c = base + __popcll(bal & ((1ull << lane) - 1ull));
                    sm.pkey[nk + c] = key;
                    sm.ctok[c] = tok;
                    sm.cstate[c] = (int16_t)cst;
                    sm.clogq[c] = lq;
                }
            }
            __syncthreads();
            const int np = nk + *ncand;
            if (tid == 0) sm.ncand[(d + 1) & 1] = 0;
            static_assert(kFlashPool <= 2 * kFlashSelThreads, "at most two pool entries a thread");
            if (np <= kFlashSelThreads)
                flash_keep<1>(sm, cur, nk, np, nb, d, M, bm, tid);
            else
                flash_keep<2>(sm, cur, nk, np, nb, d, M, bm, tid);
            __syncthreads();
            nk = min(nb, np);
            cur ^= 1;
        }
    }
    // emission in canonical order: depth asc, then (parent's frontier index, sibling rank),
    // which is the order of the keys' low words, descending
    const int n = nk;
    int dd = 0, pos = 0;
    if (tid < n) {
        const uint32_t lo = (uint32_t)sm.kkey[cur][tid];
        dd = low_depth(lo);
        const ulonglong2* k2 = (const ulonglong2*)sm.kkey[cur];
#pragma unroll 1
        for (int f = 0; f < kMaxNcap / 2; f += 8) {
            ulonglong2 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = k2[f + u];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                pos += (int)(2 * (f + u) < n && (uint32_t)x[u].x > lo) +
                       (int)(2 * (f + u) + 1 < n && (uint32_t)x[u].y > lo);
        }
        sm.korder[pos] = (int16_t)tid;
        sm.pmap[dd][sm.kfi[cur][tid]] = (int16_t)pos;
    }
    __syncthreads();
    if (tid < n)
        sm.cpar[pos] = dd > 1 ? sm.pmap[dd - 1][low_fi((uint32_t)sm.kkey[cur][tid])] : (int16_t)-1;
    __syncthreads();
    // ancestor mask: the node's own bit and its ancestors' (each node walks its own path;
    // a parent's position is below its child's)
    if (tid < n) {
        uint64_t m = 0;
        for (int p = tid, s = 0; p >= 0 && p < n && s <= kMaxB; p = sm.cpar[p], ++s) m |= 1ull << p;
        sm.mask[tid] = m;
    }
    __syncthreads();
    const size_t base = (size_t)req * Ncap;
    for (int i = tid; i < Ncap; i += kFlashSelThreads) {
        if (i < n) {
            const int e = sm.korder[i];
            a.out.token[base + i] = sm.ktok[cur][e];
            a.out.parent[base + i] = sm.cpar[i];
            a.out.depth[base + i] = (uint8_t)low_depth((uint32_t)sm.kkey[cur][e]);
            a.out.anc_mask[base + i] = sm.mask[i];
            a.out.surv[base + i] = key_surv(sm.kkey[cur][e]);
            a.out.logq[base + i] = sm.klogq[cur][e];
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
                const int st = sm.kstate[cur][e];
                const int de = low_depth((uint32_t)sm.kkey[cur][e]);
                if (st >= 0) v = sm.set[de][sm.rslot[st][i]];
            }
        }
        a.out.cand[cb + w] = v;
    }
    if (tid < 64) {
        const uint64_t ex = __ballot(tid < n && sm.kstate[cur][tid] >= 0);
        if (tid == 0) {
            a.out.n_nodes[req] = n;
            a.out.status[req] = status;
            if (a.out.n_expand) a.out.n_expand[req] = (bad_root ? 0 : 1) + __popcll(ex);
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
    const int kt = kt_for(p->k);
    if (kt == 1)
        k_flash_sets<1><<<p->R * p->B * pl.P, kFlashSetThreads, 0, st>>>(a);
    else if (kt == 2)
        k_flash_sets<2><<<p->R * p->B * pl.P, kFlashSetThreads, 0, st>>>(a);
    else if (kt == 4)
        k_flash_sets<4><<<p->R * p->B * pl.P, kFlashSetThreads, 0, st>>>(a);
    else
        k_flash_sets<8><<<p->R * p->B * pl.P, kFlashSetThreads, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (kt == 1)
        k_flash_sets_merge<1><<<p->R * p->B, 64, 0, st>>>(a);
    else if (kt == 2)
        k_flash_sets_merge<2><<<p->R * p->B, 64, 0, st>>>(a);
    else if (kt == 4)
        k_flash_sets_merge<4><<<p->R * p->B, 64, 0, st>>>(a);
    else
        k_flash_sets_merge<8><<<p->R * p->B, 64, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = a.T * ((a.SP + 7) / 8) * 8;
    if (p->head_dtype == DT_BF16 && a.lvec)
        k_flash_lse<true, true><<<grid, 256, 0, st>>>(a);
    else if (p->head_dtype == DT_BF16)
        k_flash_lse<true, false><<<grid, 256, 0, st>>>(a);
    else
        k_flash_lse<false, false><<<grid, 256, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_flash_select<<<p->R, kFlashSelThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace dt
