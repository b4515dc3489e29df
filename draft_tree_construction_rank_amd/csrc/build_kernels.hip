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

#include "dt_build_common.h"

namespace dt {

// The persistent construction kernel runs one workgroup of kWaves wavefronts per CU.
constexpr int kWaves = kBuildWaves;
constexpr int kThreads = 64 * kWaves;

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
            const uint64_t w0 = cld64(rr), w3 = cld64((const char*)rr + 24);
            hh = cld64((const char*)rr + 16);
            const int req = (int)(uint32_t)w0;
            // the head token selects the U row; -1 (no bias) gives a zero row below, and
            // U is never indexed out of range
            tok = (int)(uint32_t)(w3 >> 32);
            tok = tok < 0 ? -1 : ((uint32_t)tok < (uint32_t)a.V ? tok : 0);
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
    bool bias = false;
    if (live) {
        const RowRec* rr = level_rows(a, level) + row;
        const uint64_t w0 = cld64(rr), w3 = cld64((const char*)rr + 24);
        hh = cld64((const char*)rr + 16);
        const int req = (int)(uint32_t)w0;
        // the head token selects the U row (-1: no bias); U is never indexed out of range
        tok = (int)(uint32_t)(w3 >> 32);
        bias = tok >= 0;
        tok = (uint32_t)tok < (uint32_t)a.V ? tok : 0;
        lb = ((size_t)req * a.B + lvl) * (size_t)a.V;
    }
    // B fragments: U[tok][16 s + 8 h .. +8], zero past r and for rows without a bias
    bf16x8 uf[16];
    {
        const uint16_t* urow = (const uint16_t*)a.U + (size_t)tok * a.r;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int kk = 16 * s + 8 * h;
            const uint4 v = *(const uint4*)(urow + (kk < a.r ? kk : 0));
            uf[s] = __builtin_bit_cast(bf16x8, (kk < a.r && bias) ? v : make_uint4(0, 0, 0, 0));
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
            // the root's own token is also the chain's first token; no bias without a head
            rr.htok = a.cond == DT_COND_NONE ? -1 : root;
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
            merge_row<KT, kThreads>(a, level, S, m, sm.mrec, sm.mchild, &req, &F);
            if (F == 1) {
                // the request's only row: its select follows at once, with the children from
                // LDS (its closing publish also covers the child records)
                lds_sync();
                DT_STAMP(level, 5);
                select_request<kThreads>(a, level, req, F, nreq, sm.u.sel, sm.sh, sm.bcast + 3, sm.mchild);
                DT_STAMP(level, 4);
            } else {
                publish_wg();
                DT_STAMP(level, 5);
                if (tid == 0)
                    sm.bcast[2] = (cadd32(a.rdone + (size_t)level * a.R + req, 1u) + 1u == (unsigned)F) ? 1 : 0;
                lds_sync();
                if (sm.bcast[2]) {
                    select_request<kThreads>(a, level, req, F, nreq, sm.u.sel, sm.sh, sm.bcast + 3, nullptr);
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
        emit_request<kThreads>(a, req, failed, sm.u.em);
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
        const hipError_t e = launch_build_init(a, st);
        if (e != hipSuccess) return e;
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

hipError_t launch_build_init(const BuildArgs& a, hipStream_t st) {
    // enough workgroups to clear the per-level counters in a few stores per thread
    const size_t words = (size_t)(a.B + 2) * (a.Tmax + a.R);
    int g = (int)((words + 256 * 16 - 1) / (256 * 16));
    g = g < 1 ? 1 : (g > 256 ? 256 : g);
    hipLaunchKernelGGL(k_build_init, dim3(g), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_build(const dt_params* p, const Layout& lay, const BuildArgs& a,
                        hipStream_t st) {
    if (lay.resident) {
        bool used = false;
        const hipError_t e = launch_build_resident(p, lay, a, st, &used);
        if (used || e != hipSuccess) return e;
    }
    switch (lay.KT) {
        case 1: return launch_build_kt<1>(p, a, st);
        case 2: return launch_build_kt<2>(p, a, st);
        case 4: return launch_build_kt<4>(p, a, st);
        default: return launch_build_kt<8>(p, a, st);
    }
}

}  // namespace dt
