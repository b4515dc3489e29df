// Tree construction with the Markov head's W resident on chip for the whole round.
//
// A level-synchronous build expands every level against all of W (r x V); streamed from
// memory at every level, W (77.8 MB at r = 256, V = 151936) costs more than everything else
// a small level does.  Here each workgroup (one per CU) owns a fixed vocabulary slice of W
// -- at most 20 blocks of 32 columns -- and loads it once per round: 12 blocks into the
// AGPRs of its four wavefronts (block j in slot j / 4 of wavefront j % 4: 192 of the 256
// AGPRs a wavefront has at one wavefront per SIMD, the rest left to the compiler) and up
// to 8 into LDS (block 12 + i processed by wavefront i % 4).  Per level, every workgroup
// expands all parent rows over its own slice, in tiles of 32 rows (one MFMA B operand):
// z = L[d] + U[parent] . W on bf16 MFMA 32x32x16 with W as the A operand read straight from
// the AGPRs, then the same online log-sum-exp and ranked-list epilogue as the streaming
// kernel (dt_build_common.h); the four wavefronts' lists of a row are combined in LDS and
// one record per (row, workgroup) is published.  Merge, select and emit are the shared
// phases.  The PCTree summary's method (one backbone forward gives the whole block's
// logits; the Markov head biases each position by its parent) is what makes W the same at
// every level.
//
// The MFMA chains that read W from AGPRs are inline assembly (the compiler would copy AGPR
// operands back into VGPRs before every MFMA), so their hazards are handled here: two wait
// states before the first MFMA of a chain (its accumulator was just written by VALU
// instructions), back-to-back MFMAs on one accumulator (as the compiler issues them), and
// 24 wait states after the last one before anything reads the accumulator or reuses its
// operand registers (the compiler puts 12 there for this instruction on gfx950).
#include <hip/hip_runtime.h>

#include <mutex>

#include "dt_build_common.h"

namespace dt {

constexpr int kResWaves = 4;
constexpr int kResThreads = 64 * kResWaves;
constexpr int kResAgprSlots = 3;  // W blocks per wavefront held in AGPRs (192 of its 256)
constexpr int kResLdsSlots = 8;   // W blocks per workgroup held in LDS (128 KB)
constexpr int kResTile = 32;      // parent rows per tile
static_assert(kResMaxBlocks == kResWaves * kResAgprSlots + kResLdsSlots, "slice capacity");

template <int KT>
struct ResSmem {
    // LDS-resident W blocks: row jj (vocabulary column) chunk c (16 bytes, 8 K values) at
    // slot 32 jj + (c ^ jj), so that the fragment reads of 16 consecutive lanes hit
    // distinct banks
    uint4 wl[kResLdsSlots][kBlockCols * 32];
    union {
        float xrec[kResWaves][kResTile][rec_floats(KT)];  // per-wavefront lists of a tile
        SelSmem sel;
        EmitSmem em;
    } u;
    float mrec[kResWaves][rec_floats(KT)];
    size_t lbase[kResTile];
    uint64_t hash[kResTile];
    uint64_t rkth[kResTile];  // per row of the tile: the largest KT-th list entry seen so far
    int tok[kResTile];
    int sh[64];
    int bcast[8];
    int lrows[kMaxB + 2];
    uint64_t mchild[2][kMaxK];
};

// One MFMA chain over a block held in AGPRs: acc += W(block) . U(tile) over r = 256.
__device__ __forceinline__ void mfma_chain_agpr(f32x16& acc, const u32x4_t (&w)[16],
                                                const u32x4_t (&u)[16]) {
    asm("s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %17, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %18, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %19, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %20, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %5, %21, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %6, %22, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %7, %23, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %8, %24, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %9, %25, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %10, %26, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %11, %27, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %12, %28, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %13, %29, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %14, %30, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %15, %31, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %16, %32, %0\n\t"
        "s_nop 7\n\t"
        "s_nop 7\n\t"
        "s_nop 7"
        : "+v"(acc)
        : "a"(w[0]), "a"(w[1]), "a"(w[2]), "a"(w[3]), "a"(w[4]), "a"(w[5]), "a"(w[6]), "a"(w[7]),
          "a"(w[8]), "a"(w[9]), "a"(w[10]), "a"(w[11]), "a"(w[12]), "a"(w[13]), "a"(w[14]),
          "a"(w[15]), "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(u[5]),
          "v"(u[6]), "v"(u[7]), "v"(u[8]), "v"(u[9]), "v"(u[10]), "v"(u[11]), "v"(u[12]),
          "v"(u[13]), "v"(u[14]), "v"(u[15]));
}

// One MFMA chain over an LDS-resident block (fragments read from LDS; the compiler handles
// this chain's hazards).
__device__ __forceinline__ void mfma_chain_lds(f32x16& acc, const uint4* wb, int h, int p,
                                               const u32x4_t (&u)[16]) {
    bf16x8 wf[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) wf[s] = __builtin_bit_cast(bf16x8, wb[(2 * s + h) ^ p]);
#pragma unroll
    for (int s = 0; s < 16; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], __builtin_bit_cast(bf16x8, u[s]), acc,
                                                      0, 0, 0);
}

// The workgroup's vocabulary slice: blocks [b_beg, b_beg + nb) of 32 columns.
struct Slice {
    int b_beg, nb;
};
__device__ __forceinline__ Slice res_slice(int V, int g, int G) {
    const int NB = (V + kBlockCols - 1) / kBlockCols;
    Slice s;
    s.b_beg = (int)((long long)g * NB / G);
    s.nb = (int)((long long)(g + 1) * NB / G) - s.b_beg;
    return s;
}

// Loads the slice once: AGPR slots of this wavefront (blocks 4 i + wave; slots past the
// slice repeat its last block and are never used) and the LDS-resident blocks 12 ...  Rows
// of Wt past V read row V - 1 (their columns are masked in the epilogue).
template <int KT>
__device__ __forceinline__ void load_slice(const BuildArgs& a, const Slice& sl,
                                           u32x4_t (&wr)[kResAgprSlots][16], ResSmem<KT>& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t* Wt = (const uint16_t*)a.Wt;
#pragma unroll
    for (int i = 0; i < kResAgprSlots; ++i) {
        int j = 4 * i + wave;
        j = j < sl.nb ? j : sl.nb - 1;
        int col = (sl.b_beg + j) * kBlockCols + (lane & 31);
        col = col < a.V ? col : a.V - 1;
        const u32x4_t* src = (const u32x4_t*)(Wt + (size_t)col * 256 + 8 * (lane >> 5));
#pragma unroll
        for (int s = 0; s < 16; ++s) wr[i][s] = src[2 * s];
    }
    // the LDS blocks: 32 rows x 32 chunks of 16 bytes each, copied global -> LDS directly
    // (1 KB a wavefront per copy) so that every copy of the slice is in flight at once; lane l
    // of copy k fills slot d = 64k + l, which holds row jj = d / 32, chunk (d % 32) ^ jj
    const int nlds = sl.nb - kResWaves * kResAgprSlots;
    for (int i = 0; i < nlds; ++i) {
#pragma unroll
        for (int k = wave; k < (kBlockCols * 32) / 64; k += kResWaves) {
            const int d = 64 * k + lane;
            const int jj = d >> 5, c = (d & 31) ^ jj;
            int col = (sl.b_beg + kResWaves * kResAgprSlots + i) * kBlockCols + jj;
            col = col < a.V ? col : a.V - 1;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(Wt + (size_t)col * 256 + 8 * c),
                (__attribute__((address_space(3))) void*)(sm.wl[i] + 64 * k), 16, 0, 0);
        }
    }
    wait_vm();  // this wavefront's copies have landed (the caller's barrier orders them)
}

// Expansion of one tile (rows m0 .. m0 + 31 of the level) over the workgroup's slice; the
// tile's records (one per row, this workgroup's split) are written to the partials.
template <int KT, bool SAMPLE>
__device__ __forceinline__ void expand_res_tile(const BuildArgs& a, int level, int M, int S,
                                                int split, const Slice& sl, int m0,
                                                const u32x4_t (&wr)[kResAgprSlots][16],
                                                ResSmem<KT>& sm) {
    constexpr int RS = rec_floats(KT);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, p = lane & 31;
    const int lvl = level - 1;
    const int nrows = min(kResTile, M - m0);
    if (tid < kResTile) {
        int tok = 0;
        size_t lb = 0;
        uint64_t hh = 0;
        if (tid < nrows) {
            const RowRec* rr = level_rows(a, level) + m0 + tid + opaque_zero();
            const uint64_t w0 = cld64(rr), w3 = cld64((const char*)rr + 24);
            hh = cld64((const char*)rr + 16);
            const int req = (int)(uint32_t)w0;
            // the head token selects the U row (-1: no bias); U is never indexed out of range
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
    // B operand: U[token of row p][16 s + 8 h .. + 8], s = 0..15
    u32x4_t uf[16];
    {
        const int tk = sm.tok[p];
        const u32x4_t* urow = (const u32x4_t*)((const uint16_t*)a.U + (size_t)(tk >= 0 ? tk : 0) * 256 + 8 * h);
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < 16; ++s) uf[s] = tk >= 0 ? urow[2 * s] : zero;
    }
    const size_t lb = sm.lbase[p];
    const uint64_t hh = sm.hash[p];
    const bool live = p < nrows;
    // block logits of every block of this wavefront, issued together with the U loads
    constexpr int NLW = kResLdsSlots / kResWaves;  // LDS blocks per wavefront
    constexpr int NBW = kResAgprSlots + NLW;
    LGroups<true> lg[NBW];
    int c0s[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int j = i < kResAgprSlots ? 4 * i + wave
                                        : kResWaves * kResAgprSlots + wave + kResWaves * (i - kResAgprSlots);
        const int jc = j < sl.nb ? j : sl.nb - 1;
        c0s[i] = (sl.b_beg + jc) * kBlockCols;
        load_lgroups<true>(a, lb, c0s[i], h, true, lg[i]);
    }
    TopK<KT> top;
    Lse2 st;
    top.init();
    st.init();
#pragma unroll
    for (int i = 0; i < kResAgprSlots; ++i) {
        if (i == 1) DT_STAMP(level, 1);
        if (4 * i + wave < sl.nb) {
            f32x16 acc;
            lgroups_to_acc<true>(lg[i], acc);
            mfma_chain_agpr(acc, wr[i], uf);
            expand_epilogue<KT, SAMPLE>(a, acc, c0s[i], h, hh, live, sm.rkth + p, top, st);
        }
    }
#pragma unroll
    for (int t = 0; t < NLW; ++t) {
        const int i = wave + kResWaves * t;  // LDS slot
        if (kResWaves * kResAgprSlots + i < sl.nb) {
            f32x16 acc;
            lgroups_to_acc<true>(lg[kResAgprSlots + t], acc);
            mfma_chain_lds(acc, sm.wl[i] + p * 32, h, p, uf);
            expand_epilogue<KT, SAMPLE>(a, acc, c0s[kResAgprSlots + t], h, hh, live, sm.rkth + p,
                                        top, st);
        }
    }
    // lanes l and l ^ 32 hold the same row; then the four wavefronts' lists of each row
    st.merge_xor(32);
    top.merge_xor(32);
    if (h == 0) put_list<KT>(sm.u.xrec[wave][p], top, st);
    lds_sync();
    if (tid < kResTile * kResWaves) {
        const int row = tid / kResWaves, w = tid % kResWaves;
        TopK<KT> t;
        Lse2 s;
        get_list<KT>(sm.u.xrec[w][row], t, s);
#pragma unroll
        for (int off = 1; off < kResWaves; off <<= 1) {
            s.merge_xor(off);
            t.merge_xor(off);
        }
        if (row < nrows) {
            float v[RS];
#pragma unroll
            for (int i = 0; i < RS; ++i) v[i] = 0.0f;
            put_list<KT>(v, t, s);
            uint4* rec = (uint4*)(a.partials + ((size_t)(m0 + row) * S + split) * RS);
#pragma unroll
            for (int c = 0; c < RS / 4; ++c)
                if (c % kResWaves == w)
                    cst128(rec + c, make_uint4(__float_as_uint(v[4 * c]), __float_as_uint(v[4 * c + 1]),
                                               __float_as_uint(v[4 * c + 2]), __float_as_uint(v[4 * c + 3])));
        }
    }
    lds_sync();
}

// The level loop with W resident.  One workgroup per CU; workgroup g expands every row of
// every level over its own slice (so every workgroup must be running for a level to
// finish; the grid is one workgroup per CU of an otherwise idle device, and every wait is
// bounded).  Merge rows are handed out by per-level tickets.
template <int KT, bool SAMPLE>
__global__ __launch_bounds__(kResThreads, 1) void k_build_res(const BuildArgs a) {
    __shared__ __attribute__((aligned(16))) ResSmem<KT> sm;
    const int tid = threadIdx.x;
    const int S = (int)gridDim.x, split = (int)blockIdx.x;
    const Slice sl = res_slice(a.V, split, S);
    bool failed = false;
    if (tid < kMaxB + 2) sm.lrows[tid] = 0;
    DT_STAMP(0, 0);
    u32x4_t wr[kResAgprSlots][16];
    load_slice<KT>(a, sl, wr, sm);
    int ticket = claim_ticket(a.sync, 1, sm.bcast);  // also orders the LDS slice stores
    for (int level = 1;; ++level) {
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
        unsigned* tdone = a.tdone + (size_t)level * a.Tmax;
        for (int m0 = 0; m0 < M; m0 += kResTile) {
            expand_res_tile<KT, SAMPLE>(a, level, M, S, split, sl, m0, wr, sm);
            publish_wg();
            if (tid == 0) cadd32(tdone + m0 / kResTile, 1u);
        }
        DT_STAMP(level, 2);
        bool first_task = true;
        // merges: ticket m is parent row m, merged once every split of its tile is in
        for (; ticket < M; ticket = claim_ticket(a.sync, level, sm.bcast)) {
            const int m = ticket;
            if (!wait_at_least(a.sync, tdone + m / kResTile, (unsigned)S, sm.bcast, a.spin_limit)) {
                failed = true;
                break;
            }
            if (first_task) DT_STAMP(level, 6);
            first_task = false;
            int req, F;
            merge_row<KT, kResThreads>(a, level, S, m, sm.mrec, sm.mchild, &req, &F);
            if (F == 1) {
                lds_sync();
                DT_STAMP(level, 5);
                select_request<kResThreads>(a, level, req, F, nreq, sm.u.sel, sm.sh, sm.bcast + 3,
                                            sm.mchild);
                DT_STAMP(level, 4);
            } else {
                publish_wg();
                DT_STAMP(level, 5);
                if (tid == 0)
                    sm.bcast[2] = (cadd32(a.rdone + (size_t)level * a.R + req, 1u) + 1u == (unsigned)F) ? 1 : 0;
                lds_sync();
                if (sm.bcast[2]) {
                    select_request<kResThreads>(a, level, req, F, nreq, sm.u.sel, sm.sh,
                                                sm.bcast + 3, nullptr);
                    DT_STAMP(level, 4);
                }
            }
            lds_sync();
        }
        if (failed) break;
        ticket = claim_ticket(a.sync, level + 1, sm.bcast);
    }
    DT_STAMP(kTraceLevels - 1, 0);
    if (failed) cst32(a.sync + kSyncErr, 1u);
    for (int req = blockIdx.x; req < a.R; req += gridDim.x)
        emit_request<kResThreads>(a, req, failed, sm.u.em);
    if (blockIdx.x == 0 && a.out.level_rows) {
        lds_sync();
        for (int l = tid; l < a.B; l += blockDim.x) a.out.level_rows[l] = sm.lrows[l + 1];
    }
    DT_STAMP(kTraceLevels - 1, 1);
}

// ---------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------
// Grid of the resident kernel on the current device: one workgroup per CU, provided the
// kernel fits one per CU and the slices fit (0 otherwise).  Cached per kernel and device.
static int res_grid(const void* f, int V) {
    static std::mutex mu;
    static const void* keys[64];
    static int devs[64], vals[64], n = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int g = -1;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (int i = 0; i < n && g < 0; ++i)
            if (keys[i] == f && devs[i] == dev) g = vals[i];
        if (g < 0) {
            int per = 0, cus = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, f, kResThreads, 0) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                return 0;
            g = (per >= 1 && cus >= 1 && cus <= kMaxGrid) ? cus : 0;
            if (n < 64) {
                keys[n] = f;
                devs[n] = dev;
                vals[n] = g;
                ++n;
            }
        }
    }
    if (g < 1) return 0;
    const int NB = (V + kBlockCols - 1) / kBlockCols;
    if (NB < g || (NB + g - 1) / g > kResMaxBlocks) return 0;
    return g;
}

template <int KT, bool SAMPLE>
static hipError_t launch_res_t(const BuildArgs& a, hipStream_t st, bool* used) {
    const void* f = (const void*)k_build_res<KT, SAMPLE>;
    const int G = res_grid(f, a.V);
    *used = G > 0;
    if (G < 1) return hipSuccess;
    hipError_t e = launch_build_init(a, st);
    if (e != hipSuccess) return e;
    if (a.timing_hook) a.timing_hook(st, 0);
    hipLaunchKernelGGL((k_build_res<KT, SAMPLE>), dim3(G), dim3(kResThreads), 0, st, a);
    if (a.timing_hook) a.timing_hook(st, 1);
    return hipGetLastError();
}

hipError_t launch_build_resident(const dt_params* p, const Layout& lay, const BuildArgs& a,
                                 hipStream_t st, bool* used) {
    *used = false;
    if (!resident_params_ok(p)) return hipSuccess;
    const bool smp = p->mode == DT_SAMPLE;
    switch (lay.KT) {
        case 1: return smp ? launch_res_t<1, true>(a, st, used) : launch_res_t<1, false>(a, st, used);
        case 2: return smp ? launch_res_t<2, true>(a, st, used) : launch_res_t<2, false>(a, st, used);
        case 4: return smp ? launch_res_t<4, true>(a, st, used) : launch_res_t<4, false>(a, st, used);
        default: return smp ? launch_res_t<8, true>(a, st, used) : launch_res_t<8, false>(a, st, used);
    }
}

}  // namespace dt
