// Tree attention: one attention layer of the target's verify forward over a round's draft
// trees (PCTree summary, "From Chains to Trees", introduction: the target checks every node
// of the tree in one forward).  The root's and the nodes' keys and values follow the
// request's context in the cache; the query of a tree position sees the context, the root,
// and the slots its 64-bit ancestor mask names.
//
// Layout of the work.  A workgroup owns one (request, key/value head, query group, key
// split).  Its queries are the G grouped query heads' tree positions, concatenated
// (qi = g * (n + 1) + j), in 32-query tiles, one tile per wavefront.  The key range is walked
// in 64-key blocks: K rows are copied to LDS as they are (row-major, padded), V rows are
// transposed on the way in (keys contiguous per head-dimension row), so that both
// contractions read 16 contraction elements per lane from LDS:
//
//   S^T[key][q] = K[key][:] . Q[q][:]           A = K (LDS), B = Q (registers)
//   O^T[d][q]  += V^T[d][keys] . P^T[keys][q]    A = V^T (LDS), B = P^T (registers)
//
// With the 32x32x16 bf16 MFMA a lane holds, of the score tile, one query column and 16 keys;
// those 16 probabilities are exactly the B operand of the two P.V steps once the key order
// inside each 16-key step is permuted to match (the same permutation is applied to the
// V^T reads), so P never leaves registers.  The softmax is online in the log2 domain; the
// running maximum is only raised when a score exceeds it by more than 8 (probabilities up to
// 2^8 are harmless in fp32 and bf16), which skips almost every rescale of the accumulators.
// With several key splits, unnormalised partial outputs and (max, sum) pairs go to the
// workspace and a second kernel combines them.
#include <hip/hip_runtime.h>

#include <cmath>

#include "dt_internal.h"

namespace dt {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 abf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float af32x16;

constexpr int kAttD = 128;             // head dimension
#ifndef DT_ATTN_MAX_WAVES
#define DT_ATTN_MAX_WAVES 9
#endif
constexpr int kAttWaves = DT_ATTN_MAX_WAVES;  // query wavefronts per workgroup, at most
#ifndef DT_ATTN_BLK_SMALL
#define DT_ATTN_BLK_SMALL 32
#endif
constexpr int kAttBlkSmall = DT_ATTN_BLK_SMALL;  // keys per block below 8 wavefronts
constexpr int kAttMinWaves = 4;        // wavefronts that share the LDS fills at least
constexpr float kLazy = 8.0f;          // rescale only when the max grows by more than 2^8

struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const int32_t* ctx_len;
    const int32_t* n_nodes;
    const uint64_t* anc;
    uint16_t* O;
    float* po;       // partial outputs [units][S][G][Ncap+1][D] (S > 1)
    float2* pml;     // partial (max, sum) [units][S][G][Ncap+1]
    int R, Hq, Hkv, G, Ncap, Cmax, S, QG, NW;
    int units;       // R * Hkv
    float c2;        // scale * log2(e)
};

typedef float af32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 abf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even; v_cvt_pk_bf16_f32), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((af32x2){a, b}, abf16x2));
}

// 2^x on the transcendental unit (v_exp_f32): results below the normal range flush to
// zero, which only drops probabilities under 2^-126 of the running maximum.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short as16x4 __attribute__((ext_vector_type(4)));

// Two transposing LDS reads (four bf16 each) joined into one MFMA operand.
__device__ __forceinline__ abf16x8 tr_pair(const uint16_t* p0, const uint16_t* p1) {
    typedef __attribute__((address_space(3))) as16x4 lds_v4;
    const as16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)p0);
    const as16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)p1);
    typedef short as16x8 __attribute__((ext_vector_type(8)));
    const as16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(abf16x8, z);
}

// Workgroup barrier that waits only for this wavefront's LDS accesses: loads still in flight
// (the next block's copies) stay in flight across it.
// (s_waitcnt immediates, gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8; written with the builtin so that the compiler's own wait bookkeeping sees them.)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
__device__ __forceinline__ void att_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ bool attn_request_ok(int ctx, int n, int Ncap, int Cmax) {
    return n >= 0 && n <= Ncap && ctx >= 0 && ctx <= Cmax - n - 1;
}

// Workgroup index -> (ordered unit u, split, query group).  Workgroups are dispatched
// round-robin over the 8 XCDs; the query groups of one (unit, split) are placed 8 apart so
// that they land on the same XCD and share its L2 for the K/V blocks.
__device__ __forceinline__ void attn_decode(const AttnArgs& a, int& u, int& s, int& qg) {
    const int b = blockIdx.x;
    const int lo = b & 7, mid = (b >> 3) % a.QG, hi = (b >> 3) / a.QG;
    const int w = hi * 8 + lo;  // (unit, split) index
    u = w / a.S;
    s = w % a.S;
    qg = mid;
}

// Ordered units run the requests longest first (keys ctx_len + n_nodes + 1; invalid requests
// count zero; ties by request index), so that the dispatcher, which hands out workgroups in
// index order as compute units free up, pairs long requests with short ones instead of
// leaving a few compute units with two long ones.  Every workgroup derives the order itself:
// the key counts go to LDS and thread i ranks request i by counting the requests before it
// (R <= kLptMax; larger batches keep the request order).
constexpr int kLptMax = 1024;

__device__ __forceinline__ int attn_keys(const AttnArgs& a, int i) {
    const int ctx = a.ctx_len[i], n = a.n_nodes[i];
    return attn_request_ok(ctx, n, a.Ncap, a.Cmax) ? ctx + n + 1 : 0;
}

template <int NT>
__device__ __forceinline__ int lpt_request(const AttnArgs& a, int k, int* sL, int* sP) {
    if (a.R > kLptMax) return k;
    for (int i = threadIdx.x; i < a.R; i += NT) sL[i] = attn_keys(a, i);
    __syncthreads();
    for (int i = threadIdx.x; i < a.R; i += NT) {
        const int Li = sL[i];
        int rank = 0;
        for (int j = 0; j < a.R; ++j) {
            const int Lj = sL[j];
            rank += (Lj > Li) | ((Lj == Li) & (j < i));
        }
        sP[rank] = i;
    }
    __syncthreads();
    return sP[k];
}

// Keys go through LDS in blocks of BLK (64 with 512 threads or more, else 32).  K and V
// blocks are copied global -> LDS directly (global_load_lds: 16 bytes a lane, 1 KB a
// wavefront, i.e. four 256-byte rows) into double buffers, so a block's copies are in
// flight while the previous block is computed and one barrier per block suffices.  Rows
// are swizzled in 16-byte segments against bank conflicts: segment s of K row k sits at
// position s ^ (k % 16) (a quarter-wavefront reads 16 rows at one segment), segment s of V
// row k at s ^ 4(k % 4) (a half-wavefront's transposing reads cover four rows and four
// segments).  V is read with ds_read_b64_tr_b16: in each 16-lane group, lane 4a + b receives
// element b of the 8-byte rows addressed by lanes a, 4 + a, 8 + a and 12 + a; with lane
// 4e + a addressing V row (key) e of its half-wavefront's four keys at head-dimension columns
// 4a.. of its 16-column half, lane 4a + b receives four keys of column 4a + b, which is the
// MFMA A-operand fragment of V^T for that row.
template <int NW, int BLK>
__global__ __launch_bounds__(NW * 64, 3) void k_tree_attn(AttnArgs a) {
    constexpr int NT = NW * 64;
    __shared__ __align__(1024) uint16_t sK0[BLK * kAttD];
    __shared__ __align__(1024) uint16_t sK1[BLK * kAttD];
    __shared__ __align__(1024) uint16_t sV0[BLK * kAttD];
    __shared__ __align__(1024) uint16_t sV1[BLK * kAttD];
    __shared__ int sL[kLptMax], sP[kLptMax];

    int u, s, qg;
    attn_decode(a, u, s, qg);
    if (u >= a.units) return;
    const int r = lpt_request<NT>(a, u / a.Hkv, sL, sP), h = u % a.Hkv;
    const int unit = r * a.Hkv + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 31, hh = lane >> 5;
    const int ctx = a.ctx_len[r], n = a.n_nodes[r];
    const int Nq = a.Ncap + 1;
    const bool ok = attn_request_ok(ctx, n, a.Ncap, a.Cmax);

    // single-split mode: the first query group also writes the zero rows (positions past n,
    // or every row of an invalid request) of its G heads
    if (a.S == 1 && qg == 0) {
        const int first = ok ? n + 1 : 0;
        const int rows = a.G * (Nq - first);
        for (int i = tid; i < rows * (kAttD / 8); i += NT) {
            const int row = i / (kAttD / 8), seg = i % (kAttD / 8);
            const int g = row / (Nq - first), j = first + row % (Nq - first);
            *(uint4*)(a.O + (((size_t)r * a.Hq + h * a.G + g) * Nq + j) * kAttD + seg * 8) =
                make_uint4(0, 0, 0, 0);
        }
    }
    if (!ok) return;

    const int nq = a.G * (n + 1);
    const int tiles = (nq + 31) >> 5;
    const int t0 = qg * NW;
    if (t0 >= tiles) return;  // whole workgroup idle: uniform exit before any barrier
    const int tile = t0 + wave;
    const bool active = tile < tiles;

    const int L = ctx + n + 1;
    const int nblk = (L + BLK - 1) / BLK;
    const int b0 = (int)((long)s * nblk / a.S), b1 = (int)((long)(s + 1) * nblk / a.S);

    // this lane's query column
    const int qi = tile * 32 + c;
    const bool qv = active && qi < nq;
    const int g = qv ? qi / (n + 1) : 0;
    const int j = qv ? qi % (n + 1) : 0;
    const uint64_t qmask = j == 0 ? 0ull : a.anc[(size_t)r * a.Ncap + (j - 1)];
    abf16x8 qf[8];
    {
        const uint16_t* qp = a.Q + (((size_t)r * a.Hq + h * a.G + g) * Nq + j) * kAttD + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(abf16x8, *(const uint4*)(qp + 16 * ks));
    }

    const uint16_t* Kb = a.K + (size_t)unit * a.Cmax * kAttD;
    const uint16_t* Vb = a.V + (size_t)unit * a.Cmax * kAttD;
    // one block's K and V rows, copied by the wavefronts in 1 KB chunks (keys past the
    // request's last slot repeat it; their scores are masked)
    auto issue = [&](int b, uint16_t* kdst, uint16_t* vdst) {
        const int key0 = b * BLK;
        for (int ch = wave; ch < BLK / 4; ch += NW) {
            const int row = 4 * ch + (lane >> 4);
            const size_t src = (size_t)min(key0 + row, L - 1) * kAttD;
            const int ks = (lane & 15) ^ (row & 15), vs = (lane & 15) ^ (4 * (row & 3));
            __builtin_amdgcn_global_load_lds((const void*)(Kb + src + ks * 8),
                                             (void*)(kdst + ch * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(Vb + src + vs * 8),
                                             (void*)(vdst + ch * 512), 16, 0, 0);
        }
    };
    // per-lane part of the transposing V reads: row 4hh + e (e = (lane % 16) / 4) of each
    // 16-key step, columns 16 * ((lane / 16) % 2) + 4 * (lane % 4) of each 32-column tile
    const int tr_e = (lane & 15) >> 2, tr_a = lane & 3, tr_g = (lane >> 4) & 1;
    const int tr_row = 4 * hh + tr_e;
    const int tr_lo = 2 * tr_g + (tr_a >> 1), tr_in = 4 * (tr_a & 1);

    af32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    // one key block: wait for this thread's copies of it, barrier (every copy landed, every
    // wavefront done with the previous block and so with the buffers the next block's copies
    // go to), start the next block's copies, then every query wavefront works on it
    auto step = [&](int b, const uint16_t* __restrict__ kbuf, const uint16_t* __restrict__ vbuf,
                    uint16_t* __restrict__ knext, uint16_t* __restrict__ vnext) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        att_barrier();
        if (b + 1 < b1) issue(b + 1, knext, vnext);
        if (!active) return;
#pragma unroll
        for (int kt = 0; kt < BLK / 32; ++kt) {
            const int key0 = b * BLK + kt * 32;
            if (key0 >= L) break;
            af32x16 sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
            // row kt*32 + c, segment 2ks + hh, stored at segment (2ks + hh) ^ (c % 16)
            const uint16_t* kp = kbuf + (kt * 32 + c) * kAttD;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(abf16x8, *(const uint4*)(kp + (((2 * ks + hh) ^ (c & 15)) * 8))),
                    qf[ks], sacc, 0, 0, 0);
            // element i is key key0 + 8(i/4) + 4hh + i%4; masked keys become -inf
            const bool tail = key0 + 32 > ctx + 1;
            if (tail) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    // rel < 0: context or root; 0 <= rel < n: node rel, visible when its
                    // bit is set in this query's mask (the shift amount is masked to stay
                    // defined; its bit only counts when 0 <= rel < n <= 64)
                    const int rel = key0 + 8 * (i >> 2) + 4 * hh + (i & 3) - ctx - 1;
                    const bool bit = (qmask >> ((unsigned)rel & 63u)) & 1ull;
                    const bool vis = (rel < 0) | ((rel < n) & bit);
                    sacc[i] = vis ? sacc[i] : -INFINITY;
                }
            }
            float mx = sacc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
            // the maximum in the log2 domain (the scale is positive)
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.c2;
            const bool raise = mx > m + kLazy;
            if (__any(raise)) {
                const float mn = raise ? mx : m;
                const float alpha = raise ? ex2(m - mn) : 1.0f;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
                lsum *= alpha;
                m = mn;
            }
            const float mu = m == -INFINITY ? 0.0f : m;
            uint32_t pw[8];
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = ex2(fmaf(sacc[i], a.c2, -mu));
                const float p1 = ex2(fmaf(sacc[i + 1], a.c2, -mu));
                lsum += p0 + p1;
                pw[i >> 1] = pack_bf16x2(p0, p1);
            }
            const abf16x8 pb0 = __builtin_bit_cast(abf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            const abf16x8 pb1 = __builtin_bit_cast(abf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
            // V^T fragments: keys kt*32 + 16kk + {4hh + 0..3, 8 + 4hh + 0..3} (the same order
            // as this lane's probabilities), head-dimension row 32dt + c
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const int col = (((4 * dt) ^ (4 * tr_e)) + tr_lo) * 8 + tr_in;
                const uint16_t* vp = vbuf + (kt * 32 + tr_row) * kAttD + col;
                const abf16x8 v0 = tr_pair(vp, vp + 8 * kAttD);
                const abf16x8 v1 = tr_pair(vp + 16 * kAttD, vp + 24 * kAttD);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb0, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb1, o[dt], 0, 0, 0);
            }
        }
    };
    if (b0 < b1) issue(b0, sK0, sV0);
    // unrolled by two so that each step names its buffers statically
    for (int b = b0; b < b1; b += 2) {
        step(b, sK0, sV0, sK1, sV1);
        if (b + 1 < b1) step(b + 1, sK1, sV1, sK0, sV0);
    }
    if (!active) return;
    const float lt = lsum + __shfl_xor(lsum, 32);
    if (!qv) return;
    // element i of o[dt] is head-dimension row 32dt + 8(i/4) + 4hh + i%4 of this query
    if (a.S == 1) {
        const float inv = 1.0f / lt;
        uint16_t* op = a.O + (((size_t)r * a.Hq + h * a.G + g) * Nq + j) * kAttD + 4 * hh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float e0 = o[dt][4 * q4], e1 = o[dt][4 * q4 + 1];
                const float e2 = o[dt][4 * q4 + 2], e3 = o[dt][4 * q4 + 3];
                const uint2 w = make_uint2(pack_bf16x2(e0 * inv, e1 * inv),
                                           pack_bf16x2(e2 * inv, e3 * inv));
                *(uint2*)(op + 32 * dt + 8 * q4) = w;
            }
    } else {
        const size_t row = (((size_t)unit * a.S + s) * a.G + g) * Nq + j;
        float* pp = a.po + row * kAttD + 4 * hh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(float4*)(pp + 32 * dt + 8 * q4) =
                    make_float4(o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]);
        if (hh == 0) a.pml[row] = make_float2(m, lt);
    }
}

// Combines the key splits: one 64-thread workgroup per (request, query head, tree position).
__global__ __launch_bounds__(64) void k_tree_attn_combine(AttnArgs a) {
    const int Nq = a.Ncap + 1;
    const int row = blockIdx.x;  // (r * Hq + hq) * Nq + j
    const int j = row % Nq, hq = (row / Nq) % a.Hq, r = row / (Nq * a.Hq);
    const int h = hq / a.G, g = hq % a.G;
    const int ctx = a.ctx_len[r], n = a.n_nodes[r];
    uint16_t* op = a.O + (size_t)row * kAttD + 2 * threadIdx.x;
    if (!attn_request_ok(ctx, n, a.Ncap, a.Cmax) || j > n) {
        *(uint32_t*)op = 0u;
        return;
    }
    const size_t base = (((size_t)(r * a.Hkv + h) * a.S) * a.G + g) * Nq + j;
    const size_t sstride = (size_t)a.G * Nq;
    float M = -INFINITY;
    for (int s = 0; s < a.S; ++s) M = fmaxf(M, a.pml[base + s * sstride].x);
    float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s = 0; s < a.S; ++s) {
        const float2 ml = a.pml[base + s * sstride];
        if (ml.x == -INFINITY) continue;
        const float w = ex2(ml.x - M);
        const float2 v = *(const float2*)(a.po + (base + s * sstride) * kAttD + 2 * threadIdx.x);
        l += w * ml.y;
        o0 += w * v.x;
        o1 += w * v.y;
    }
    const float inv = 1.0f / l;
    *(uint32_t*)op = pack_bf16x2(o0 * inv, o1 * inv);
}

AttnPlan attn_plan(const dt_attn_params* p) {
    AttnPlan pl{};
    pl.G = p->Hq / p->Hkv;
    const int tiles = (pl.G * (p->Ncap + 1) + 31) / 32;
    pl.QG = (tiles + kAttWaves - 1) / kAttWaves;
    pl.NW = (tiles + pl.QG - 1) / pl.QG;
    if (pl.NW < kAttMinWaves) pl.NW = kAttMinWaves;
    const long units = (long)p->R * p->Hkv;
    // enough workgroups to cover the chip about twice, each split at least 128 keys
    const long want = (512 + units * pl.QG - 1) / (units * pl.QG);
    const long maxs = p->Cmax / 128 > 1 ? p->Cmax / 128 : 1;
    pl.S = (int)(want < 1 ? 1 : (want > maxs ? maxs : want));
    if (pl.S > 1) {
        const size_t rows = (size_t)units * pl.S * pl.G * (p->Ncap + 1);
        pl.po_bytes = (rows * kAttD * sizeof(float) + 255) & ~(size_t)255;
        pl.total = pl.po_bytes + ((rows * sizeof(float2) + 255) & ~(size_t)255);
    }
    return pl;
}

hipError_t launch_tree_attention(const dt_attn_params* p, const AttnPlan& pl, const void* Q,
                                 const void* K, const void* V, const int32_t* ctx_len,
                                 const int32_t* n_nodes, const uint64_t* anc, void* O,
                                 char* ws, hipStream_t st) {
    AttnArgs a{};
    a.Q = (const uint16_t*)Q;
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.ctx_len = ctx_len;
    a.n_nodes = n_nodes;
    a.anc = anc;
    a.O = (uint16_t*)O;
    a.po = pl.S > 1 ? (float*)ws : nullptr;
    a.pml = pl.S > 1 ? (float2*)(ws + pl.po_bytes) : nullptr;
    a.R = p->R;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.G = pl.G;
    a.Ncap = p->Ncap;
    a.Cmax = p->Cmax;
    a.S = pl.S;
    a.QG = pl.QG;
    a.NW = pl.NW;
    a.units = p->R * p->Hkv;
    a.c2 = p->scale * 1.4426950408889634f;
    const long w = (long)a.units * a.S;
    const int grid = (int)(((w + 7) / 8) * 8 * a.QG);
    switch (pl.NW) {
        case 4: k_tree_attn<4, kAttBlkSmall><<<grid, 256, 0, st>>>(a); break;
        case 5: k_tree_attn<5, kAttBlkSmall><<<grid, 320, 0, st>>>(a); break;
        case 6: k_tree_attn<6, kAttBlkSmall><<<grid, 384, 0, st>>>(a); break;
        case 7: k_tree_attn<7, kAttBlkSmall><<<grid, 448, 0, st>>>(a); break;
        case 8: k_tree_attn<8, 64><<<grid, 512, 0, st>>>(a); break;
        default: k_tree_attn<9, 64><<<grid, 576, 0, st>>>(a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.S == 1) return e;
    k_tree_attn_combine<<<a.R * a.Hq * (a.Ncap + 1), 64, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace dt
