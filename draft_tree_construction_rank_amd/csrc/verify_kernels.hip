// Verification kernels for gfx950.
//
// Greedy accept-walk (PCTree setup: greedy verification): one workgroup per request walks
// from the root; each step is a row argmax over the vocabulary (bandwidth-bound, 16-byte
// loads spread over 1024 threads) followed by a lookup of the argmax among the current
// node's children (at most 64 tree nodes, held in LDS).
#include <hip/hip_runtime.h>

#include "dt_device.h"
#include "dt_mma.h"

namespace dt {

struct ArgMax {
    float v;
    int i;
};

__device__ __forceinline__ ArgMax amax(ArgMax a, ArgMax b) {
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

// Within one thread indices arrive in increasing order, so a strict comparison keeps the
// lowest index among equal values.
__device__ __forceinline__ void amax_seq(ArgMax& a, float v, int i) {
    if (v > a.v) {
        a.v = v;
        a.i = i;
    }
}

__device__ __forceinline__ ArgMax wave_amax(ArgMax a) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ArgMax o;
        o.v = __shfl_xor(a.v, off);
        o.i = __shfl_xor(a.i, off);
        a = amax(a, o);
    }
    return a;
}

// Workgroup reduction of per-thread candidates; every thread gets the result.
__device__ ArgMax block_amax(ArgMax best, ArgMax* sh) {
    const int tid = threadIdx.x;
    best = wave_amax(best);
    const int wv = tid >> 6, nw = blockDim.x >> 6;
    if ((tid & 63) == 0) sh[wv] = best;
    __syncthreads();
    if (tid < 64) {
        ArgMax b = (tid < nw) ? sh[tid] : ArgMax{-INFINITY, 0x7fffffff};
        b = wave_amax(b);
        if (tid == 0) sh[0] = b;
    }
    __syncthreads();
    const ArgMax r = sh[0];
    __syncthreads();
    return r;
}

// Argmax (ties: lower index) of units [lo, hi) of one row over the whole workgroup; a unit
// is a 16-byte segment when `vec` (V a multiple of 8 bf16 / 4 float values), else one value.
// Each thread keeps kBatch independent loads in flight before it uses any of them.
template <bool BF16, int kBatch>
__device__ ArgMax range_argmax(const void* row, int lo, int hi, bool vec, ArgMax* sh) {
    ArgMax best{-INFINITY, 0x7fffffff};
    const int tid = threadIdx.x, nt = blockDim.x;
    if (BF16) {
        const uint16_t* p = (const uint16_t*)row;
        if (vec) {
            for (int i0 = lo + tid; i0 < hi; i0 += nt * kBatch) {
                uint4 w[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int i = i0 + u * nt;
                    w[u] = i < hi ? ((const uint4*)p)[i] : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int i = i0 + u * nt;
                    if (i < hi) {
                        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            amax_seq(best, bf16_lo(ws[e]), i * 8 + 2 * e);
                            amax_seq(best, bf16_hi(ws[e]), i * 8 + 2 * e + 1);
                        }
                    }
                }
            }
        } else {
            for (int i = lo + tid; i < hi; i += nt) amax_seq(best, bf16_to_f32(p[i]), i);
        }
    } else {
        const float* p = (const float*)row;
        if (vec) {
            for (int i0 = lo + tid; i0 < hi; i0 += nt * kBatch) {
                float4 w[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int i = i0 + u * nt;
                    w[u] = i < hi ? ((const float4*)p)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int i = i0 + u * nt;
                    if (i < hi) {
                        amax_seq(best, w[u].x, i * 4);
                        amax_seq(best, w[u].y, i * 4 + 1);
                        amax_seq(best, w[u].z, i * 4 + 2);
                        amax_seq(best, w[u].w, i * 4 + 3);
                    }
                }
            }
        } else {
            for (int i = lo + tid; i < hi; i += nt) amax_seq(best, p[i], i);
        }
    }
    return block_amax(best, sh);
}

template <bool BF16>
__device__ __forceinline__ int row_units(int V, bool vec) {
    return vec ? (BF16 ? V >> 3 : V >> 2) : V;
}

// Root rows, split: workgroup (request, j) writes the argmax of the j-th of S equal parts of
// the request's row 0 to part[request][j].
template <bool BF16>
__global__ __launch_bounds__(256) void k_verify_root(int V, int Ncap, int S, const void* target,
                                                     ArgMax* part) {
    __shared__ ArgMax sh[4];
    const int req = blockIdx.x / S, j = blockIdx.x % S;
    const bool vec = BF16 ? (V & 7) == 0 : (V & 3) == 0;
    const int n = row_units<BF16>(V, vec);
    const int lo = (int)((long long)j * n / S), hi = (int)((long long)(j + 1) * n / S);
    const char* rp = (const char*)target + (size_t)req * (Ncap + 1) * (size_t)V * (BF16 ? 2 : 4);
    const ArgMax am = range_argmax<BF16, 8>(rp, lo, hi, vec, sh);
    if (threadIdx.x == 0) part[(size_t)req * S + j] = am;
}

// The walk: one workgroup per request.  Row 0's argmax comes from the S partials of
// k_verify_root; every later row is reduced here.
template <bool BF16>
__global__ __launch_bounds__(1024) void k_verify_greedy(int B, int V, int Ncap, int S,
                                                        const void* target, const ArgMax* part,
                                                        dt_tree tree, dt_verify_out out) {
    __shared__ ArgMax sh[16];
    __shared__ int s_tok[kMaxNcap], s_par[kMaxNcap];
    __shared__ int s_child;
    const int req = blockIdx.x, tid = threadIdx.x;
    const int n = tree.n_nodes[req];
    // a bad root or a build whose internal wait gave up: nothing is emitted
    const bool bad = (tree.status[req] & (DT_REQ_BAD_ROOT | DT_REQ_SYNC_TIMEOUT)) != 0;
    if (tid < Ncap) {
        s_tok[tid] = tree.token[(size_t)req * Ncap + tid];
        s_par[tid] = tree.parent[(size_t)req * Ncap + tid];
    }
    for (int i = tid; i < B; i += blockDim.x) out.path[(size_t)req * B + i] = -1;
    for (int i = tid; i <= B; i += blockDim.x) out.out_tokens[(size_t)req * (B + 1) + i] = -1;
    __syncthreads();
    if (bad) {
        if (tid == 0) {
            out.accept_len[req] = 0;
            out.n_out[req] = 0;
        }
        return;
    }
    const bool vec = BF16 ? (V & 7) == 0 : (V & 3) == 0;
    const size_t esz = BF16 ? 2 : 4;
    int v = -1, row = 0, nacc = 0;
    for (;;) {
        ArgMax am;
        if (row == 0) {
            // S <= 64 partials, in index order of their vocabulary parts
            ArgMax c{-INFINITY, 0x7fffffff};
            if (tid < S) c = part[(size_t)req * S + tid];
            am = block_amax(c, sh);
        } else {
            const char* rp = (const char*)target + ((size_t)req * (Ncap + 1) + row) * (size_t)V * esz;
            am = range_argmax<BF16, 20>(rp, 0, row_units<BF16>(V, vec), vec, sh);
        }
        if (tid == 0) s_child = -1;
        __syncthreads();
        if (tid < n && s_par[tid] == v && s_tok[tid] == am.i) s_child = tid;
        __syncthreads();
        const int w = s_child;
        __syncthreads();
        if (tid == 0) out.out_tokens[(size_t)req * (B + 1) + nacc] = am.i;
        if (w < 0) break;
        if (tid == 0) out.path[(size_t)req * B + nacc] = w;
        ++nacc;
        v = w;
        row = w + 1;
    }
    if (tid == 0) {
        out.accept_len[req] = nacc;
        out.n_out[req] = nacc + 1;
    }
}

hipError_t launch_verify_greedy(const dt_params* p, const Layout& lay, char* ws,
                                const dt_tree* tree, const void* target,
                                const dt_verify_out* out, hipStream_t st) {
    ArgMax* part = (ArgMax*)(ws + lay.gpart);
    const int S = lay.gsplits;
    if (p->logits_dtype == DT_BF16) {
        hipLaunchKernelGGL(k_verify_root<true>, dim3(p->R * S), dim3(256), 0, st, p->V, p->Ncap,
                           S, target, part);
        hipLaunchKernelGGL(k_verify_greedy<true>, dim3(p->R), dim3(1024), 0, st, p->B, p->V,
                           p->Ncap, S, target, (const ArgMax*)part, *tree, *out);
    } else {
        hipLaunchKernelGGL(k_verify_root<false>, dim3(p->R * S), dim3(256), 0, st, p->V, p->Ncap,
                           S, target, part);
        hipLaunchKernelGGL(k_verify_greedy<false>, dim3(p->R), dim3(1024), 0, st, p->B, p->V,
                           p->Ncap, S, target, (const ArgMax*)part, *tree, *out);
    }
    return hipGetLastError();
}


// =======================================================================================
// Lossless sample verify (TreeSpark lossless section).  The requests walk in lock-step,
// one node per step; a step is two launches:
//   k_vs_rows_blocks (k_vs_rows for float32 heads or logits) - for every request still
//                walking at a node of depth < B: the node's draft row
//                y_q = (L[d] + U[t] . Wt) * log2(e)/T on MFMA, stored to vrow, plus per-split
//                (max, sum) of y_q and of the target row;
//   k_vs_split - the rejection chain, each request on SC workgroups that split the
//                vocabulary: every workgroup of a request takes the same decisions (they
//                depend only on values every workgroup computes identically), and each
//                vocabulary-wide reduction (a residual mass, a draw) is one partial per
//                slice, exchanged through tagged slots and summed in slice order.  A
//                workgroup keeps its slice's p and q in registers for the whole step.
// Residuals in closed form: after j rejections the target law is max(p - a_j q, 0) / S_j
// with a_0 = 0, S_0 = 1, a_{j+1} = a_j + S_j / c_j, c_j = 1 - (q mass of the rejected
// siblings), S_{j+1} = sum max(p - a_{j+1} q, 0), and the draft law is q / c_j on the
// siblings not yet tried.  This equals the literal update p_{j+1} = max(p_j - q_j, 0)/Z,
// q_{j+1} = q_j without x_j renormalised (induction on j: a rejected x_j has
// p_j(x_j) < q_j(x_j), so it stays at zero residual for every later a).  Acceptance of x_j:
// u_j * q(x_j) * S_j < max(p(x_j) - a_j q(x_j), 0) * c_j.
// =======================================================================================
__global__ __launch_bounds__(256) void k_vs_init(int R, int B, uint32_t round,
                                                 const int32_t* root_token, dt_tree tree,
                                                 VState* state, uint64_t* vred, dt_verify_out out) {
    const int req = blockIdx.x * blockDim.x + threadIdx.x;
    if (req >= R) return;
    VState s;
    // a bad root or a build whose internal wait gave up: nothing is emitted
    s.active = (tree.status[req] & (DT_REQ_BAD_ROOT | DT_REQ_SYNC_TIMEOUT)) ? 0 : 1;
    s.v = -1;
    s.row = 0;
    s.depth = 0;
    s.token = root_token[req];
    s.nacc = 0;
    s.nemit = 0;
    s.pad = 0;
    s.hash = root_hash(round, req, s.token);
    state[req] = s;
    // the chain's exchange slots: no slot may hold a tag of this round's steps yet
    for (int i = 0; i < kVsPhases * kVsMaxSplits; ++i) vred[(size_t)req * kVsPhases * kVsMaxSplits + i] = 0ull;
    for (int i = 0; i < B; ++i) out.path[(size_t)req * B + i] = -1;
    for (int i = 0; i <= B; ++i) out.out_tokens[(size_t)req * (B + 1) + i] = -1;
    out.accept_len[req] = 0;
    out.n_out[req] = 0;
}

struct VsArgs {
    const void* L;
    const void* U;
    const void* Wt;
    const void* target;
    const VState* state;
    float* vrow;
    float* vpart;
    int R, B, V, r, Ncap, NC, S;
    float y2scale;
    int bf16;
    int vec;  // bf16 logits, V a multiple of 8, 16-byte aligned L and target: 16-byte loads
};

template <bool HEAD_BF16>
__global__ __launch_bounds__(256) void k_vs_rows(const VsArgs a) {
    const int T = (a.R + kTileRows - 1) / kTileRows;
    const int tile = blockIdx.x / a.S, split = blockIdx.x % a.S;
    if (tile >= T) return;
    const int m0 = tile * kTileRows;
    const int nrows = min(kTileRows, a.R - m0);
    __shared__ __attribute__((aligned(16))) uint16_t sA[HEAD_BF16 ? kTileRows * kAStride : 1];
    __shared__ __attribute__((aligned(16))) float sAf[HEAD_BF16 ? 1 : kTileRows * kAfStride];
    __shared__ float sZ[kTileRows * kZStride];
    __shared__ int sLive[kTileRows];
    __shared__ int sAny;
    const int tid = threadIdx.x;
    if (tid == 0) sAny = 0;
    __syncthreads();
    if (tid < kTileRows) {
        int live = 0;
        if (tid < nrows) {
            const VState& s = a.state[m0 + tid];
            live = s.active && s.depth < a.B;
        }
        sLive[tid] = live;
        if (live) atomicOr(&sAny, 1);
    }
    __syncthreads();
    if (!sAny) return;
    load_a_tile<HEAD_BF16>(a.U, a.r, nrows, [&](int row) {
        const int t = sLive[row] ? a.state[m0 + row].token : 0;
        return (uint32_t)t < (uint32_t)a.V ? t : 0;  // never index U out of range
    }, sA, sAf);
    __syncthreads();

    const int erow = tid >> 2, epart = tid & 3;
    const bool eactive = erow < nrows && sLive[erow];
    const int req = m0 + erow;
    VState st;
    if (eactive) st = a.state[req];
    const size_t lbase = eactive ? ((size_t)req * a.B + st.depth) * (size_t)a.V : 0;
    const size_t tbase = eactive ? ((size_t)req * (a.Ncap + 1) + st.row) * (size_t)a.V : 0;
    Lse2 lq, lp;
    lq.init();
    lp.init();
    const int c_beg = (int)((long long)split * a.NC / a.S);
    const int c_end = (int)((long long)(split + 1) * a.NC / a.S);
    const bool two = nrows > 32;
    for (int c = c_beg; c < c_end; ++c) {
        const int col0 = c * kChunkCols;
        mma_chunk<HEAD_BF16>(a.Wt, a.V, a.r, col0, two, sA, sAf, sZ);
        if (eactive) {
            const int cb = col0 + epart * 32;
            const float* zr = sZ + erow * kZStride + epart * 32;
            float* vr = a.vrow + (size_t)req * a.V;
            float mq = -INFINITY, mp = -INFINITY;
            float yq[32], yp[32];
            if (a.vec && cb + 32 <= a.V) {
                // whole 32-column part inside the row: 16-byte loads of the block and target
                // logits, 16-byte stores of the draft row
                const uint4* lv = (const uint4*)((const uint16_t*)a.L + lbase + cb);
                const uint4* tv = (const uint4*)((const uint16_t*)a.target + tbase + cb);
                uint4 lw[4], tw[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    lw[g] = lv[g];
                    tw[g] = tv[g];
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t l4[4] = {lw[g].x, lw[g].y, lw[g].z, lw[g].w};
                    const uint32_t t4[4] = {tw[g].x, tw[g].y, tw[g].z, tw[g].w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int j = 8 * g + 2 * h;
                        yq[j] = (zr[j] + bf16_lo(l4[h])) * a.y2scale;
                        yq[j + 1] = (zr[j + 1] + bf16_hi(l4[h])) * a.y2scale;
                        yp[j] = bf16_lo(t4[h]) * a.y2scale;
                        yp[j + 1] = bf16_hi(t4[h]) * a.y2scale;
                    }
                }
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    mq = fmaxf(mq, yq[j]);
                    mp = fmaxf(mp, yp[j]);
                }
                float4* vo = (float4*)(vr + cb);
#pragma unroll
                for (int g = 0; g < 8; ++g)
                    vo[g] = make_float4(yq[4 * g], yq[4 * g + 1], yq[4 * g + 2], yq[4 * g + 3]);
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const int x = cb + j;
                    if (x < a.V) {
                        yq[j] = (zr[j] + load_logit(a.L, lbase + x, a.bf16)) * a.y2scale;
                        yp[j] = load_logit(a.target, tbase + x, a.bf16) * a.y2scale;
                        vr[x] = yq[j];
                        mq = fmaxf(mq, yq[j]);
                        mp = fmaxf(mp, yp[j]);
                    } else {
                        yq[j] = -INFINITY;
                        yp[j] = -INFINITY;
                    }
                }
            }
            // (the hardware exp2: terms below 2^-126 of the block maximum flush to zero, far
            // below float32 resolution of a sum that holds the maximum's 1)
            float sq = 0.0f, sp = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                if (cb + j < a.V) {
                    sq += __builtin_amdgcn_exp2f(yq[j] - mq);
                    sp += __builtin_amdgcn_exp2f(yp[j] - mp);
                }
            }
            if (mq != -INFINITY) {
                lq.merge(mq, sq);
                lp.merge(mp, sp);
            }
        }
        __syncthreads();
    }
    lq.merge_xor(1);
    lq.merge_xor(2);
    lp.merge_xor(1);
    lp.merge_xor(2);
    if (eactive && epart == 0) {
        float* rec = a.vpart + ((size_t)req * a.S + split) * 4;
        rec[0] = lq.m;
        rec[1] = lq.s;
        rec[2] = lp.m;
        rec[3] = lp.s;
    }
}

// bf16 head and logits, V a multiple of 8, 16-byte aligned rows: the draft rows on the
// expansion's transposed block (W as the MFMA A operand straight from memory, the walking
// requests' U rows from LDS as B, the block logits as the accumulators' initial values), so
// that lane l holds request m0 + 32q + l % 32 at 16 columns of each 32-column block; the
// draft row is stored and both online log-sum-exps run on those registers.  A workgroup
// takes up to 64 requests (two row blocks) over one vocabulary split, its four wavefronts
// the split's blocks w, w + 4, ...; the next block's W fragments, block logits and target
// logits are in flight while the current block's epilogue runs.  Workgroup b runs on XCD
// b % 8 and takes split (b / 8 / T) * 8 + b % 8 of tile (b / 8) % T.
constexpr int kVsTile = 64;
constexpr int kVsRowWaves = 4;

// Four groups of 4 bf16 of a row at the lane's columns c0 + 8j + 4h (clamped into the row
// past V; those columns are masked by the epilogue).
__device__ __forceinline__ void vs_row_words(const VsArgs& a, const void* base, size_t rb, int c0,
                                             int h, uint2 (&g)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = c0 + 8 * j + 4 * h;
        g[j] = *(const uint2*)((const uint16_t*)base + rb + (c < a.V ? c : a.V - 4));
    }
}

// z = L + U.W of one request at the lane's 16 columns and tg its target words there: stores
// the draft row and folds both rows into the online log-sum-exps (log2 units).
__device__ __forceinline__ void vs_row_epi(const VsArgs& a, const f32x16& z, const uint2 (&tg)[4],
                                           int c0, int h, float* vr, Lse2& lq, Lse2& lp) {
    const bool full = c0 + kBlockCols <= a.V;
    float yq[16], yp[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float t4[4] = {bf16_lo(tg[j].x), bf16_hi(tg[j].x), bf16_lo(tg[j].y), bf16_hi(tg[j].y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool in = full || c0 + 8 * j + 4 * h + i < a.V;
            yq[4 * j + i] = in ? z[4 * j + i] * a.y2scale : -INFINITY;
            yp[4 * j + i] = in ? t4[i] * a.y2scale : -INFINITY;
        }
        const int c = c0 + 8 * j + 4 * h;
        if (full) {
            *(float4*)(vr + c) = make_float4(yq[4 * j], yq[4 * j + 1], yq[4 * j + 2], yq[4 * j + 3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (c + i < a.V) vr[c + i] = yq[4 * j + i];
        }
    }
    float mq = yq[0], mp = yp[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
        mq = fmaxf(mq, yq[e]);
        mp = fmaxf(mp, yp[e]);
    }
    float sq = 0.0f, sp = 0.0f;
    if (mq != -INFINITY) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {  // (hardware exp2, as in k_vs_rows)
            sq += __builtin_amdgcn_exp2f(yq[e] - mq);
            sp += __builtin_amdgcn_exp2f(yp[e] - mp);
        }
        lq.merge(mq, sq);
        lp.merge(mp, sp);
    }
}

__global__ __launch_bounds__(kVsRowWaves * 64) void k_vs_rows_blocks(const VsArgs a) {
    __shared__ __align__(16) uint16_t sA[kVsTile * kAStride];
    __shared__ int sTok[kVsTile];
    static_assert(kVsTile == kTileRows, "one A tile of two 32-row blocks");
    __shared__ size_t sLb[kVsTile], sTb[kVsTile];
    __shared__ int sLive[kVsTile];
    __shared__ Lse2 sW[2][kVsRowWaves][kVsTile];
    __shared__ int sAny;
    const int T = (a.R + kVsTile - 1) / kVsTile;
    const int b = blockIdx.x, idx = b >> 3;
    const int tile = idx % T, split = (idx / T) * 8 + (b & 7);
    if (split >= a.S) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, p0 = lane & 31;
    const int m0 = tile * kVsTile;
    const int nrows = min(kVsTile, a.R - m0);
    if (tid == 0) sAny = 0;
    __syncthreads();
    if (tid < kVsTile) {
        int live = 0, tok = -1;
        size_t lb = 0, tb = 0;
        if (tid < nrows) {
            const VState s = a.state[m0 + tid];
            live = s.active && s.depth < a.B;
            if (live) {
                const int req = m0 + tid;
                tok = (uint32_t)s.token < (uint32_t)a.V ? s.token : 0;  // never index U out of range
                lb = ((size_t)req * a.B + s.depth) * (size_t)a.V;
                tb = ((size_t)req * (a.Ncap + 1) + s.row) * (size_t)a.V;
            }
        }
        sLive[tid] = live;
        sTok[tid] = tok;
        sLb[tid] = lb;
        sTb[tid] = tb;
        if (live) atomicOr(&sAny, 1);
    }
    __syncthreads();
    if (!sAny) return;
    load_a_tile<true>(a.U, a.r, nrows, [&](int row) { return sTok[row]; }, sA, nullptr);
    __syncthreads();
    const int NB = (a.V + kBlockCols - 1) / kBlockCols;
    const int b_beg = (int)((long)split * NB / a.S), b_end = (int)((long)(split + 1) * NB / a.S);
    const int nq = (nrows + 31) >> 5;
    Lse2 lq[2], lp[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        lq[q].init();
        lp[q].init();
    }
    // the tile's block and target logits are loaded with the block's W fragments, one block
    // ahead
    bf16x8 wf[16];
    uint2 nl[2][4], nt[2][4];
    const size_t la0 = sLb[p0], la1 = sLb[32 + p0], ta0 = sTb[p0], ta1 = sTb[32 + p0];
    auto prefetch = [&](int c0) {
        load_wfrag(a.Wt, a.V, a.r, c0, wf);
        vs_row_words(a, a.L, la0, c0, h, nl[0]);
        vs_row_words(a, a.target, ta0, c0, h, nt[0]);
        if (nq > 1) {
            vs_row_words(a, a.L, la1, c0, h, nl[1]);
            vs_row_words(a, a.target, ta1, c0, h, nt[1]);
        }
    };
    auto to_acc = [&](const uint2 (&g)[4], f32x16& acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[4 * j + 0] = bf16_lo(g[j].x);
            acc[4 * j + 1] = bf16_hi(g[j].x);
            acc[4 * j + 2] = bf16_lo(g[j].y);
            acc[4 * j + 3] = bf16_hi(g[j].y);
        }
    };
    int blk = b_beg + wave;
    if (blk < b_end) prefetch(blk * kBlockCols);
    for (; blk < b_end; blk += kVsRowWaves) {
        const int c0 = blk * kBlockCols;
        const bool more = blk + kVsRowWaves < b_end;
        {
            const bool two = nq > 1;
            f32x16 acc0, acc1;
            uint2 t0[4], t1[4];  // this block's target words (nt is refilled for the next)
            to_acc(nl[0], acc0);
#pragma unroll
            for (int j = 0; j < 4; ++j) t0[j] = nt[0][j];
            if (two) {
                to_acc(nl[1], acc1);
#pragma unroll
                for (int j = 0; j < 4; ++j) t1[j] = nt[1][j];
            }
            mma_wfrag(wf, two, sA, acc0, acc1);
            if (more) prefetch(c0 + kVsRowWaves * kBlockCols);
            if (sLive[p0]) vs_row_epi(a, acc0, t0, c0, h, a.vrow + (size_t)(m0 + p0) * a.V, lq[0], lp[0]);
            if (two && sLive[32 + p0])
                vs_row_epi(a, acc1, t1, c0, h, a.vrow + (size_t)(m0 + 32 + p0) * a.V, lq[1], lp[1]);
        }
    }
    // lanes l and l ^ 32 hold the same request; then the wavefronts' blocks
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        lq[q].merge_xor(32);
        lp[q].merge_xor(32);
        if (h == 0) {
            sW[0][wave][32 * q + p0] = lq[q];
            sW[1][wave][32 * q + p0] = lp[q];
        }
    }
    __syncthreads();
    if (tid < nrows && sLive[tid]) {
        Lse2 tq, tp;
        tq.init();
        tp.init();
#pragma unroll
        for (int w = 0; w < kVsRowWaves; ++w) {
            tq.merge(sW[0][w][tid].m, sW[0][w][tid].s);
            tp.merge(sW[1][w][tid].m, sW[1][w][tid].s);
        }
        float* rec = a.vpart + ((size_t)(m0 + tid) * a.S + split) * 4;
        rec[0] = tq.m;
        rec[1] = tq.s;
        rec[2] = tp.m;
        rec[3] = tp.s;
    }
}

// Block-wide float sum in a fixed order (deterministic); every thread gets the total.
__device__ float block_sum_f(float v, float* sh) {
    const int tid = threadIdx.x, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if ((tid & 63) == 0) sh[tid >> 6] = v;
    __syncthreads();
    float t = 0.0f;
    for (int i = 0; i < nw; ++i) t += sh[i];
    __syncthreads();
    return t;
}

struct ChainArgs {
    const void* target;
    const VState* state;  // this step's walk states
    VState* next;         // next step's walk states
    const float* vrow;
    const float* vpart;
    uint64_t* vred;
    dt_tree tree;
    dt_verify_out out;
    int R, B, V, k, Ncap, S, SC;
    float y2scale, invT;
    uint32_t seed_lo, seed_hi, spin_limit;
    int bf16;
    int vec;  // bf16 target, V a multiple of 8, 16-byte aligned target: 16-byte loads
};

// Per-request exchange of one partial per slice.  Each reduction of a step has its own slot
// per slice (phase j < k: the residual mass after sibling j; kMaxK: the draw), used at most
// once a step, and a slot word carries the step's tag (walk step + 1, at most 33) in its low
// byte: a workgroup writes its partial and tag in one 64-bit store, and SC threads wait
// (bounded) until every slot of the request holds this step's tag.  Slots are zeroed at the
// start of a round, and a step is one launch, so no slot can hold a stale word with the
// current tag.  Every thread then reads the SC words, in slice order.
__device__ __forceinline__ bool vs_exchange(const ChainArgs& a, int req, int sp, int phase,
                                            uint64_t val, uint32_t tag, uint64_t* parts,
                                            uint64_t* shp) {
    uint64_t* red = a.vred + ((size_t)req * kVsPhases + phase) * kVsMaxSplits;
    const int tid = threadIdx.x;
    if (tid == 0) cst64(red + sp, val | tag);
    int ok = 1;
    if (tid < a.SC) {
        uint64_t w = cld64(red + tid);
        uint32_t it = 0;
        while ((uint32_t)(w & 0xFFu) != tag) {
            __builtin_amdgcn_s_sleep(2);
            if (++it > a.spin_limit) {
                ok = 0;
                break;
            }
            w = cld64(red + tid);
        }
        shp[tid] = w;
    }
    ok = __syncthreads_and(ok);
    if (ok)
        for (int i = 0; i < a.SC; ++i) parts[i] = shp[i];
    __syncthreads();
    return ok != 0;
}

// A draw's slot word: key order in the high half, the complemented token (24 bits) above the
// tag, so that the largest word is the largest key, then the lowest token; 0 above the tag:
// no candidate in the slice.
__device__ __forceinline__ uint64_t vs_draw_word(float key, int tok) {
    return ((uint64_t)ord32(key) << 32) | ((uint64_t)(~(uint32_t)tok & 0xFFFFFFu) << 8);
}

// E = -ln u, an Exp(1) variate, for u = (m + 1/2) 2^-24 with m = the top 24 bits of w (the
// uniform of u01).  A Gumbel variate is -ln E, so ranking x + Gumbel is ranking x - ln E and,
// for positive weights d, ranking d + Gumbel in the log domain is ranking d / E.  For m < 2^23
// u is exact in float32 and E = -ln u; above, v = 1 - u is exact: below 2^-6 the series
// v + v^2/2 + ... + v^5/5 (truncation below 2e-10 relative), otherwise -ln of the rounded u
// (relative error below 2e-6).
__device__ __forceinline__ float exp1_variate(uint32_t w) {
    const uint32_t m = w >> 8;
    const float u = ((float)m + 0.5f) * (1.0f / 16777216.0f);
    const float v = ((float)(16777216u - m) - 0.5f) * (1.0f / 16777216.0f);
    const float poly = v * (1.0f + v * (0.5f + v * (1.0f / 3.0f + v * (0.25f + v * 0.2f))));
    return (m >= (1u << 23) && v < 0.015625f) ? poly : -logf(u);
}

// The chain keeps its slice of p and q in registers: thread t of a workgroup owns the
// 8-element groups g_lo + t + kVsThreads * i of the slice, for i < kVsCached (loaded once a
// step, before the first sibling's test), and recomputes any groups beyond those from memory
// on every pass (only vocabularies above kVsThreads * kVsCached * 8 * kVsMaxSplits words).
constexpr int kVsThreads = 256;
constexpr int kVsCached = 6;
static_assert(kVsChainWords == kVsThreads * kVsCached * 8, "chain slice capacity");

// Eight target logits (raw, not tempered) of group g; -inf past the vocabulary.
__device__ __forceinline__ void vs_load_t8(const ChainArgs& a, size_t tbase, int g, float (&t)[8]) {
    const int x0 = 8 * g;
    if (a.vec) {
        const uint4 w = *(const uint4*)((const uint16_t*)a.target + tbase + x0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            t[2 * h] = bf16_lo(ws[h]);
            t[2 * h + 1] = bf16_hi(ws[h]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            t[e] = x0 + e < a.V ? load_logit(a.target, tbase + x0 + e, a.bf16) : -INFINITY;
    }
}

// Eight draft logits (log2 units) of group g; -inf past the vocabulary.
__device__ __forceinline__ void vs_load_y8(const ChainArgs& a, const float* yq, int g, float (&y)[8]) {
    const int x0 = 8 * g;
    if (a.vec) {
        const float4 v0 = *(const float4*)(yq + x0), v1 = *(const float4*)(yq + x0 + 4);
        y[0] = v0.x; y[1] = v0.y; y[2] = v0.z; y[3] = v0.w;
        y[4] = v1.x; y[5] = v1.y; y[6] = v1.z; y[7] = v1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x0 + e < a.V ? yq[x0 + e] : -INFINITY;
    }
}

// p and q (normalised, linear units) from the raw logits; 0 past the vocabulary.
__device__ __forceinline__ void vs_pq8(const ChainArgs& a, const float (&t)[8], const float (&y)[8],
                                       float lse_q, float lse_p, float (&p)[8], float (&q)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        p[e] = exp2f(t[e] * a.y2scale - lse_p);
        q[e] = exp2f(y[e] - lse_q);
    }
}

// Exponential-race entries of one group of the residual max(p - alpha q, 0) (index 8g + e):
// the key d / E ranks like ln d + Gumbel.
__device__ __forceinline__ void vs_resid_draw8(const ChainArgs& a, uint64_t hash, int g,
                                               const float (&p)[8], const float (&q)[8],
                                               float alpha, ArgMax& best) {
    float d[8];
    bool any = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        d[e] = p[e] - alpha * q[e];
        any |= d[e] > 0.0f;
    }
    if (!any) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4 w = rand4((uint32_t)(2 * g + h), STREAM_RESID, hash, a.seed_lo, a.seed_hi);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float de = d[4 * h + e];
            if (de > 0.0f)
                amax_seq(best, de * __builtin_amdgcn_rcpf(exp1_variate(ws[e])), 8 * g + 4 * h + e);
        }
    }
}

__global__ __launch_bounds__(kVsThreads) void k_vs_split(const ChainArgs a) {
    __shared__ float shf[8];
    __shared__ ArgMax sha[8];
    __shared__ Lse2 shl[2][8];
    __shared__ int s_tok[kMaxNcap], s_par[kMaxNcap];
    __shared__ int s_x[kMaxK];
    __shared__ float s_yx[kMaxK], s_tx[kMaxK];
    __shared__ uint64_t shp[kVsMaxSplits];
    const int req = blockIdx.x / a.SC, sp = blockIdx.x % a.SC, tid = threadIdx.x;
    VState st = a.state[req];
    if (!st.active) {
        if (sp == 0 && tid == 0) a.next[req] = st;
        return;
    }
    const uint32_t tag = (uint32_t)st.nemit + 1u;
    const int n = a.tree.n_nodes[req];
    if (tid < a.Ncap) {
        s_tok[tid] = a.tree.token[(size_t)req * a.Ncap + tid];
        s_par[tid] = a.tree.parent[(size_t)req * a.Ncap + tid];
    }
    // this workgroup's slice: 8-element groups [g_lo, g_hi)
    const int G8 = (a.V + 7) >> 3;
    const int g_lo = (int)((long long)sp * G8 / a.SC), g_hi = (int)((long long)(sp + 1) * G8 / a.SC);
    const int g_rest = g_lo + tid + kVsThreads * kVsCached;  // first group not cached
    const size_t tbase = ((size_t)req * (a.Ncap + 1) + st.row) * (size_t)a.V;
    const float* yq = a.vrow + (size_t)req * a.V;
    int emitted = -1;
    bool descend = false, failed = false;
    uint64_t parts[kVsMaxSplits];
    auto pick = [&](const uint64_t* ps) -> int {
        uint64_t b = 0;
        for (int i = 0; i < a.SC; ++i) b = ps[i] > b ? ps[i] : b;
        return (b >> 8) ? (int)(~(uint32_t)(b >> 8) & 0xFFFFFFu) : -1;
    };
    auto ranked = [&](ArgMax best) -> uint64_t {
        best = block_amax(best, sha);
        return best.v == -INFINITY ? 0ull : vs_draw_word(best.v, best.i);
    };
    if (st.depth == a.B) {
        // a draw from p: Gumbel-max over target / T
        ArgMax best{-INFINITY, 0x7fffffff};
        for (int g = g_lo + tid; g < g_hi; g += kVsThreads) {
            float t[8];
            vs_load_t8(a, tbase, g, t);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 w = rand4((uint32_t)(2 * g + h), STREAM_RESID, st.hash, a.seed_lo,
                                      a.seed_hi);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int x = 8 * g + 4 * h + e;
                    if (x < a.V) amax_seq(best, t[4 * h + e] * a.invT - logf(exp1_variate(ws[e])), x);
                }
            }
        }
        const uint64_t mine = ranked(best);
        if (vs_exchange(a, req, sp, kMaxK, mine, tag, parts, shp)) emitted = pick(parts);
        else failed = true;
    } else {
        // the drawn siblings' raw logits, fetched while the normalisers are formed
        const int32_t* cand = a.tree.cand + ((size_t)req * (a.Ncap + 1) + st.row) * a.k;
        if (tid < a.k) {
            const int x = cand[tid];
            // an empty slot (a ranked list shorter than k, only possible with non-finite
            // draft logits) is no drawn sibling
            const bool ok = x >= 0 && x < a.V;
            s_x[tid] = ok ? x : -1;
            s_yx[tid] = ok ? yq[x] : 0.0f;
            s_tx[tid] = ok ? load_logit(a.target, tbase + x, a.bf16) : 0.0f;
        }
        // the slice's raw logits: every load in flight at once (groups past the slice load
        // its first group and are zeroed when converted)
        float ct[kVsCached][8], cy[kVsCached][8];
#pragma unroll
        for (int i = 0; i < kVsCached; ++i) {
            const int g = g_lo + tid + kVsThreads * i;
            vs_load_t8(a, tbase, g < g_hi ? g : g_lo, ct[i]);
            vs_load_y8(a, yq, g < g_hi ? g : g_lo, cy[i]);
        }
        // normalisers of q and p (log2 units), from the draft-row partials
        Lse2 lq, lp;
        lq.init();
        lp.init();
        {
            constexpr int kRecs = 4;  // records a thread loads before merging (S <= 1024)
            float4 rec[kRecs];
#pragma unroll
            for (int i = 0; i < kRecs; ++i) {
                const int s = tid + kVsThreads * i;
                rec[i] = s < a.S ? *(const float4*)(a.vpart + ((size_t)req * a.S + s) * 4)
                                 : make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
            }
#pragma unroll
            for (int i = 0; i < kRecs; ++i) {
                lq.merge(rec[i].x, rec[i].y);
                lp.merge(rec[i].z, rec[i].w);
            }
            for (int s = tid + kVsThreads * kRecs; s < a.S; s += kVsThreads) {
                const float* r = a.vpart + ((size_t)req * a.S + s) * 4;
                lq.merge(r[0], r[1]);
                lp.merge(r[2], r[3]);
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            lq.merge_xor(off);
            lp.merge_xor(off);
        }
        if ((tid & 63) == 0) {
            shl[0][tid >> 6] = lq;
            shl[1][tid >> 6] = lp;
        }
        __syncthreads();
        lq.init();
        lp.init();
        for (int i = 0; i < kVsThreads / 64; ++i) {
            lq.merge(shl[0][i].m, shl[0][i].s);
            lp.merge(shl[1][i].m, shl[1][i].s);
        }
        const float lse_q = lq.m + log2f(lq.s), lse_p = lp.m + log2f(lp.s);
        float cp[kVsCached][8], cq[kVsCached][8];
#pragma unroll
        for (int i = 0; i < kVsCached; ++i) {
            vs_pq8(a, ct[i], cy[i], lse_q, lse_p, cp[i], cq[i]);
            if (g_lo + tid + kVsThreads * i >= g_hi) {
#pragma unroll
                for (int e = 0; e < 8; ++e) cp[i][e] = cq[i][e] = 0.0f;
            }
        }
        float alpha = 0.0f, S = 1.0f, c = 1.0f;
        for (int j = 0; j < a.k; ++j) {
            const int x = s_x[j];
            if (x < 0) continue;
            const float qx = exp2f(s_yx[j] - lse_q);
            const float px = exp2f(s_tx[j] * a.y2scale - lse_p);
            const uint4 w = rand4((uint32_t)(j >> 2), STREAM_ACCEPT, st.hash, a.seed_lo, a.seed_hi);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
            const float u = u01(ws[j & 3]);
            if (u * qx * S < fmaxf(px - alpha * qx, 0.0f) * c) {
                emitted = x;
                descend = true;
                break;
            }
            alpha += S / c;
            c -= qx;
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < kVsCached; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) part += fmaxf(cp[i][e] - alpha * cq[i][e], 0.0f);
            for (int g = g_rest; g < g_hi; g += kVsThreads) {
                float t8[8], y8[8], p8[8], q8[8];
                vs_load_t8(a, tbase, g, t8);
                vs_load_y8(a, yq, g, y8);
                vs_pq8(a, t8, y8, lse_q, lse_p, p8, q8);
#pragma unroll
                for (int e = 0; e < 8; ++e) part += fmaxf(p8[e] - alpha * q8[e], 0.0f);
            }
            part = block_sum_f(part, shf);
            if (!vs_exchange(a, req, sp, j, (uint64_t)__float_as_uint(part) << 32, tag, parts, shp)) {
                failed = true;
                break;
            }
            S = 0.0f;
            for (int i = 0; i < a.SC; ++i) S += __uint_as_float((uint32_t)(parts[i] >> 32));
            if (!(S > 0.0f)) {
                emitted = x;
                descend = true;
                break;
            }
        }
        if (emitted < 0 && !failed) {
            // every sibling rejected: a draw from the residual max(p - alpha q, 0)
            ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
            for (int i = 0; i < kVsCached; ++i) {
                const int g = g_lo + tid + kVsThreads * i;
                if (g < g_hi) vs_resid_draw8(a, st.hash, g, cp[i], cq[i], alpha, best);
            }
            for (int g = g_rest; g < g_hi; g += kVsThreads) {
                float t8[8], y8[8], p8[8], q8[8];
                vs_load_t8(a, tbase, g, t8);
                vs_load_y8(a, yq, g, y8);
                vs_pq8(a, t8, y8, lse_q, lse_p, p8, q8);
                vs_resid_draw8(a, st.hash, g, p8, q8, alpha, best);
            }
            const uint64_t mine = ranked(best);
            if (vs_exchange(a, req, sp, kMaxK, mine, tag, parts, shp)) emitted = pick(parts);
            else failed = true;
        }
    }
    __syncthreads();
    if (sp != 0 || tid != 0) return;
    if (failed) {
        // an internal wait gave up: the walk ends, n_out = -1 reports it
        st.active = 0;
        a.out.accept_len[req] = st.nacc;
        a.out.n_out[req] = -1;
        a.next[req] = st;
        return;
    }
    int w = -1;
    if (descend) {
        for (int i = 0; i < n; ++i)
            if (s_par[i] == st.v && s_tok[i] == emitted) w = i;
    }
    a.out.out_tokens[(size_t)req * (a.B + 1) + st.nemit] = emitted;
    st.nemit += 1;
    if (w >= 0) {
        a.out.path[(size_t)req * a.B + st.nacc] = w;
        st.nacc += 1;
        st.v = w;
        st.row = w + 1;
        st.depth += 1;
        st.token = emitted;
        st.hash = child_hash(st.hash, emitted);
    } else {
        st.active = 0;
        a.out.accept_len[req] = st.nacc;
        a.out.n_out[req] = st.nemit;
    }
    a.next[req] = st;
}

hipError_t launch_verify_sample(const dt_params* p, const Layout& lay, char* ws,
                                const dt_tree* tree, const void* L, const void* U,
                                const void* Wt, const int32_t* root_token, const void* target,
                                const dt_verify_out* out, hipStream_t st) {
    VState* state = (VState*)(ws + lay.vstate);  // two buffers of R: this step's, the next's
    uint64_t* vred = (uint64_t*)(ws + lay.vred);
    hipLaunchKernelGGL(k_vs_init, dim3((p->R + 255) / 256), dim3(256), 0, st, p->R, p->B,
                       p->round, root_token, *tree, state, vred, *out);
    VsArgs va{};
    va.L = L;
    va.U = U;
    va.Wt = Wt;
    va.target = target;
    va.vrow = (float*)(ws + lay.vrow);
    va.vpart = (float*)(ws + lay.vpart);
    va.R = p->R;
    va.B = p->B;
    va.V = p->V;
    va.r = p->r;
    va.Ncap = p->Ncap;
    va.NC = lay.NC;
    va.S = lay.vsplits;
    va.y2scale = (float)(1.4426950408889634 / (double)p->temperature);
    va.bf16 = p->logits_dtype == DT_BF16;
    const bool al16 = (((uintptr_t)L | (uintptr_t)target) & 15) == 0;
    va.vec = va.bf16 && (p->V & 7) == 0 && al16;
    ChainArgs ca{};
    ca.target = target;
    ca.vrow = va.vrow;
    ca.vpart = va.vpart;
    ca.vred = vred;
    ca.tree = *tree;
    ca.out = *out;
    ca.R = p->R;
    ca.B = p->B;
    ca.V = p->V;
    ca.k = p->k;
    ca.Ncap = p->Ncap;
    ca.S = lay.vsplits;
    ca.SC = lay.vcsplits;
    ca.y2scale = va.y2scale;
    ca.invT = (float)(1.0 / (double)p->temperature);
    ca.seed_lo = (uint32_t)p->seed;
    ca.seed_hi = (uint32_t)(p->seed >> 32);
    ca.spin_limit = kSpinLimit;
    ca.bf16 = va.bf16;
    ca.vec = va.vec;
    // bf16 head and 16-byte-ready logits: the transposed-block rows pass over 64-request
    // tiles and a multiple of 8 splits (about 512 workgroups; never more splits than the
    // partial records hold); otherwise the LDS-tile pass
    const bool blocks = p->head_dtype == DT_BF16 && va.vec;
    dim3 grid;
    if (blocks) {
        const int tiles = (p->R + kVsTile - 1) / kVsTile;
        const int NB = (p->V + kBlockCols - 1) / kBlockCols;
        int sp = (512 / tiles) & ~7;
        sp = sp < 8 ? 8 : sp;
        sp = sp > lay.vsplits ? lay.vsplits : sp;
        sp = sp > NB ? NB : sp;
        va.S = ca.S = sp;
        grid = dim3(tiles * ((sp + 7) / 8) * 8);
    } else {
        grid = dim3(((p->R + kTileRows - 1) / kTileRows) * lay.vsplits);
    }
    for (int step = 0; step <= p->B; ++step) {
        va.state = state + (size_t)(step & 1) * p->R;
        ca.state = va.state;
        ca.next = state + (size_t)((step + 1) & 1) * p->R;
        if (blocks)
            hipLaunchKernelGGL(k_vs_rows_blocks, grid, dim3(kVsRowWaves * 64), 0, st, va);
        else if (p->head_dtype == DT_BF16)
            hipLaunchKernelGGL(k_vs_rows<true>, grid, dim3(256), 0, st, va);
        else
            hipLaunchKernelGGL(k_vs_rows<false>, grid, dim3(256), 0, st, va);
        hipLaunchKernelGGL(k_vs_split, dim3(p->R * lay.vcsplits), dim3(kVsThreads), 0, st, ca);
    }
    return hipGetLastError();
}

}  // namespace dt
