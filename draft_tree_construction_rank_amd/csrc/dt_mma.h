// The Markov-bias contraction tile shared by the expansion and sample-verify kernels:
// C[64 rows x 128 columns] = A[64 x r] . Wt[128 cols x r]^T on gfx950 MFMA (bf16 32x32x16 with
// fp32 accumulation; f32 32x32x2 for float32 heads), written to an LDS tile.
#pragma once

#include <hip/hip_runtime.h>

#include "dt_internal.h"

namespace dt {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kAStride = 256 + 8;  // bf16 elements per LDS row of A (padding against conflicts)
constexpr int kAfStride = 66;      // floats per LDS row of A for float32 heads (r <= 64)
constexpr int kZStride = kChunkCols + 4;

// Zero that the compiler cannot see through: added to the thread index where per-thread
// address arithmetic would otherwise be hoisted out of a persistent loop and kept (spilled)
// for the kernel's lifetime.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// A tile: rows < nrows take U[token_of(row)] (a zero row where token_of(row) < 0), other
// rows and columns >= r are zero.  NT threads (the workgroup size).  Ends with the
// caller's __syncthreads().
template <bool HEAD_BF16, int NT = 256, typename TokFn>
__device__ __forceinline__ void load_a_tile(const void* U, int r, int nrows, TokFn token_of,
                                            uint16_t* sA, float* sAf) {
    const int tid = threadIdx.x + opaque_zero();
    if constexpr (HEAD_BF16) {
        // 64 rows x 33 16-byte segments: every address is clamped into the row so that all
        // loads of a thread are unconditional and can be in flight together.
        constexpr int segs = kAStride / 8;
        constexpr int per = (kTileRows * segs + NT - 1) / NT;
        uint4 v[per];
#pragma unroll
        for (int q = 0; q < per; ++q) {
            const int i = tid + q * NT;
            const int row = i / segs, seg = i % segs;
            const int t = (i < kTileRows * segs && row < nrows) ? token_of(row) : 0;
            const bool ok = i < kTileRows * segs && row < nrows && seg * 8 < r && t >= 0;
            const int tok = t >= 0 ? t : 0;
            const uint4 x = *(const uint4*)((const uint16_t*)U + (size_t)tok * r +
                                            (seg * 8 < r ? seg * 8 : 0));
            v[q] = ok ? x : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < per; ++q) {
            const int i = tid + q * NT;
            if (i < kTileRows * segs) *(uint4*)(sA + (i / segs) * kAStride + (i % segs) * 8) = v[q];
        }
    } else {
        for (int i = tid; i < kTileRows * kAfStride; i += NT) {
            const int row = i / kAfStride, kk = i % kAfStride;
            float v = 0.0f;
            if (row < nrows && kk < r) {
                const int t = token_of(row);
                if (t >= 0) v = ((const float*)U)[(size_t)t * r + kk];
            }
            sAf[i] = v;
        }
    }
}

// One 64 x 128 chunk starting at column col0 (columns >= V give zeros).  Wave w computes
// columns col0 + 32w .. +32; `two` selects whether rows 32..63 are live.  Ends with a
// __syncthreads() so the tile in sZ is visible to the whole workgroup.
template <bool HEAD_BF16>
__device__ __forceinline__ void mma_chunk(const void* Wt, int V, int r, int col0, bool two,
                                          const uint16_t* sA, const float* sAf, float* sZ) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bcol = col0 + wave * 32 + (lane & 31);
    f32x16 acc0, acc1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        acc0[i] = 0.0f;
        acc1[i] = 0.0f;
    }
    if constexpr (HEAD_BF16) {
        // Two halves of 8 K-steps: 8 unconditional 16-byte loads from clamped addresses are
        // issued back to back, then 8 (or 16) MFMAs.  Columns past V read column V-1 (their
        // results are never used); K offsets past r read offset 0 (multiplied by the zero
        // padding of the A tile), so all 16 K-steps always run.
        const int khalf = (lane >> 5) * 8;
        const uint16_t* wrow = (const uint16_t*)Wt + (size_t)(bcol < V ? bcol : V - 1) * r;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 bfr[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int kk = (h * 8 + s) * 16 + khalf;
                bfr[s] = __builtin_bit_cast(bf16x8, *(const uint4*)(wrow + (kk < r ? kk : 0)));
            }
            if (two) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int ko = (h * 8 + s) * 16 + khalf;
                    const uint4 a0 = *(const uint4*)(sA + (lane & 31) * kAStride + ko);
                    const uint4 a1 = *(const uint4*)(sA + (32 + (lane & 31)) * kAStride + ko);
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0),
                                                                   bfr[s], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1),
                                                                   bfr[s], acc1, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int ko = (h * 8 + s) * 16 + khalf;
                    const uint4 a0 = *(const uint4*)(sA + (lane & 31) * kAStride + ko);
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0),
                                                                   bfr[s], acc0, 0, 0, 0);
                }
            }
        }
    } else {
        const int nsteps = (r + 1) >> 1;
        const int kh = lane >> 5;
        for (int s = 0; s < nsteps; ++s) {
            const int kk = s * 2 + kh;
            const float b = (bcol < V && kk < r) ? ((const float*)Wt)[(size_t)bcol * r + kk] : 0.0f;
            const float a0 = sAf[(lane & 31) * kAfStride + kk];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b, acc0, 0, 0, 0);
            if (two) {
                const float a1 = sAf[(32 + (lane & 31)) * kAfStride + kk];
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b, acc1, 0, 0, 0);
            }
        }
    }
    // 32x32 result layout: element i of lane l is row 8*(i/4) + 4*(l/32) + i%4, column l%32.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        sZ[row * kZStride + wave * 32 + (lane & 31)] = acc0[i];
        if (two) sZ[(32 + row) * kZStride + wave * 32 + (lane & 31)] = acc1[i];
    }
    __syncthreads();
}

// Transposed block for the expansion: D[c][p] = Wt[c0 + c] . A[p] for 32 vocabulary columns c
// and the tile's parent rows p, with the head rows of W as the MFMA A operand and the parent
// rows (from LDS) as the B operand.  In the 32x32 output layout lane l then holds parent row
// p = l%32 (acc0; row 32 + l%32 in acc1) at columns c0 + 8(e/4) + 4(l/32) + e%4, e = 0..15,
// so a parent row's online softmax and top-k run on the accumulators directly.  Columns past
// V read column V-1 and K offsets past r read offset 0 (the LDS rows are zero there).
//
// bf16 heads: the 16 A fragments of a block (16 KB per wavefront) are loaded by
// load_wfrag() into registers, so the caller can issue the next block's loads before it
// works on the current one.
__device__ __forceinline__ void load_wfrag(const void* Wt, int V, int r, int c0, bf16x8 (&wf)[16]) {
    const int lane = threadIdx.x & 63;
    const int col = c0 + (lane & 31);
    // recomputed at every call: hoisted out of the persistent loop, the sixteen offsets were
    // spilled and reloaded one round trip at a time
    const int khalf = (lane >> 5) * 8 + opaque_zero();
    const uint16_t* wrow = (const uint16_t*)Wt + (size_t)(col < V ? col : V - 1) * r;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int kk = s * 16 + khalf;
        wf[s] = __builtin_bit_cast(bf16x8, *(const uint4*)(wrow + (kk < r ? kk : 0)));
    }
}

// Accumulates onto acc0 (and acc1 when `two`); the caller initialises them.
__device__ __forceinline__ void mma_wfrag(const bf16x8 (&wf)[16], bool two, const uint16_t* sA,
                                          f32x16& acc0, f32x16& acc1) {
    const int lane = threadIdx.x & 63;
    const uint16_t* b0 = sA + (lane & 31) * kAStride + (lane >> 5) * 8;
    if (two) {
        const uint16_t* b1 = b0 + 32 * kAStride;
        // B fragments in groups of four: the LDS latency overlaps the MFMAs of the group before
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint4 u0[4], u1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u0[q] = *(const uint4*)(b0 + (4 * g + q) * 16);
                u1[q] = *(const uint4*)(b1 + (4 * g + q) * 16);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[4 * g + q],
                                                               __builtin_bit_cast(bf16x8, u0[q]), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[4 * g + q],
                                                               __builtin_bit_cast(bf16x8, u1[q]), acc1, 0, 0, 0);
            }
        }
    } else {
        uint4 u0[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) u0[s] = *(const uint4*)(b0 + s * 16);
#pragma unroll
        for (int s = 0; s < 16; ++s)
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], __builtin_bit_cast(bf16x8, u0[s]),
                                                           acc0, 0, 0, 0);
    }
}

// float32 heads (r <= 64): the whole transposed block, f32 32x32x2 MFMA.
// Accumulates onto acc0 (and acc1 when `two`); the caller initialises them.
__device__ __forceinline__ void xblock_mma_f32(const void* Wt, int V, int r, int c0, bool two,
                                               const float* sAf, f32x16& acc0, f32x16& acc1) {
    const int lane = threadIdx.x & 63;
    const int col = c0 + (lane & 31);
    const int kh = lane >> 5;
    const float* wrow = (const float*)Wt + (size_t)(col < V ? col : V - 1) * r;
    const float* b0 = sAf + (lane & 31) * kAfStride + kh;
    const int nsteps = (r + 1) >> 1;
    for (int s = 0; s < nsteps; ++s) {
        const int kk = 2 * s + kh;
        const float w = wrow[kk < r ? kk : 0];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(w, b0[2 * s], acc0, 0, 0, 0);
        if (two) acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(w, b0[32 * kAfStride + 2 * s], acc1, 0, 0, 0);
    }
}

}  // namespace dt
