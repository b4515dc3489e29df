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

// A tile: rows < nrows take U[token_of(row)], other rows and columns >= r are zero.
// 256 threads.  Ends with the caller's __syncthreads().
template <bool HEAD_BF16, typename TokFn>
__device__ __forceinline__ void load_a_tile(const void* U, int r, int nrows, TokFn token_of,
                                            uint16_t* sA, float* sAf) {
    const int tid = threadIdx.x;
    if constexpr (HEAD_BF16) {
        const int segs = kAStride / 8;  // 16-byte segments per LDS row (incl. padding)
        for (int i = tid; i < kTileRows * segs; i += 256) {
            const int row = i / segs, seg = i % segs;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < nrows && seg * 8 < r)
                v = *(const uint4*)((const uint16_t*)U + (size_t)token_of(row) * r + seg * 8);
            *(uint4*)(sA + row * kAStride + seg * 8) = v;
        }
    } else {
        for (int i = tid; i < kTileRows * kAfStride; i += 256) {
            const int row = i / kAfStride, kk = i % kAfStride;
            float v = 0.0f;
            if (row < nrows && kk < r) v = ((const float*)U)[(size_t)token_of(row) * r + kk];
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
        const int nsteps = (r + 15) >> 4;
        bf16x8 bfr[16];
        const int khalf = (lane >> 5) * 8;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (s < nsteps && bcol < V && s * 16 + khalf < r)
                v = *(const uint4*)((const uint16_t*)Wt + (size_t)bcol * r + s * 16 + khalf);
            bfr[s] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (s < nsteps) {
                const uint4 a0 = *(const uint4*)(sA + (lane & 31) * kAStride + s * 16 + khalf);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0),
                                                               bfr[s], acc0, 0, 0, 0);
                if (two) {
                    const uint4 a1 =
                        *(const uint4*)(sA + (32 + (lane & 31)) * kAStride + s * 16 + khalf);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a1), bfr[s], acc1, 0, 0, 0);
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

}  // namespace dt
