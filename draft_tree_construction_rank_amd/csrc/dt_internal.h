// Internal layout shared by the host code and the kernels of libdtree (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dtree.h"

namespace dt {

constexpr int kTileRows = 64;    // parent rows per expansion tile (two 32-row MFMA blocks)
constexpr int kChunkCols = 128;  // vocabulary columns per chunk (four waves x 32 columns)
constexpr int kMaxNcap = 64;
constexpr int kMaxB = 32;
constexpr int kMaxK = 8;
constexpr int kSelectSlots = 1024;  // >= Ncap + Ncap * k
constexpr int kMaxSplits = 256;     // vocabulary splits per parent row (merge work bound)

// A frontier entry: a node that is (or was) expanded at some level.  self = the low word of
// its selection key (0xFFFFFFFF for the root).
struct alignas(8) FrontEntry {
    uint32_t self;
    int32_t token;
    float s;
    uint32_t pad;
    uint64_t hash;
};

// A generated child.
struct alignas(8) ChildRec {
    int32_t token;
    float s;
    float logq;
    uint32_t pad;
    uint64_t hash;
};

// Offsets (bytes) of every workspace region; sizes depend only on the parameters.
struct Layout {
    size_t rows;      // int2 [R*Ncap]: (request, frontier index) of every parent row
    size_t sync;      // unsigned [kSyncWords]: level counters (offset 0)
    size_t roff;      // int [R]: first parent row of each request at the current level
    size_t pdone;     // int [R]: merge parts finished per request
    size_t front;     // FrontEntry [R][B+1][Ncap]
    size_t fcount;    // int [R][B+1]: frontier size per level (level 0 = the root)
    size_t arena;     // ChildRec [R][B][Ncap][k]
    size_t ckeys;     // u64 [R][Ncap*k]: keys of the children generated at this level
    size_t skeys;     // u64 [R][Ncap]: the selected set, best first
    size_t scount;    // int [R]
    size_t nbeff;     // int [R]: budget after clamping
    size_t rstat;     // int [R]: per-request status bits
    size_t partials;  // float [64*max(G, tiles)][2+3*KT]: per (row, vocabulary split) partials
    size_t vrow;      // float [R][V]: sample verify, draft row (log2 units, then q) of the node
    size_t vprow;     // float [R][V]: sample verify, target probabilities p of the node
    size_t vstate;    // VState [R]
    size_t vpart;     // float [R][vsplits][4]: sample verify partial (max, sum) of q and p
    size_t total;
    int G;            // largest grid of the construction kernel
    int NC;           // vocabulary chunks of 128 columns
    int KT;           // top-k list length used by the kernels (1, 2, 4 or 8)
    int vsplits;      // vocabulary splits per request in sample verify
};

Layout make_layout(const dt_params* p);

inline int kt_for(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8; }

// Floats per partial record of the expansion: (max, sum) + KT x (key, y, token), padded to
// a multiple of 4 for 16-byte accesses.
__host__ __device__ constexpr int rec_floats(int KT) { return ((2 + 3 * KT) + 3) & ~3; }

// Walk state of one request in sample verify.
struct alignas(8) VState {
    int active, v, row, depth, token, nacc, nemit, pad;
    uint64_t hash;
};

// Control words at the start of the workspace.
constexpr int kSyncFinish = 3;  // workgroups done with the select phase
constexpr int kSyncRows = 4;    // parent rows at the current level
constexpr int kSyncWords = 8;

// Arguments of the tree-construction kernels (passed by value).
struct BuildArgs {
    void (*timing_hook)(hipStream_t, int);  // host-only: brackets each expansion launch
    const void* L;
    const void* U;
    const void* Wt;
    const int32_t* root_token;
    const int32_t* n_budget;
    const float* tau;
    unsigned* sync;
    int2* rows;
    int* roff;
    int* pdone;
    FrontEntry* front;
    int* fcount;
    ChildRec* arena;
    uint64_t* ckeys;
    uint64_t* skeys;
    int* scount;
    int* nbeff;
    int* rstat;
    float* partials;
    dt_tree out;
    int R, B, k, V, r, Ncap, NC;
    float y2scale;  // log2(e) / T' : converts z to log2-unit tempered logits
    float invT;     // 1 / T' (sample ranking key)
    uint32_t seed_lo, seed_hi, round;
    int logits_bf16;
    float cal[16];
};

// Host-side launchers (enqueue only).
hipError_t launch_build(const dt_params* p, const Layout& lay, const BuildArgs& a,
                        hipStream_t st);
hipError_t launch_verify_greedy(const dt_params* p, const dt_tree* tree, const void* target,
                                const dt_verify_out* out, hipStream_t st);
hipError_t launch_verify_sample(const dt_params* p, const Layout& lay, char* ws,
                                const dt_tree* tree, const void* L, const void* U,
                                const void* Wt, const int32_t* root_token, const void* target,
                                const dt_verify_out* out, hipStream_t st);

}  // namespace dt
