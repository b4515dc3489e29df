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
constexpr int kMaxSplits = 512;     // vocabulary splits per parent row (merge work bound)
constexpr int kMaxGrid = 256;       // largest grid of the persistent construction kernel
                                    // (one workgroup per CU of an MI355X)
constexpr int kBlockCols = 32;      // vocabulary columns per MFMA block of the expansion
constexpr int kBuildWaves = 8;      // wavefronts per workgroup of the construction kernel
constexpr int kGroupRows = 32 * kBuildWaves;  // parent rows per group-mode expansion item
constexpr size_t kScratchBytes = DT_NOALLOC_SCRATCH_BYTES;  // device scratch of tree_build_noalloc
constexpr int kMaxDevices = 64;
constexpr uint32_t kSpinLimit = 1u << 25;  // default polls of one bounded wait (about 2 s)
constexpr int kResMaxBlocks = 20;  // W-resident kernel: largest vocabulary slice (32-column blocks)
constexpr int kCountRows = 32;     // rows per tdone counter (the smallest expansion tile)

// A frontier entry: a node that is (or was) expanded at some level.  self = the low word of
// its selection key (0xFFFFFFFF for the root).
struct alignas(8) FrontEntry {
    uint32_t self;
    int32_t token;
    float s;
    uint32_t pad;
    uint64_t hash;
};

// A generated child (also what the select reads to rank it: token and survival in the first
// word, the random-stream hash in the third).
struct alignas(8) ChildRec {
    int32_t token;
    float s;
    float logq;
    uint32_t pad;
    uint64_t hash;
};

// A parent row of a level: written by the select that kept the node (by k_build_init for the
// roots) and read by the expansion (token, hash, request) and the merge (survival, hash, F).
struct alignas(16) RowRec {
    int32_t req;
    int32_t fi;     // the node's index in the request's frontier at this level (canonical)
    int32_t token;
    float s;        // the node's survival
    uint64_t hash;  // the node's random stream
    int32_t F;      // parent rows of this request at this level
    int32_t htok;   // head token: whose U row biases the expansion (-1: no bias)
};

// Offsets (bytes) of every workspace region; sizes depend only on the parameters.
struct Layout {
    size_t rows;      // RowRec [2][R*Ncap]: parent rows of a level (double-buffered by level)
    size_t sync;      // unsigned [kSyncWords]: generation, error flag, per-level counters
    size_t tdone;     // unsigned [B+2][tiles]: expansion items finished per level and row tile
    size_t rdone;     // unsigned [B+2][R]: parent rows merged per level and request
    size_t front;     // FrontEntry [R][B+1][Ncap]
    size_t fcount;    // int [R][B+1]: frontier size per level (level 0 = the root)
    size_t arena;     // ChildRec [R][B][Ncap][k]
    size_t skeys;     // u64 [R][Ncap]: the selected set, best first
    size_t scount;    // int [R]
    size_t nbeff;     // int [R]: budget after clamping
    size_t rstat;     // int [R]: per-request status bits
    size_t partials;  // float [64*max(G, tiles)][2+3*KT]: per (row, vocabulary split) partials
    size_t vrow;      // float [R][V]: sample verify, draft row of the node (log2 units)
    size_t vstate;    // VState [R]
    size_t vpart;     // float [R][vsplits][4]: sample verify partial (max, sum) of q and p
    size_t vred;      // u64 [R][kVsPhases][kVsMaxSplits]: per-slice partials of a step's
                      // reductions (residual masses, draws), tagged with the step
    size_t gpart;     // (float, int) [R][gsplits]: greedy verify, split argmax of the root rows
    size_t trace;     // u64 [kMaxGrid][kTraceLevels][16]: phase timestamps (DT_TRACE builds only)
    size_t build_total;  // extent of the regions tree_build uses (a prefix of the layout)
    size_t total;
    int G;            // largest grid of the construction kernel (sizes the partial records)
    int NC;           // vocabulary chunks of 128 columns
    int KT;           // top-k list length used by the kernels (1, 2, 4 or 8)
    int vsplits;      // vocabulary splits per request in sample verify (draft rows)
    int vcsplits;     // workgroups per request of the rejection chain
    int gsplits;      // vocabulary splits per request of the root-row argmax in greedy verify
    bool resident;    // partials sized for the W-resident kernel
};

// allow_resident: size the partial records for the W-resident kernel too (one record per
// row and workgroup), which needs more workspace than the streaming kernel.
Layout make_layout(const dt_params* p, bool allow_resident = true);

inline int kt_for(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8; }

// Floats per partial record of the expansion: (max, sum) + KT x (key, y, token), padded to
// a multiple of 4 for 16-byte accesses.
__host__ __device__ constexpr int rec_floats(int KT) { return ((2 + 3 * KT) + 3) & ~3; }

// Walk state of one request in sample verify (nemit: steps taken, one token emitted each).
struct alignas(8) VState {
    int active, v, row, depth, token, nacc, nemit, pad;
    uint64_t hash;
};
constexpr int kVsMaxSplits = 16;     // chain workgroups per request at most
constexpr int kVsChainWords = 256 * 6 * 8;  // vocabulary words a chain workgroup keeps in
                                            // registers (threads x cached groups x 8)
constexpr int kVsPhases = kMaxK + 1;  // reductions of one step: k residual masses, one draw

// Control words at the start of the workspace.  Per-level words are indexed by the level
// (1..B+1) so that a late workgroup never reads the next level's value.
constexpr int kSyncGen = 0;     // u64: (parent rows of the next level << 32) | (requests with rows
                                // at the next level << 8) | last level whose selects are done
constexpr int kSyncErr = 2;     // set when a bounded wait gives up
constexpr int kSyncAlloc = 8;   // u64 [level]: rows allocated for that level
constexpr int kSyncDone = 80;   // u64 [level]: (selects done << 48) | (requests with rows at
                                // the next level << 32) | rows of the next level
constexpr int kSyncClaim = 160; // u32 [level]: work tickets handed out (expansion items, then
                                // merge rows)
constexpr int kSyncWords = 208;
__host__ __device__ constexpr uint64_t pack_gen(int level, int nreq, int rows) {
    return ((uint64_t)(uint32_t)rows << 32) | ((uint64_t)(uint32_t)nreq << 8) | (uint64_t)level;
}

// Phase timestamps of the construction kernel, written only by builds compiled with
// DT_TRACE: per workgroup and level, sixteen wall-clock stamps (slot meanings at DT_STAMP).
constexpr int kTraceLevels = 40;

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
    unsigned* tdone;
    unsigned* rdone;
    RowRec* rows;
    FrontEntry* front;
    int* fcount;
    ChildRec* arena;
    uint64_t* skeys;
    int* scount;
    int* nbeff;
    int* rstat;
    float* partials;
    dt_tree out;
    uint64_t* trace;  // phase timestamps (DT_TRACE builds only; null otherwise)
    int R, B, k, V, r, Ncap, NC;
    int Tmax;  // row tiles of kTileRows for R * Ncap rows (stride of tdone per level)
    float y2scale;  // log2(e) / T' : converts z to log2-unit tempered logits
    float invT;     // 1 / T' (sample ranking key)
    uint32_t seed_lo, seed_hi, round;
    int logits_bf16;
    uint32_t spin_limit;  // iterations of a bounded wait before it gives up
    int cond;             // DT_COND_*: head token of a row (own token, chain token, none)
    float cal[16];
};

// Host-side launchers (enqueue only).
hipError_t launch_build(const dt_params* p, const Layout& lay, const BuildArgs& a,
                        hipStream_t st);
// tdone counters per level: one per kCountRows parent rows (both kernels index them by a
// row tile of at least that many rows).
inline int max_tiles(int R, int Ncap) { return (R * Ncap + kCountRows - 1) / kCountRows; }
// W-resident construction (build_resident.hip): bf16 head and logits, r = 256, V a
// multiple of 8, and rounds of at most kResMaxRows parent rows per level (R * Ncap): every
// workgroup of that kernel expands every row over its slice, which loses to the streaming
// kernel once levels get wide (measured: 64 requests of 64 nodes ran 1.3x to 2x slower).
// The slice-size check needs the device and happens at launch.
constexpr int kResMaxRows = 128;
inline bool resident_params_ok(const dt_params* p) {
    return p->head_dtype == DT_BF16 && p->logits_dtype == DT_BF16 && p->r == 256 &&
           (p->V & 7) == 0 && p->R * p->Ncap <= kResMaxRows;
}
// Set-up kernel of a round (control words, counters, roots); shared by both kernels.
hipError_t launch_build_init(const BuildArgs& a, hipStream_t st);
// Enqueues the W-resident kernel if it applies on the current device (*used); otherwise
// enqueues nothing.
hipError_t launch_build_resident(const dt_params* p, const Layout& lay, const BuildArgs& a,
                                 hipStream_t st, bool* used);
hipError_t launch_verify_greedy(const dt_params* p, const Layout& lay, char* ws,
                                const dt_tree* tree, const void* target,
                                const dt_verify_out* out, hipStream_t st);
hipError_t launch_verify_sample(const dt_params* p, const Layout& lay, char* ws,
                                const dt_tree* tree, const void* L, const void* U,
                                const void* Wt, const int32_t* root_token, const void* target,
                                const dt_verify_out* out, hipStream_t st);

// Tree attention (attn_kernels.hip): G grouped query heads per key/value head, QG query
// groups of NW wavefronts (one 32-query tile each), S key splits; with S > 1 the workspace
// holds po_bytes of partial outputs, then the (max, sum) pairs.
struct AttnPlan {
    int G, QG, NW, S;
    size_t po_bytes, total;
};
AttnPlan attn_plan(const dt_attn_params* p);
hipError_t launch_tree_attention(const dt_attn_params* p, const AttnPlan& pl, const void* Q,
                                 const void* K, const void* V, const int32_t* ctx_len,
                                 const int32_t* n_nodes, const uint64_t* anc, void* O,
                                 char* ws, hipStream_t st);

// Two-stage M-ary tree (flash_kernels.hip): M = k tokens per depth, NS = 1 + M (B - 1)
// states a request, T tiles of 64 states, SP vocabulary splits; the workspace holds the
// token sets, the per-(state, split) log-sum-exp records, every state's children's
// conditional logits, then stage 1's part lists (P parts a block row).
struct FlashPlan {
    int M, NS, T, SP, P;
    size_t sets_bytes, zc_off, setp_off, total;
};
FlashPlan flash_plan(const dt_params* p);
hipError_t launch_build_flash(const dt_params* p, const FlashPlan& pl, const void* L,
                              const void* U, const void* Wt, const int32_t* root_token,
                              const int32_t* n_budget, const float* tau, const dt_tree* out,
                              char* ws, hipStream_t st);

}  // namespace dt
