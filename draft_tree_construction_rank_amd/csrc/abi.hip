// Host side of libdtree: argument validation, workspace layout and the launch sequence.
// Every entry point validates on the host and returns before enqueuing anything when an
// argument is bad; otherwise it only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "dt_internal.h"

namespace dt {

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(const dt_params* p, bool allow_resident) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return o;
    };
    const size_t R = p->R, B = p->B, N = p->Ncap, k = p->k, V = p->V;
    L.NC = (int)((V + kChunkCols - 1) / kChunkCols);
    L.KT = kt_for(p->k);
    L.G = kMaxGrid;
    const size_t tmax = (R * N + kTileRows - 1) / kTileRows;
    // records: (parent row, vocabulary split) pairs; a level of T row groups of g rows uses
    // at most g * max(G, T) of them (g = kTileRows in tile mode, kGroupRows in group mode),
    // because splits_for() keeps S <= max(1, G / T): more splits would write past this region
    size_t cap_rows = (size_t)kGroupRows * (tmax > (size_t)L.G ? tmax : (size_t)L.G);
    // the W-resident kernel writes one record per parent row and workgroup
    L.resident = allow_resident && resident_params_ok(p);
    if (L.resident && R * N * (size_t)kMaxGrid > cap_rows) cap_rows = R * N * (size_t)kMaxGrid;
    L.sync = take(kSyncWords * sizeof(unsigned));
    L.tdone = take((B + 2) * (size_t)max_tiles((int)R, (int)N) * sizeof(unsigned));
    L.rdone = take((B + 2) * R * sizeof(unsigned));
    L.rows = take(2 * R * N * sizeof(RowRec));
    L.front = take(R * (B + 1) * N * sizeof(FrontEntry));
    L.fcount = take(R * (B + 1) * sizeof(int));
    L.arena = take(R * B * N * k * sizeof(ChildRec));
    L.skeys = take(R * N * sizeof(uint64_t));
    L.scount = take(R * sizeof(int));
    L.nbeff = take(R * sizeof(int));
    L.rstat = take(R * sizeof(int));
    L.partials = take(cap_rows * rec_floats(L.KT) * sizeof(float));
    L.build_total = off;  // everything below is used by the verifiers only
    L.vsplits = 0;
    L.vrow = L.vstate = L.vpart = L.vred = 0;
    L.vcsplits = 0;
    if (p->mode == DT_SAMPLE) {
        // sample verify: ceil(R/64) request tiles x vsplits vocabulary splits, grid <= 1024
        const int tiles = (int)((R + kTileRows - 1) / kTileRows);
        int s = 1024 / tiles;
        if (s >= 8) s &= ~7;
        if (s > L.NC) s = L.NC;
        if (s < 1) s = 1;
        L.vsplits = s;
        // rejection chain: about 512 workgroups over all requests, at least enough that a
        // workgroup's slice fits the groups its threads cache (kVsChainWords), at most
        // kVsMaxSplits each and at most one per 8-word group of the vocabulary
        int c = (int)(512 / R);
        const int need = (int)((V + kVsChainWords - 1) / kVsChainWords);
        if (c < need) c = need;
        c = c < 1 ? 1 : (c > kVsMaxSplits ? kVsMaxSplits : c);
        if ((size_t)c > (V + 7) / 8) c = (int)((V + 7) / 8);
        L.vcsplits = c;
        L.vrow = take(R * V * sizeof(float));
        L.vstate = take(2 * R * sizeof(VState));
        L.vpart = take(R * (size_t)L.vsplits * 4 * sizeof(float));
        L.vred = take(R * (size_t)kVsPhases * kVsMaxSplits * sizeof(uint64_t));
    }
    {
        // greedy verify: the root rows are split over about 1024 workgroups, each of at least
        // 256 sixteen-byte segments of the row
        const size_t segs = (V + 7) / 8;
        size_t s = 1024 / R;
        if (s > 64) s = 64;
        if (s > segs / 256) s = segs / 256;
        if (s < 1) s = 1;
        L.gsplits = (int)s;
        L.gpart = take(R * s * 8);
    }
#ifdef DT_TRACE
    // phase timestamps (instrumented builds only): last, and counted in the build's extent
    L.trace = take((size_t)kMaxGrid * kTraceLevels * 16 * sizeof(uint64_t));
    L.build_total = off;
#endif
    L.total = off;
    return L;
}

static dt_status validate(const dt_params* p) {
    if (!p) return DT_EINVAL;
    if (p->R < 1 || p->R > 4096) return DT_EINVAL;
    if (p->B < 1 || p->B > kMaxB) return DT_EINVAL;
    if (p->k < 1 || p->k > kMaxK) return DT_EINVAL;
    if (p->V < 1 || p->V > (1 << 24) || p->k > p->V) return DT_EINVAL;
    if (p->Ncap < 1 || p->Ncap > kMaxNcap) return DT_EINVAL;
    if (p->logits_dtype != DT_F32 && p->logits_dtype != DT_BF16) return DT_EINVAL;
    if (p->head_dtype != DT_F32 && p->head_dtype != DT_BF16) return DT_EINVAL;
    if (p->mode != DT_GREEDY && p->mode != DT_SAMPLE) return DT_EINVAL;
    if (p->head_dtype == DT_BF16 && (p->r < 8 || p->r > 256 || (p->r & 7) != 0)) return DT_EINVAL;
    if (p->head_dtype == DT_F32 && (p->r < 1 || p->r > 64)) return DT_EINVAL;
    if (!std::isfinite(p->temperature) || !(p->temperature > 0.0f)) return DT_EINVAL;
    for (int i = 0; i < 16; ++i) {
        const float c = p->cal[i];
        if (!(c >= 0.0f && c <= 1.0f)) return DT_EINVAL;
        if (i > 0 && c < p->cal[i - 1]) return DT_EINVAL;
    }
    if (p->cond != DT_COND_PARENT && p->cond != DT_COND_CHAIN && p->cond != DT_COND_NONE)
        return DT_EINVAL;
    if (p->cond != DT_COND_PARENT && p->mode != DT_GREEDY) return DT_EINVAL;
    return DT_OK;
}

static bool tree_ptrs_ok(const dt_tree* t) {
    return t && t->token && t->parent && t->depth && t->anc_mask && t->surv && t->logq &&
           t->n_nodes && t->cand && t->status;
}

static bool verify_ptrs_ok(const dt_verify_out* o) {
    return o && o->accept_len && o->path && o->out_tokens && o->n_out;
}

// ---- optional event timing of the expansion kernel
struct Timing {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;
    size_t used = 0;
};
static Timing g_timing;

static void timing_mark(hipStream_t st) {
    if (!g_timing.on) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.used == g_timing.pool.size()) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        g_timing.pool.push_back(e);
    }
    (void)hipEventRecord(g_timing.pool[g_timing.used++], st);
}

static void timing_hook(hipStream_t st, int) { timing_mark(st); }

// ---- bound of the construction kernel's internal waits: kSpinLimit polls, or the value of
// the environment variable DT_WAIT_LIMIT (a test hook: a small bound makes a round give up
// and report DT_REQ_SYNC_TIMEOUT while every kernel still exits normally)
static uint32_t wait_limit() {
    const char* e = std::getenv("DT_WAIT_LIMIT");
    if (!e || !*e) return kSpinLimit;
    char* end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    if (end == e || v < 1 || v > kSpinLimit) return kSpinLimit;
    return (uint32_t)v;
}

// ---- tree_build: argument checks and the enqueue shared by both entry points
static dt_status check_build_args(const dt_params* p, const void* block_logits, const void* U,
                                  const void* Wt, const int32_t* root_token,
                                  const int32_t* n_budget, const float* tau, const dt_tree* out) {
    const dt_status v = validate(p);
    if (v != DT_OK) return v;
    if (!block_logits || !U || !Wt || !root_token || !n_budget || !tau || !tree_ptrs_ok(out))
        return DT_EINVAL;
    if (((uintptr_t)U & 15) || ((uintptr_t)Wt & 15) || ((uintptr_t)block_logits & 15))
        return DT_EINVAL;
    return DT_OK;
}

static dt_status enqueue_build(const dt_params* p, const Layout& lay, const void* block_logits,
                               const void* U, const void* Wt, const int32_t* root_token,
                               const int32_t* n_budget, const float* tau, const dt_tree* out,
                               char* ws, hipStream_t st, bool timed) {
    const float Teff = (p->mode == DT_SAMPLE) ? p->temperature : 1.0f;
    BuildArgs a{};
    a.timing_hook = timed ? timing_hook : nullptr;
    a.L = block_logits;
    a.U = U;
    a.Wt = Wt;
    a.root_token = root_token;
    a.n_budget = n_budget;
    a.tau = tau;
    a.sync = (unsigned*)(ws + lay.sync);
    a.rows = (RowRec*)(ws + lay.rows);
    a.tdone = (unsigned*)(ws + lay.tdone);
    a.rdone = (unsigned*)(ws + lay.rdone);
    a.front = (FrontEntry*)(ws + lay.front);
    a.fcount = (int*)(ws + lay.fcount);
    a.arena = (ChildRec*)(ws + lay.arena);
    a.skeys = (uint64_t*)(ws + lay.skeys);
    a.scount = (int*)(ws + lay.scount);
    a.nbeff = (int*)(ws + lay.nbeff);
    a.rstat = (int*)(ws + lay.rstat);
    a.partials = (float*)(ws + lay.partials);
    a.out = *out;
#ifdef DT_TRACE
    a.trace = (uint64_t*)(ws + lay.trace);
#endif
    a.R = p->R;
    a.B = p->B;
    a.k = p->k;
    a.V = p->V;
    a.r = p->r;
    a.Ncap = p->Ncap;
    a.NC = lay.NC;
    a.Tmax = max_tiles(p->R, p->Ncap);
    a.y2scale = (float)(1.4426950408889634 / (double)Teff);
    a.invT = (float)(1.0 / (double)Teff);
    a.seed_lo = (uint32_t)p->seed;
    a.seed_hi = (uint32_t)(p->seed >> 32);
    a.round = p->round;
    a.logits_bf16 = p->logits_dtype == DT_BF16;
    a.spin_limit = wait_limit();
    a.cond = (int)p->cond;
    for (int i = 0; i < 16; ++i) a.cal[i] = p->cal[i];
    if (launch_build(p, lay, a, st) != hipSuccess) return DT_EDEVICE;
    return DT_OK;
}

// ---- scratch of tree_build_noalloc: the construction workspace for callers that cannot
// allocate.  One copy per device (each device that runs the library holds it until the
// process ends).  In host code `scratch` only names the symbol: its device address is looked
// up once per device with hipGetSymbolAddress and kept in g_scratch; kernels only ever get
// that address.  Calls on one device share the array, so overlapping calls race.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchPtrs {
    std::mutex mu;
    char* ptr[kMaxDevices] = {};
};
static ScratchPtrs g_scratch;

static char* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch.mu);
    if (!g_scratch.ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch.ptr[dev] = (char*)ptr;
    }
    return g_scratch.ptr[dev];
}

// ---- tree attention
static dt_status validate_attn(const dt_attn_params* p) {
    if (!p) return DT_EINVAL;
    if (p->R < 1 || p->R > 65536 || p->Hkv < 1 || p->Hkv > 256 || p->Hq < p->Hkv ||
        p->Hq % p->Hkv != 0 || p->Hq / p->Hkv > 16)
        return DT_EINVAL;
    if (p->D != 128 || p->Ncap < 1 || p->Ncap > kMaxNcap || p->Cmax < 2 || p->Cmax > (1 << 24))
        return DT_EINVAL;
    if (!std::isfinite(p->scale) || !(p->scale > 0.0f)) return DT_EINVAL;
    return DT_OK;
}

}  // namespace dt

using namespace dt;

extern "C" {

const char* dt_status_string(int32_t code) {
    switch (code) {
        case DT_OK: return "DT_OK";
        case DT_EINVAL: return "DT_EINVAL: invalid argument";
        case DT_ENOSPC: return "DT_ENOSPC: workspace too small";
        case DT_EDEVICE: return "DT_EDEVICE: HIP launch or device error";
    }
    return "unknown dt_status";
}

dt_status dt_build_workspace_bytes(const dt_params* p, size_t* bytes) {
    const dt_status v = validate(p);
    if (v != DT_OK) return v;
    if (!bytes) return DT_EINVAL;
    *bytes = make_layout(p).total;
    return DT_OK;
}

dt_status tree_build(const dt_params* p, const void* block_logits, const void* U, const void* Wt,
                     const int32_t* root_token, const int32_t* n_budget, const float* tau,
                     const dt_tree* out, void* workspace, size_t ws_bytes, void* stream) {
    const dt_status v = check_build_args(p, block_logits, U, Wt, root_token, n_budget, tau, out);
    if (v != DT_OK) return v;
    if (!workspace || ((uintptr_t)workspace & 255)) return DT_EINVAL;
    // the W-resident kernel's layout when the workspace holds it (dt_build_workspace_bytes
    // returns that size), else the streaming kernel's
    Layout lay = make_layout(p, true);
    if (ws_bytes < lay.total) lay = make_layout(p, false);
    if (ws_bytes < lay.total) return DT_ENOSPC;
    return enqueue_build(p, lay, block_logits, U, Wt, root_token, n_budget, tau, out,
                         (char*)workspace, (hipStream_t)stream, g_timing.on);
}

dt_status tree_build_noalloc(const dt_params* p, const void* block_logits, const void* U,
                             const void* Wt, const int32_t* root_token, const int32_t* n_budget,
                             const float* tau, const dt_tree* out, void* stream) {
    const dt_status v = check_build_args(p, block_logits, U, Wt, root_token, n_budget, tau, out);
    if (v != DT_OK) return v;
    Layout lay = make_layout(p, true);
    if (lay.build_total > kScratchBytes) lay = make_layout(p, false);
    if (lay.build_total > kScratchBytes) return DT_ENOSPC;
    char* ws = scratch_ptr();
    if (!ws) return DT_EDEVICE;
    return enqueue_build(p, lay, block_logits, U, Wt, root_token, n_budget, tau, out, ws,
                         (hipStream_t)stream, false);
}

dt_status tree_verify_greedy(const dt_params* p, const dt_tree* tree, const void* target_logits,
                             const dt_verify_out* out, void* workspace, size_t ws_bytes,
                             void* stream) {
    const dt_status v = validate(p);
    if (v != DT_OK) return v;
    if (!tree_ptrs_ok(tree) || !target_logits || !verify_ptrs_ok(out) || !workspace)
        return DT_EINVAL;
    if (((uintptr_t)target_logits & 15) || ((uintptr_t)workspace & 255)) return DT_EINVAL;
    const Layout lay = make_layout(p);
    if (ws_bytes < lay.total) return DT_ENOSPC;
    if (launch_verify_greedy(p, lay, (char*)workspace, tree, target_logits, out,
                             (hipStream_t)stream) != hipSuccess)
        return DT_EDEVICE;
    return DT_OK;
}

dt_status tree_verify_sample(const dt_params* p, const dt_tree* tree, const void* block_logits,
                             const void* U, const void* Wt, const int32_t* root_token,
                             const void* target_logits, const dt_verify_out* out,
                             void* workspace, size_t ws_bytes, void* stream) {
    const dt_status v = validate(p);
    if (v != DT_OK) return v;
    if (p->mode != DT_SAMPLE) return DT_EINVAL;
    if (!tree_ptrs_ok(tree) || !block_logits || !U || !Wt || !root_token || !target_logits ||
        !verify_ptrs_ok(out) || !workspace)
        return DT_EINVAL;
    if (((uintptr_t)U & 15) || ((uintptr_t)Wt & 15) || ((uintptr_t)block_logits & 15) ||
        ((uintptr_t)target_logits & 15) || ((uintptr_t)workspace & 255))
        return DT_EINVAL;
    const Layout lay = make_layout(p);
    if (ws_bytes < lay.total) return DT_ENOSPC;
    if (launch_verify_sample(p, lay, (char*)workspace, tree, block_logits, U, Wt, root_token,
                             target_logits, out, (hipStream_t)stream) != hipSuccess)
        return DT_EDEVICE;
    return DT_OK;
}

dt_status dt_attn_workspace_bytes(const dt_attn_params* p, size_t* bytes) {
    const dt_status v = validate_attn(p);
    if (v != DT_OK) return v;
    if (!bytes) return DT_EINVAL;
    *bytes = attn_plan(p).total;
    return DT_OK;
}

dt_status tree_attention(const dt_attn_params* p, const void* Q, const void* K, const void* V,
                         const int32_t* ctx_len, const dt_tree* tree, void* O,
                         void* workspace, size_t ws_bytes, void* stream) {
    const dt_status v = validate_attn(p);
    if (v != DT_OK) return v;
    if (!Q || !K || !V || !ctx_len || !tree || !tree->n_nodes || !tree->anc_mask || !O)
        return DT_EINVAL;
    if (((uintptr_t)Q & 15) || ((uintptr_t)K & 15) || ((uintptr_t)V & 15) || ((uintptr_t)O & 15))
        return DT_EINVAL;
    const AttnPlan pl = attn_plan(p);
    if (pl.total > 0) {
        if (!workspace || ((uintptr_t)workspace & 255)) return DT_EINVAL;
        if (ws_bytes < pl.total) return DT_ENOSPC;
    }
    if (launch_tree_attention(p, pl, Q, K, V, ctx_len, tree->n_nodes, tree->anc_mask, O,
                              (char*)workspace, (hipStream_t)stream) != hipSuccess)
        return DT_EDEVICE;
    return DT_OK;
}

static dt_status validate_flash(const dt_params* p) {
    const dt_status v = validate(p);
    if (v != DT_OK) return v;
    if (p->mode != DT_GREEDY || p->cond != DT_COND_PARENT) return DT_EINVAL;
    return DT_OK;
}

dt_status dt_flash_workspace_bytes(const dt_params* p, size_t* bytes) {
    const dt_status v = validate_flash(p);
    if (v != DT_OK) return v;
    if (!bytes) return DT_EINVAL;
    *bytes = flash_plan(p).total;
    return DT_OK;
}

dt_status tree_build_flash(const dt_params* p, const void* block_logits, const void* U,
                           const void* Wt, const int32_t* root_token, const int32_t* n_budget,
                           const float* tau, const dt_tree* out, void* workspace,
                           size_t ws_bytes, void* stream) {
    const dt_status v = validate_flash(p);
    if (v != DT_OK) return v;
    if (!block_logits || !U || !Wt || !root_token || !n_budget || !tau || !tree_ptrs_ok(out) ||
        !workspace)
        return DT_EINVAL;
    if (((uintptr_t)block_logits & 15) || ((uintptr_t)U & 15) || ((uintptr_t)Wt & 15) ||
        ((uintptr_t)workspace & 255))
        return DT_EINVAL;
    const FlashPlan pl = flash_plan(p);
    if (ws_bytes < pl.total) return DT_ENOSPC;
    if (launch_build_flash(p, pl, block_logits, U, Wt, root_token, n_budget, tau, out,
                           (char*)workspace, (hipStream_t)stream) != hipSuccess)
        return DT_EDEVICE;
    return DT_OK;
}

dt_status dt_load_policy(const dt_policy* pol, float load, int32_t R, float* tau,
                         int32_t* n_budget) {
    if (!pol || !tau || !n_budget || R < 1) return DT_EINVAL;
    if (!std::isfinite(load) || load < 0.0f || load > 1.0f) return DT_EINVAL;
    if (!std::isfinite(pol->tau_max) || pol->tau_max < 0.0f || pol->tau_max > 1.0f) return DT_EINVAL;
    if (pol->Ncap < 1 || pol->Ncap > kMaxNcap || pol->capacity < 0) return DT_EINVAL;
    const double avail = (1.0 - (double)load) * (double)pol->capacity;
    long long n = (long long)std::floor(avail / (double)R);
    n = n < 1 ? 1 : (n > pol->Ncap ? pol->Ncap : n);
    const float t = pol->tau_max * load;
    for (int32_t i = 0; i < R; ++i) {
        tau[i] = t;
        n_budget[i] = (int32_t)n;
    }
    return DT_OK;
}

dt_status dt_timing_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.on = on != 0;
    g_timing.used = 0;
    return DT_OK;
}

dt_status dt_timing_read(double* total_ms, int32_t* launches) {
    if (!total_ms || !launches) return DT_EINVAL;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    double tot = 0.0;
    const size_t pairs = g_timing.used / 2;
    if (pairs > 0 && hipEventSynchronize(g_timing.pool[2 * pairs - 1]) != hipSuccess)
        return DT_EDEVICE;
    for (size_t i = 0; i < pairs; ++i) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, g_timing.pool[2 * i], g_timing.pool[2 * i + 1]) != hipSuccess)
            return DT_EDEVICE;
        tot += ms;
    }
    *total_ms = tot;
    *launches = (int32_t)pairs;
    g_timing.used = 0;
    return DT_OK;
}

}  // extern "C"
