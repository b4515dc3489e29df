/* dtree.h - C ABI of libdtree.so: parent-conditioned draft-tree construction and
 * verification for a semi-autoregressive block drafter, on one AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *  - "From Chains to Trees: Parent-Conditioned Drafting for Semi-Autoregressive Speculative
 *    Decoding" (PCTree summary): one backbone forward gives logits for every position of the
 *    block; a light Markov head biases the block by the previous token; the chain becomes a
 *    budget-limited tree with k children per parent and N nodes (method paragraph, main
 *    setting k = 4, N = 32); k = 1 is the greedy chain; verification is greedy.
 *  - "TreeSpark: adaptive draft trees" (kongchang article): the parent-conditioned
 *    distribution is calibrated to an edge-acceptance estimate, path survival (the product
 *    of edge estimates) drives best-first expansion and per-round stopping, and lossless
 *    decoding samples siblings without replacement and matches residuals in recursive
 *    rejection (core-idea and lossless sections).
 *
 * Conventions shared by every call
 *  - Every array pointer is caller-owned DEVICE memory (e.g. from PyTorch) unless noted;
 *    the library never allocates or frees device memory and keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work; outputs
 *    are valid once the stream has been synchronised.  Calls on different streams with
 *    different workspaces are independent.
 *  - `workspace` is caller-owned device memory of at least dt_build_workspace_bytes() bytes,
 *    256-byte aligned (DT_EINVAL if misaligned or NULL, DT_ENOSPC if smaller); its contents
 *    on entry do not matter and on return are unspecified.  A verify call may use another
 *    workspace than the tree_build call that made its tree.
 *  - Host-side argument errors return synchronously before anything is enqueued.
 *    Device-side data errors are reported per request in `status` and never abort.
 *  - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *  - tree_build's kernel hands its work out through per-level tickets, so a round completes
 *    whatever number of its workgroups is resident at once (for example while another
 *    kernel holds compute units).  Its internal waits are bounded (about two seconds); the
 *    environment variable DT_WAIT_LIMIT, if set to a number of polls, lowers that bound
 *    (a test hook that makes a round give up and report DT_REQ_SYNC_TIMEOUT).
 *
 * Markov head form: bias[p][c] = sum_j U[p][j] * W[j][c], a rank-r head shared by all block
 * positions (the pages fix what the head does, not its form).  W is passed TRANSPOSED,
 * as Wt[V][r] (row c holds W[:, c]), so both tables are row-per-token.
 */
#ifndef DTREE_H
#define DTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DT_OK = 0,
    DT_EINVAL = 1,  /* bad argument (checked on the host, nothing enqueued) */
    DT_ENOSPC = 2,  /* workspace smaller than dt_build_workspace_bytes() */
    DT_EDEVICE = 3  /* a HIP call or kernel launch failed */
} dt_status;

enum { DT_F32 = 0, DT_BF16 = 1 };   /* storage dtypes */
enum { DT_GREEDY = 0, DT_SAMPLE = 1 };
/* Which token's Markov-head row biases a node's expansion (dt_params.cond).
 *  DT_COND_PARENT  the node's own token: the parent-conditioned tree (PCTree summary,
 *                  method paragraph).
 *  DT_COND_CHAIN   the drafter's greedy chain token at the node's depth: every sibling at
 *                  one depth reuses the chain's distribution for that depth (the
 *                  "Shared-Markov tree" control of the PCTree summary).  Greedy mode only.
 *  DT_COND_NONE    no bias: each depth's block row alone, the per-position marginal that
 *                  ranks candidates without their parent (TreeSpark article, the first
 *                  flaw of existing draft trees).  Greedy mode only. */
enum { DT_COND_PARENT = 0, DT_COND_CHAIN = 1, DT_COND_NONE = 2 };

/* Per-request status bits written to dt_tree.status. */
enum {
    DT_REQ_BAD_ROOT = 1,       /* root_token outside [0, V): empty tree, nothing emitted */
    DT_REQ_BUDGET_CLAMPED = 2, /* n_budget outside [0, Ncap]: clamped into range */
    DT_REQ_SYNC_TIMEOUT = 4    /* an internal wait between workgroups gave up (about two
                                  seconds): the tree is reported empty and the verifiers
                                  emit nothing for the request (n_out = 0), as for a bad
                                  root */
};

/* Round parameters (host struct, read synchronously). */
typedef struct dt_params {
    int32_t R;            /* requests in the batch, >= 1 */
    int32_t B;            /* block positions = maximum tree depth, 1..32 */
    int32_t k;            /* children per expanded parent, 1..8, k <= V */
    int32_t V;            /* vocabulary size, 1..2^24 */
    int32_t r;            /* Markov-head rank: bf16 head 8..256 and a multiple of 8; f32 head 1..64 */
    int32_t Ncap;         /* node capacity per request (tree arrays' width), 1..64 */
    int32_t logits_dtype; /* DT_BF16 | DT_F32: block logits and target logits */
    int32_t head_dtype;   /* DT_BF16 | DT_F32: U and Wt */
    int32_t mode;         /* DT_GREEDY: rank children by logit, q at T = 1.
                             DT_SAMPLE: Gumbel-top-k children, q at `temperature`. */
    float temperature;    /* > 0, finite; used in DT_SAMPLE mode */
    float cal[16];        /* calibration table: edge estimate for q in [i/16, (i+1)/16);
                             values in [0, 1] and non-decreasing */
    uint64_t seed;        /* key of the counter-based generator (sample mode) */
    uint32_t round;       /* round counter, folded into every node's random stream */
    uint32_t cond;        /* DT_COND_*; 0 (DT_COND_PARENT) is the parent-conditioned tree */
} dt_params;

/* Emitted trees.  Node order is canonical: depth ascending, then the path of sibling ranks
 * from the root ascending (parents precede children).  Slots >= n_nodes hold token -1,
 * parent -2, depth 0, mask 0, surv 0, logq 0. */
typedef struct dt_tree {
    int32_t* token;     /* [R][Ncap] draft token of each node */
    int16_t* parent;    /* [R][Ncap] parent's node index; -1 = the root */
    uint8_t* depth;     /* [R][Ncap] 1..B */
    uint64_t* anc_mask; /* [R][Ncap] bit j set iff node j is this node or one of its
                           ancestors (the root is not a node): the tree-attention mask */
    float* surv;        /* [R][Ncap] path survival (float32 product of table entries) */
    float* logq;        /* [R][Ncap] log of the node's probability under its parent's
                           parent-conditioned draft distribution */
    int32_t* n_nodes;   /* [R] */
    int32_t* cand;      /* [R][Ncap+1][k] ranked children of every expanded node: row 0 =
                           the root, row i+1 = node i; -1 for nodes never expanded */
    int32_t* status;    /* [R] DT_REQ_* bits */
    int32_t* n_expand;  /* [R] optional (NULL = not written): expansions made */
    int32_t* level_rows;/* [B] optional (NULL = not written): parents expanded at each
                           level, summed over requests */
} dt_tree;

/* Verification outputs. */
typedef struct dt_verify_out {
    int32_t* accept_len; /* [R] accepted tree nodes (0..B) */
    int32_t* path;       /* [R][B] accepted node indices in order, -1 padded */
    int32_t* out_tokens; /* [R][B+1] accepted tokens, then the round's final token, -1 pad */
    int32_t* n_out;      /* [R] tokens emitted this round: accept_len + 1 (0 for a bad root) */
} dt_verify_out;

/* Workspace needed by tree_build, tree_verify_greedy and tree_verify_sample for these
 * parameters (one size covers all three).  Writes *bytes on the host.  DT_EINVAL on bad
 * parameters. */
dt_status dt_build_workspace_bytes(const dt_params* p, size_t* bytes);

/* Build one round's draft trees for R requests.
 *  block_logits [R][B][V]  (logits_dtype): row d of request i = the drafter's logits for
 *                          block position d; a node at depth d is expanded with row d
 *  U            [V][r]     (head_dtype): parent-token embedding of the Markov head
 *  Wt           [V][r]     (head_dtype): W transposed (child-token embedding)
 *  root_token   [R] int32: the last committed token (depth 0; not a node)
 *  n_budget     [R] int32: node budget N per request, 0..Ncap
 *  tau          [R] float: stopping threshold; nodes with survival < tau are never kept
 *                          (tau <= 0 disables stopping)
 *  out          host struct of device pointers (dt_tree), fully overwritten
 * Expansion of node v (token t, depth d): z[c] = L[d][c] + U[t] . Wt[c] (t replaced by the
 * chain token of depth d, or the bias dropped, under p->cond); q = softmax(z / T')
 * with T' = 1 (greedy) or temperature (sample); the k children are the largest z (greedy;
 * ties to the lower token id) or the largest z/T + Gumbel noise (sample); a child's survival
 * is fl32(s_parent * cal[min(15, floor(16 q))]), the root's is 1; logq = log q.  The tree is
 * the best n_budget nodes with survival >= tau under the order (survival desc, depth asc,
 * sibling-rank path asc), which equals best-first expansion with per-round stopping. */
dt_status tree_build(const dt_params* p, const void* block_logits, const void* U,
                     const void* Wt, const int32_t* root_token, const int32_t* n_budget,
                     const float* tau, const dt_tree* out, void* workspace, size_t ws_bytes,
                     void* stream);

/* tree_build for callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and results as tree_build without
 * the workspace: the construction workspace is a fixed device array of
 * DT_NOALLOC_SCRATCH_BYTES inside the library, one per device, reserved when the library's
 * code is loaded on that device and kept until the process ends.  No device or host memory
 * is allocated by the call (no hipMalloc, hipFree or allocating library routine), and
 * timing (dt_timing_enable) does not apply to it.  DT_ENOSPC if dt_build_workspace_bytes()'s
 * construction part for these parameters exceeds DT_NOALLOC_SCRATCH_BYTES (for example
 * R = 64, B = 16, Ncap = 64 and k <= 8 fit).  Every call on one device uses the same array:
 * calls that overlap on one device (concurrent streams or host threads) race and must be
 * serialised by the caller; successive calls on one stream are fine (each clears what it
 * needs at its start). */
#define DT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dt_status tree_build_noalloc(const dt_params* p, const void* block_logits, const void* U,
                             const void* Wt, const int32_t* root_token, const int32_t* n_budget,
                             const float* tau, const dt_tree* out, void* stream);

/* Greedy accept-walk (PCTree setup: greedy verification).
 *  tree          the dt_tree written by tree_build (device arrays; read only)
 *  target_logits [R][Ncap+1][V] (logits_dtype): row 0 = the root, row i+1 = node i
 * From the root: t* = argmax of the current row (ties: lower id); if a child of the current
 * node carries t*, accept it and continue from it; otherwise t* is the final (bonus) token.
 * The root rows' argmax is split over many workgroups (partials in `workspace`); the walk
 * below the root runs one workgroup per request. */
dt_status tree_verify_greedy(const dt_params* p, const dt_tree* tree, const void* target_logits,
                             const dt_verify_out* out, void* workspace, size_t ws_bytes,
                             void* stream);

/* Lossless sample verify (TreeSpark lossless section), p->mode must be DT_SAMPLE and the
 * tree built in that mode with the same seed and round.  At each visited node v:
 * p = softmax(target_row / T), q = softmax(z_v / T) (recomputed from block_logits, U, Wt);
 * the k drawn siblings cand[v] are tried in draw order; x_j is accepted iff
 * u_j * q_j(x_j) < p_j(x_j), else p and q become the residual laws
 * p_{j+1} = max(p_j - q_j, 0) / Z and q_{j+1} = q_j without x_j, renormalised.  An accepted
 * sibling that is a tree node is descended into; one that is not ends the round; if all are
 * rejected the round ends with a draw from the final residual; at depth B it ends with a
 * draw from p.  Each request's vocabulary-wide reductions are split over several
 * workgroups that wait for each other (bounded, about two seconds); a request whose wait
 * gave up reports n_out = -1. */
dt_status tree_verify_sample(const dt_params* p, const dt_tree* tree, const void* block_logits,
                             const void* U, const void* Wt, const int32_t* root_token,
                             const void* target_logits, const dt_verify_out* out,
                             void* workspace, size_t ws_bytes, void* stream);

/* Load-adaptive per-round tree sizing (TreeSpark article, core idea: path survival drives
 * best-first expansion, per-round stopping and a load-adaptive serving policy; as load rises
 * the tree shrinks back toward a chain).  The pages give no formula; this is the reading
 * taken.  Under calibration a node's survival estimates the probability that its path is
 * accepted, so the stopping threshold acts as the price of one more verified token:
 *   tau[i]      = tau_max * load
 *   n_budget[i] = clamp(floor((1 - load) * capacity / R), 1, Ncap)
 * with load in [0, 1] the share of the target forward's token capacity (capacity tokens per
 * round for this batch) taken by other work.  Host function: tau and n_budget are HOST
 * arrays of R entries (copy them to the device for tree_build).  DT_EINVAL for R < 1,
 * Ncap outside 1..64, capacity < 0, or load / tau_max not finite or outside [0, 1]. */
typedef struct dt_policy {
    float tau_max;    /* threshold at full load, in [0, 1] */
    int32_t capacity; /* target-forward tokens per round available to this batch at no load */
    int32_t Ncap;     /* largest node budget per request (the tree arrays' width) */
} dt_policy;
dt_status dt_load_policy(const dt_policy* pol, float load, int32_t R, float* tau,
                         int32_t* n_budget);

/* ---- Two-stage M-ary tree ------------------------------------------------------------------
 * The TreeFlash construction (TreeFlash explainer, technical summary, methodology: two-stage
 * inference construction) on this library's Markov head, M = p->k.  Stage 1: for every block
 * row j, the M tokens with the largest unconditioned block logits (ties: lower id) are the
 * only tokens of the tree at depth j + 1.  Stage 2: the parent-conditioned law of every state
 * (row j, token t) -- t = root_token for j = 0, t in stage 1's set of row j - 1 otherwise --
 * is evaluated over the whole vocabulary, z = L[j] + U[t] . W, q(c) = softmax(z)_c for the M
 * tokens c of row j's set; the 1 + M (B - 1) states are independent, so this is one parallel
 * pass.  Final selection: the best-first top-N with per-round stopping of tree_build (same
 * calibration, survival, global order and canonical emission) over the lattice in which a node
 * of depth j with token t has as children row j's set, ranked by their conditional logits.
 * Greedy mode and DT_COND_PARENT only (DT_EINVAL otherwise).  Outputs as tree_build; cand rows
 * hold the M ranked children; level_rows is not written. */
dt_status dt_flash_workspace_bytes(const dt_params* p, size_t* bytes);
dt_status tree_build_flash(const dt_params* p, const void* block_logits, const void* U,
                           const void* Wt, const int32_t* root_token, const int32_t* n_budget,
                           const float* tau, const dt_tree* out, void* workspace,
                           size_t ws_bytes, void* stream);

/* ---- Tree attention: the verify forward's attention over a round's trees -------------
 * One attention layer of the target model that scores every tree position in one pass
 * (PCTree summary, introduction: the target checks all nodes of the tree in one forward;
 * TreeSpark article, introduction: one verification pass over several continuations).
 * Tree position j of request r is the root (j = 0, the round's last emitted token) or node
 * j - 1 of the emitted tree.  Its key and value sit in the cache at slot ctx_len[r] + j,
 * after the request's context.  The query of position j sees every context slot, the
 * root's slot, and, for a node, the slots of the nodes set in its ancestor mask (itself and
 * its ancestors): each node is scored as if its own path were the whole continuation.
 * Scores scale * q.k, softmax over the visible slots, output = the weighted sum of values.
 * Query head hq uses key/value head hq / (Hq / Hkv). */
typedef struct dt_attn_params {
    int32_t R;     /* requests, 1..65536 */
    int32_t Hq;    /* query heads, a multiple of Hkv, Hq / Hkv <= 16 */
    int32_t Hkv;   /* key/value heads, 1..256 */
    int32_t D;     /* head dimension: 128 */
    int32_t Ncap;  /* tree capacity, 1..64: Q and O hold Ncap + 1 positions per head */
    int32_t Cmax;  /* cache slots per (request, key/value head), 2..2^24 */
    float scale;   /* score scale, finite and > 0 (usually 1/sqrt(D)) */
} dt_attn_params;

/* Workspace for tree_attention (0 when the call needs none).  DT_EINVAL on bad parameters. */
dt_status dt_attn_workspace_bytes(const dt_attn_params* p, size_t* bytes);

/* Q        [R][Hq][Ncap+1][D] bf16, row j = tree position j.
 * K, V     [R][Hkv][Cmax][D]  bf16 caches; slots ctx_len[r] .. ctx_len[r] + n_nodes[r]
 *          hold the tree's keys and values.
 * ctx_len  [R] int32 context entries before the root.
 * tree     the emitted trees: only n_nodes and anc_mask are read (tree_build's output, or
 *          any trees whose masks have bit i set only for i < n_nodes).
 * O        [R][Hq][Ncap+1][D] bf16 output.  Rows past n_nodes, and every row of a request
 *          whose n_nodes is outside [0, Ncap] or whose tree does not fit the cache
 *          (ctx_len < 0 or ctx_len + n_nodes + 1 > Cmax), are written as zeros.
 * workspace  device memory of dt_attn_workspace_bytes() bytes, 256-byte aligned (may be
 *          NULL when that size is 0).
 * Q, K, V and O must be 16-byte aligned.  Arithmetic: bf16 MFMA products with fp32
 * accumulation, fp32 online softmax, probabilities rounded to bf16 for the value product. */
dt_status tree_attention(const dt_attn_params* p, const void* Q, const void* K, const void* V,
                         const int32_t* ctx_len, const dt_tree* tree, void* O,
                         void* workspace, size_t ws_bytes, void* stream);

/* Text for a status code; any integer is accepted (unknown codes give a fixed text). */
const char* dt_status_string(int32_t code);

/* Measurement support (host only, not thread-safe): when enabled, the library brackets each
 * launch of the fused Markov-bias/top-k kernel with HIP events on the caller's stream.
 * dt_timing_read() synchronises those events and returns the summed kernel time and the
 * number of timed launches since the last enable, then clears the record. */
dt_status dt_timing_enable(int32_t on);
dt_status dt_timing_read(double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* DTREE_H */
