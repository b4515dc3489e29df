/* Plain CPU oracle for parent-conditioned draft-tree construction and verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or call this
 * code; only the test suite, the smoke check and the CPU-baseline leg of the benchmark use
 * it.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and passage):
 *  - "From Chains to Trees: Parent-Conditioned Drafting for Semi-Autoregressive Speculative
 *    Decoding" (PCTree summary): block logits from one backbone forward, a Markov head that
 *    biases the block by the previous token, expansion of each parent by its own
 *    conditional distribution into k children, budget N, k = 1 = greedy chain, greedy
 *    verification.
 *  - "TreeSpark: adaptive draft trees" (kongchang article), core-idea and lossless
 *    sections: calibration of the parent-conditioned probability to an edge-acceptance
 *    estimate, path survival driving best-first expansion and per-round stopping, siblings
 *    sampled without replacement and recursive rejection with residual matching.
 *
 * All probabilities are computed in float64 from the exact stored inputs (bf16 values are
 * passed as the float32 numbers they equal).  Survival is a float32 product, as specified,
 * so that its ordering is bit-identical on every implementation.
 */
#ifndef DTREE_ORACLE_H
#define DTREE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_GREEDY = 0, OR_SAMPLE = 1 };
enum { OR_STREAM_GUMBEL = 1, OR_STREAM_ACCEPT = 2, OR_STREAM_RESID = 3 };
enum { OR_STATUS_BAD_ROOT = 1, OR_STATUS_BUDGET_CLAMPED = 2 };
/* Which token's head row biases a node's expansion: its own (parent-conditioned tree), the
 * greedy chain's token at its depth (Shared-Markov control), or none (per-position
 * marginals).  The last two are greedy-mode variants. */
enum { OR_COND_PARENT = 0, OR_COND_CHAIN = 1, OR_COND_NONE = 2 };

typedef struct {
    int32_t R, B, k, V, r, Ncap;
    int32_t mode;         /* OR_GREEDY | OR_SAMPLE */
    double temperature;   /* used in sample mode; greedy mode uses 1 */
    float cal[16];        /* calibration table, values in [0, 1] */
    uint64_t seed;
    uint32_t round;
    int32_t req_base;     /* request id of row 0 of every [R] array: request i's random
                             streams are keyed by req_base + i */
    int32_t cond;         /* OR_COND_* */
} or_params;

/* Emitted trees, canonical (depth, path-lex) order; caller-owned host arrays. */
typedef struct {
    int32_t* token;    /* [R][Ncap], -1 past n_nodes */
    int16_t* parent;   /* [R][Ncap], -1 = root, -2 past n_nodes */
    uint8_t* depth;    /* [R][Ncap], 0 past n_nodes */
    uint64_t* mask;    /* [R][Ncap], ancestors and self, 0 past n_nodes */
    float* surv;       /* [R][Ncap] */
    float* logq;       /* [R][Ncap] */
    int32_t* n_nodes;  /* [R] */
    int32_t* cand;     /* [R][Ncap+1][k]: drawn/ranked children of root (row 0), node i (row i+1) */
    int32_t* status;   /* [R] */
    int32_t* n_expand; /* [R] number of expansions made (root included) */
} or_tree;

typedef struct {
    int32_t* accept_len; /* [R] */
    int32_t* path;       /* [R][B], canonical node indices, -1 pad */
    int32_t* out_tokens; /* [R][B+1], -1 pad */
    int32_t* n_out;      /* [R] */
} or_verify;

/* Smallest distance to a decision boundary seen while computing one request. */
typedef struct {
    double key_gap;   /* adjacent gaps among each expansion's top-(k+1) ranking keys */
    double q_edge;    /* |q - i/16| over interior bin edges i = 1..15, every child */
    double accept;    /* |u - p_j(x)/q_j(x)| over every accept test (sample verify) */
    double draw_gap;  /* top-2 gap of every Gumbel-max draw (sample verify) */
    double argmax_gap;/* top-2 gap of every target-row argmax (greedy verify) */
} or_margin;

/* Counter-based randomness (Philox4x32-10, Salmon et al. SC'11; SplitMix64 output mix). */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint64_t or_mix64(uint64_t x);
uint64_t or_root_hash(uint32_t round, int32_t request, int32_t root_token);
uint64_t or_child_hash(uint64_t parent_hash, int32_t token);
double or_uniform(uint64_t seed, uint64_t hash, uint32_t stream, uint32_t index);

/* One expansion.  Writes z[V] (float64), lse, and the k ranked children (token, y value).
 * `token` selects the head row U[token]; token < 0 means no bias.  Returns the smallest
 * adjacent gap among the top-(k+1) ranking keys. */
double or_expand(const or_params* P, const float* L_req, const float* U, const float* Wt,
                 int32_t depth, int32_t token, uint64_t hash, double* z, double* lse,
                 int32_t* child_tok, double* child_y);

/* Tree construction: literal best-first with a priority queue (method 0) or the
 * level-synchronous expand-then-select form (method 1).  L is [R][B][V]. */
int or_build(const or_params* P, const float* L, const float* U, const float* Wt,
             const int32_t* root_token, const int32_t* n_budget, const float* tau,
             int32_t method, or_tree* out, or_margin* margins /* [R] or NULL */);

/* Two-stage M-ary tree (M = P->k; greedy mode): per block row the M largest unconditioned
 * logits form the depth's token set; every (row, token) state's parent-conditioned law is
 * evaluated; best-first top-N over the resulting lattice.  Same outputs as or_build. */
int or_build_flash(const or_params* P, const float* L, const float* U, const float* Wt,
                   const int32_t* root_token, const int32_t* n_budget, const float* tau,
                   or_tree* out, or_margin* margins /* [R] or NULL */);

/* Greedy accept-walk; target is [R][Ncap+1][V]. */
int or_verify_greedy(const or_params* P, const or_tree* tree, const float* target,
                     or_verify* out, or_margin* margins);

/* Lossless sample verify (recursive rejection with residuals); draft rows recomputed. */
int or_verify_sample(const or_params* P, const or_tree* tree, const float* L, const float* U,
                     const float* Wt, const int32_t* root_token, const float* target,
                     or_verify* out, or_margin* margins);

/* Rejection chain at one node with explicit probabilities: acc[j] = probability that draw
 * x_j is accepted given x_1..x_{j-1} were rejected; resid[V] = residual law after all k
 * rejections.  Uses the same residual update as or_verify_sample. */
void or_chain_probs(const double* p, const double* q, int32_t V, const int32_t* x, int32_t k,
                    double* acc, double* resid);

/* Statistical driver: n_rounds full rounds (build + sample verify) of request 0, with the
 * target given as a table target_tab[d][t][V] (row for a node of depth d and token t; the
 * root uses depth 0 and root_token).  Records the first two emitted tokens per round
 * (second = -1 when the round emitted one token). */
int or_sample_rounds(const or_params* P, const float* L, const float* U, const float* Wt,
                     int32_t root_token, int32_t n_budget, float tau, const float* target_tab,
                     int64_t n_rounds, int32_t* first, int32_t* second);

/* Negative controls for the statistical pins (0 = faithful). 1: q is not reduced after a
 * rejection (the rejected sibling keeps its mass); 2: the target law is not replaced by the
 * residual after a rejection; 3: the draw at a depth-B node uses its parent's target row. */
void or_set_fault(int32_t mode);

#ifdef __cplusplus
}
#endif
#endif
