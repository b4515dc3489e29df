/* Plain CPU oracle for parent-conditioned draft-tree construction and verification.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the benchmark).  It is
 * deliberately slow and literal: one node at a time, float64 sums in index order, a
 * priority queue popped by linear scan.  It shares nothing with the HIP library.
 *
 * Every function names the passage of the pages it follows; see dtree_oracle.h for the
 * list of pages.  Where the pages leave a step open, the reading taken is stated inline.
 * Parity status: every function here is pinned by a CPU test (closed forms, brute force,
 * exact enumeration, invariants or published known-answer vectors).
 */
#include "dtree_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int g_fault = 0;
void or_set_fault(int32_t mode) { g_fault = mode; }

/* ------------------------------------------------------------------------------------ */
/* Counter-based randomness.                                                              */
/* Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw ("Parallel random numbers:  */
/* as easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies with the Weyl key   */
/* schedule.  SplitMix64's output function (Steele, Lea and Flood, OOPSLA 2014) hashes      */
/* token paths.                                                                            */
/* ------------------------------------------------------------------------------------ */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

uint64_t or_mix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* A node's random stream is keyed by its token path (not by its slot in the tree), so its
 * draws do not depend on which other nodes were selected. */
uint64_t or_root_hash(uint32_t round, int32_t request, int32_t root_token)
{
    uint64_t a = or_mix64(((uint64_t)round << 32) | (uint64_t)(uint32_t)request);
    return or_mix64(a ^ (uint64_t)(uint32_t)root_token);
}

uint64_t or_child_hash(uint64_t parent_hash, int32_t token)
{
    return or_mix64(parent_hash ^ (uint64_t)(uint32_t)token);
}

/* Uniform in (0, 1): word (index mod 4) of Philox at counter (index/4, stream, hash), key =
 * seed; the top 24 bits plus one half, times 2^-24. */
double or_uniform(uint64_t seed, uint64_t hash, uint32_t stream, uint32_t index)
{
    uint32_t ctr[4] = {index >> 2, stream, (uint32_t)hash, (uint32_t)(hash >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    uint32_t w = out[index & 3u];
    return ((double)(w >> 8) + 0.5) * (1.0 / 16777216.0);
}

static double gumbel(uint64_t seed, uint64_t hash, uint32_t stream, uint32_t index)
{
    double u = or_uniform(seed, hash, stream, index);
    return -log(-log(u));
}

/* ------------------------------------------------------------------------------------ */
/* Expansion of one node (PCTree summary, method paragraph: the Markov head biases the      */
/* block's position logits by the previous token, and each parent is expanded by its own   */
/* conditional distribution; TreeSpark core idea: that distribution is read from the        */
/* drafter's Markov head).  Head form: z[c] = L[d][c] + sum_j U[t][j] * W[j][c], one head   */
/* shared by all positions; W is stored transposed (Wt[c][j]).                              */
/* Children: the k largest z (ties: lower token id) in greedy mode; in sample mode the k    */
/* largest y[c] + G[c] with y = z/T and Gumbel noise G (Gumbel-top-k, which draws k        */
/* siblings without replacement from softmax(y) - TreeSpark lossless section).              */
/* ------------------------------------------------------------------------------------ */
double or_expand(const or_params* P, const float* L_req, const float* U, const float* Wt,
                 int32_t depth, int32_t token, uint64_t hash, double* y, double* lse,
                 int32_t* child_tok, double* child_y)
{
    const int V = P->V, r = P->r, k = P->k;
    const double T = (P->mode == OR_SAMPLE) ? P->temperature : 1.0;
    const float* Lrow = L_req + (size_t)depth * (size_t)V;
    const float* u = token >= 0 ? U + (size_t)token * (size_t)r : NULL;

    for (int c = 0; c < V; ++c) {
        const float* w = Wt + (size_t)c * (size_t)r;
        double bias = 0.0;
        if (u)
            for (int j = 0; j < r; ++j) bias += (double)u[j] * (double)w[j];
        double z = (double)Lrow[c] + bias;
        y[c] = z / T;
    }
    double m = y[0];
    for (int c = 1; c < V; ++c)
        if (y[c] > m) m = y[c];
    double s = 0.0;
    for (int c = 0; c < V; ++c) s += exp(y[c] - m);
    *lse = m + log(s);

    double* key = (double*)malloc(sizeof(double) * (size_t)V);
    unsigned char* taken = (unsigned char*)calloc((size_t)V, 1);
    for (int c = 0; c < V; ++c)
        key[c] = (P->mode == OR_SAMPLE) ? y[c] + gumbel(P->seed, hash, OR_STREAM_GUMBEL, (uint32_t)c)
                                         : y[c];
    /* k+1 passes of "largest key, lower id on ties"; the (k+1)-th only measures the gap. */
    const int npick = (k + 1 < V) ? k + 1 : V;
    double prev = 0.0, gap = INFINITY;
    for (int j = 0; j < npick; ++j) {
        int best = -1;
        for (int c = 0; c < V; ++c) {
            if (taken[c]) continue;
            if (best < 0 || key[c] > key[best]) best = c;
        }
        taken[best] = 1;
        if (j > 0 && prev - key[best] < gap) gap = prev - key[best];
        prev = key[best];
        if (j < k) {
            child_tok[j] = best;
            child_y[j] = y[best];
        }
    }
    free(key);
    free(taken);
    return gap;
}

/* ------------------------------------------------------------------------------------ */
/* Node store and the global order.                                                       */
/* ------------------------------------------------------------------------------------ */
typedef struct {
    int32_t token, depth, parent, rank, child0;
    float s, logq;
    uint64_t hash;
} node_t;

typedef struct {
    node_t* v;
    int n, cap;
    int use_head;      /* 0: a node's own token is its head token */
    int32_t head[33];  /* else: head token of every node at depth d (-1: no bias) */
} store_t;

static int store_add(store_t* st, node_t nd)
{
    if (st->n == st->cap) {
        st->cap = st->cap ? st->cap * 2 : 256;
        st->v = (node_t*)realloc(st->v, sizeof(node_t) * (size_t)st->cap);
    }
    st->v[st->n] = nd;
    return st->n++;
}

/* Sibling-rank sequence from the root; returns its length (the depth). */
static int rank_path(const store_t* st, int idx, int32_t* out)
{
    int d = st->v[idx].depth;
    for (int i = d - 1; i >= 0; --i) {
        out[i] = st->v[idx].rank;
        idx = st->v[idx].parent;
    }
    return d;
}

static int pathlex_less(const store_t* st, int a, int b)
{
    int32_t pa[64], pb[64];
    int la = rank_path(st, a, pa), lb = rank_path(st, b, pb);
    int n = la < lb ? la : lb;
    for (int i = 0; i < n; ++i)
        if (pa[i] != pb[i]) return pa[i] < pb[i];
    return la < lb;
}

/* Global order used by best-first expansion and by the select: survival descending, then
 * depth ascending, then sibling-rank path ascending (TreeSpark core idea: expand the path
 * most likely to survive first; the tie rules are this library's reading). */
static int key_better(const store_t* st, int a, int b)
{
    const node_t* A = &st->v[a];
    const node_t* Bn = &st->v[b];
    if (A->s != Bn->s) return A->s > Bn->s;
    if (A->depth != Bn->depth) return A->depth < Bn->depth;
    return pathlex_less(st, a, b);
}

static int canon_less(const store_t* st, int a, int b)
{
    if (st->v[a].depth != st->v[b].depth) return st->v[a].depth < st->v[b].depth;
    return pathlex_less(st, a, b);
}

static void upd_min(double* m, double v)
{
    if (v < *m) *m = v;
}

/* Calibration and survival (TreeSpark core idea: the parent-conditioned probability is
 * mapped through a calibration table to an edge-acceptance estimate; path survival is the
 * product along the path).  Reading: 16 equal-width bins on q in [0, 1], piecewise
 * constant; survival is a float32 product in depth order. */
static int cal_bin(double q)
{
    int b = (int)floor(16.0 * q);
    if (b > 15) b = 15;
    if (b < 0) b = 0;
    return b;
}

static double q_edge_distance(double q)
{
    double best = INFINITY;
    for (int i = 1; i < 16; ++i) {
        double d = fabs(q - (double)i / 16.0);
        if (d < best) best = d;
    }
    return best;
}

static void expand_in_store(const or_params* P, const float* L_req, const float* U,
                            const float* Wt, store_t* st, int idx, double* ybuf,
                            or_margin* mg)
{
    const int k = P->k;
    int32_t ctok[8];
    double cy[8], lse;
    node_t par = st->v[idx];
    const int32_t head = st->use_head ? st->head[par.depth] : par.token;
    double gap = or_expand(P, L_req, U, Wt, par.depth, head, par.hash, ybuf, &lse, ctok, cy);
    if (mg) upd_min(&mg->key_gap, gap);
    int first = -1;
    for (int j = 0; j < k; ++j) {
        double q = exp(cy[j] - lse);
        if (mg) upd_min(&mg->q_edge, q_edge_distance(q));
        float a = P->cal[cal_bin(q)];
        node_t ch;
        ch.token = ctok[j];
        ch.depth = par.depth + 1;
        ch.parent = idx;
        ch.rank = j;
        ch.child0 = -1;
        ch.s = par.s * a; /* float x float, rounded to float */
        ch.logq = (float)(cy[j] - lse);
        ch.hash = or_child_hash(par.hash, ctok[j]);
        int id = store_add(st, ch);
        if (j == 0) first = id;
    }
    st->v[idx].child0 = first;
}

/* Emission (reading: canonical order = depth, then sibling-rank path; parents precede
 * children; the ancestor mask holds the node's own bit and its ancestors' bits, not the
 * root's). */
static void emit_tree(const or_params* P, const store_t* st, int* sel, int nsel, int req,
                      or_tree* out)
{
    const int Ncap = P->Ncap, k = P->k;
    for (int i = 1; i < nsel; ++i) { /* insertion sort into canonical order */
        int x = sel[i], j = i - 1;
        while (j >= 0 && canon_less(st, x, sel[j])) {
            sel[j + 1] = sel[j];
            --j;
        }
        sel[j + 1] = x;
    }
    int* canon = (int*)malloc(sizeof(int) * (size_t)st->n);
    for (int i = 0; i < st->n; ++i) canon[i] = -1;
    for (int i = 0; i < nsel; ++i) canon[sel[i]] = i;

    size_t base = (size_t)req * (size_t)Ncap;
    for (int i = 0; i < Ncap; ++i) {
        out->token[base + i] = -1;
        out->parent[base + i] = -2;
        out->depth[base + i] = 0;
        out->mask[base + i] = 0;
        out->surv[base + i] = 0.0f;
        out->logq[base + i] = 0.0f;
    }
    for (int i = 0; i < nsel; ++i) {
        const node_t* nd = &st->v[sel[i]];
        int par = (nd->parent == 0) ? -1 : canon[nd->parent];
        out->token[base + i] = nd->token;
        out->parent[base + i] = (int16_t)par;
        out->depth[base + i] = (uint8_t)nd->depth;
        out->mask[base + i] = ((par >= 0) ? out->mask[base + par] : 0ull) | (1ull << i);
        out->surv[base + i] = nd->s;
        out->logq[base + i] = nd->logq;
    }
    out->n_nodes[req] = nsel;
    size_t cb = (size_t)req * (size_t)(Ncap + 1) * (size_t)k;
    for (int row = 0; row <= Ncap; ++row)
        for (int j = 0; j < k; ++j) out->cand[cb + (size_t)row * k + j] = -1;
    if (st->n > 0 && st->v[0].child0 >= 0)
        for (int j = 0; j < k; ++j) out->cand[cb + j] = st->v[st->v[0].child0 + j].token;
    for (int i = 0; i < nsel; ++i) {
        int c0 = st->v[sel[i]].child0;
        if (c0 < 0) continue;
        for (int j = 0; j < k; ++j)
            out->cand[cb + (size_t)(i + 1) * k + j] = st->v[c0 + j].token;
    }
    free(canon);
}

/* Best-first with a priority queue (TreeSpark core idea: best-first expansion and
 * per-round stopping; PCTree: budget N).  Pop the best pending node by the global order;
 * stop when the budget is full, nothing is pending, or the best survival falls below tau
 * (reading: s == tau is kept). */
static int build_heap(const or_params* P, const float* L_req, const float* U, const float* Wt,
                      store_t* st, int nb, float tau, int* sel, double* ybuf, or_margin* mg,
                      int* n_expand)
{
    int npend = 0, nsel = 0;
    int* pend = (int*)malloc(sizeof(int) * (size_t)(P->k * (nb + 1) + 1));
    expand_in_store(P, L_req, U, Wt, st, 0, ybuf, mg);
    *n_expand = 1;
    for (int j = 0; j < P->k; ++j) pend[npend++] = st->v[0].child0 + j;
    while (nsel < nb && npend > 0) {
        int bi = 0;
        for (int i = 1; i < npend; ++i)
            if (key_better(st, pend[i], pend[bi])) bi = i;
        int best = pend[bi];
        pend[bi] = pend[--npend];
        if (st->v[best].s < tau) break;
        sel[nsel++] = best;
        if (st->v[best].depth < P->B) {
            expand_in_store(P, L_req, U, Wt, st, best, ybuf, mg);
            ++*n_expand;
            for (int j = 0; j < P->k; ++j) pend[npend++] = st->v[best].child0 + j;
        }
    }
    free(pend);
    return nsel;
}

/* Level-synchronous form: at level d expand every depth-(d-1) node of the current set,
 * then keep the best nb of (set + new children) with s >= tau.  Equal to best-first because
 * survival never increases along a path (cal <= 1), so every node ranks below its
 * ancestors. */
static int build_levelsync(const or_params* P, const float* L_req, const float* U,
                           const float* Wt, store_t* st, int nb, float tau, int* sel,
                           double* ybuf, int* n_expand)
{
    int nsel = 0;
    int cap = nb + 64 * P->k + 1;
    int* cand = (int*)malloc(sizeof(int) * (size_t)cap);
    int* front = (int*)malloc(sizeof(int) * (size_t)(nb + 1));
    int nfront = 1;
    front[0] = 0;
    *n_expand = 0;
    for (int d = 1; d <= P->B && nfront > 0; ++d) {
        int nc = 0;
        for (int i = 0; i < nsel; ++i) cand[nc++] = sel[i];
        for (int f = 0; f < nfront; ++f) {
            expand_in_store(P, L_req, U, Wt, st, front[f], ybuf, NULL);
            ++*n_expand;
            for (int j = 0; j < P->k; ++j) cand[nc++] = st->v[front[f]].child0 + j;
        }
        int nk = 0;
        for (int i = 0; i < nc; ++i)
            if (!(st->v[cand[i]].s < tau)) cand[nk++] = cand[i];
        for (int i = 1; i < nk; ++i) {
            int x = cand[i], j = i - 1;
            while (j >= 0 && key_better(st, x, cand[j])) {
                cand[j + 1] = cand[j];
                --j;
            }
            cand[j + 1] = x;
        }
        nsel = nk < nb ? nk : nb;
        for (int i = 0; i < nsel; ++i) sel[i] = cand[i];
        nfront = 0;
        for (int i = 0; i < nsel; ++i)
            if (st->v[sel[i]].depth == d) front[nfront++] = sel[i];
    }
    free(cand);
    free(front);
    return nsel;
}

/* Head tokens of the Shared-Markov control (PCTree summary, mechanism paragraph): first walk
 * the drafter's greedy chain -- c_0 = the root, c_{d+1} = the argmax (ties: lower id) of the
 * head-biased row L[d] + U[c_d] . W -- then every node at depth d is expanded with the chain's
 * distribution of that depth, i.e. with head token c_d.  Without a head, every node's
 * head is -1. */
static void head_tokens(const or_params* P, const float* L_req, const float* U, const float* Wt,
                        int32_t root, double* ybuf, store_t* st)
{
    st->use_head = P->cond != OR_COND_PARENT;
    if (P->cond == OR_COND_NONE) {
        for (int d = 0; d <= P->B; ++d) st->head[d] = -1;
        return;
    }
    if (P->cond != OR_COND_CHAIN) return;
    or_params Q = *P;
    Q.k = 1;
    Q.mode = OR_GREEDY;
    st->head[0] = root;
    for (int d = 0; d + 1 < P->B; ++d) {
        int32_t t;
        double y, lse;
        or_expand(&Q, L_req, U, Wt, d, st->head[d], 0, ybuf, &lse, &t, &y);
        st->head[d + 1] = t;
    }
}

int or_build(const or_params* P, const float* L, const float* U, const float* Wt,
             const int32_t* root_token, const int32_t* n_budget, const float* tau,
             int32_t method, or_tree* out, or_margin* margins)
{
    if (P->k < 1 || P->k > 8 || P->B < 1 || P->B > 32 || P->Ncap < 1 || P->Ncap > 64) return -1;
    double* ybuf = (double*)malloc(sizeof(double) * (size_t)P->V);
    int* sel = (int*)malloc(sizeof(int) * 128);
    for (int req = 0; req < P->R; ++req) {
        const float* L_req = L + (size_t)req * (size_t)P->B * (size_t)P->V;
        or_margin* mg = margins ? &margins[req] : NULL;
        int status = 0;
        int nb = n_budget[req];
        if (nb < 0 || nb > P->Ncap) {
            status |= OR_STATUS_BUDGET_CLAMPED;
            nb = nb < 0 ? 0 : P->Ncap;
        }
        store_t st = {0};
        int nsel = 0, nexp = 0;
        if (root_token[req] < 0 || root_token[req] >= P->V) {
            status |= OR_STATUS_BAD_ROOT;
        } else {
            node_t root;
            root.token = root_token[req];
            root.depth = 0;
            root.parent = -1;
            root.rank = 0;
            root.child0 = -1;
            root.s = 1.0f;
            root.logq = 0.0f;
            root.hash = or_root_hash(P->round, P->req_base + req, root_token[req]);
            store_add(&st, root);
            head_tokens(P, L_req, U, Wt, root_token[req], ybuf, &st);
            if (method == 0)
                nsel = build_heap(P, L_req, U, Wt, &st, nb, tau[req], sel, ybuf, mg, &nexp);
            else
                nsel = build_levelsync(P, L_req, U, Wt, &st, nb, tau[req], sel, ybuf, &nexp);
        }
        emit_tree(P, &st, sel, nsel, req, out);
        out->status[req] = status;
        out->n_expand[req] = nexp;
        free(st.v);
    }
    free(ybuf);
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Two-stage M-ary tree (TreeFlash explainer, technical summary, methodology: two-stage    */
/* inference construction), carried onto this library's Markov head.                     */
/* ------------------------------------------------------------------------------------ */
/* Stage 1: for every block row j, S_j = the M tokens with the largest unconditioned block
 * logits L[j] (ties: lower id); S_j is the only token set the tree uses at depth j + 1.
 * Stage 2: the parent-conditioned law of every state (row j, token t) -- t = the root for
 * j = 0, t in S_{j-1} for j >= 1 -- is evaluated over the whole vocabulary, z = L[j] +
 * U[t] . W, lse = log sum exp z, and for each c in S_j: q(c) = exp(z_c - lse); the M
 * siblings are ranked by (z desc, token asc).  Final selection: best-first top-N with
 * per-round stopping (the same order, calibration and survival as the parent-conditioned
 * tree) over the lattice in which a node of depth j with token t has the children S_j with
 * the q of state (j, t).  M = P->k; greedy mode. */
typedef struct {
    int M, B;
    int32_t* set;  /* [B][M] S_j, logit order */
    int32_t* tok;  /* [B][M][M] state (j, slot) -> children in sibling order */
    double* z;     /* [B][M][M] their conditional logits */
    double* lse;   /* [B][M] */
} flash_t;

static int flash_slot(const flash_t* F, int j, int32_t t)
{
    if (j == 0) return 0;
    for (int s = 0; s < F->M; ++s)
        if (F->set[(size_t)(j - 1) * F->M + s] == t) return s;
    return -1;
}

static void flash_stages(const or_params* P, const float* L_req, const float* U,
                         const float* Wt, int32_t root, flash_t* F, double* ybuf,
                         or_margin* mg)
{
    const int M = F->M, V = P->V;
    /* stage 1: M passes of "largest logit, lower id on ties" per row */
    unsigned char* taken = (unsigned char*)malloc((size_t)V);
    for (int j = 0; j < F->B; ++j) {
        const float* row = L_req + (size_t)j * (size_t)V;
        memset(taken, 0, (size_t)V);
        for (int s = 0; s < M; ++s) {
            int best = -1;
            for (int c = 0; c < V; ++c)
                if (!taken[c] && (best < 0 || (double)row[c] > (double)row[best])) best = c;
            taken[best] = 1;
            F->set[(size_t)j * M + s] = best;
        }
    }
    free(taken);
    /* stage 2: every state's conditional law over V, gathered at S_j */
    or_params Q = *P;
    Q.k = 1;
    Q.mode = OR_GREEDY;
    for (int j = 0; j < F->B; ++j) {
        const int nstate = j == 0 ? 1 : M;
        for (int s = 0; s < nstate; ++s) {
            const int32_t t = j == 0 ? root : F->set[(size_t)(j - 1) * M + s];
            int32_t ct;
            double cy, lse;
            or_expand(&Q, L_req, U, Wt, j, t, 0, ybuf, &lse, &ct, &cy);
            const size_t st = (size_t)j * M + s;
            F->lse[st] = lse;
            int32_t* tk = F->tok + st * M;
            double* zz = F->z + st * M;
            for (int i = 0; i < M; ++i) {
                tk[i] = F->set[(size_t)j * M + i];
                zz[i] = ybuf[tk[i]];
            }
            for (int i = 1; i < M; ++i) { /* insertion sort: z desc, token asc */
                int32_t xt = tk[i];
                double xz = zz[i];
                int a = i - 1;
                while (a >= 0 && (zz[a] < xz || (zz[a] == xz && tk[a] > xt))) {
                    tk[a + 1] = tk[a];
                    zz[a + 1] = zz[a];
                    --a;
                }
                tk[a + 1] = xt;
                zz[a + 1] = xz;
            }
            if (mg)
                for (int i = 1; i < M; ++i) upd_min(&mg->key_gap, zz[i - 1] - zz[i]);
        }
    }
}

static void expand_flash(const or_params* P, const flash_t* F, store_t* st, int idx,
                         or_margin* mg)
{
    const int M = F->M;
    node_t par = st->v[idx];
    const int j = par.depth;
    const size_t sti = (size_t)j * M + flash_slot(F, j, par.token);
    int first = -1;
    for (int i = 0; i < M; ++i) {
        const double lq = F->z[sti * M + i] - F->lse[sti];
        const double q = exp(lq);
        if (mg) upd_min(&mg->q_edge, q_edge_distance(q));
        node_t ch;
        ch.token = F->tok[sti * M + i];
        ch.depth = j + 1;
        ch.parent = idx;
        ch.rank = i;
        ch.child0 = -1;
        ch.s = par.s * P->cal[cal_bin(q)]; /* float x float, rounded to float */
        ch.logq = (float)lq;
        ch.hash = or_child_hash(par.hash, ch.token);
        int id = store_add(st, ch);
        if (i == 0) first = id;
    }
    st->v[idx].child0 = first;
}

int or_build_flash(const or_params* P, const float* L, const float* U, const float* Wt,
                   const int32_t* root_token, const int32_t* n_budget, const float* tau,
                   or_tree* out, or_margin* margins)
{
    if (P->k < 1 || P->k > 8 || P->k > P->V || P->B < 1 || P->B > 32 || P->Ncap < 1 ||
        P->Ncap > 64 || P->mode != OR_GREEDY)
        return -1;
    const int M = P->k, B = P->B;
    double* ybuf = (double*)malloc(sizeof(double) * (size_t)P->V);
    int* sel = (int*)malloc(sizeof(int) * 128);
    flash_t F;
    F.M = M;
    F.B = B;
    F.set = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * M);
    F.tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * M * M);
    F.z = (double*)malloc(sizeof(double) * (size_t)B * M * M);
    F.lse = (double*)malloc(sizeof(double) * (size_t)B * M);
    for (int req = 0; req < P->R; ++req) {
        const float* L_req = L + (size_t)req * (size_t)B * (size_t)P->V;
        or_margin* mg = margins ? &margins[req] : NULL;
        int status = 0, nsel = 0, nexp = 0;
        int nb = n_budget[req];
        if (nb < 0 || nb > P->Ncap) {
            status |= OR_STATUS_BUDGET_CLAMPED;
            nb = nb < 0 ? 0 : P->Ncap;
        }
        store_t st = {0};
        if (root_token[req] < 0 || root_token[req] >= P->V) {
            status |= OR_STATUS_BAD_ROOT;
        } else {
            flash_stages(P, L_req, U, Wt, root_token[req], &F, ybuf, mg);
            node_t root;
            root.token = root_token[req];
            root.depth = 0;
            root.parent = -1;
            root.rank = 0;
            root.child0 = -1;
            root.s = 1.0f;
            root.logq = 0.0f;
            root.hash = or_root_hash(P->round, P->req_base + req, root_token[req]);
            store_add(&st, root);
            /* best-first with a priority queue, as build_heap, over the lattice */
            int npend = 0;
            int* pend = (int*)malloc(sizeof(int) * (size_t)(M * (nb + 1) + 1));
            expand_flash(P, &F, &st, 0, mg);
            nexp = 1;
            for (int i = 0; i < M; ++i) pend[npend++] = st.v[0].child0 + i;
            while (nsel < nb && npend > 0) {
                int bi = 0;
                for (int i = 1; i < npend; ++i)
                    if (key_better(&st, pend[i], pend[bi])) bi = i;
                int best = pend[bi];
                pend[bi] = pend[--npend];
                if (st.v[best].s < tau[req]) break;
                sel[nsel++] = best;
                if (st.v[best].depth < B) {
                    expand_flash(P, &F, &st, best, mg);
                    ++nexp;
                    for (int i = 0; i < M; ++i) pend[npend++] = st.v[best].child0 + i;
                }
            }
            free(pend);
        }
        emit_tree(P, &st, sel, nsel, req, out);
        out->status[req] = status;
        out->n_expand[req] = nexp;
        free(st.v);
    }
    free(F.set);
    free(F.tok);
    free(F.z);
    free(F.lse);
    free(ybuf);
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Verification.                                                                           */
/* ------------------------------------------------------------------------------------ */
static int find_child(const or_tree* T, const or_params* P, int req, int parent, int32_t tok)
{
    size_t base = (size_t)req * (size_t)P->Ncap;
    for (int i = 0; i < T->n_nodes[req]; ++i)
        if (T->parent[base + i] == parent && T->token[base + i] == tok) return i;
    return -1;
}

/* Greedy accept-walk (PCTree setup: greedy verification).  At the current node take the
 * target row's argmax (ties: lower id); descend while a child carries that token; the
 * first unmatched argmax is the bonus token. */
int or_verify_greedy(const or_params* P, const or_tree* T, const float* target,
                     or_verify* out, or_margin* margins)
{
    const int V = P->V, B = P->B, Ncap = P->Ncap;
    for (int req = 0; req < P->R; ++req) {
        for (int i = 0; i < B; ++i) out->path[(size_t)req * B + i] = -1;
        for (int i = 0; i <= B; ++i) out->out_tokens[(size_t)req * (B + 1) + i] = -1;
        if (T->status[req] & OR_STATUS_BAD_ROOT) {
            out->accept_len[req] = 0;
            out->n_out[req] = 0;
            continue;
        }
        int v = -1, row = 0, nacc = 0;
        for (;;) {
            const float* t = target + ((size_t)req * (Ncap + 1) + row) * (size_t)V;
            int best = 0;
            for (int c = 1; c < V; ++c)
                if (t[c] > t[best]) best = c;
            if (margins) {
                double second = -INFINITY;
                for (int c = 0; c < V; ++c)
                    if (c != best && t[c] > second) second = t[c];
                upd_min(&margins[req].argmax_gap, (double)t[best] - second);
            }
            out->out_tokens[(size_t)req * (B + 1) + nacc] = best;
            int w = find_child(T, P, req, v, best);
            if (w < 0) break;
            out->path[(size_t)req * B + nacc] = w;
            ++nacc;
            v = w;
            row = w + 1;
        }
        out->accept_len[req] = nacc;
        out->n_out[req] = nacc + 1;
    }
    return 0;
}

/* One rejection step (TreeSpark lossless section: after a rejected sibling the target law
 * becomes the normalised residual max(p - q, 0) and the rejected sibling leaves the draft
 * law, which is renormalised).  Returns 0 when the residual mass is zero, which in exact
 * arithmetic cannot follow a rejection (reading: treated as an accept). */
static int residual_step(double* pj, double* qj, int32_t x, int V)
{
    double Z = 0.0;
    for (int y = 0; y < V; ++y) {
        double d = pj[y] - qj[y];
        if (d > 0.0) Z += d;
    }
    if (!(Z > 0.0)) return 0;
    if (g_fault != 2) {
        for (int y = 0; y < V; ++y) {
            double d = pj[y] - qj[y];
            pj[y] = (d > 0.0 ? d : 0.0) / Z;
        }
    }
    if (g_fault != 1) {
        qj[x] = 0.0;
        double S = 0.0;
        for (int y = 0; y < V; ++y) S += qj[y];
        for (int y = 0; y < V; ++y) qj[y] /= S;
    }
    return 1;
}

void or_chain_probs(const double* p, const double* q, int32_t V, const int32_t* x, int32_t k,
                    double* acc, double* resid)
{
    double* pj = (double*)malloc(sizeof(double) * (size_t)V);
    double* qj = (double*)malloc(sizeof(double) * (size_t)V);
    memcpy(pj, p, sizeof(double) * (size_t)V);
    memcpy(qj, q, sizeof(double) * (size_t)V);
    int j = 0;
    for (; j < k; ++j) {
        double a = pj[x[j]] / qj[x[j]];
        acc[j] = a < 1.0 ? a : 1.0;
        if (acc[j] >= 1.0) break;
        if (!residual_step(pj, qj, x[j], V)) {
            acc[j] = 1.0;
            break;
        }
    }
    for (int i = j + 1; i < k; ++i) acc[i] = 1.0;
    memcpy(resid, pj, sizeof(double) * (size_t)V);
    free(pj);
    free(qj);
}

/* Gumbel-max draw from log-weights lw (entries with lw = -inf excluded); ties: lower id. */
static int gumbel_argmax(const double* lw, int V, uint64_t seed, uint64_t hash, double* gap)
{
    int best = -1;
    double bk = -INFINITY, second = -INFINITY;
    for (int c = 0; c < V; ++c) {
        if (lw[c] == -INFINITY) continue;
        double key = lw[c] + gumbel(seed, hash, OR_STREAM_RESID, (uint32_t)c);
        if (best < 0 || key > bk) {
            second = bk;
            bk = key;
            best = c;
        } else if (key > second) {
            second = key;
        }
    }
    *gap = bk - second;
    return best;
}

/* Lossless sample verify (TreeSpark lossless section; Leviathan et al. 2023 acceptance
 * rule as recalled on the same page).  At each visited node v: p = softmax(target/T),
 * q = softmax(z_v/T).  The drawn siblings are tried in draw order; x_j is accepted iff
 * u_j * q_j(x_j) < p_j(x_j); after a rejection p and q become the residual laws.  Reading
 * for pruned trees: a drawn sibling that is not in the tree is still tested and, when
 * accepted, ends the round as a leaf.  If every sibling is rejected the round ends with a
 * draw from the final residual; at a depth-B node the round ends with a draw from p. */
int or_verify_sample(const or_params* P, const or_tree* T, const float* L, const float* U,
                     const float* Wt, const int32_t* root_token, const float* target,
                     or_verify* out, or_margin* margins)
{
    const int V = P->V, B = P->B, Ncap = P->Ncap, k = P->k;
    const double Temp = P->temperature;
    double* y = (double*)malloc(sizeof(double) * (size_t)V);
    double* yp = (double*)malloc(sizeof(double) * (size_t)V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    double* lw = (double*)malloc(sizeof(double) * (size_t)V);
    for (int req = 0; req < P->R; ++req) {
        or_margin* mg = margins ? &margins[req] : NULL;
        for (int i = 0; i < B; ++i) out->path[(size_t)req * B + i] = -1;
        for (int i = 0; i <= B; ++i) out->out_tokens[(size_t)req * (B + 1) + i] = -1;
        if (T->status[req] & OR_STATUS_BAD_ROOT) {
            out->accept_len[req] = 0;
            out->n_out[req] = 0;
            continue;
        }
        const float* L_req = L + (size_t)req * (size_t)B * (size_t)V;
        int v = -1, row = 0, prow = 0, depth = 0, nacc = 0, nemit = 0;
        int32_t token = root_token[req];
        uint64_t hash = or_root_hash(P->round, P->req_base + req, token);
        for (;;) {
            /* fault 3 (negative control): the depth-B draw reads the parent's target row */
            const int trow = (depth == B && g_fault == 3) ? prow : row;
            const float* t = target + ((size_t)req * (Ncap + 1) + trow) * (size_t)V;
            for (int c = 0; c < V; ++c) yp[c] = (double)t[c] / Temp;
            double gap;
            if (depth == B) {
                int x = gumbel_argmax(yp, V, P->seed, hash, &gap);
                if (mg) upd_min(&mg->draw_gap, gap);
                out->out_tokens[(size_t)req * (B + 1) + nemit++] = x;
                break;
            }
            double mp = yp[0];
            for (int c = 1; c < V; ++c)
                if (yp[c] > mp) mp = yp[c];
            double sp = 0.0;
            for (int c = 0; c < V; ++c) sp += exp(yp[c] - mp);
            for (int c = 0; c < V; ++c) p[c] = exp(yp[c] - mp) / sp;
            int32_t ctok[8];
            double cy[8], lse;
            or_expand(P, L_req, U, Wt, depth, token, hash, y, &lse, ctok, cy);
            for (int c = 0; c < V; ++c) q[c] = exp(y[c] - lse);
            const int32_t* cand = T->cand + ((size_t)req * (Ncap + 1) + row) * (size_t)k;
            int accepted = -1;
            for (int j = 0; j < k; ++j) {
                int32_t x = cand[j];
                /* reading: a ranked list shorter than k (only possible when the draft row
                 * holds non-finite values) leaves slot j empty (-1); an empty slot is no
                 * drawn sibling and is skipped */
                if (x < 0 || x >= V) continue;
                double u = or_uniform(P->seed, hash, OR_STREAM_ACCEPT, (uint32_t)j);
                if (mg && q[x] > 0.0) upd_min(&mg->accept, fabs(u - p[x] / q[x]));
                if (u * q[x] < p[x]) {
                    accepted = x;
                    break;
                }
                if (!residual_step(p, q, x, V)) {
                    accepted = x;
                    break;
                }
            }
            if (accepted >= 0) {
                out->out_tokens[(size_t)req * (B + 1) + nemit++] = accepted;
                int w = find_child(T, P, req, v, accepted);
                if (w < 0) break; /* accepted sibling outside the tree: ends the round */
                out->path[(size_t)req * B + nacc++] = w;
                v = w;
                prow = row;
                row = w + 1;
                depth += 1;
                token = accepted;
                hash = or_child_hash(hash, accepted);
                continue;
            }
            for (int c = 0; c < V; ++c) lw[c] = p[c] > 0.0 ? log(p[c]) : -INFINITY;
            int x = gumbel_argmax(lw, V, P->seed, hash, &gap);
            if (mg) upd_min(&mg->draw_gap, gap);
            out->out_tokens[(size_t)req * (B + 1) + nemit++] = x;
            break;
        }
        out->accept_len[req] = nacc;
        out->n_out[req] = nemit;
    }
    free(y);
    free(yp);
    free(p);
    free(q);
    free(lw);
    return 0;
}

int or_sample_rounds(const or_params* P0, const float* L, const float* U, const float* Wt,
                     int32_t root_token, int32_t n_budget, float tau, const float* target_tab,
                     int64_t n_rounds, int32_t* first, int32_t* second)
{
    or_params P = *P0;
    P.R = 1;
    const int V = P.V, Ncap = P.Ncap, k = P.k, B = P.B;
    or_tree T;
    T.token = (int32_t*)malloc(sizeof(int32_t) * Ncap);
    T.parent = (int16_t*)malloc(sizeof(int16_t) * Ncap);
    T.depth = (uint8_t*)malloc((size_t)Ncap);
    T.mask = (uint64_t*)malloc(sizeof(uint64_t) * Ncap);
    T.surv = (float*)malloc(sizeof(float) * Ncap);
    T.logq = (float*)malloc(sizeof(float) * Ncap);
    T.n_nodes = (int32_t*)malloc(sizeof(int32_t));
    T.cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(Ncap + 1) * k);
    T.status = (int32_t*)malloc(sizeof(int32_t));
    T.n_expand = (int32_t*)malloc(sizeof(int32_t));
    or_verify O;
    O.accept_len = (int32_t*)malloc(sizeof(int32_t));
    O.path = (int32_t*)malloc(sizeof(int32_t) * B);
    O.out_tokens = (int32_t*)malloc(sizeof(int32_t) * (B + 1));
    O.n_out = (int32_t*)malloc(sizeof(int32_t));
    float* target = (float*)malloc(sizeof(float) * (size_t)(Ncap + 1) * V);
    for (int64_t n = 0; n < n_rounds; ++n) {
        P.round = (uint32_t)n;
        or_build(&P, L, U, Wt, &root_token, &n_budget, &tau, 0, &T, NULL);
        memcpy(target, target_tab + (size_t)root_token * V, sizeof(float) * V);
        for (int i = 0; i < T.n_nodes[0]; ++i)
            memcpy(target + (size_t)(i + 1) * V,
                   target_tab + ((size_t)T.depth[i] * V + (size_t)T.token[i]) * V,
                   sizeof(float) * V);
        or_verify_sample(&P, &T, L, U, Wt, &root_token, target, &O, NULL);
        first[n] = O.out_tokens[0];
        second[n] = O.n_out[0] > 1 ? O.out_tokens[1] : -1;
    }
    free(T.token); free(T.parent); free(T.depth); free(T.mask); free(T.surv); free(T.logq);
    free(T.n_nodes); free(T.cand); free(T.status); free(T.n_expand);
    free(O.accept_len); free(O.path); free(O.out_tokens); free(O.n_out);
    free(target);
    return 0;
}
