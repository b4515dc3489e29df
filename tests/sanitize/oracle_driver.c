/* Sanitizer driver for the oracle: runs every exported oracle function on small random
 * instances (both build methods, both modes, every head variant, the sampling driver and
 * the chain probabilities) and checks the return codes and that the two build methods
 * agree.  Built with -fsanitize=address,undefined by tests/test_sanitizers.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dtree_oracle.h"

static double rnd(uint64_t* s) {
    *s = *s * 6364136223846793005ull + 1442695040888963407ull;
    return ((*s >> 11) + 0.5) / 9007199254740992.0;
}

static double gauss(uint64_t* s) {
    const double u = rnd(s), v = rnd(s);
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

typedef struct {
    int32_t *token, *n_nodes, *cand, *status, *n_expand, *acc, *path, *outt, *nout;
    int16_t* parent;
    uint8_t* depth;
    uint64_t* mask;
    float *surv, *logq;
} bufs;

static void alloc_tree(bufs* b, int R, int Ncap, int k, int B, or_tree* t, or_verify* v) {
    b->token = calloc((size_t)R * Ncap, 4);
    b->parent = calloc((size_t)R * Ncap, 2);
    b->depth = calloc((size_t)R * Ncap, 1);
    b->mask = calloc((size_t)R * Ncap, 8);
    b->surv = calloc((size_t)R * Ncap, 4);
    b->logq = calloc((size_t)R * Ncap, 4);
    b->n_nodes = calloc(R, 4);
    b->cand = calloc((size_t)R * (Ncap + 1) * k, 4);
    b->status = calloc(R, 4);
    b->n_expand = calloc(R, 4);
    b->acc = calloc(R, 4);
    b->path = calloc((size_t)R * B, 4);
    b->outt = calloc((size_t)R * (B + 1), 4);
    b->nout = calloc(R, 4);
    *t = (or_tree){b->token, b->parent, b->depth, b->mask, b->surv, b->logq, b->n_nodes,
                   b->cand, b->status, b->n_expand};
    *v = (or_verify){b->acc, b->path, b->outt, b->nout};
}

static void free_tree(bufs* b) {
    free(b->token); free(b->parent); free(b->depth); free(b->mask); free(b->surv);
    free(b->logq); free(b->n_nodes); free(b->cand); free(b->status); free(b->n_expand);
    free(b->acc); free(b->path); free(b->outt); free(b->nout);
}

static int run_case(uint64_t seed, int R, int B, int k, int V, int r, int Ncap, int mode,
                    int cond, double T) {
    uint64_t s = seed;
    float* L = malloc(sizeof(float) * R * B * V);
    float* U = malloc(sizeof(float) * V * r);
    float* Wt = malloc(sizeof(float) * V * r);
    float* tgt = malloc(sizeof(float) * R * (Ncap + 1) * V);
    int32_t *root = malloc(4 * R), *nb = malloc(4 * R);
    float* tau = malloc(4 * R);
    for (int i = 0; i < R * B * V; ++i) L[i] = (float)(2.0 * gauss(&s));
    for (int i = 0; i < V * r; ++i) U[i] = (float)(gauss(&s) / sqrt(r));
    for (int i = 0; i < V * r; ++i) Wt[i] = (float)(gauss(&s) / sqrt(r));
    for (int i = 0; i < R * (Ncap + 1) * V; ++i) tgt[i] = (float)(2.0 * gauss(&s));
    for (int i = 0; i < R; ++i) {
        root[i] = (int32_t)(rnd(&s) * V);
        nb[i] = i == 0 ? Ncap : (int32_t)(rnd(&s) * (Ncap + 1));
        tau[i] = i == 1 ? 0.3f : 0.0f;
    }
    root[R - 1] = V + 3; /* a bad root: empty tree, status bit */
    or_params P;
    memset(&P, 0, sizeof(P));
    P.R = R; P.B = B; P.k = k; P.V = V; P.r = r; P.Ncap = Ncap; P.mode = mode;
    P.temperature = T; P.seed = seed; P.round = 7; P.req_base = 0; P.cond = cond;
    for (int i = 0; i < 16; ++i) P.cal[i] = (float)((i + 0.5) / 16.0);
    bufs b0, b1;
    or_tree t0, t1;
    or_verify v0, v1;
    alloc_tree(&b0, R, Ncap, k, B, &t0, &v0);
    alloc_tree(&b1, R, Ncap, k, B, &t1, &v1);
    or_margin* mg = calloc(R, sizeof(or_margin));
    int bad = 0;
    bad |= or_build(&P, L, U, Wt, root, nb, tau, 0, &t0, mg) != 0;
    bad |= or_build(&P, L, U, Wt, root, nb, tau, 1, &t1, NULL) != 0;
    bad |= memcmp(b0.token, b1.token, 4 * (size_t)R * Ncap) != 0;
    bad |= memcmp(b0.mask, b1.mask, 8 * (size_t)R * Ncap) != 0;
    if (mode == OR_GREEDY)
        bad |= or_verify_greedy(&P, &t0, tgt, &v0, mg) != 0;
    else
        bad |= or_verify_sample(&P, &t0, L, U, Wt, root, tgt, &v0, mg) != 0;
    if (mode == OR_SAMPLE && cond == OR_COND_PARENT) {
        float* tab = malloc(sizeof(float) * (B + 1) * V * V);
        for (int i = 0; i < (B + 1) * V * V; ++i) tab[i] = (float)(1.5 * gauss(&s));
        int32_t first[200], second[200];
        bad |= or_sample_rounds(&P, L, U, Wt, root[0], Ncap, 0.0f, tab, 200, first, second) != 0;
        free(tab);
    }
    free_tree(&b0);
    free_tree(&b1);
    free(mg); free(L); free(U); free(Wt); free(tgt); free(root); free(nb); free(tau);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run_case(1, 3, 3, 2, 40, 4, 8, OR_GREEDY, OR_COND_PARENT, 1.0);
    bad |= run_case(2, 4, 4, 3, 33, 8, 12, OR_GREEDY, OR_COND_CHAIN, 1.0);
    bad |= run_case(3, 3, 3, 3, 29, 4, 10, OR_GREEDY, OR_COND_NONE, 1.0);
    bad |= run_case(4, 3, 3, 2, 24, 4, 6, OR_SAMPLE, OR_COND_PARENT, 0.6);
    bad |= run_case(5, 2, 1, 3, 16, 4, 3, OR_SAMPLE, OR_COND_PARENT, 1.5);
    bad |= run_case(6, 2, 5, 1, 50, 2, 64, OR_GREEDY, OR_COND_PARENT, 1.0);
    for (int f = 1; f <= 3; ++f) {
        or_set_fault(f);
        bad |= run_case(10 + f, 2, 2, 3, 16, 4, 5, OR_SAMPLE, OR_COND_PARENT, 1.0);
    }
    or_set_fault(0);
    {
        double p[7] = {0.1, 0.2, 0.05, 0.3, 0.15, 0.1, 0.1}, q[7] = {0.3, 0.1, 0.1, 0.1, 0.2, 0.1, 0.1};
        int32_t x[3] = {0, 4, 1};
        double acc[3], res[7];
        or_chain_probs(p, q, 7, x, 3, acc, res);
        double sum = 0.0;
        for (int i = 0; i < 7; ++i) sum += res[i];
        bad |= fabs(sum - 1.0) > 1e-12;
    }
    uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4];
    or_philox4x32_10(ctr, key, out);
    (void)or_uniform(1, or_child_hash(or_root_hash(1, 2, 3), 4), 1, 5);
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
