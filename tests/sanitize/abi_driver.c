/* Sanitizer driver for the library's host-side code: parameter validation, workspace and
 * attention planning, argument rejection (every call here returns before anything reaches
 * a device), the load policy and the status strings.  Linked against a build of libdtree
 * whose host code is compiled with -fsanitize=address,undefined by tests/test_sanitizers.py
 * (no GPU is needed). */
#include <stdio.h>
#include <string.h>

#include "dtree.h"

static dt_params base(void) {
    dt_params p;
    memset(&p, 0, sizeof(p));
    p.R = 4; p.B = 16; p.k = 4; p.V = 151936; p.r = 256; p.Ncap = 64;
    p.logits_dtype = DT_BF16; p.head_dtype = DT_BF16; p.mode = DT_GREEDY; p.temperature = 1.0f;
    for (int i = 0; i < 16; ++i) p.cal[i] = (i + 0.5f) / 16.0f;
    return p;
}

int main(void) {
    int bad = 0;
    size_t n = 0;
    /* workspace sizes over a sweep of shapes, both modes */
    for (int R = 1; R <= 4096; R *= 4)
        for (int k = 1; k <= 8; k *= 2)
            for (int mode = 0; mode < 2; ++mode) {
                dt_params p = base();
                p.R = R; p.k = k; p.mode = mode; p.Ncap = 1 + (R * k) % 64;
                bad |= dt_build_workspace_bytes(&p, &n) != DT_OK || n == 0;
            }
    dt_params p = base();
    p.B = 33;
    bad |= dt_build_workspace_bytes(&p, &n) != DT_EINVAL;
    p = base();
    p.cal[3] = 0.01f; /* decreasing table */
    bad |= dt_build_workspace_bytes(&p, &n) != DT_EINVAL;
    /* argument rejection before any device work */
    p = base();
    dt_tree t;
    memset(&t, 0, sizeof(t));
    char fake[64];
    bad |= tree_build(&p, NULL, fake, fake, NULL, NULL, NULL, &t, NULL, 0, NULL) != DT_EINVAL;
    dt_build_workspace_bytes(&p, &n);
    void* al = (void*)(((unsigned long)fake + 255) & ~255ul);
    dt_tree t2;
    t2.token = (int32_t*)al; t2.parent = (int16_t*)al; t2.depth = (uint8_t*)al;
    t2.anc_mask = (uint64_t*)al; t2.surv = (float*)al; t2.logq = (float*)al;
    t2.n_nodes = (int32_t*)al; t2.cand = (int32_t*)al; t2.status = (int32_t*)al;
    t2.n_expand = NULL; t2.level_rows = NULL;
    bad |= tree_build(&p, al, al, al, al, al, al, &t2, (void*)0x100000, n - 1, NULL) != DT_ENOSPC;
    dt_params big = base();
    big.R = 4096; big.k = 8; big.B = 32;
    bad |= tree_build_noalloc(&big, al, al, al, al, al, al, &t2, NULL) != DT_ENOSPC;
    dt_verify_out v;
    memset(&v, 0, sizeof(v));
    bad |= tree_verify_greedy(&p, &t2, al, &v, al, n, NULL) != DT_EINVAL;
    bad |= tree_verify_sample(&p, &t2, al, al, al, al, al, &v, al, n, NULL) != DT_EINVAL;
    /* attention planning and rejection */
    for (int R = 1; R <= 256; R *= 2)
        for (int Hq = 8; Hq <= 64; Hq *= 2) {
            dt_attn_params a = {R, Hq, 8, 128, 64, 2113, 0.088f};
            bad |= dt_attn_workspace_bytes(&a, &n) != DT_OK;
        }
    dt_attn_params a = {1, 32, 8, 128, 64, 2113, 0.088f};
    dt_attn_workspace_bytes(&a, &n);
    bad |= tree_attention(&a, al, al, al, al, &t2, al, NULL, 0, NULL) != DT_EINVAL;
    a.D = 64;
    bad |= dt_attn_workspace_bytes(&a, &n) != DT_EINVAL;
    /* load policy */
    dt_policy pol = {0.5f, 256, 64};
    float tau[64];
    int32_t nb[64];
    for (int i = 0; i <= 20; ++i)
        bad |= dt_load_policy(&pol, i / 20.0f, 64, tau, nb) != DT_OK;
    bad |= dt_load_policy(&pol, 1.5f, 64, tau, nb) != DT_EINVAL;
    for (int s = -1; s < 6; ++s) bad |= dt_status_string(s) == NULL;
    double ms;
    int32_t launches;
    bad |= dt_timing_enable(0) != DT_OK;
    bad |= dt_timing_read(&ms, &launches) != DT_OK || launches != 0;
    printf(bad ? "abi driver: FAILED\n" : "abi driver: ok\n");
    return bad;
}
