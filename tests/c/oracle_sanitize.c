/*
 * oracle_sanitize.c - drives every oracle function on small deterministic
 * inputs; built with the address and undefined-behaviour sanitizers by
 * tests/test_oracle_sanitize.py, so that an out-of-bounds access, a leak or
 * undefined arithmetic anywhere in the oracle fails the test.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "peg_oracle.h"

static uint32_t state = 12345u;
static uint32_t next(void) {
    state = state * 1103515245u + 12345u;
    return state >> 8;
}

#define CHECK(x)                                          \
    do {                                                  \
        if ((x) != 0) {                                   \
            fprintf(stderr, "oracle call failed: %s\n", #x); \
            return 1;                                     \
        }                                                 \
    } while (0)

static int run(int64_t T, int32_t K, int32_t E, int32_t C, int32_t m, int64_t H) {
    int64_t total = T * K;
    int32_t* top = malloc(sizeof(int32_t) * (size_t)(total + 1));
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)(total + 1));
    int32_t* bid = malloc(sizeof(int32_t) * (size_t)(total + 1));
    int32_t* rows = malloc(sizeof(int32_t) * (size_t)(total + 1));
    int32_t *tpe = malloc(sizeof(int32_t) * E), *bins = malloc(sizeof(int32_t) * E);
    int32_t *pb = malloc(sizeof(int32_t) * E), *base = malloc(sizeof(int32_t) * E), *lim = malloc(sizeof(int32_t) * E);
    float* w = malloc(sizeof(float) * (size_t)(total + 1));
    for (int64_t a = 0; a < total; ++a) {
        top[a] = (int32_t)(next() % (uint32_t)(E + 1)) - 1; /* -1 .. E-1 */
        w[a] = (float)(next() % 1000) / 1000.0f;
    }
    int64_t n = pego_route_prep(top, T, K, E, m, idx, bid, tpe, bins, pb);
    if (n < 0) return 1;
    CHECK(pego_assignment_rows(T, K, E, PEGO_BINNED, C, idx, bid, bins, pb, rows));
    CHECK(pego_assignment_rows(T, K, E, PEGO_PADDED, C, idx, bid, bins, pb, rows));
    for (int32_t e = 0; e < E; ++e) {
        base[e] = e * C;
        lim[e] = e * C + (int32_t)(next() % (uint32_t)(C + 1));
    }
    CHECK(pego_assignment_rows_windows(T, K, E, idx, bid, bins, base, lim, rows));
    int64_t R_bin = (int64_t)E * C, R_pad = E ? pb[E - 1] : 0;
    int64_t R = R_bin > R_pad ? R_bin : R_pad;
    float* x = malloc(sizeof(float) * (size_t)(T * H + 1));
    float* g = malloc(sizeof(float) * (size_t)(T * H + 1));
    float* y = malloc(sizeof(float) * (size_t)(R * H + 1));
    float* out = malloc(sizeof(float) * (size_t)(T * H + 1));
    double* scale = malloc(sizeof(double) * (size_t)(T * (H > K ? H : K) + 1));
    float* wg = malloc(sizeof(float) * (size_t)(total + 1));
    for (int64_t i = 0; i < T * H; ++i) {
        x[i] = (float)((int)(next() % 2001) - 1000) / 100.0f;
        g[i] = (float)((int)(next() % 2001) - 1000) / 100.0f;
    }
    for (int layout = 0; layout < 2; ++layout) {
        int64_t Rl = layout == PEGO_BINNED ? R_bin : R_pad;
        CHECK(pego_gather(x, T, H * 4, K, E, layout, C, idx, bid, bins, pb, Rl, NULL, 0, y));
        CHECK(pego_scatter_combine(y, PEGO_F32, Rl, T, H, K, E, layout, C, idx, bid, bins, pb, w, NULL, 0, out, scale));
        CHECK(pego_wgrad(y, g, PEGO_F32, Rl, T, H, K, E, layout, C, idx, bid, bins, pb, NULL, 0, wg, scale));
        CHECK(pego_combine_backward_dy(g, PEGO_F32, T, H, K, E, layout, C, idx, bid, bins, pb, w, Rl, NULL, 0, y));
    }
    (void)pego_validate_routing(idx, bid, bins, pb, T, K, E, n);
    /* compaction: a routing map of T rows x E experts, topk = min(E, 3) */
    uint8_t* rmap = malloc((size_t)(T * E + 1));
    float* probs = malloc(sizeof(float) * (size_t)(T * E + 1));
    for (int64_t i = 0; i < T * E; ++i) {
        rmap[i] = (uint8_t)(next() % 3 == 0);
        probs[i] = (float)(next() % 1000) / 1000.0f;
    }
    int32_t topk = E < 3 ? E : 3;
    float* pout = malloc(sizeof(float) * (size_t)(T * topk + 1));
    int32_t* rexp = malloc(sizeof(int32_t) * (size_t)(T * topk + 1));
    float* dense = malloc(sizeof(float) * (size_t)(T * E + 1));
    CHECK(pego_routing_map_compact(probs, PEGO_F32, rmap, T, E, topk, pout, rexp));
    CHECK(pego_routing_map_compact_backward(pout, rexp, T, E, topk, dense));
    /* gating on the probs as scores, both gating functions */
    int32_t* gtop = malloc(sizeof(int32_t) * (size_t)(T * K + 1));
    float* gw = malloc(sizeof(float) * (size_t)(T * K + 1));
    if (K <= E) {
        CHECK(pego_router_topk(probs, PEGO_F32, T, E, K, 0, 1, gtop, gw));
        CHECK(pego_router_topk(probs, PEGO_F32, T, E, K, 1, 0, gtop, gw));
    }
    free(top); free(idx); free(bid); free(rows); free(tpe); free(bins); free(pb); free(base); free(lim); free(w);
    free(x); free(g); free(y); free(out); free(scale); free(wg); free(rmap); free(probs); free(pout); free(rexp);
    free(dense); free(gtop); free(gw);
    return 0;
}

int main(void) {
    int rc = 0;
    rc |= run(0, 2, 4, 3, 2, 5);
    rc |= run(1, 1, 1, 1, 1, 1);
    rc |= run(17, 2, 5, 3, 4, 7);
    rc |= run(40, 4, 6, 9, 3, 3);
    rc |= run(33, 8, 8, 20, 8, 9);
    if (rc) return 1;
    printf("oracle sanitize ok\n");
    return 0;
}
