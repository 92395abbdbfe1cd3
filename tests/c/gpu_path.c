/*
 * gpu_path.c - the routing path driven from plain C through include/peg.h,
 * with no Python in the process: device buffers come from the HIP runtime,
 * every call goes to libpeg.so, and every output is compared with the CPU
 * oracle (oracle/peg_oracle.h) on the same seeded batch. Test
 * infrastructure; tests/test_gpu_c_driver.py runs it on a GPU.
 *
 * Cases: both layouts (binned with a capacity that drops routes, padded to a
 * multiple), bf16 rows of a width that leaves a ragged tail, absent routes.
 * Index outputs and the gathered tensor must match bit for bit; the combine
 * and wgrad must be within |gpu - oracle| <= rtol*|oracle| + 1e-5*scale,
 * rtol 2e-2 for the bf16 combine and 1e-5 for the float wgrad, where scale
 * is the oracle's sum of the magnitudes of the terms. The combine backward
 * (dout = the gradient rows; one pass at K = 2, the dy gather then the
 * wgrad kernel at K = 4): dy within one bf16 rounding of the oracle's, its
 * wgrad equal to the wgrad kernel's bit for bit.
 *
 * Exit status 0 and a last line "gpu_path ok" when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "peg.h"
#include "peg_oracle.h"

static int failures = 0;

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, \
                    __LINE__);                                                        \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

#define PEG_OK_(call)                                                                      \
    do {                                                                                   \
        peg_status s_ = (call);                                                            \
        if (s_ != PEG_OK) {                                                                \
            fprintf(stderr, "peg error %s at %s:%d\n", peg_status_string(s_), __FILE__, __LINE__); \
            exit(3);                                                                       \
        }                                                                                  \
    } while (0)

/* xorshift64*: the seeded input stream (inputs only, no routing arithmetic) */
static uint64_t rng_state;
static uint64_t rng_next(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1DULL;
}
static double rng_unit(void) { return (double)(rng_next() >> 11) / 9007199254740992.0; }

/* a bf16 bit pattern of a value in [-2, 2): the upper half of its float bits */
static uint16_t bf16_bits(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* element count for a host allocation: at least 1, so malloc never sees 0 */
static size_t at_least1(int64_t n) { return n > 0 ? (size_t)n : 1; }

static void* dev_copy(const void* host, size_t bytes) {
    void* p = NULL;
    if (bytes == 0) return NULL;
    HIP_OK(hipMalloc(&p, bytes));
    if (host) HIP_OK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
    return p;
}

static void* host_copy(const void* dev, size_t bytes) {
    void* p = calloc(bytes ? bytes : 1, 1);
    if (bytes) HIP_OK(hipMemcpy(p, dev, bytes, hipMemcpyDeviceToHost));
    return p;
}

static void expect_bytes(const void* gpu, const void* want, size_t bytes, const char* what, const char* tag) {
    if (memcmp(gpu, want, bytes) != 0) {
        fprintf(stderr, "FAIL %s: %s differs\n", tag, what);
        ++failures;
    }
}

static void expect_close(double g, double o, double scale, double rtol, const char* what, const char* tag,
                         int64_t i) {
    if (!(fabs(g - o) <= rtol * fabs(o) + 1e-5 * scale)) {
        if (failures < 20) fprintf(stderr, "FAIL %s: %s[%lld] gpu %.9g oracle %.9g\n", tag, what, (long long)i, g, o);
        ++failures;
    }
}

static void run_case(const char* tag, int64_t T, int64_t H, int32_t K, int32_t E, int32_t layout, int32_t capacity,
                     int32_t pad_multiple, uint64_t seed) {
    const int64_t n_ids = T * K;
    rng_state = seed * 0x9E3779B97F4A7C15ULL + 1;
    int32_t* top = malloc(sizeof(int32_t) * at_least1(n_ids));
    float* weights = malloc(sizeof(float) * at_least1(n_ids));
    uint16_t* x = malloc(2 * at_least1(T * H));
    uint16_t* grad = malloc(2 * at_least1(T * H));
    for (int64_t t = 0; t < T; ++t) {
        /* K distinct experts per token, about one route in eight absent */
        for (int32_t k = 0; k < K; ++k) {
            int32_t e, clash;
            do {
                e = (int32_t)(rng_next() % (uint64_t)E);
                clash = 0;
                for (int32_t j = 0; j < k; ++j) clash |= top[t * K + j] == e;
            } while (clash);
            top[t * K + k] = e;
        }
        for (int32_t k = 0; k < K; ++k) {
            if (rng_next() % 8 == 0) top[t * K + k] = -1;
            weights[t * K + k] = (float)rng_unit();
        }
    }
    for (int64_t i = 0; i < T * H; ++i) {
        x[i] = bf16_bits(4.0 * rng_unit() - 2.0);
        grad[i] = bf16_bits(4.0 * rng_unit() - 2.0);
    }

    /* GPU: route_prep, gather, combine, wgrad through the C ABI */
    const size_t ws_bytes = peg_workspace_bytes(T, K, E);
    void* ws = dev_copy(NULL, ws_bytes);
    int32_t* d_top = dev_copy(top, sizeof(int32_t) * n_ids);
    float* d_w = dev_copy(weights, sizeof(float) * n_ids);
    void* d_x = dev_copy(x, 2 * (size_t)(T * H));
    void* d_grad = dev_copy(grad, 2 * (size_t)(T * H));
    int32_t* d_idx = dev_copy(NULL, sizeof(int32_t) * n_ids);
    int32_t* d_bid = dev_copy(NULL, sizeof(int32_t) * n_ids);
    int32_t* d_tpe = dev_copy(NULL, sizeof(int32_t) * E);
    int32_t* d_bins = dev_copy(NULL, sizeof(int32_t) * E);
    int32_t* d_pbins = layout == PEG_PADDED ? dev_copy(NULL, sizeof(int32_t) * E) : NULL;
    int32_t* d_slot = dev_copy(NULL, sizeof(int32_t) * n_ids);
    PEG_OK_(peg_route_prep(d_top, T, K, E, layout, capacity, pad_multiple, d_idx, d_bid, d_tpe, d_bins, d_pbins,
                           d_slot, ws, ws_bytes, NULL));
    HIP_OK(hipDeviceSynchronize());

    int64_t R;
    if (layout == PEG_PADDED) {
        int32_t last = 0;
        HIP_OK(hipMemcpy(&last, d_pbins + (E - 1), sizeof(int32_t), hipMemcpyDeviceToHost));
        R = last;
    } else {
        R = (int64_t)E * capacity;
    }
    void* d_y = dev_copy(NULL, 2 * (size_t)(R * H));
    uint32_t* d_err = dev_copy(NULL, sizeof(uint32_t));
    if (layout == PEG_PADDED) {
        HIP_OK(hipMemset(d_err, 0, sizeof(uint32_t)));
        PEG_OK_(peg_gather_padded(d_x, PEG_BF16, T, H, K, E, d_idx, d_bid, d_bins, d_pbins, d_slot, d_y, R, d_err,
                                  ws, ws_bytes, NULL));
    } else {
        PEG_OK_(peg_gather_binned(d_x, PEG_BF16, T, H, K, E, capacity, d_idx, d_bid, d_bins, d_slot, d_y, ws,
                                  ws_bytes, NULL));
    }
    void* d_out = dev_copy(NULL, 2 * (size_t)(T * H));
    float* d_wg = dev_copy(NULL, sizeof(float) * n_ids);
    PEG_OK_(peg_scatter_combine(d_y, PEG_BF16, layout, T, H, K, E, capacity, d_idx, d_bid, d_bins, d_pbins, d_slot,
                                d_w, d_out, ws, ws_bytes, NULL));
    PEG_OK_(peg_wgrad(d_y, d_grad, PEG_BF16, layout, T, H, K, E, capacity, d_idx, d_bid, d_bins, d_pbins, d_slot,
                      d_wg, ws, ws_bytes, NULL));
    /* the combine backward with dout = grad: one pass for K <= 2, the dy
       gather then the wgrad kernel for larger K */
    void* d_dy = dev_copy(NULL, 2 * (size_t)(R * H));
    float* d_wgb = dev_copy(NULL, sizeof(float) * n_ids);
    PEG_OK_(peg_combine_backward(d_y, d_grad, d_w, PEG_BF16, layout, T, H, K, E, capacity, d_idx, d_bid, d_bins,
                                 d_pbins, d_slot, d_dy, R, d_wgb, ws, ws_bytes, NULL));
    HIP_OK(hipDeviceSynchronize());

    int32_t* g_idx = host_copy(d_idx, sizeof(int32_t) * n_ids);
    int32_t* g_bid = host_copy(d_bid, sizeof(int32_t) * n_ids);
    int32_t* g_tpe = host_copy(d_tpe, sizeof(int32_t) * E);
    int32_t* g_bins = host_copy(d_bins, sizeof(int32_t) * E);
    int32_t* g_slot = host_copy(d_slot, sizeof(int32_t) * n_ids);
    uint16_t* g_y = host_copy(d_y, 2 * (size_t)(R * H));
    uint16_t* g_out = host_copy(d_out, 2 * (size_t)(T * H));
    float* g_wg = host_copy(d_wg, sizeof(float) * n_ids);
    uint16_t* g_dy = host_copy(d_dy, 2 * (size_t)(R * H));
    float* g_wgb = host_copy(d_wgb, sizeof(float) * n_ids);

    /* oracle on the same inputs */
    int32_t* o_idx = malloc(sizeof(int32_t) * at_least1(n_ids));
    int32_t* o_bid = malloc(sizeof(int32_t) * at_least1(n_ids));
    int32_t* o_tpe = malloc(sizeof(int32_t) * E);
    int32_t* o_bins = malloc(sizeof(int32_t) * E);
    int32_t* o_pbins = layout == PEG_PADDED ? malloc(sizeof(int32_t) * E) : NULL;
    int32_t* o_slot = malloc(sizeof(int32_t) * at_least1(n_ids));
    if (pego_route_prep(top, T, K, E, pad_multiple, o_idx, o_bid, o_tpe, o_bins, o_pbins) < 0 ||
        pego_assignment_rows(T, K, E, layout, capacity, o_idx, o_bid, o_bins, o_pbins, o_slot) != 0) {
        fprintf(stderr, "FAIL %s: oracle refused the case\n", tag);
        exit(4);
    }
    uint16_t* o_y = calloc(at_least1(R * H), 2);
    uint16_t* o_out = calloc(at_least1(T * H), 2);
    double* o_out_scale = calloc(at_least1(T * H), sizeof(double));
    float* o_wg = calloc(at_least1(n_ids), sizeof(float));
    double* o_wg_scale = calloc(at_least1(n_ids), sizeof(double));
    pego_gather(x, T, 2 * H, K, E, layout, capacity, o_idx, o_bid, o_bins, o_pbins, R, NULL, 0, o_y);
    pego_scatter_combine(o_y, PEGO_BF16, R, T, H, K, E, layout, capacity, o_idx, o_bid, o_bins, o_pbins, weights,
                         NULL, 0, o_out, o_out_scale);
    pego_wgrad(o_y, grad, PEGO_BF16, R, T, H, K, E, layout, capacity, o_idx, o_bid, o_bins, o_pbins, NULL, 0, o_wg,
               o_wg_scale);
    uint16_t* o_dy = calloc(at_least1(R * H), 2);
    if (pego_combine_backward_dy(grad, PEGO_BF16, T, H, K, E, layout, capacity, o_idx, o_bid, o_bins, o_pbins,
                                 weights, R, NULL, 0, o_dy) != 0) {
        fprintf(stderr, "FAIL %s: oracle refused the backward\n", tag);
        exit(4);
    }

    expect_bytes(g_idx, o_idx, sizeof(int32_t) * n_ids, "indices", tag);
    expect_bytes(g_bid, o_bid, sizeof(int32_t) * n_ids, "bin_ids", tag);
    expect_bytes(g_tpe, o_tpe, sizeof(int32_t) * E, "tokens_per_expert", tag);
    expect_bytes(g_bins, o_bins, sizeof(int32_t) * E, "bins", tag);
    if (layout == PEG_PADDED) {
        int32_t* g_pbins = host_copy(d_pbins, sizeof(int32_t) * E);
        expect_bytes(g_pbins, o_pbins, sizeof(int32_t) * E, "padded_bins", tag);
        free(g_pbins);
    }
    expect_bytes(g_slot, o_slot, sizeof(int32_t) * n_ids, "slot_row", tag);
    if (layout == PEG_PADDED) {
        uint32_t flag = 1;
        HIP_OK(hipMemcpy(&flag, d_err, sizeof(uint32_t), hipMemcpyDeviceToHost));
        const uint32_t zero = 0;
        expect_bytes(&flag, &zero, sizeof(uint32_t), "gather_padded error flag (expected clear)", tag);
    }
    expect_bytes(g_y, o_y, 2 * (size_t)(R * H), "gathered expert tensor", tag);
    for (int64_t i = 0; i < T * H; ++i)
        expect_close(pego_load(g_out, PEGO_BF16, i), pego_load(o_out, PEGO_BF16, i), o_out_scale[i], 2e-2,
                     "combine", tag, i);
    for (int64_t i = 0; i < n_ids; ++i)
        expect_close(g_wg[i], o_wg[i], o_wg_scale[i], 1e-5, "wgrad", tag, i);
    for (int64_t i = 0; i < R * H; ++i) {  /* one rounding of a product: S = |oracle| */
        const double o = pego_load(o_dy, PEGO_BF16, i);
        expect_close(pego_load(g_dy, PEGO_BF16, i), o, fabs(o), 2e-2, "combine backward dy", tag, i);
    }
    expect_bytes(g_wgb, g_wg, sizeof(float) * n_ids, "combine backward wgrad (== the wgrad kernel's)", tag);
    printf("%s: T%lld H%lld K%d E%d R%lld checked\n", tag, (long long)T, (long long)H, K, E, (long long)R);
    fflush(stdout);

    void* dev_bufs[] = {ws, d_top, d_w, d_x, d_grad, d_idx, d_bid, d_tpe, d_bins, d_pbins, d_slot, d_y, d_err,
                        d_out, d_wg, d_dy, d_wgb};
    for (size_t i = 0; i < sizeof(dev_bufs) / sizeof(dev_bufs[0]); ++i)
        if (dev_bufs[i]) HIP_OK(hipFree(dev_bufs[i]));
    void* host_bufs[] = {top, weights, x, grad, g_idx, g_bid, g_tpe, g_bins, g_slot, g_y, g_out, g_wg, g_dy, g_wgb,
                         o_idx, o_bid, o_tpe, o_bins, o_pbins, o_slot, o_y, o_out, o_out_scale, o_wg, o_wg_scale,
                         o_dy};
    for (size_t i = 0; i < sizeof(host_bufs) / sizeof(host_bufs[0]); ++i) free(host_bufs[i]);
}

int main(void) {
    int n = 0;
    HIP_OK(hipGetDeviceCount(&n));
    if (n < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    /* binned: capacity below the mean load, so routes are dropped */
    run_case("binned", 777, 136, 2, 8, PEG_BINNED, 150, 0, 1);
    /* padded to a multiple of 16, four routes per token over 33 experts */
    run_case("padded", 1000, 264, 4, 33, PEG_PADDED, 0, 16, 2);
    /* 8192 ids: the multi-tile form of route_prep */
    run_case("padded-tiled", 4096, 72, 2, 8, PEG_PADDED, 0, 128, 3);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("gpu_path ok\n");
    return 0;
}
