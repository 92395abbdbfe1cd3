/*
 * peg_oracle.c - plain, slow CPU oracle of the MoE token-routing data path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg. It shares no code with the GPU library.
 *
 * Style: scalar loops in the order the pages state the method, double
 * precision for every floating-point sum, one round-to-nearest-even to the
 * output type at the end. No blocking, fusion, vectorisation or threads.
 *
 * Page references (title, section):
 *   [BIN] "Build Triton-Ascend Binned MoE Routing"
 *   [PAD] "Build Triton-Ascend Padded MoE Routing"
 *   [MOK] "core.transformer.moe.megakernel.mok.route_adapter"
 *   [FMD] "Fused MoE Dispatch (Triton, universal)"
 *
 * Parity status per function is stated in the function comments; each is
 * pinned by the CPU tests against brute force, library routines, closed
 * forms and the pages' invariants. One case is parity unpinned: a routing
 * map row with more than topk routes (pego_routing_map_compact), where no
 * page fixes which routes are kept.
 */
#include "peg_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary32 / bfloat16 / binary16).                */
/* ------------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t h) {
    /* bfloat16 is the upper half of a binary32: widening is exact. */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double f16_bits_to_double(uint16_t h) {
    /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int fr = h & 0x3FF;
    double v;
    if (ex == 0) {
        v = ldexp((double)fr, -24); /* subnormal: fr * 2^(1-15-10) */
    } else if (ex == 31) {
        v = fr ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + fr), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
    }
    return sign ? -v : v;
}

/*
 * Round a finite nonzero magnitude `a` to a binary format with `p`
 * significand bits (implicit bit included) and normal exponents
 * [emin, emax], ties to even. Returns the rounded magnitude (a double that
 * the target format represents exactly), or INFINITY on overflow.
 */
static double round_to_format(double a, int p, int emin, int emax) {
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1 */
    int expo = e2 - 1;
    if (expo < emin) expo = emin;            /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, expo - (p - 1));
    double m = a / quantum;                  /* exact: division by a power of two */
    double r = nearbyint(m);                 /* default rounding mode: ties to even */
    double v = r * quantum;
    if (v >= ldexp(1.0, emax + 1)) return INFINITY;
    return v;
}

uint16_t pego_round_bf16(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    double r = isinf(a) ? INFINITY : round_to_format(a, 8, -126, 127);
    if (isinf(r)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

uint16_t pego_round_f16(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFE00u : 0x7E00u);
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    double r = isinf(a) ? INFINITY : round_to_format(a, 11, -14, 15);
    if (isinf(r)) return (uint16_t)(sign | 0x7C00u);
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14)) {
        /* subnormal: value = fr * 2^-24 */
        uint16_t fr = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | fr);
    }
    int e2;
    double f = frexp(r, &e2);               /* r = f * 2^e2, f in [0.5, 1) */
    int ex = (e2 - 1) + 15;                 /* biased exponent */
    uint16_t fr = (uint16_t)(ldexp(f, 11) - 1024.0); /* fraction bits */
    return (uint16_t)(sign | (uint16_t)(ex << 10) | fr);
}

double pego_load(const void* base, int32_t dtype, int64_t idx) {
    if (dtype == PEGO_F32) return (double)((const float*)base)[idx];
    if (dtype == PEGO_BF16) return bf16_bits_to_double(((const uint16_t*)base)[idx]);
    return f16_bits_to_double(((const uint16_t*)base)[idx]);
}

void pego_store(void* base, int32_t dtype, int64_t idx, double v) {
    if (dtype == PEGO_F32) {
        ((float*)base)[idx] = (float)v; /* C conversion: current mode, ties to even */
    } else if (dtype == PEGO_BF16) {
        ((uint16_t*)base)[idx] = pego_round_bf16(v);
    } else {
        ((uint16_t*)base)[idx] = pego_round_f16(v);
    }
}

static int dtype_ok(int32_t dtype) {
    return dtype == PEGO_F32 || dtype == PEGO_BF16 || dtype == PEGO_F16;
}

/* ------------------------------------------------------------------------ */
/* Routing preparation.                                                     */
/* ------------------------------------------------------------------------ */

/*
 * [PAD] Workflow steps 1-3 ([BIN] Workflow steps 1-2):
 *   1. sort the assignments by expert -> indices (assignment ids) and the
 *      aligned, nondecreasing bin_ids. The pages do not fix the order inside
 *      an expert; the reading taken is ascending assignment id (a stable
 *      sort), which makes the result unique. It is realised here by the
 *      plainest selection: for each expert in turn, scan every assignment
 *      id in increasing order and append the ones routed to it.
 *   2. bins[e] = real cumulative count through expert e (inclusive).
 *   3. padded_bins[e] = cumulative count with each count rounded up to the
 *      padding multiple.
 * Assignment a = t*K + k; a value outside [0, E) in top_experts means "no
 * route" and is left out. Sorted positions [n, T*K) are set to -1.
 */
int64_t pego_route_prep(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                        int32_t pad_multiple, int32_t* indices, int32_t* bin_ids,
                        int32_t* tokens_per_expert, int32_t* bins, int32_t* padded_bins) {
    if (T < 0 || K < 1 || E < 1 || !top_experts || !indices || !bin_ids || !bins) return -1;
    if (padded_bins && pad_multiple < 1) return -1;
    int64_t total = T * (int64_t)K;

    /* step 1: selection sort by expert, ascending assignment id within one */
    int64_t pos = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int64_t a = 0; a < total; ++a) {
            if (top_experts[a] == e) {
                indices[pos] = (int32_t)a;
                bin_ids[pos] = e;
                ++pos;
            }
        }
    }
    int64_t n = pos;
    for (int64_t i = n; i < total; ++i) {
        indices[i] = -1;
        bin_ids[i] = -1;
    }

    /* step 2: counts and their inclusive running sum */
    int64_t run = 0, prun = 0;
    for (int32_t e = 0; e < E; ++e) {
        int64_t count = 0;
        for (int64_t i = 0; i < n; ++i)
            if (bin_ids[i] == e) ++count;
        if (tokens_per_expert) tokens_per_expert[e] = (int32_t)count;
        run += count;
        bins[e] = (int32_t)run;
        /* step 3: round the count up to the multiple, then accumulate */
        if (padded_bins) {
            int64_t rounded = ((count + pad_multiple - 1) / pad_multiple) * pad_multiple;
            prun += rounded;
            padded_bins[e] = (int32_t)prun;
        }
    }
    return n;
}

/*
 * Rows of the sorted positions [0, n) in the expert tensor ([BIN] and [PAD]
 * Implementation Pattern). Every expert owns one segment of rows: in the
 * binned layout expert e's segment is the `capacity` rows from e*capacity;
 * in the padded layout it starts where the previous expert's padded segment
 * ends (padded_bins[e-1], or 0 for the first expert). The walk below goes
 * through the experts in turn; for each it visits the sorted positions in
 * order, and every position of that expert receives the next unused row of
 * the segment. A binned segment that has run out of rows drops the position
 * (row -1). Returns a malloc'd array of n entries (at least one), or NULL
 * when a position names no expert in [0, E) or memory runs out.
 */
static int64_t* position_rows(int64_t n, int32_t E, int32_t layout, int32_t capacity,
                              const int32_t* bin_ids, const int32_t* padded_bins) {
    int64_t* row_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    if (!row_of) return NULL;
    for (int64_t i = 0; i < n; ++i) row_of[i] = -2; /* not handed a row yet */
    for (int32_t e = 0; e < E; ++e) {
        int64_t segment_base;
        if (layout == PEGO_BINNED) segment_base = (int64_t)e * capacity;
        else segment_base = e == 0 ? 0 : padded_bins[e - 1];
        int64_t handed_out = 0;
        for (int64_t i = 0; i < n; ++i) {
            if (bin_ids[i] != e) continue;
            if (layout == PEGO_BINNED && handed_out >= capacity) row_of[i] = -1; /* segment full */
            else row_of[i] = segment_base + handed_out;
            ++handed_out;
        }
    }
    for (int64_t i = 0; i < n; ++i) {
        if (row_of[i] == -2) { /* bin_ids[i] is not an expert */
            free(row_of);
            return NULL;
        }
    }
    return row_of;
}

static int64_t valid_count(const int32_t* bins, int32_t E, int64_t total) {
    int64_t n = bins[E - 1];
    if (n < 0) n = 0;
    if (n > total) n = total;
    return n;
}

/*
 * Row of every assignment id ([BIN] Workflow step 5 / [PAD] step 6: the
 * scatter is indexed by assignment id, each id unique): rows_out[a] is the
 * expert-tensor row holding assignment a, -1 if a has no route or was
 * dropped by the capacity limit.
 */
int pego_assignment_rows(int64_t T, int32_t K, int32_t E, int32_t layout, int32_t capacity,
                         const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                         const int32_t* padded_bins, int32_t* rows_out) {
    if (T < 0 || K < 1 || E < 1 || !indices || !bin_ids || !bins || !rows_out) return -1;
    if (layout == PEGO_BINNED && capacity < 1) return -1;
    if (layout == PEGO_PADDED && !padded_bins) return -1;
    int64_t total = T * (int64_t)K;
    for (int64_t a = 0; a < total; ++a) rows_out[a] = -1;
    int64_t n = valid_count(bins, E, total);
    int64_t* row_of = position_rows(n, E, layout, capacity, bin_ids, padded_bins);
    if (!row_of) return -1;
    for (int64_t i = 0; i < n; ++i) {
        int32_t a = indices[i];
        if (a < 0 || a >= total) { free(row_of); return -1; }
        rows_out[a] = (int32_t)row_of[i];
    }
    free(row_of);
    return 0;
}

/*
 * Rows of every assignment id when each expert owns a caller-given window of
 * rows [row_base[e], row_limit[e]): the Implementation Pattern's segments of
 * [BIN] and [PAD] with each expert's segment start and end supplied. The
 * same walk as position_rows: experts in turn, each one's sorted positions
 * in order, every position taking the next row of the expert's window from
 * row_base[e] up; once a window's rows reach row_limit[e], the remaining
 * assignments of that expert are dropped (-1).
 * (Used for one shard of a token-sharded batch: the windows then start where
 * the earlier shards' assignments of each expert end.)
 */
int pego_assignment_rows_windows(int64_t T, int32_t K, int32_t E, const int32_t* indices,
                                 const int32_t* bin_ids, const int32_t* bins,
                                 const int32_t* row_base, const int32_t* row_limit,
                                 int32_t* rows_out) {
    if (T < 0 || K < 1 || E < 1 || !indices || !bin_ids || !bins || !row_base || !row_limit || !rows_out)
        return -1;
    int64_t total = T * (int64_t)K;
    for (int64_t a = 0; a < total; ++a) rows_out[a] = -1;
    int64_t n = valid_count(bins, E, total);
    for (int64_t i = 0; i < n; ++i) {
        if (bin_ids[i] < 0 || bin_ids[i] >= E) return -1;
        if (indices[i] < 0 || indices[i] >= total) return -1;
    }
    for (int32_t e = 0; e < E; ++e) {
        int64_t next_row = row_base[e];
        for (int64_t i = 0; i < n; ++i) {
            if (bin_ids[i] != e) continue;
            rows_out[indices[i]] = next_row < row_limit[e] ? (int32_t)next_row : -1;
            ++next_row;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gathers.                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * [BIN] Goal / Workflow step 3 / Ascend Guardrails and [PAD] Workflow
 * steps 4-5 / Ascend Guardrails: the expert tensor of R rows starts as
 * zeros; each kept sorted position i copies token indices[i] / K into its
 * row. Rows are moved as raw bytes.
 *
 * rows == NULL: out holds all R rows. Otherwise out holds nrows rows and
 * out[j] is row rows[j] of the expert tensor (a sample of it).
 */
int pego_gather(const void* x, int64_t T, int64_t row_bytes, int32_t K, int32_t E,
                int32_t layout, int32_t capacity, const int32_t* indices,
                const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
                int64_t R, const int64_t* rows, int64_t nrows, void* out) {
    if (T < 0 || row_bytes < 0 || K < 1 || E < 1 || R < 0 || !x || !bins || !out) return -1;
    if (layout == PEGO_BINNED && capacity < 1) return -1;
    if (layout == PEGO_PADDED && !padded_bins) return -1;
    int64_t total = T * (int64_t)K;

    /* source token of each row of the expert tensor; -1 = zero row */
    int64_t* src = (int64_t*)malloc(sizeof(int64_t) * (size_t)(R > 0 ? R : 1));
    if (!src) return -1;
    for (int64_t r = 0; r < R; ++r) src[r] = -1;
    int64_t n = valid_count(bins, E, total);
    int64_t* row_of = position_rows(n, E, layout, capacity, bin_ids, padded_bins);
    if (!row_of) { free(src); return -1; }
    for (int64_t i = 0; i < n; ++i) {
        int64_t row = row_of[i];
        if (row < 0 || row >= R) continue; /* dropped, or beyond the tensor */
        int64_t token = indices[i] / K;
        if (indices[i] < 0 || token >= T) { free(src); free(row_of); return -1; }
        src[row] = token;
    }
    free(row_of);

    const uint8_t* xb = (const uint8_t*)x;
    uint8_t* ob = (uint8_t*)out;
    int64_t count = rows ? nrows : R;
    for (int64_t j = 0; j < count; ++j) {
        int64_t r = rows ? rows[j] : j;
        uint8_t* dst = ob + j * row_bytes;
        if (r < 0 || r >= R || src[r] < 0) {
            memset(dst, 0, (size_t)row_bytes);
        } else {
            memcpy(dst, xb + src[r] * row_bytes, (size_t)row_bytes);
        }
    }
    free(src);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Scatter-combine.                                                         */
/* ------------------------------------------------------------------------ */

/*
 * [BIN] Workflow step 5: load every kept expert row, store it (scaled by its
 * weight when weights are given) into its unique assignment slot, then
 * reduce the TOP_K slots of each token. [PAD] Workflow step 6 and Ascend
 * Guardrails: the same through padded storage, weight of sorted position i
 * = weights[indices[i]].
 *
 * The slot buffer of the pages is kept here as a row reference per
 * assignment (slot_src); the reduction then reads the referenced rows.
 * Sums run in double over k ascending and are rounded once to dtype.
 * tokens == NULL: all T tokens, out [T, H]. Otherwise out [ntok, H] holds
 * the listed tokens. scale (optional, same shape, double) receives the sum
 * of the magnitudes of the terms, the scale of the rounding error.
 */
int pego_scatter_combine(const void* y, int32_t dtype, int64_t R, int64_t T, int64_t H,
                         int32_t K, int32_t E, int32_t layout, int32_t capacity,
                         const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                         const int32_t* padded_bins, const float* weights,
                         const int64_t* tokens, int64_t ntok, void* out, double* scale) {
    if (!dtype_ok(dtype) || T < 0 || H < 0 || K < 1 || E < 1 || !y || !out || !bins) return -1;
    if (layout == PEGO_BINNED && capacity < 1) return -1;
    if (layout == PEGO_PADDED && !padded_bins) return -1;
    int64_t total = T * (int64_t)K;
    int64_t* slot_src = (int64_t*)malloc(sizeof(int64_t) * (size_t)(total > 0 ? total : 1));
    if (!slot_src) return -1;
    for (int64_t a = 0; a < total; ++a) slot_src[a] = -1;
    int64_t n = valid_count(bins, E, total);
    int64_t* row_of = position_rows(n, E, layout, capacity, bin_ids, padded_bins);
    if (!row_of) { free(slot_src); return -1; }
    for (int64_t i = 0; i < n; ++i) {
        int64_t row = row_of[i];
        if (row < 0) continue; /* beyond capacity: never read */
        int64_t a = indices[i];
        if (a < 0 || a >= total || row >= R) { free(slot_src); free(row_of); return -1; }
        slot_src[a] = row;
    }
    free(row_of);

    int64_t count = tokens ? ntok : T;
    for (int64_t j = 0; j < count; ++j) {
        int64_t t = tokens ? tokens[j] : j;
        if (t < 0 || t >= T) { free(slot_src); return -1; }
        for (int64_t h = 0; h < H; ++h) {
            double sum = 0.0, mag = 0.0;
            for (int32_t k = 0; k < K; ++k) {
                int64_t a = t * K + k;
                int64_t row = slot_src[a];
                if (row < 0) continue;
                double w = weights ? (double)weights[a] : 1.0;
                double term = w * pego_load(y, dtype, row * H + h);
                sum += term;
                mag += fabs(term);
            }
            pego_store(out, dtype, j * H + h, sum);
            if (scale) scale[j * H + h] = mag;
        }
    }
    free(slot_src);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Router-weight gradient.                                                  */
/* ------------------------------------------------------------------------ */

/*
 * [BIN] Workflow step 6: for each kept sorted position i, the dot product
 * of its expert row with the gradient row of token indices[i] // TOP_K;
 * [PAD] Workflow step 6: the same with the padded mapping. The result is
 * stored at assignment id indices[i]; every other assignment gets 0.
 * The dot runs in double and is rounded once to float.
 * tokens == NULL: wgrad [T*K]. Otherwise wgrad [ntok*K] holds the K
 * assignments of each listed token. scale: sum of |y*grad| per output.
 */
int pego_wgrad(const void* y, const void* grad, int32_t dtype, int64_t R, int64_t T, int64_t H,
               int32_t K, int32_t E, int32_t layout, int32_t capacity, const int32_t* indices,
               const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
               const int64_t* tokens, int64_t ntok, float* wgrad, double* scale) {
    if (!dtype_ok(dtype) || T < 0 || H < 0 || K < 1 || E < 1 || !y || !grad || !wgrad || !bins)
        return -1;
    if (layout == PEGO_BINNED && capacity < 1) return -1;
    if (layout == PEGO_PADDED && !padded_bins) return -1;
    int64_t total = T * (int64_t)K;

    /* sorted position holding each assignment id (-1: not in indices) */
    int64_t* pos_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)(total > 0 ? total : 1));
    if (!pos_of) return -1;
    for (int64_t a = 0; a < total; ++a) pos_of[a] = -1;
    int64_t n = valid_count(bins, E, total);
    for (int64_t i = 0; i < n; ++i) {
        int64_t a = indices[i];
        if (a < 0 || a >= total) { free(pos_of); return -1; }
        pos_of[a] = i;
    }
    int64_t* row_of = position_rows(n, E, layout, capacity, bin_ids, padded_bins);
    if (!row_of) { free(pos_of); return -1; }

    int64_t count = tokens ? ntok : T;
    for (int64_t j = 0; j < count; ++j) {
        int64_t t = tokens ? tokens[j] : j;
        if (t < 0 || t >= T) { free(pos_of); free(row_of); return -1; }
        for (int32_t k = 0; k < K; ++k) {
            int64_t o = j * K + k;
            wgrad[o] = 0.0f;
            if (scale) scale[o] = 0.0;
            int64_t i = pos_of[t * K + k];
            if (i < 0) continue; /* no route */
            int64_t row = row_of[i];
            if (row >= R) { free(pos_of); free(row_of); return -1; }
            if (row < 0) continue; /* beyond capacity */
            double dot = 0.0, mag = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double p = pego_load(y, dtype, row * H + h) * pego_load(grad, dtype, t * H + h);
                dot += p;
                mag += fabs(p);
            }
            wgrad[o] = (float)dot;
            if (scale) scale[o] = mag;
        }
    }
    free(pos_of);
    free(row_of);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of the combine with respect to the expert tensor.               */
/* ------------------------------------------------------------------------ */

/*
 * The combine of [BIN] Workflow step 5 / [PAD] Workflow step 6 is linear in
 * the expert tensor: out[t] = sum over kept k of w[t*K+k] * y[row(t*K+k)].
 * Its gradient with respect to y, given the upstream gradient dout [T, H],
 * is therefore: every kept sorted position i with assignment a = indices[i]
 * gets w[a] * dout[a / K] in its row (the weighted gather of dout through
 * the same mapping; the [PAD] front matter lists this use of the padded
 * storage); every other row of the R-row tensor is zero. Without
 * weights (factor 1) the rows are copied as raw bits. The product runs in
 * double and is rounded once to dtype. rows == NULL: dy holds all R rows;
 * otherwise dy[j] is row rows[j] (a sample).
 */
int pego_combine_backward_dy(const void* dout, int32_t dtype, int64_t T, int64_t H, int32_t K, int32_t E,
                             int32_t layout, int32_t capacity, const int32_t* indices, const int32_t* bin_ids,
                             const int32_t* bins, const int32_t* padded_bins, const float* weights, int64_t R,
                             const int64_t* rows, int64_t nrows, void* dy) {
    if (!dtype_ok(dtype) || T < 0 || H < 0 || K < 1 || E < 1 || R < 0 || !dout || !bins || !dy) return -1;
    if (layout == PEGO_BINNED && capacity < 1) return -1;
    if (layout == PEGO_PADDED && !padded_bins) return -1;
    int64_t total = T * (int64_t)K;
    /* assignment held by each row of the expert tensor; -1 = zero row */
    int64_t* src = (int64_t*)malloc(sizeof(int64_t) * (size_t)(R > 0 ? R : 1));
    if (!src) return -1;
    for (int64_t r = 0; r < R; ++r) src[r] = -1;
    int64_t n = valid_count(bins, E, total);
    int64_t* row_of = position_rows(n, E, layout, capacity, bin_ids, padded_bins);
    if (!row_of) { free(src); return -1; }
    for (int64_t i = 0; i < n; ++i) {
        int64_t row = row_of[i];
        if (row < 0 || row >= R) continue;
        if (indices[i] < 0 || indices[i] >= total) { free(src); free(row_of); return -1; }
        src[row] = indices[i];
    }
    free(row_of);
    int eb = dtype == PEGO_F32 ? 4 : 2;
    int64_t count = rows ? nrows : R;
    for (int64_t j = 0; j < count; ++j) {
        int64_t r = rows ? rows[j] : j;
        int64_t a = (r >= 0 && r < R) ? src[r] : -1;
        if (a < 0) {
            memset((uint8_t*)dy + j * H * eb, 0, (size_t)(H * eb));
            continue;
        }
        int64_t t = a / K;
        if (!weights) {
            memcpy((uint8_t*)dy + j * H * eb, (const uint8_t*)dout + t * H * eb, (size_t)(H * eb));
            continue;
        }
        double w = (double)weights[a];
        for (int64_t h = 0; h < H; ++h) pego_store(dy, dtype, j * H + h, w * pego_load(dout, dtype, t * H + h));
    }
    free(src);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Routing-map compaction.                                                  */
/* ------------------------------------------------------------------------ */

/*
 * [MOK] RoutingMapToIndices / routing_map_to_mok_inputs: the dense map is
 * the authoritative route set (no top-k over probs). Each row is walked in
 * increasing expert index; routed experts fill the output slots in that
 * order, at most topk of them; the rest of the row is padded with index -1
 * and probability 0. Probabilities are returned as float32.
 * A row with more than topk routes keeps its topk lowest expert ids: the
 * page gives topk as the most routes a token emits and does not say which
 * ones survive; this is the reading taken. Parity unpinned for such rows:
 * no page value fixes the choice (the pins check it against the same
 * reading written as a plain row walk).
 */
int pego_routing_map_compact(const void* probs, int32_t probs_dtype, const uint8_t* routing_map,
                             int64_t T, int32_t E, int32_t topk, float* probs_out,
                             int32_t* route_experts) {
    if (!dtype_ok(probs_dtype) || T < 0 || E < 1 || topk < 1 || !probs || !routing_map ||
        !probs_out || !route_experts)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        int32_t j = 0;
        for (int32_t e = 0; e < E; ++e) {
            if (routing_map[t * E + e] != 0 && j < topk) {
                route_experts[t * topk + j] = e;
                probs_out[t * topk + j] = (float)pego_load(probs, probs_dtype, t * E + e);
                ++j;
            }
        }
        for (; j < topk; ++j) {
            route_experts[t * topk + j] = -1;
            probs_out[t * topk + j] = 0.0f;
        }
    }
    return 0;
}

/*
 * [MOK] RoutingMapToIndices backward: the gradient of each compact slot is
 * written back at the dense position of its expert; everything else is 0.
 */
int pego_routing_map_compact_backward(const float* grad_probs_out, const int32_t* route_experts,
                                      int64_t T, int32_t E, int32_t topk, float* grad_probs) {
    if (T < 0 || E < 1 || topk < 1 || !grad_probs_out || !route_experts || !grad_probs) return -1;
    for (int64_t i = 0; i < T * (int64_t)E; ++i) grad_probs[i] = 0.0f;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < topk; ++j) {
            int32_t e = route_experts[t * topk + j];
            if (e >= 0 && e < E) grad_probs[t * E + e] = grad_probs_out[t * topk + j];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Router top-k gating.                                                     */
/* ------------------------------------------------------------------------ */

/* Ranking of two router scores: NaN ranks below every number; numbers by
 * value (so -0 and +0 tie). */
static int score_above(double a, double b) {
    if (isnan(a)) return 0;
    if (isnan(b)) return 1;
    return a > b;
}

/*
 * [FMD] pipeline figure (router scores -> top-k gating -> permute) and Usage
 * (gating "softmax" or "sigmoid"). The pages name the two gating functions
 * and nothing more; the readings taken:
 *   - the K experts of a token are its K highest scores, listed from the
 *     highest down, the lower expert id first among equal scores; the
 *     ranking uses the scores themselves (softmax and sigmoid are
 *     increasing, so this is the ranking of the probabilities without the
 *     ties that rounding them would add);
 *   - softmax: p_e = exp(l_e - m) / sum_j exp(l_j - m) over all E experts,
 *     m = the highest score; sigmoid: p_e = 1 / (1 + exp(-l_e));
 *   - normalize != 0: the K weights are p / (sum of the K selected p), the
 *     renormalisation the workloads' router uses; else the K weights are p.
 * Everything is evaluated in double in that order and rounded once to
 * float32; NaN or infinite scores give whatever those formulas give. Domain:
 * for sigmoid, finite scores above -700 (below that exp(-l) overflows double
 * and the renormalised weights would become 0/0 instead of their finite
 * value).
 * gating: 0 = softmax, 1 = sigmoid.
 */
int pego_router_topk(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                     int32_t gating, int32_t normalize, int32_t* top_experts, float* weights) {
    if (!dtype_ok(dtype) || T < 0 || E < 1 || K < 1 || K > E || (gating != 0 && gating != 1) ||
        (T > 0 && (!logits || !top_experts || !weights)))
        return -1;
    double* l = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)K);
    if (!l || !taken || !p) {
        free(l);
        free(taken);
        free(p);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            l[e] = pego_load(logits, dtype, t * E + e);
            taken[e] = 0;
        }
        /* selection: K rounds, each takes the best remaining expert; the scan
         * runs over increasing ids and replaces only on a strictly higher
         * rank, so the lower id wins a tie */
        for (int32_t k = 0; k < K; ++k) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || score_above(l[e], l[best])) best = e;
            }
            taken[best] = 1;
            top_experts[t * K + k] = best;
        }
        if (gating == 0) {
            double m = l[top_experts[t * K]];
            double denom = 0.0;
            for (int32_t e = 0; e < E; ++e) denom += exp(l[e] - m);
            for (int32_t k = 0; k < K; ++k) p[k] = exp(l[top_experts[t * K + k]] - m) / denom;
        } else {
            for (int32_t k = 0; k < K; ++k) p[k] = 1.0 / (1.0 + exp(-l[top_experts[t * K + k]]));
        }
        double sel = 0.0;
        for (int32_t k = 0; k < K; ++k) sel += p[k];
        for (int32_t k = 0; k < K; ++k) weights[t * K + k] = (float)(normalize ? p[k] / sel : p[k]);
    }
    free(l);
    free(taken);
    free(p);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Validation of the routing preconditions.                                 */
/* ------------------------------------------------------------------------ */

#define FLAG_BINS_NOT_MONOTONIC 0x1u
#define FLAG_BINS_TOTAL 0x2u
#define FLAG_BIN_IDS 0x4u
#define FLAG_PADDED_BINS 0x8u
#define FLAG_INDICES 0x10u

/*
 * [BIN] Ascend Guardrails: bins monotonic, last bin equal to the number of
 * indices, bin_ids consistent with the bin boundaries, assignment ids unique.
 * [PAD] Ascend Guardrails: padded_bins monotonic with every padded segment
 * at least as long as its real count.
 * The expected expert of position i is the number of experts e whose
 * inclusive bin end bins[e] is <= i (for monotonic bins: the expert whose
 * segment holds i).
 */
uint32_t pego_validate_routing(const int32_t* indices, const int32_t* bin_ids,
                               const int32_t* bins, const int32_t* padded_bins, int64_t T,
                               int32_t K, int32_t E, int64_t n_indices) {
    uint32_t flags = 0;
    int64_t total = T * (int64_t)K;
    for (int32_t e = 0; e < E; ++e) {
        int64_t prev = e == 0 ? 0 : bins[e - 1];
        if (bins[e] < prev) flags |= FLAG_BINS_NOT_MONOTONIC;
    }
    if (n_indices >= 0 && bins[E - 1] != n_indices) flags |= FLAG_BINS_TOTAL;
    int64_t n = n_indices >= 0 ? n_indices : bins[E - 1];
    if (n < 0) n = 0;
    if (n > total) n = total;
    for (int64_t i = 0; i < n; ++i) {
        int32_t expect = 0;
        for (int32_t e = 0; e < E; ++e)
            if (bins[e] <= i) ++expect;
        if (bin_ids[i] != expect) flags |= FLAG_BIN_IDS;
    }
    if (padded_bins) {
        for (int32_t e = 0; e < E; ++e) {
            int64_t pprev = e == 0 ? 0 : padded_bins[e - 1];
            int64_t prev = e == 0 ? 0 : bins[e - 1];
            if (padded_bins[e] < pprev) flags |= FLAG_PADDED_BINS;
            if ((int64_t)padded_bins[e] - pprev < (int64_t)bins[e] - prev) flags |= FLAG_PADDED_BINS;
        }
    }
    uint8_t* seen = (uint8_t*)calloc((size_t)(total > 0 ? total : 1), 1);
    if (!seen) return 0xFFFFFFFFu;
    for (int64_t i = 0; i < n; ++i) {
        int32_t a = indices[i];
        if (a < 0 || a >= total) {
            flags |= FLAG_INDICES;
            continue;
        }
        if (seen[a]) flags |= FLAG_INDICES;
        seen[a] = 1;
    }
    free(seen);
    return flags;
}
