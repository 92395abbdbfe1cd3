/*
 * peg.h - C ABI of the MI355X (gfx950) MoE token-routing data path:
 * sorted-expert-bin dispatch (binned and padded gathers), the inverse
 * weighted top-k scatter-combine, the router-weight gradient (wgrad), and
 * dense routing-map compaction.
 *
 * Sources (web pages; cited by title and section):
 *   [BIN]  "Build Triton-Ascend Binned MoE Routing": Goal, Workflow,
 *          Implementation Pattern, Ascend Guardrails, Verification.
 *   [PAD]  "Build Triton-Ascend Padded MoE Routing": same sections.
 *   [MOK]  "core.transformer.moe.megakernel.mok.route_adapter" (Megatron-Core
 *          API page): RoutingMapToIndices, routing_map_to_mok_inputs.
 *   [FMD]  "Fused MoE Dispatch (Triton, universal)": the pipeline diagram
 *          (router scores, top-k gating, permute ... unpermute + weighted
 *          combine) and Usage (gating "softmax" or "sigmoid").
 *
 * Conventions shared by every call
 *   - T tokens, H hidden size, E experts, K = TOP_K routes per token.
 *   - Assignment id a = t*K + k names route k of token t; token = a / K
 *     ([BIN] Workflow step 6, [PAD] Implementation Pattern).
 *   - All tensors are dense, row-major, rows of H elements with stride H.
 *   - Index arrays are int32; T*K must be < 2^31. Byte offsets are 64-bit.
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream` and returns; no call
 *     synchronises the host, allocates or frees memory.
 *   - The caller owns every buffer. Scratch comes from a caller-provided
 *     device workspace `ws` of `ws_bytes` bytes, at least
 *     peg_workspace_bytes(T, K, E); it must not be shared by calls that may
 *     run concurrently. Workspace contents need no initialisation.
 *   - Host-side argument checks return a status synchronously and enqueue
 *     nothing. No C++ exception crosses this boundary.
 *   - Data preconditions of the routing arrays (bin_ids nondecreasing,
 *     bins consistent, unique assignment ids; [BIN]/[PAD] Workflow and Ascend
 *     Guardrails) are NOT checked by the hot calls; peg_validate_routing
 *     checks them on demand. Whatever the routing arrays hold, no call reads
 *     or writes outside the buffers whose sizes this header states.
 */
#ifndef PEG_H_
#define PEG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t peg_status;
#define PEG_OK 0
#define PEG_ERR_NULL_ARG 1      /* a required pointer is NULL */
#define PEG_ERR_BAD_SHAPE 2     /* a size is out of range (see each call) */
#define PEG_ERR_BAD_DTYPE 3     /* unsupported dtype / layout code */
#define PEG_ERR_WORKSPACE 4     /* ws is NULL or ws_bytes is too small */
#define PEG_ERR_LAUNCH 5        /* the HIP runtime rejected a launch */
#define PEG_ERR_ALIGNMENT 6     /* a pointer is not aligned to its element */
#define PEG_ERR_SCRATCH_LIMIT 7 /* the sizes need more than the static scratch of an
                                   allocation-free entry point */

/* Element types. Gathers move bits and accept any of them. */
#define PEG_F32 0
#define PEG_BF16 1
#define PEG_F16 2

/* Expert-tensor layouts. */
#define PEG_BINNED 0 /* [E, C, H]: row = e*C + offset, offsets >= C dropped ([BIN]) */
#define PEG_PADDED 1 /* [padded_bins[E-1], H]: row = padded_start(e) + offset ([PAD]) */

/* Limits enforced by the host checks. Besides the limits each call lists,
 * every call returns PEG_ERR_BAD_SHAPE when one of its launches would exceed
 * 2^32 - 1 threads (a HIP dispatch counts its threads in 32 bits), before
 * it writes any output (a call given slot_row = NULL may have rebuilt the row
 * map into its workspace by then): for the row kernels (2 to 8 waves of 64
 * per token, 4 waves per block) this is T above about 33.5 million tokens
 * at 2 waves per token down to 8.4 million at 8. */
#define PEG_MAX_EXPERTS 1024

/* Bits of the flag word written by peg_validate_routing and of the
 * err_flag word of peg_gather_padded. */
#define PEG_FLAG_BINS_NOT_MONOTONIC 0x1u   /* bins[e] < bins[e-1] or bins[0] < 0 */
#define PEG_FLAG_BINS_TOTAL 0x2u           /* bins[E-1] != number of indices */
#define PEG_FLAG_BIN_IDS 0x4u              /* bin_ids[i] != e for bins[e-1] <= i < bins[e] */
#define PEG_FLAG_PADDED_BINS 0x8u          /* padded_bins not monotonic, or a padded segment < its count */
#define PEG_FLAG_INDICES 0x10u             /* an index outside [0, T*K) or repeated */
#define PEG_FLAG_OUT_ROWS 0x20u            /* padded_bins[E-1] > out_rows: rows beyond were skipped */

/* Human-readable name of a status code (static string, never NULL). */
const char* peg_status_string(peg_status s);

/* ABI version, (major << 16) | minor. */
int32_t peg_abi_version(void);

/* Bytes of device workspace that every call below needs for these sizes
 * (0 only if T*K == 0 and E == 0). Pure host arithmetic. Returns 0 for
 * negative or out-of-range sizes. */
size_t peg_workspace_bytes(int64_t T, int32_t K, int32_t E);

/*
 * peg_route_prep - routing preparation.
 * [BIN] Workflow steps 1-2; [PAD] Workflow steps 1-3.
 *
 * Sorts the valid assignments by expert, stably (ascending assignment id
 * within an expert), and builds the per-expert bins.
 *   top_experts [T*K] int32: expert id of assignment a; any value outside
 *                  [0, E) (normally -1) means "no route" and the assignment
 *                  is left out of the sort.
 *   layout         PEG_BINNED or PEG_PADDED: selects how slot_row is filled.
 *   capacity       C >= 1, rows per expert of the binned layout (binned only).
 *   pad_multiple   m >= 1 (required when padded_bins != NULL or layout is
 *                  padded; ignored otherwise).
 * Outputs (all written in full):
 *   indices [T*K]  positions [0, n): valid assignment ids sorted by expert;
 *                  positions [n, T*K): -1. n = bins[E-1] = number of valid
 *                  assignments.
 *   bin_ids [T*K]  positions [0, n): expert of indices[i] (nondecreasing);
 *                  positions [n, T*K): -1.
 *   tokens_per_expert [E] real count of each expert (may be NULL).
 *   bins [E]       inclusive cumulative counts: bins[e] = sum_{j<=e} count[j].
 *   padded_bins [E] inclusive cumulative sums of count[j] rounded up to a
 *                  multiple of m (may be NULL for the binned layout).
 *   slot_row [T*K] row of assignment a in the expert tensor of `layout`,
 *                  or -1 if a has no route or (binned) was dropped because
 *                  its offset within its expert is >= C (may be NULL).
 *                  This inverse map is what the gather, scatter and wgrad
 *                  kernels consume; passing it to them skips a rebuild.
 * Errors: NULL_ARG (top_experts/indices/bin_ids/bins, or ws), BAD_SHAPE
 * (T < 0, K < 1, E < 1, E > PEG_MAX_EXPERTS, T*K >= 2^31, C < 1 for binned,
 * m < 1 where required), BAD_DTYPE (layout), WORKSPACE, LAUNCH.
 */
peg_status peg_route_prep(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                          int32_t layout, int32_t capacity, int32_t pad_multiple,
                          int32_t* indices, int32_t* bin_ids, int32_t* tokens_per_expert,
                          int32_t* bins, int32_t* padded_bins, int32_t* slot_row,
                          void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's own device scratch behind peg_route_prep_noalloc
 * (one copy per GPU, held until the process ends). */
#define PEG_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * peg_route_prep_noalloc - peg_route_prep for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and outputs, bit for
 * bit, without the workspace. It allocates nothing and frees nothing; its
 * scratch (the per-tile expert counts of batches of 8192 assignments and
 * more) is a static array of PEG_NOALLOC_SCRATCH_BYTES in the library's
 * device memory, one per GPU.
 *   Limit: the count table takes ceil(T*K / tile) * E * 4 bytes, the tile
 *   being 1024 assignments for E <= 512 and 512 above (smaller for batches
 *   under 64 tiles); sizes beyond the scratch return PEG_ERR_SCRATCH_LIMIT
 *   and enqueue nothing. The scratch holds up to 4,194,304 assignments at
 *   E = 64, 1,048,576 at E = 256 and 131,072 at E = 1024.
 *   The scratch needs no clearing (every entry a call reads, it writes
 *   first). Every call on one GPU uses that GPU's one array: calls that may
 *   overlap on one GPU (other streams, other host threads) race and must be
 *   serialised by the caller. The stream must belong to the calling thread's
 *   current device (the array of that device is used).
 * Errors: those of peg_route_prep (without WORKSPACE), SCRATCH_LIMIT.
 */
peg_status peg_route_prep_noalloc(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                                  int32_t layout, int32_t capacity, int32_t pad_multiple,
                                  int32_t* indices, int32_t* bin_ids, int32_t* tokens_per_expert,
                                  int32_t* bins, int32_t* padded_bins, int32_t* slot_row, void* stream);

/*
 * peg_gather_binned - binned dispatch into [E, C, H].
 * [BIN] Goal, Workflow step 3, Implementation Pattern, Ascend Guardrails
 * (zero-initialised output, nothing beyond capacity).
 *
 * For every sorted position i < n with offset o = i - start(e) < C
 * (e = bin_ids[i], start(e) = bins[e-1] or 0): out[e*C + o] = x[indices[i]/K],
 * copied bit for bit. Every other row of out (unused capacity) is zero.
 *   x   [T, H] of dtype; out [E*C, H] of dtype, every row written.
 *   slot_row [T*K] from peg_route_prep(layout = PEG_BINNED, same C), or NULL:
 *       then it is rebuilt from indices/bin_ids/bins into ws.
 *   indices, bin_ids [T*K] and bins [E] as produced by peg_route_prep
 *       (indices and bin_ids are only read when slot_row is NULL).
 * Errors: NULL_ARG, BAD_SHAPE (T < 0, H < 1, K < 1, E out of range, C < 1,
 * E*C*H too large for int64), BAD_DTYPE, ALIGNMENT (x or out not aligned to
 * the element size), WORKSPACE, LAUNCH.
 */
peg_status peg_gather_binned(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K,
                             int32_t E, int32_t capacity, const int32_t* indices,
                             const int32_t* bin_ids, const int32_t* bins,
                             const int32_t* slot_row, void* out, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * peg_gather_padded - padded dispatch into [padded_bins[E-1], H].
 * [PAD] Goal, Workflow steps 4-5, Implementation Pattern, Ascend Guardrails
 * (zero gaps, padded_bins[-1] rows).
 *
 * For every sorted position i < n: out[pstart(e) + (i - start(e))] =
 * x[indices[i]/K] bit for bit (pstart(e) = padded_bins[e-1] or 0); every gap
 * row of [0, R), R = padded_bins[E-1], is zero. Any monotonic padded_bins
 * whose segments hold their counts is accepted (not only the minimal
 * round-up). Rows [R, out_rows) are not touched.
 *   out [out_rows, H]: allocated rows; rows at or beyond out_rows are never
 *       written. If R > out_rows the rows beyond are skipped and
 *       PEG_FLAG_OUT_ROWS is OR-ed into *err_flag (when err_flag != NULL).
 *   slot_row from peg_route_prep(layout = PEG_PADDED, same padded_bins), or
 *       NULL (rebuilt from indices/bin_ids/bins/padded_bins into ws).
 * Errors: as peg_gather_binned, plus BAD_SHAPE for out_rows < 0.
 */
peg_status peg_gather_padded(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K,
                             int32_t E, const int32_t* indices, const int32_t* bin_ids,
                             const int32_t* bins, const int32_t* padded_bins,
                             const int32_t* slot_row, void* out, int64_t out_rows,
                             uint32_t* err_flag, void* ws, size_t ws_bytes, void* stream);

/*
 * peg_scatter_combine - inverse of the gathers: weighted top-k combine.
 * [BIN] Workflow step 5; [PAD] Workflow step 6 and Ascend Guardrails (weights
 * indexed by assignment id); [FMD] pipeline diagram, its final stage (undo
 * the permutation, combine with the gating weights).
 *
 * out[t, :] = sum over k = 0..K-1 (ascending) with assignment a = t*K + k
 * kept, of w[a] * y[row(a), :], accumulated in fp32 and rounded once to the
 * dtype of y (round to nearest even). Rows of y that are unused capacity,
 * padding, or dropped are never read. A token with no kept route gets a
 * zero row.
 *   y [R, H] of dtype (expert tensor in `layout`); out [T, H] of dtype.
 *   y may be NULL for a padded tensor of no rows (padded_bins[E-1] = 0):
 *       then no row is read (and every output row is zero).
 *   weights [T*K] f32 by assignment id, or NULL (every factor is 1).
 *   capacity: binned only. padded_bins: padded only. indices/bin_ids/bins/
 *   padded_bins are read only when slot_row is NULL.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, ALIGNMENT, WORKSPACE, LAUNCH.
 */
peg_status peg_scatter_combine(const void* y, int32_t dtype, int32_t layout, int64_t T,
                               int64_t H, int32_t K, int32_t E, int32_t capacity,
                               const int32_t* indices, const int32_t* bin_ids,
                               const int32_t* bins, const int32_t* padded_bins,
                               const int32_t* slot_row, const float* weights, void* out,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * peg_wgrad - router-weight gradient.
 * [BIN] Workflow step 6; [PAD] Workflow step 6; fp32 accumulation per the
 * Ascend Guardrails of both.
 *
 * wgrad[a] = sum_h y[row(a), h] * grad[a/K, h] for every kept assignment a,
 * accumulated in fp32; wgrad[a] = 0 for dropped or unrouted assignments.
 *   y [R, H] and grad [T, H] both of dtype; wgrad [T*K] f32, fully written.
 *   y may be NULL for a padded tensor of no rows (then every wgrad is 0).
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, ALIGNMENT, WORKSPACE, LAUNCH.
 */
peg_status peg_wgrad(const void* y, const void* grad, int32_t dtype, int32_t layout, int64_t T,
                     int64_t H, int32_t K, int32_t E, int32_t capacity, const int32_t* indices,
                     const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
                     const int32_t* slot_row, float* wgrad, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * peg_combine_backward - backward of the combine, together with wgrad.
 * The combine ([BIN] Workflow step 5, [PAD] Workflow step 6) is linear in the
 * expert tensor; its gradient with respect to that tensor, given the upstream
 * gradient dout of the combine output, sends dout back through the same row
 * mapping (the [PAD] front matter lists this use of the padded storage).
 * wgrad is [BIN]/[PAD] Workflow step 6 with grad = dout.
 *
 * For K <= 2 one pass over dout computes both; for larger K two launches
 * on the stream do, a weighted gather of dout into dy, then the wgrad
 * kernel of peg_wgrad (at K = 8 the pair measured 6-14% faster than the
 * one pass on a clean cache and within 2% of it when called back to back;
 * at K = 2 the one pass is faster):
 *   dy[row(a)] = w[a] * dout[a/K] for every kept assignment a (fp32 product,
 *                one rounding to dtype; raw bit copy when weights == NULL);
 *                every other row of [0, dy_rows) is zero: the gap rows of
 *                the layout and, when dy_rows > R, the rows [R, dy_rows);
 *   wgrad[a]   = <y[row(a)], dout[a/K]> as peg_wgrad.
 *   y [R, H], dout [T, H], dy [dy_rows, H], all of dtype; weights [T*K] f32
 *   or NULL; wgrad [T*K] f32, fully written. R = E*C (binned) or
 *   padded_bins[E-1] (padded); y may be NULL for a padded tensor of no rows
 *   (every wgrad is then 0). Rows of dy at or past dy_rows are never
 *   written (a route whose row is there gets no dy row; its wgrad is still
 *   computed). The other arguments are as for peg_wgrad.
 * Errors: NULL_ARG, BAD_SHAPE (also dy_rows < 0), BAD_DTYPE, ALIGNMENT,
 * WORKSPACE, LAUNCH.
 */
peg_status peg_combine_backward(const void* y, const void* dout, const float* weights, int32_t dtype,
                                int32_t layout, int64_t T, int64_t H, int32_t K, int32_t E, int32_t capacity,
                                const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                                const int32_t* padded_bins, const int32_t* slot_row, void* dy, int64_t dy_rows,
                                float* wgrad, void* ws, size_t ws_bytes, void* stream);

/*
 * peg_route_prep_windows - the routing preparation of peg_route_prep with
 * each expert's rows in a caller-given window [row_base[e], row_limit[e]).
 * [BIN]/[PAD] Workflow steps 1-2 (stable sort by expert, inclusive bins) and
 * the Implementation Pattern's row formula (segment start + offset inside the
 * expert, dropped past the segment's end) with the segment start and end
 * supplied per expert.
 *
 * indices, bin_ids, tokens_per_expert and bins are exactly those of
 * peg_route_prep for this batch. slot_row[a] = row_base[e] + offset of a
 * inside expert e (ascending assignment id), or -1 if that is at or past
 * row_limit[e] (dropped) or a has no route. Windows [e*C, (e+1)*C) give the
 * binned layout; for one shard of a batch cut into contiguous token ranges,
 * windows starting at e*C + (assignments of e in the earlier shards) place
 * the shard's rows, and drop its assignments, exactly as one call over the
 * whole batch would (the earlier shards' counts come from their
 * tokens_per_expert: an all-gather of E counts per shard and a prefix sum).
 *   row_base, row_limit [E] int32 device, 0 <= row_base[e];
 *   other arguments as for peg_route_prep; ws: peg_workspace_bytes(T, K, E).
 * Errors: NULL_ARG, BAD_SHAPE, WORKSPACE, LAUNCH.
 */
peg_status peg_route_prep_windows(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                                  const int32_t* row_base, const int32_t* row_limit, int32_t* indices,
                                  int32_t* bin_ids, int32_t* tokens_per_expert, int32_t* bins,
                                  int32_t* slot_row, void* ws, size_t ws_bytes, void* stream);

/*
 * peg_gather_rows - dispatch by a row map alone: out[slot_row[a]] =
 * x[a / K] for every assignment a with 0 <= slot_row[a] < out_rows (raw
 * bytes). [BIN] Workflow step 3 / [PAD] Workflow step 4 (copy each kept
 * token row to its expert row) without the zero-fill of unused rows: rows no
 * assignment maps to are left as they are, for a caller that assembles one
 * expert tensor from several calls (shards) and clears it itself.
 * A row at or past out_rows is skipped and sets PEG_FLAG_OUT_ROWS in
 * *err_flag (if err_flag != NULL).
 *   x [T, H] of dtype; slot_row [T*K] int32 device; out [out_rows, H].
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, ALIGNMENT, LAUNCH.
 */
peg_status peg_gather_rows(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K,
                           const int32_t* slot_row, void* out, int64_t out_rows, uint32_t* err_flag,
                           void* stream);

/* Gating functions of peg_router_topk. */
#define PEG_GATING_SOFTMAX 0
#define PEG_GATING_SIGMOID 1

/*
 * peg_router_topk - router top-k gating: scores -> top_experts and weights,
 * the inputs of peg_route_prep and of the weighted combine.
 * [FMD] pipeline diagram (router scores -> top-k gating -> permute) and
 * Usage (gating softmax or sigmoid).
 *
 * For each token t, with scores l = logits[t, 0..E-1]:
 *   top_experts[t, 0..K-1] = the K experts of highest score, highest first;
 *     equal scores: the lower expert id first; NaN ranks below every
 *     number; -0 and +0 are equal. The selection is exact (no rounding
 *     takes part in it).
 *   p = exp(l - max l) / sum_e exp(l_e - max l) over all E experts
 *     (PEG_GATING_SOFTMAX) or 1 / (1 + exp(-l)) (PEG_GATING_SIGMOID);
 *   weights[t, k] = p of expert top_experts[t, k], divided by the sum of the
 *     K chosen p when normalize != 0. fp32 arithmetic; NaN or infinite
 *     scores give what those formulas give in IEEE arithmetic. Renormalised
 *     sigmoid weights stay finite for any finite scores (the common factor
 *     exp(max l) is cancelled when max l < 0); an unnormalised p below about
 *     1e-38 may come back as 0.
 *   logits [T, E] of dtype (PEG_F32, PEG_BF16 or PEG_F16);
 *   top_experts [T, K] int32 and weights [T, K] f32, fully written.
 * Errors: NULL_ARG, BAD_SHAPE (T < 0, E < 1, E > PEG_MAX_EXPERTS, K < 1,
 * K > E, T*E >= 2^31), BAD_DTYPE (also an unknown gating), ALIGNMENT, LAUNCH.
 */
peg_status peg_router_topk(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                           int32_t gating, int32_t normalize, int32_t* top_experts, float* weights,
                           void* stream);

/*
 * peg_route_prep_logits - router top-k gating fused with the routing
 * preparation: one call from router scores to everything peg_route_prep
 * writes. [FMD] pipeline diagram (router scores -> top-k gating -> permute)
 * and [PAD]/[BIN] Workflow steps 1-3.
 *
 * Writes top_experts [T, K] and weights [T, K] exactly as peg_router_topk
 * does, and indices, bin_ids, tokens_per_expert, bins, padded_bins and
 * slot_row exactly as peg_route_prep(top_experts, ...) does. The gating pass
 * also counts the experts of each tile of assignment ids, so no separate
 * histogram pass reads top_experts back.
 *   Arguments: those of peg_router_topk, then those of peg_route_prep after
 *   its top_experts (layout, capacity, pad_multiple, indices, bin_ids,
 *   tokens_per_expert, bins, padded_bins, slot_row, ws, ws_bytes).
 *   ws: at least peg_workspace_bytes(T, K, E).
 * Errors: those of both calls.
 */
peg_status peg_route_prep_logits(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                                 int32_t gating, int32_t normalize, int32_t layout, int32_t capacity,
                                 int32_t pad_multiple, int32_t* top_experts, float* weights,
                                 int32_t* indices, int32_t* bin_ids, int32_t* tokens_per_expert,
                                 int32_t* bins, int32_t* padded_bins, int32_t* slot_row, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * peg_routing_map_compact - dense routing map -> fixed-width routes.
 * [MOK] RoutingMapToIndices and routing_map_to_mok_inputs.
 *
 * For each row t: the experts e with routing_map[t, e] != 0 taken in
 * increasing e; the first min(count, topk) fill route_experts[t, 0..] with e
 * and probs_out[t, 0..] with probs[t, e] widened to f32; the remaining slots
 * get -1 and 0.0. The map is authoritative: probs never select routes.
 *   probs [T, E] of probs_dtype (PEG_F32, PEG_BF16 or PEG_F16);
 *   routing_map [T, E] bytes, nonzero = routed;
 *   probs_out [T, topk] f32; route_experts [T, topk] int32.
 * Errors: NULL_ARG, BAD_SHAPE (T < 0, E < 1, E > PEG_MAX_EXPERTS, topk < 1,
 * topk > E), BAD_DTYPE, ALIGNMENT, LAUNCH.
 */
peg_status peg_routing_map_compact(const void* probs, int32_t probs_dtype,
                                   const uint8_t* routing_map, int64_t T, int32_t E,
                                   int32_t topk, float* probs_out, int32_t* route_experts,
                                   void* stream);

/*
 * peg_routing_map_compact_backward - router-gradient scatter of the
 * compaction. [MOK] RoutingMapToIndices (backward) and the backward kernel
 * listed under Functions.
 *
 * grad_probs[t, e] = grad_probs_out[t, j] where route_experts[t, j] == e
 * (j < topk, route_experts[t, j] in [0, E)); every other element is 0.
 *   grad_probs_out [T, topk] f32; route_experts [T, topk] int32 as returned
 *   by peg_routing_map_compact; grad_probs [T, E] f32, fully written.
 * Errors: NULL_ARG, BAD_SHAPE, LAUNCH.
 */
peg_status peg_routing_map_compact_backward(const float* grad_probs_out,
                                            const int32_t* route_experts, int64_t T,
                                            int32_t E, int32_t topk, float* grad_probs,
                                            void* stream);

/*
 * peg_validate_routing - on-demand check of the routing preconditions.
 * [BIN] Ascend Guardrails (bins monotonic, bins[-1] equals the number of
 * indices, bin_ids consistent with the bin boundaries, unique assignment
 * ids); [PAD] Ascend Guardrails (padded segments no smaller than counts).
 *
 * Writes into *flags (device uint32, overwritten) the OR of PEG_FLAG_* bits
 * for every violated condition; 0 means valid.
 *   n_indices: the number of indices the caller holds (len(indices)); if
 *       < 0, the total check is skipped and n = bins[E-1] is used.
 *   padded_bins may be NULL (padded checks skipped).
 * Errors: NULL_ARG, BAD_SHAPE, WORKSPACE, LAUNCH.
 */
peg_status peg_validate_routing(const int32_t* indices, const int32_t* bin_ids,
                                const int32_t* bins, const int32_t* padded_bins, int64_t T,
                                int32_t K, int32_t E, int64_t n_indices, uint32_t* flags,
                                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PEG_H_ */
