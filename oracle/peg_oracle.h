/*
 * peg_oracle.h - plain, slow CPU oracle of the MoE token-routing data path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code. The GPU library
 * shares no code, header, table or helper with it, and neither includes or
 * calls the other.
 *
 * Every function follows the page passage it cites, in the pages' own order:
 *   [BIN] "Build Triton-Ascend Binned MoE Routing": Workflow,
 *         Implementation Pattern, Ascend Guardrails.
 *   [PAD] "Build Triton-Ascend Padded MoE Routing": same sections.
 *   [MOK] "core.transformer.moe.megakernel.mok.route_adapter":
 *         RoutingMapToIndices, routing_map_to_mok_inputs.
 *   [FMD] "Fused MoE Dispatch (Triton, universal)": pipeline figure, Usage
 *         (router top-k gating, softmax or sigmoid).
 * Floating point is evaluated in double (fp64) and rounded once to the
 * output type with round-to-nearest-even.
 *
 * Return value of the int functions: 0 on success, -1 on an argument the
 * oracle refuses (it never reads or writes out of bounds).
 */
#ifndef PEG_ORACLE_H_
#define PEG_ORACLE_H_

#include <stdint.h>

#define PEGO_F32 0
#define PEGO_BF16 1
#define PEGO_F16 2
#define PEGO_BINNED 0
#define PEGO_PADDED 1

/* Number conversions, written from the IEEE 754 formats. */
double pego_load(const void* base, int32_t dtype, int64_t idx);
void pego_store(void* base, int32_t dtype, int64_t idx, double v);
uint16_t pego_round_bf16(double v);
uint16_t pego_round_f16(double v);

/* Routing preparation: returns n (valid assignments) or -1. */
int64_t pego_route_prep(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                        int32_t pad_multiple, int32_t* indices, int32_t* bin_ids,
                        int32_t* tokens_per_expert, int32_t* bins, int32_t* padded_bins);

/* Row of every assignment in the expert tensor (-1: unrouted or dropped). */
int pego_assignment_rows(int64_t T, int32_t K, int32_t E, int32_t layout, int32_t capacity,
                         const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                         const int32_t* padded_bins, int32_t* rows_out);

/* Rows within caller-given per-expert windows [row_base[e], row_limit[e]). */
int pego_assignment_rows_windows(int64_t T, int32_t K, int32_t E, const int32_t* indices,
                                 const int32_t* bin_ids, const int32_t* bins,
                                 const int32_t* row_base, const int32_t* row_limit,
                                 int32_t* rows_out);

int pego_gather(const void* x, int64_t T, int64_t row_bytes, int32_t K, int32_t E,
                int32_t layout, int32_t capacity, const int32_t* indices,
                const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
                int64_t R, const int64_t* rows, int64_t nrows, void* out);

int pego_scatter_combine(const void* y, int32_t dtype, int64_t R, int64_t T, int64_t H,
                         int32_t K, int32_t E, int32_t layout, int32_t capacity,
                         const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                         const int32_t* padded_bins, const float* weights,
                         const int64_t* tokens, int64_t ntok, void* out, double* scale);

int pego_wgrad(const void* y, const void* grad, int32_t dtype, int64_t R, int64_t T, int64_t H,
               int32_t K, int32_t E, int32_t layout, int32_t capacity, const int32_t* indices,
               const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
               const int64_t* tokens, int64_t ntok, float* wgrad, double* scale);

int pego_combine_backward_dy(const void* dout, int32_t dtype, int64_t T, int64_t H, int32_t K, int32_t E,
                             int32_t layout, int32_t capacity, const int32_t* indices, const int32_t* bin_ids,
                             const int32_t* bins, const int32_t* padded_bins, const float* weights, int64_t R,
                             const int64_t* rows, int64_t nrows, void* dy);

int pego_routing_map_compact(const void* probs, int32_t probs_dtype, const uint8_t* routing_map,
                             int64_t T, int32_t E, int32_t topk, float* probs_out,
                             int32_t* route_experts);

int pego_routing_map_compact_backward(const float* grad_probs_out, const int32_t* route_experts,
                                      int64_t T, int32_t E, int32_t topk, float* grad_probs);

/* Router top-k gating: gating 0 = softmax, 1 = sigmoid; K <= E. */
int pego_router_topk(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                     int32_t gating, int32_t normalize, int32_t* top_experts, float* weights);

uint32_t pego_validate_routing(const int32_t* indices, const int32_t* bin_ids,
                               const int32_t* bins, const int32_t* padded_bins, int64_t T,
                               int32_t K, int32_t E, int64_t n_indices);

#endif
