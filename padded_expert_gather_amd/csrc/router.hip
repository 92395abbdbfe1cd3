// router.hip - router top-k gating on gfx950: per-token scores -> the K
// chosen experts and their weights, the input of route_prep; and the same
// gating fused with route_prep's histogram pass.
//
// Source: "Fused MoE Dispatch (Triton, universal)", the pipeline figure
// (router scores, then top-k gating, then permute) and Usage (gating by
// softmax or by sigmoid). What is computed, per token t with scores l[t, :]:
//   * the K experts with the highest scores, highest first, the lower
//     expert id first among equal scores (NaN ranks below every number,
//     -0 and +0 are equal);
//   * p = softmax over all E scores (shifted by the highest score), or the
//     logistic sigmoid of each chosen score;
//   * weights = p of the chosen experts, renormalised over the K when asked.
//
// Design: a group of G lanes (8, or 16/32 when E > 256) owns one token, so
// a wave serves 64/G tokens; lane g holds the scores of experts g, g + G,
// g + 2G, ... (CPL <= 32 of them) as order-preserving 32-bit keys. K rounds
// of [group maximum of the keys, group minimum of the ids holding it, the
// owner clears the winner] give the K experts in rank order, exactly (no
// float arithmetic decides the selection). Group reductions use DPP lane
// moves (quad permutes, half-row and row mirrors), plain VALU operations;
// only groups wider than a 16-lane row also cross rows through the LDS
// crossbar. Result k is kept by lane k % G, so the K outputs of a token are
// written by the group's lanes side by side, and the weights of all K are
// evaluated after the rounds, by all lanes at once.
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

// Order-preserving image of a float's value as an unsigned integer: larger
// values give larger images (every number maps to 0x007FFFFF or more); NaN
// gives 1, below every number; -0 maps as +0; 0 is left free to mark an
// expert that is absent or already chosen.
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f != f) return 1u;
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) == 0u) b = 0u;  // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of score_key for every key a number gives (1 decodes to NaN).
__device__ __forceinline__ float key_score(uint32_t k) {
    if (k <= 1u) return __uint_as_float(0x7FC00000u);
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Maximum / minimum over the G lanes of a group, every lane of it gets the
// result (DPP lane moves inside 16-lane rows, the LDS crossbar beyond).
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    v = max(v, (uint32_t)dpp_read<kDppQuadXor1>((int)v));
    v = max(v, (uint32_t)dpp_read<kDppQuadXor2>((int)v));
    v = max(v, (uint32_t)dpp_read<kDppHalfMirror>((int)v));
    if constexpr (G >= 16) v = max(v, (uint32_t)dpp_read<kDppRowMirror>((int)v));
#pragma unroll
    for (int d = 16; d < G; d <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, G));
    return v;
}

template <int G>
__device__ __forceinline__ uint32_t group_min(uint32_t v) {
    v = min(v, (uint32_t)dpp_read<kDppQuadXor1>((int)v));
    v = min(v, (uint32_t)dpp_read<kDppQuadXor2>((int)v));
    v = min(v, (uint32_t)dpp_read<kDppHalfMirror>((int)v));
    if constexpr (G >= 16) v = min(v, (uint32_t)dpp_read<kDppRowMirror>((int)v));
#pragma unroll
    for (int d = 16; d < G; d <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d, G));
    return v;
}

// Sum over the G lanes of a group, the same value in every lane (each step
// adds two partial sums that the pair of lanes holds in swapped order, and
// float addition is commutative).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_read_f<kDppQuadXor1>(v);
    v += dpp_read_f<kDppQuadXor2>(v);
    v += dpp_read_f<kDppHalfMirror>(v);
    if constexpr (G >= 16) v += dpp_read_f<kDppRowMirror>(v);
#pragma unroll
    for (int d = 16; d < G; d <<= 1) v += __shfl_xor(v, d, G);
    return v;
}

template <int DT>
__device__ __forceinline__ float load_score(const void* p, int64_t i) {
    if constexpr (DT == PEG_F32) return reinterpret_cast<const float*>(p)[i];
    else return decode<DT>(reinterpret_cast<const uint16_t*>(p)[i]);
}

// Gating of token t by the G lanes of a group (lane g): on return, lane g
// holds the results k = j * G + g (k < K, j < KS) in sel_e[j] (expert) and
// sel_w[j] (weight). KS = 1 when K <= G. Every lane of the group must call it.
//
// A round picks the highest score key over the group (a 32-bit maximum),
// then the lowest expert id holding it (a 32-bit minimum over the lanes whose
// key ties); the winner's key is cleared. The scores of the chosen experts
// are kept and turned into weights after the K rounds, all lanes at once.
// exp is the hardware base-2 exponential of x * log2(e) (__expf): its
// relative error grows with |x| as about |x| * 2^-24, well inside the 1e-5
// tolerance for the score gaps that carry weight.
template <int DT, int G, int CPL, int KS>
__device__ __forceinline__ void gate_token(const void* __restrict__ logits, int64_t t, int32_t E, int32_t K,
                                           int32_t gating, int32_t normalize, int g, int32_t (&sel_e)[KS],
                                           float (&sel_w)[KS]) {
    static_assert(G >= 8 && G <= kWave && (G & (G - 1)) == 0, "group of 8..64 lanes");
    uint32_t key[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = g + j * G;
        key[j] = e < E ? score_key(load_score<DT>(logits, t * E + e)) : 0u;
    }
    uint32_t top = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) top = max(top, key[j]);
    top = group_max<G>(top);
    const float m = key_score(top);  // the highest score (NaN if every score is)
    // softmax denominator over all E scores
    float denom = 1.0f;
    if (gating == 0) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            if (g + j * G < E) s += __expf(key_score(key[j]) - m);
        denom = group_sum<G>(s);
    }
    float sel_l[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        sel_e[j] = 0;
        sel_l[j] = 0.0f;
    }
    for (int k = 0; k < K; ++k) {
        uint32_t best = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) best = max(best, key[j]);
        best = group_max<G>(best);
        // lowest id among the group's keys equal to best: within a lane the
        // ids rise with j, so its first such slot
        uint32_t id = 0xFFFFFFFFu;
#pragma unroll
        for (int j = CPL - 1; j >= 0; --j)
            if (key[j] == best) id = (uint32_t)(g + j * G);
        const int32_t e = (int32_t)group_min<G>(id);
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            if (g + j * G == e) key[j] = 0u;
        if constexpr (KS == 1) {
            if (k == g) {
                sel_e[0] = e;
                sel_l[0] = key_score(best);
            }
        } else {
            if (k % G == g) {
#pragma unroll
                for (int j = 0; j < KS; ++j)
                    if (j == k / G) {
                        sel_e[j] = e;
                        sel_l[j] = key_score(best);
                    }
            }
        }
    }
    // Renormalised sigmoid with a negative top score m: every chosen sigmoid
    // carries the factor exp(m), which cancels in the ratio; it is taken out
    // (q = exp(l - m) / (1 + exp(l)) instead of 1 / (1 + exp(-l))) so that
    // exp(-l) cannot overflow fp32 and turn the weights into 0 / 0.
    const bool shifted = gating != 0 && normalize && m < 0.0f;
    float sel_sum = 0.0f;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        float p = 0.0f;
        if (j * G + g < K) {
            const float l = sel_l[j];
            if (gating == 0) p = __expf(l - m) / denom;
            else if (shifted) p = __expf(l - m) / (1.0f + __expf(l));
            else p = 1.0f / (1.0f + __expf(-l));
        }
        sel_w[j] = p;
        sel_sum += p;
    }
    if (normalize) {
        sel_sum = group_sum<G>(sel_sum);
#pragma unroll
        for (int j = 0; j < KS; ++j) sel_w[j] = sel_w[j] / sel_sum;
    }
}

// G lanes per token, CPL scores per lane (E <= G * CPL), KS result slots per
// lane (K <= G * KS).
template <int DT, int G, int CPL, int KS>
__global__ __launch_bounds__(kBlock) void router_topk_kernel(const void* __restrict__ logits, int64_t T, int32_t E,
                                                             int32_t K, int32_t gating, int32_t normalize,
                                                             int32_t* __restrict__ top_experts,
                                                             float* __restrict__ weights) {
    constexpr int TPB = kBlock / G;
    const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / G;
    if (t >= T) return;  // whole groups leave together: reductions stay within live groups
    const int g = threadIdx.x % G;
    int32_t sel_e[KS];
    float sel_w[KS];
    gate_token<DT, G, CPL, KS>(logits, t, E, K, gating, normalize, g, sel_e, sel_w);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int k = j * G + g;
        if (k < K) {
            top_experts[t * K + k] = sel_e[j];
            weights[t * K + k] = sel_w[j];
        }
    }
}

// Gating fused with the first pass of the routing preparation: block b owns
// the assignment ids [b * tile, (b + 1) * tile) and gates every token that
// has an id there (a token that straddles two tiles is gated by both blocks,
// identically; the block holding its first id writes its outputs). The
// block's expert histogram of its ids goes to counts[b * E + e], the
// table the placement pass reads.
constexpr int kHistThreads = 1024;  // gating lanes of a tile: 128 tokens per pass at 8 lanes per token

template <int DT, int G, int CPL, int KS>
__global__ __launch_bounds__(kHistThreads) void router_hist_kernel(const void* __restrict__ logits, int64_t T, int32_t E,
                                                             int32_t K, int32_t gating, int32_t normalize,
                                                             int64_t tile, int64_t ntiles,
                                                             int32_t* __restrict__ top_experts,
                                                             float* __restrict__ weights,
                                                             int32_t* __restrict__ counts) {
    constexpr int TPB = kHistThreads / G;
    __shared__ int hist[PEG_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += kHistThreads) hist[e] = 0;
    lds_barrier();
    const int64_t total = T * (int64_t)K;
    const int64_t lo = (int64_t)blockIdx.x * tile;
    const int64_t hi = lo + tile < total ? lo + tile : total;
    const int64_t t_first = lo / K;
    const int64_t t_last = (hi - 1) / K;  // hi > lo: every launched tile holds an id
    const int g = threadIdx.x % G;
    for (int64_t t0 = t_first; t0 <= t_last; t0 += TPB) {
        const int64_t t = t0 + threadIdx.x / G;
        if (t > t_last) continue;  // whole groups skip together
        int32_t sel_e[KS];
        float sel_w[KS];
        gate_token<DT, G, CPL, KS>(logits, t, E, K, gating, normalize, g, sel_e, sel_w);
        const bool owner = t * K >= lo;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int k = j * G + g;
            if (k < K) {
                const int64_t a = t * K + k;
                if (a >= lo && a < hi) atomicAdd(&hist[sel_e[j]], 1);
                if (owner) {
                    top_experts[a] = sel_e[j];
                    weights[a] = sel_w[j];
                }
            }
        }
    }
    lds_barrier();
    for (int e = threadIdx.x; e < E; e += kHistThreads) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Launch arguments of both gating kernels.
struct GateArgs {
    const void* logits;
    int64_t T;
    int32_t E, K, gating, normalize;
    int32_t* top;
    float* w;
    int64_t tile, ntiles;  // fused histogram only (ntiles > 0)
    int32_t* counts;
};

template <int DT, int G, int CPL, int KS>
static peg_status gate_launch(hipStream_t s, const GateArgs& a) {
    if (a.ntiles > 0) {
        if (!grid_fits(a.ntiles, kHistThreads)) return PEG_ERR_BAD_SHAPE;
        return launch(router_hist_kernel<DT, G, CPL, KS>, dim3((unsigned)a.ntiles), dim3(kHistThreads), 0, s,
                      a.logits, a.T, a.E, a.K, a.gating, a.normalize, a.tile, a.ntiles, a.top, a.w, a.counts);
    }
    constexpr int TPB = kBlock / G;
    if (!grid_fits((a.T + TPB - 1) / TPB, kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)((a.T + TPB - 1) / TPB));
    return launch(router_topk_kernel<DT, G, CPL, KS>, grid, dim3(kBlock), 0, s, a.logits, a.T, a.E, a.K, a.gating,
                  a.normalize, a.top, a.w);
}

template <int DT, int G, int CPL>
static peg_status gate_go(hipStream_t s, const GateArgs& a) {
    if (a.K <= G) return gate_launch<DT, G, CPL, 1>(s, a);
    return gate_launch<DT, G, CPL, CPL>(s, a);
}

template <int DT>
static peg_status gate_dispatch(hipStream_t s, const GateArgs& a) {
    if (a.E <= 8) return gate_go<DT, 8, 1>(s, a);
    if (a.E <= 16) return gate_go<DT, 8, 2>(s, a);
    if (a.E <= 32) return gate_go<DT, 8, 4>(s, a);
    if (a.E <= 64) return gate_go<DT, 8, 8>(s, a);
    if (a.E <= 128) return gate_go<DT, 8, 16>(s, a);
    if (a.E <= 256) return gate_go<DT, 8, 32>(s, a);
    if (a.E <= 512) return gate_go<DT, 16, 32>(s, a);
    return gate_go<DT, 32, 32>(s, a);
}

static peg_status gate(int32_t dtype, hipStream_t s, const GateArgs& a) {
    if (dtype == PEG_F32) return gate_dispatch<PEG_F32>(s, a);
    if (dtype == PEG_BF16) return gate_dispatch<PEG_BF16>(s, a);
    return gate_dispatch<PEG_F16>(s, a);
}

static peg_status gate_checks(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K, int32_t gating,
                              const int32_t* top_experts, const float* weights) {
    if (!dtype_ok(dtype) || (gating != PEG_GATING_SOFTMAX && gating != PEG_GATING_SIGMOID))
        return PEG_ERR_BAD_DTYPE;
    if (T < 0 || E < 1 || E > PEG_MAX_EXPERTS || K < 1 || K > E) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / E) return PEG_ERR_BAD_SHAPE;
    if (T > 0 && (!logits || !top_experts || !weights)) return PEG_ERR_NULL_ARG;
    if (!aligned(logits, elem_bytes(dtype)) || !aligned(top_experts, 4) || !aligned(weights, 4))
        return PEG_ERR_ALIGNMENT;
    return PEG_OK;
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_router_topk(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                                   int32_t gating, int32_t normalize, int32_t* top_experts, float* weights,
                                   void* stream) {
    PEG_CHECK(gate_checks(logits, dtype, T, E, K, gating, top_experts, weights));
    if (T == 0) return PEG_OK;
    const GateArgs a{logits, T, E, K, gating, normalize ? 1 : 0, top_experts, weights, 0, 0, nullptr};
    return gate(dtype, reinterpret_cast<hipStream_t>(stream), a);
}

PEG_API peg_status peg_route_prep_logits(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                                         int32_t gating, int32_t normalize, int32_t layout, int32_t capacity,
                                         int32_t pad_multiple, int32_t* top_experts, float* weights,
                                         int32_t* indices, int32_t* bin_ids, int32_t* tokens_per_expert,
                                         int32_t* bins, int32_t* padded_bins, int32_t* slot_row, void* ws,
                                         size_t ws_bytes, void* stream) {
    PEG_CHECK(gate_checks(logits, dtype, T, E, K, gating, top_experts, weights));
    // the routing-preparation checks of peg_route_prep
    if (!layout_ok(layout)) return PEG_ERR_BAD_DTYPE;
    if (T > kMaxAssign / K) return PEG_ERR_BAD_SHAPE;
    const int64_t total = T * (int64_t)K;
    if (layout == PEG_BINNED && (capacity < 1 || (int64_t)E * capacity > kMaxAssign)) return PEG_ERR_BAD_SHAPE;
    const bool need_pad = padded_bins != nullptr || layout == PEG_PADDED;
    if (need_pad && pad_multiple < 1) return PEG_ERR_BAD_SHAPE;
    if (need_pad && total + (int64_t)E * (pad_multiple - 1) > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    if (!bins || (total > 0 && (!indices || !bin_ids))) return PEG_ERR_NULL_ARG;
    if (layout == PEG_PADDED && !padded_bins) return PEG_ERR_NULL_ARG;
    if (!ws || ws_bytes < ws_need(T, K, E)) return PEG_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int items = fused_items(total, K, E);
    const int64_t ntiles = tiles_of(total, items);
    int32_t* counts = reinterpret_cast<int32_t*>(ws);
    if (ntiles > 0) {
        const GateArgs a{logits, T, E, K, gating, normalize ? 1 : 0, top_experts, weights,
                         (int64_t)kBlock * items, ntiles, counts};
        PEG_CHECK(gate(dtype, s, a));
    }
    return prep_place(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids, tokens_per_expert,
                      bins, padded_bins, slot_row, counts, items, s);
}
