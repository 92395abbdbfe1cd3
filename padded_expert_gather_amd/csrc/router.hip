// router.hip - router top-k gating on gfx950: per-token scores -> the K
// chosen experts and their weights, the input of route_prep.
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
// g + 2G, ... (CPL <= 32 of them). Each score becomes a 64-bit key,
// (order-preserving image of the float) << 32 | (~expert id), so that one
// unsigned maximum picks the highest score and, on ties, the lowest id. K
// rounds of [lane maximum over its keys, maximum over the group, the owner
// retires the winner] give the K experts in rank order, exactly (no float
// arithmetic decides the selection). Group reductions use DPP lane moves
// (quad permutes, half-row and row mirrors), which are plain VALU
// operations; only groups wider than a 16-lane row also cross rows through
// the LDS crossbar. Result k is kept by lane k % G, so the K outputs of a
// token are written by the group's lanes side by side.
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

// Order-preserving image of a float's value as an unsigned integer: larger
// values give larger images; NaN gives 0, below every number; -0 maps as +0.
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f != f) return 0u;
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) == 0u) b = 0u;  // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of score_key for every key a number gives (0 decodes to NaN).
__device__ __forceinline__ float key_score(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7FC00000u);
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
    const uint64_t o = ((uint64_t)(uint32_t)dpp_read<CTRL>((int)(v >> 32)) << 32) |
                       (uint32_t)dpp_read<CTRL>((int)(uint32_t)v);
    return o > v ? o : v;
}

// Maximum over the G lanes of a group; every lane of it gets the result.
template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t v) {
    v = max_step<kDppQuadXor1>(v);
    v = max_step<kDppQuadXor2>(v);
    v = max_step<kDppHalfMirror>(v);
    if constexpr (G >= 16) v = max_step<kDppRowMirror>(v);
#pragma unroll
    for (int d = 16; d < G; d <<= 1) {
        const uint64_t o = __shfl_xor(v, d, G);
        v = o > v ? o : v;
    }
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

// G lanes per token, CPL scores per lane (E <= G * CPL).
template <int DT, int G, int CPL>
__global__ __launch_bounds__(kBlock) void router_topk_kernel(const void* __restrict__ logits, int64_t T, int32_t E,
                                                             int32_t K, int32_t gating, int32_t normalize,
                                                             int32_t* __restrict__ top_experts,
                                                             float* __restrict__ weights) {
    static_assert(G >= 8 && G <= kWave && (G & (G - 1)) == 0, "group of 8..64 lanes");
    constexpr int TPB = kBlock / G;
    const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / G;
    if (t >= T) return;  // whole groups leave together: reductions stay within live groups
    const int g = threadIdx.x % G;
    uint64_t key[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int e = g + j * G;
        key[j] = e < E ? ((uint64_t)score_key(load_score<DT>(logits, t * E + e)) << 32) |
                             (uint64_t)(0xFFFFFFFFu - (uint32_t)e)
                       : 0ull;
    }
    uint64_t top = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) top = key[j] > top ? key[j] : top;
    top = group_max<G>(top);
    const float m = key_score((uint32_t)(top >> 32));  // the highest score (NaN if every score is)
    // softmax denominator over all E scores
    float denom = 1.0f;
    if (gating == 0) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            if (g + j * G < E) s += expf(key_score((uint32_t)(key[j] >> 32)) - m);
        denom = group_sum<G>(s);
    }
    // Renormalised sigmoid with a negative top score m: every chosen sigmoid
    // carries the factor exp(m), which cancels in the ratio; it is taken out
    // (q = exp(l - m) / (1 + exp(l)) instead of 1 / (1 + exp(-l))) so that
    // exp(-l) cannot overflow fp32 and turn the weights into 0 / 0.
    const bool shifted = gating != 0 && normalize && m < 0.0f;
    // K selection rounds; result k lands in slot k / G of lane k % G.
    int32_t sel_e[CPL];
    float sel_p[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        sel_e[j] = 0;
        sel_p[j] = 0.0f;
    }
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) best = key[j] > best ? key[j] : best;
        best = group_max<G>(best);
        const int32_t e = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
        if (e % G == g) {
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                if (j == e / G) key[j] = 0;
        }
        if (k % G == g) {
            const float l = key_score((uint32_t)(best >> 32));
            float p;
            if (gating == 0) p = expf(l - m) / denom;
            else if (shifted) p = expf(l - m) / (1.0f + expf(l));
            else p = 1.0f / (1.0f + expf(-l));
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                if (j == k / G) {
                    sel_e[j] = e;
                    sel_p[j] = p;
                }
        }
    }
    float sel_sum = 0.0f;
    if (normalize) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) sel_sum += sel_p[j];  // slots past K hold 0
        sel_sum = group_sum<G>(sel_sum);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int k = j * G + g;
        if (k < K) {
            top_experts[t * K + k] = sel_e[j];
            weights[t * K + k] = normalize ? sel_p[j] / sel_sum : sel_p[j];
        }
    }
}

template <int DT, int G, int CPL>
static peg_status router_go(hipStream_t s, const void* logits, int64_t T, int32_t E, int32_t K, int32_t gating,
                            int32_t normalize, int32_t* top, float* w) {
    constexpr int TPB = kBlock / G;
    const dim3 grid((unsigned)((T + TPB - 1) / TPB));
    return launch(router_topk_kernel<DT, G, CPL>, grid, dim3(kBlock), 0, s, logits, T, E, K, gating, normalize, top,
                  w);
}

template <int DT>
static peg_status router_dispatch(hipStream_t s, const void* logits, int64_t T, int32_t E, int32_t K,
                                  int32_t gating, int32_t normalize, int32_t* top, float* w) {
#define PEG_ROUTER(GG, CC) return router_go<DT, GG, CC>(s, logits, T, E, K, gating, normalize, top, w)
    if (E <= 8) PEG_ROUTER(8, 1);
    if (E <= 16) PEG_ROUTER(8, 2);
    if (E <= 32) PEG_ROUTER(8, 4);
    if (E <= 64) PEG_ROUTER(8, 8);
    if (E <= 128) PEG_ROUTER(8, 16);
    if (E <= 256) PEG_ROUTER(8, 32);
    if (E <= 512) PEG_ROUTER(16, 32);
    PEG_ROUTER(32, 32);
#undef PEG_ROUTER
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_router_topk(const void* logits, int32_t dtype, int64_t T, int32_t E, int32_t K,
                                   int32_t gating, int32_t normalize, int32_t* top_experts, float* weights,
                                   void* stream) {
    if (!dtype_ok(dtype) || (gating != PEG_GATING_SOFTMAX && gating != PEG_GATING_SIGMOID))
        return PEG_ERR_BAD_DTYPE;
    if (T < 0 || E < 1 || E > PEG_MAX_EXPERTS || K < 1 || K > E) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / E) return PEG_ERR_BAD_SHAPE;
    if (T > 0 && (!logits || !top_experts || !weights)) return PEG_ERR_NULL_ARG;
    if (!aligned(logits, elem_bytes(dtype)) || !aligned(top_experts, 4) || !aligned(weights, 4))
        return PEG_ERR_ALIGNMENT;
    if (T == 0) return PEG_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int32_t norm = normalize ? 1 : 0;
    if (dtype == PEG_F32) return router_dispatch<PEG_F32>(s, logits, T, E, K, gating, norm, top_experts, weights);
    if (dtype == PEG_BF16) return router_dispatch<PEG_BF16>(s, logits, T, E, K, gating, norm, top_experts, weights);
    return router_dispatch<PEG_F16>(s, logits, T, E, K, gating, norm, top_experts, weights);
}
