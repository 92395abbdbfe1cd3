// compact.hip - dense routing map -> fixed-width routes, and its backward.
//
// Source: "core.transformer.moe.megakernel.mok.route_adapter",
// RoutingMapToIndices and routing_map_to_mok_inputs: the map is the
// authoritative route set; each row is compacted in increasing expert index;
// rows with fewer than topk routes are padded with index -1 and probability
// 0; probabilities come back as float32; the backward scatters the compact
// router gradients back to the dense row.
//
// One wave64 per row: a ballot over 64 experts at a time, the lane's slot is
// the running count plus the popcount of the routed lanes below it.
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

constexpr int kRowsPerBlock = kBlock / kWave;

template <int PDT>
__global__ __launch_bounds__(kBlock) void compact_kernel(const void* __restrict__ probs,
                                                         const uint8_t* __restrict__ rmap, int64_t T, int32_t E,
                                                         int32_t topk, float* __restrict__ probs_out,
                                                         int32_t* __restrict__ route_experts) {
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= T) return;
    const int lane = lane_id();
    const uint8_t* mrow = rmap + row * E;
    float* prow = probs_out + row * topk;
    int32_t* irow = route_experts + row * topk;
    int count = 0;  // wave-uniform
    for (int e0 = 0; e0 < E && count < topk; e0 += kWave) {
        const int e = e0 + lane;
        const bool routed = e < E && mrow[e] != 0;
        const uint64_t mask = __ballot(routed);
        const int slot = count + __popcll(mask & lanes_below());
        if (routed && slot < topk) {
            float p;
            if constexpr (PDT == PEG_F32) p = reinterpret_cast<const float*>(probs)[row * E + e];
            else p = decode<PDT>(reinterpret_cast<const uint16_t*>(probs)[row * E + e]);
            irow[slot] = e;
            prow[slot] = p;
        }
        count += __popcll(mask);
    }
    if (count > topk) count = topk;
    for (int j = count + lane; j < topk; j += kWave) {
        irow[j] = -1;
        prow[j] = 0.0f;
    }
}

__global__ __launch_bounds__(kBlock) void compact_backward_kernel(const float* __restrict__ grad_out,
                                                                  const int32_t* __restrict__ route_experts,
                                                                  int64_t T, int32_t E, int32_t topk,
                                                                  float* __restrict__ grad_dense) {
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= T) return;
    const int lane = lane_id();
    const int32_t* irow = route_experts + row * topk;
    const float* grow = grad_out + row * topk;
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        if (e >= E) continue;
        float v = 0.0f;
        for (int j = 0; j < topk; ++j)  // same address for all lanes: broadcast loads
            if (irow[j] == e) v = grow[j];
        grad_dense[row * E + e] = v;
    }
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_routing_map_compact(const void* probs, int32_t probs_dtype, const uint8_t* routing_map,
                                           int64_t T, int32_t E, int32_t topk, float* probs_out,
                                           int32_t* route_experts, void* stream) {
    if (!dtype_ok(probs_dtype)) return PEG_ERR_BAD_DTYPE;
    if (T < 0 || E < 1 || E > PEG_MAX_EXPERTS || topk < 1 || topk > E) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / E) return PEG_ERR_BAD_SHAPE;
    if (T > 0 && (!probs || !routing_map || !probs_out || !route_experts)) return PEG_ERR_NULL_ARG;
    if (!aligned(probs, elem_bytes(probs_dtype)) || !aligned(probs_out, 4) || !aligned(route_experts, 4))
        return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!grid_fits((T + kRowsPerBlock - 1) / kRowsPerBlock, kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)((T + kRowsPerBlock - 1) / kRowsPerBlock));
    if (probs_dtype == PEG_F32)
        return launch(compact_kernel<PEG_F32>, grid, dim3(kBlock), 0, s, probs, routing_map, T, E, topk, probs_out,
                      route_experts);
    if (probs_dtype == PEG_BF16)
        return launch(compact_kernel<PEG_BF16>, grid, dim3(kBlock), 0, s, probs, routing_map, T, E, topk, probs_out,
                      route_experts);
    return launch(compact_kernel<PEG_F16>, grid, dim3(kBlock), 0, s, probs, routing_map, T, E, topk, probs_out,
                  route_experts);
}

PEG_API peg_status peg_routing_map_compact_backward(const float* grad_probs_out, const int32_t* route_experts,
                                                    int64_t T, int32_t E, int32_t topk, float* grad_probs,
                                                    void* stream) {
    if (T < 0 || E < 1 || E > PEG_MAX_EXPERTS || topk < 1 || topk > E) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / E) return PEG_ERR_BAD_SHAPE;
    if (T > 0 && (!grad_probs_out || !route_experts || !grad_probs)) return PEG_ERR_NULL_ARG;
    if (!aligned(grad_probs_out, 4) || !aligned(route_experts, 4) || !aligned(grad_probs, 4))
        return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!grid_fits((T + kRowsPerBlock - 1) / kRowsPerBlock, kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)((T + kRowsPerBlock - 1) / kRowsPerBlock));
    return launch(compact_backward_kernel, grid, dim3(kBlock), 0, s, grad_probs_out, route_experts, T, E, topk,
                  grad_probs);
}
