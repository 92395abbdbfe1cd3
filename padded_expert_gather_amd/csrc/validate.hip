// validate.hip - on-demand check of the routing preconditions.
//
// Sources: "Build Triton-Ascend Binned MoE Routing", Ascend Guardrails (bins
// monotonic, last bin equal to the number of indices, bin_ids consistent
// with the bin boundaries, unique assignment ids for stores without atomics);
// "Build Triton-Ascend Padded MoE Routing", Ascend Guardrails (padded bins
// monotonic, padded segments no shorter than the real counts).
//
// The expected expert of sorted position i is the number of experts e with
// bins[e] <= i (for monotonic bins: the expert whose segment holds i).
// Uniqueness uses a bitmap of T*K bits in the workspace.
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

__global__ __launch_bounds__(kBlock) void validate_clear_kernel(uint32_t* __restrict__ bitmap, int64_t words,
                                                                uint32_t* __restrict__ flags) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < words; i += (int64_t)gridDim.x * kBlock)
        bitmap[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0;
}

__global__ __launch_bounds__(1024) void validate_bins_kernel(const int32_t* __restrict__ bins,
                                                             const int32_t* __restrict__ padded_bins, int32_t E,
                                                             int64_t n_indices, uint32_t* __restrict__ flags) {
    const int e = threadIdx.x;
    uint32_t f = 0;
    if (e < E) {
        const int64_t prev = e ? bins[e - 1] : 0;
        if (bins[e] < prev) f |= PEG_FLAG_BINS_NOT_MONOTONIC;
        if (padded_bins) {
            const int64_t pprev = e ? padded_bins[e - 1] : 0;
            if (padded_bins[e] < pprev || (int64_t)padded_bins[e] - pprev < (int64_t)bins[e] - prev)
                f |= PEG_FLAG_PADDED_BINS;
        }
        if (e == E - 1 && n_indices >= 0 && (int64_t)bins[e] != n_indices) f |= PEG_FLAG_BINS_TOTAL;
    }
    if (f) atomicOr(flags, f);
}

__global__ __launch_bounds__(kBlock) void validate_positions_kernel(const int32_t* __restrict__ indices,
                                                                    const int32_t* __restrict__ bin_ids,
                                                                    const int32_t* __restrict__ bins, int32_t E,
                                                                    int64_t total, int64_t n_indices,
                                                                    uint32_t* __restrict__ bitmap,
                                                                    uint32_t* __restrict__ flags) {
    __shared__ int sb[PEG_MAX_EXPERTS];
    __shared__ int s_mono;
    if (threadIdx.x == 0) s_mono = 1;
    for (int e = threadIdx.x; e < E; e += kBlock) sb[e] = bins[e];
    __syncthreads();
    for (int e = threadIdx.x + 1; e < E; e += kBlock)
        if (sb[e] < sb[e - 1]) s_mono = 0;
    __syncthreads();
    const bool mono = s_mono != 0;
    int64_t n = n_indices >= 0 ? n_indices : (int64_t)sb[E - 1];
    n = n < 0 ? 0 : (n > total ? total : n);
    uint32_t f = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
        int expect = 0;
        if (mono) {  // first e with sb[e] > i
            int a = 0, b = E;
            while (a < b) {
                const int m = (a + b) >> 1;
                if ((int64_t)sb[m] <= i) a = m + 1;
                else b = m;
            }
            expect = a;
        } else {
            for (int e = 0; e < E; ++e) expect += (int64_t)sb[e] <= i;
        }
        if (bin_ids[i] != expect) f |= PEG_FLAG_BIN_IDS;
        const int a = indices[i];
        if (a < 0 || a >= total) {
            f |= PEG_FLAG_INDICES;
        } else {
            const uint32_t bit = 1u << (a & 31);
            const uint32_t old = atomicOr(&bitmap[a >> 5], bit);
            if (old & bit) f |= PEG_FLAG_INDICES;
        }
    }
    if (f) atomicOr(flags, f);
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_validate_routing(const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                                        const int32_t* padded_bins, int64_t T, int32_t K, int32_t E,
                                        int64_t n_indices, uint32_t* flags, void* ws, size_t ws_bytes,
                                        void* stream) {
    if (T < 0 || K < 1 || E < 1 || E > PEG_MAX_EXPERTS || T > kMaxAssign / K) return PEG_ERR_BAD_SHAPE;
    const int64_t total = T * (int64_t)K;
    if (n_indices > total) return PEG_ERR_BAD_SHAPE;
    if (!bins || !flags || (total > 0 && (!indices || !bin_ids))) return PEG_ERR_NULL_ARG;
    if (!ws || ws_bytes < ws_need(T, K, E)) return PEG_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws);
    const int64_t words = (total + 31) / 32;
    int64_t blocks = (words + kBlock - 1) / kBlock;
    blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
    PEG_CHECK(launch(validate_clear_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, bitmap, words, flags));
    PEG_CHECK(launch(validate_bins_kernel, dim3(1), dim3(1024), 0, s, bins, padded_bins, E, n_indices, flags));
    int64_t pblocks = (total + kBlock - 1) / kBlock;
    pblocks = pblocks < 1 ? 1 : (pblocks > 4096 ? 4096 : pblocks);
    return launch(validate_positions_kernel, dim3((unsigned)pblocks), dim3(kBlock), 0, s, indices, bin_ids, bins, E,
                  total, n_indices, bitmap, flags);
}
