// slots.hip - assignment -> expert-tensor row map rebuilt from the sorted
// routing arrays, for callers that bring their own indices / bin_ids / bins.
//
// Row of a sorted position follows the Implementation Pattern of "Build
// Triton-Ascend Binned MoE Routing" (expert*capacity + offset, offsets past
// the capacity dropped) and of "Build Triton-Ascend Padded MoE Routing"
// (padded start + offset). Entries outside their valid range are ignored, so
// malformed arrays never cause an out-of-bounds write.
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

__global__ __launch_bounds__(kBlock) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) p[i] = v;
}

__global__ __launch_bounds__(kBlock) void rebuild_kernel(int64_t total, int32_t E, int32_t layout, int32_t capacity,
                                                         const int32_t* __restrict__ indices,
                                                         const int32_t* __restrict__ bin_ids,
                                                         const int32_t* __restrict__ bins,
                                                         const int32_t* __restrict__ padded_bins,
                                                         int32_t* __restrict__ slot_row) {
    int64_t n = bins[E - 1];
    n = n < 0 ? 0 : (n > total ? total : n);
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
        const int e = bin_ids[i];
        const int a = indices[i];
        if ((unsigned)e >= (unsigned)E || a < 0 || a >= total) continue;
        const int64_t offset = i - (e ? bins[e - 1] : 0);
        int64_t row = -1;
        if (offset >= 0) {
            if (layout == PEG_BINNED) row = offset < capacity ? (int64_t)e * capacity + offset : -1;
            else row = (e ? padded_bins[e - 1] : 0) + offset;
        }
        slot_row[a] = (row >= 0 && row <= 0x7fffffff) ? (int32_t)row : -1;
    }
}

static unsigned grid_for(int64_t n) {
    int64_t b = (n + kBlock - 1) / kBlock;
    if (b > 65536) b = 65536;
    return (unsigned)(b < 1 ? 1 : b);
}

peg_status rebuild_slot_row(int64_t total, int32_t E, int32_t layout, int32_t capacity, const int32_t* indices,
                            const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
                            int32_t* slot_row, hipStream_t s) {
    if (total == 0) return PEG_OK;
    PEG_CHECK(launch(fill_i32_kernel, dim3(grid_for(total)), dim3(kBlock), 0, s, slot_row, total, -1));
    return launch(rebuild_kernel, dim3(grid_for(total)), dim3(kBlock), 0, s, total, E, layout, capacity, indices,
                  bin_ids, bins, padded_bins, slot_row);
}

}  // namespace peg
