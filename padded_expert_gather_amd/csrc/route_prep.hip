// route_prep.hip - routing preparation on gfx950: per-expert histogram,
// inclusive bins / padded bins by wave64 scans, and a stable counting sort
// of the assignment ids by expert.
//
// Sources: "Build Triton-Ascend Padded MoE Routing", Workflow steps 1-3 (sort
// by expert, real cumulative bins, bins of counts rounded up to the padding
// multiple) and Implementation Pattern (row of a sorted position);
// "Build Triton-Ascend Binned MoE Routing", Workflow steps 1-3 (inclusive
// bins, capacity cut-off) and Implementation Pattern.
//
// Three launches, no global atomics, deterministic:
//   1. tile_hist   : one block per tile of 256*ITEMS assignment ids; LDS
//                    histogram of its expert ids -> counts[e][tile].
//   2. tile_scan   : one 1024-thread block; exclusive scan of counts in
//                    expert-major order, which is directly the first sorted
//                    position of (expert e, tile) -> bins, padded_bins.
//   3. tile_place  : every tile re-reads its ids; a wave64 "multisplit"
//                    (ballots over the bits of the expert id) gives each id
//                    its rank among equal ids of its 64-id chunk; per-chunk
//                    counts scanned in LDS give the rank inside the tile.
//                    Position = tile base + chunk prefix + rank, which keeps
//                    ascending assignment id inside each expert (stable).
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

template <int ITEMS>
__global__ __launch_bounds__(kBlock) void tile_hist_kernel(const int32_t* __restrict__ top, int64_t total,
                                                           int32_t E, int64_t ntiles,
                                                           int32_t* __restrict__ counts) {
    __shared__ int hist[PEG_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += kBlock) hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * (kBlock * ITEMS);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        int64_t a = base + j * kBlock + threadIdx.x;
        if (a < total) {
            int v = top[a];
            if ((unsigned)v < (unsigned)E) atomicAdd(&hist[v], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kBlock) counts[(int64_t)e * ntiles + blockIdx.x] = hist[e];
}

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;

__global__ __launch_bounds__(kScanThreads) void tile_scan_kernel(int32_t* __restrict__ counts, int64_t ntiles,
                                                                 int32_t E, int32_t pad_multiple,
                                                                 int32_t* __restrict__ tokens_per_expert,
                                                                 int32_t* __restrict__ bins,
                                                                 int32_t* __restrict__ padded_bins) {
    __shared__ int scratch[kScanThreads / kWave];
    const int64_t L = ntiles * (int64_t)E;
    int carry = 0;
    for (int64_t base = 0; base < L; base += (int64_t)kScanThreads * kScanPer) {
        const int64_t my = base + (int64_t)threadIdx.x * kScanPer;
        int v[kScanPer];
        int s = 0;
#pragma unroll
        for (int i = 0; i < kScanPer; ++i) {
            v[i] = (my + i < L) ? counts[my + i] : 0;
            s += v[i];
        }
        int total;
        int run = carry + block_exclusive_scan<kScanThreads>(s, scratch, &total);
#pragma unroll
        for (int i = 0; i < kScanPer; ++i) {
            if (my + i < L) {
                counts[my + i] = run;  // first sorted position of (expert, tile)
                run += v[i];
            }
        }
        carry += total;
    }
    __syncthreads();  // the bases written above are read by other threads below

    // Inclusive bin end of expert e = first position of expert e+1.
    const int e = threadIdx.x;
    int end_e = 0, end_prev = 0;
    if (e < E && ntiles > 0) {
        end_e = (e + 1 < E) ? counts[(int64_t)(e + 1) * ntiles] : carry;
        end_prev = e > 0 ? counts[(int64_t)e * ntiles] : 0;
    }
    const int count = end_e - end_prev;
    if (e < E) {
        bins[e] = end_e;
        if (tokens_per_expert) tokens_per_expert[e] = count;
    }
    if (padded_bins) {
        int rounded = (e < E) ? ((count + pad_multiple - 1) / pad_multiple) * pad_multiple : 0;
        int total;
        int pre = block_exclusive_scan<kScanThreads>(rounded, scratch, &total);
        if (e < E) padded_bins[e] = pre + rounded;
    }
}

template <int ITEMS>
__global__ __launch_bounds__(kBlock) void tile_place_kernel(
    const int32_t* __restrict__ top, int64_t total, int32_t E, int32_t nbits, const int32_t* __restrict__ base_pos,
    int64_t ntiles, const int32_t* __restrict__ bins, const int32_t* __restrict__ padded_bins, int32_t layout,
    int32_t capacity, int32_t* __restrict__ indices, int32_t* __restrict__ bin_ids, int32_t* __restrict__ slot_row) {
    constexpr int NCH = ITEMS * (kBlock / kWave);  // 64-id chunks per tile
    extern __shared__ int chunk_cnt[];              // [NCH][E]
    for (int i = threadIdx.x; i < NCH * E; i += kBlock) chunk_cnt[i] = 0;
    __syncthreads();

    const int w = threadIdx.x / kWave;
    const int64_t base = (int64_t)blockIdx.x * (kBlock * ITEMS);
    int ex[ITEMS], rank[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = base + j * kBlock + threadIdx.x;
        const int v = a < total ? top[a] : -1;
        const bool valid = (unsigned)v < (unsigned)E;
        uint64_t same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (v >> b) & 1;
            const uint64_t ones = __ballot(valid && bit);
            same &= bit ? ones : ~ones;
        }
        ex[j] = valid ? v : -1;
        rank[j] = __popcll(same & lanes_below());
        if (valid && rank[j] == 0) chunk_cnt[(j * (kBlock / kWave) + w) * E + v] = __popcll(same);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kBlock) {
        int run = 0;
        for (int c = 0; c < NCH; ++c) {
            int t = chunk_cnt[c * E + e];
            chunk_cnt[c * E + e] = run;
            run += t;
        }
    }
    __syncthreads();

    const int n = bins[E - 1];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = base + j * kBlock + threadIdx.x;
        if (a >= total) continue;
        const int e = ex[j];
        if (e >= 0) {
            const int pos = base_pos[(int64_t)e * ntiles + blockIdx.x] +
                            chunk_cnt[(j * (kBlock / kWave) + w) * E + e] + rank[j];
            indices[pos] = (int32_t)a;
            bin_ids[pos] = e;
            if (slot_row) {
                const int offset = pos - (e ? bins[e - 1] : 0);
                int row;
                if (layout == PEG_BINNED) row = offset < capacity ? e * capacity + offset : -1;
                else row = (e ? padded_bins[e - 1] : 0) + offset;
                slot_row[a] = row;
            }
        } else if (slot_row) {
            slot_row[a] = -1;
        }
        if (a >= n) {  // sorted positions past the last valid one
            indices[a] = -1;
            bin_ids[a] = -1;
        }
    }
}

template <int ITEMS>
static peg_status prep_launch(const int32_t* top, int64_t total, int32_t E, int32_t layout, int32_t capacity,
                              int32_t pad_multiple, int32_t* indices, int32_t* bin_ids, int32_t* tpe,
                              int32_t* bins, int32_t* padded_bins, int32_t* slot_row, int32_t* counts,
                              hipStream_t s) {
    const int64_t ntiles = prep_tiles(total, E);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    PEG_CHECK(launch(tile_hist_kernel<ITEMS>, dim3((unsigned)ntiles), dim3(kBlock), 0, s, top, total, E, ntiles,
                     counts));
    PEG_CHECK(launch(tile_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, ntiles, E, pad_multiple, tpe,
                     bins, padded_bins));
    const size_t lds = (size_t)ITEMS * (kBlock / kWave) * E * sizeof(int);
    PEG_CHECK(launch(tile_place_kernel<ITEMS>, dim3((unsigned)ntiles), dim3(kBlock), lds, s, top, total, E,
                     nbits, counts, ntiles, bins, padded_bins, layout, capacity, indices, bin_ids, slot_row));
    return PEG_OK;
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_route_prep(const int32_t* top_experts, int64_t T, int32_t K, int32_t E, int32_t layout,
                                  int32_t capacity, int32_t pad_multiple, int32_t* indices, int32_t* bin_ids,
                                  int32_t* tokens_per_expert, int32_t* bins, int32_t* padded_bins,
                                  int32_t* slot_row, void* ws, size_t ws_bytes, void* stream) {
    if (!layout_ok(layout)) return PEG_ERR_BAD_DTYPE;
    if (T < 0 || K < 1 || E < 1 || E > PEG_MAX_EXPERTS) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / K) return PEG_ERR_BAD_SHAPE;
    const int64_t total = T * (int64_t)K;
    if (layout == PEG_BINNED && capacity < 1) return PEG_ERR_BAD_SHAPE;
    if (layout == PEG_BINNED && (int64_t)E * capacity > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    const bool need_pad = padded_bins != nullptr || layout == PEG_PADDED;
    if (need_pad && pad_multiple < 1) return PEG_ERR_BAD_SHAPE;
    if (need_pad && total + (int64_t)E * (pad_multiple - 1) > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    if (!bins || (total > 0 && (!top_experts || !indices || !bin_ids))) return PEG_ERR_NULL_ARG;
    if (layout == PEG_PADDED && !padded_bins) return PEG_ERR_NULL_ARG;
    if (!ws) return PEG_ERR_WORKSPACE;
    if (ws_bytes < ws_need(T, K, E)) return PEG_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int32_t* counts = reinterpret_cast<int32_t*>(ws);
    const int items = prep_items(E);
    if (items == 8)
        return prep_launch<8>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                              tokens_per_expert, bins, padded_bins, slot_row, counts, s);
    if (items == 4)
        return prep_launch<4>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                              tokens_per_expert, bins, padded_bins, slot_row, counts, s);
    return prep_launch<2>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                          tokens_per_expert, bins, padded_bins, slot_row, counts, s);
}
