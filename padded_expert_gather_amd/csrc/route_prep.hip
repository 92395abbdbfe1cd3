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
// Ranking inside a 64-id chunk is a wave64 "multisplit": ballots over the bits
// of the expert id give every lane the mask of lanes holding the same expert;
// its rank is the popcount of that mask below the lane. Every wave owns a
// contiguous run of ids and walks its chunks in order, keeping per-expert
// running counts in LDS; a scan over the waves per expert then gives each
// wave's base. Positions therefore follow ascending assignment id inside
// every expert (a stable sort). No global atomics; the result is
// deterministic.
//
// Paths:
//   small: T*K < 8192 and its count table fits in LDS -> one 1024-thread
//          block does everything (histogram, scans, placement) in one launch;
//   tiled: tiles of 256*ITEMS ids (ITEMS shrinks for small inputs so that
//          there are at least 64 tiles); a histogram launch, then a placement
//          launch in which every block reads the (experts x tiles) count
//          table and derives its own bases (block 0 also writes the bins);
//          when that table is large, a single-block scan launch in between
//          computes the bases once.
#include <atomic>
#include <mutex>

#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

// Mask of the lanes of this wave whose expert id equals this lane's (0 for
// a lane without a valid id): one ballot per bit of the id; a lane keeps the
// lanes that agree with it on every bit.
__device__ __forceinline__ uint64_t same_expert_mask(int v, bool valid, int nbits, int /*E*/) {
    uint64_t same = __builtin_amdgcn_ballot_w64(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (v >> b) & 1;
        const uint64_t ones = __builtin_amdgcn_ballot_w64(bit);
        same &= bit ? ones : ~ones;
    }
    return valid ? same : 0;
}

// Ranks of a wave's ITEMS chunks of 64 ids, the ids in order (chunk j, lane
// l): rank[j] = lanes below this one with the same expert in chunk j;
// pre[j] = ids of the same expert in the wave's earlier chunks, read from the
// wave's running counts wcnt[E] in LDS (all lanes read, then the first lane
// of each expert adds the chunk's count; a wave's LDS operations complete in
// order, so the next chunk reads the updated counts). wcnt ends holding the
// wave's totals. Invalid ids (outside [0, E)) become -1 and are not counted.
template <int ITEMS>
__device__ __forceinline__ void wave_ranks(int (&v)[ITEMS], int E, int nbits, int* wcnt, int (&rank)[ITEMS],
                                           int (&pre)[ITEMS]) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const bool valid = (unsigned)v[j] < (unsigned)E;
        const uint64_t same = same_expert_mask(v[j], valid, nbits, E);
        rank[j] = rank_below(same);
        pre[j] = valid ? wcnt[v[j]] : 0;
        if (valid && rank[j] == 0) wcnt[v[j]] = pre[j] + __popcll(same);
        if (!valid) v[j] = -1;
    }
}

// Exclusive scan over the NW waves of each expert's count, in place in
// wcnt[NW][E] (each entry becomes the ids of that expert in the earlier
// waves); tot[e] (optional) receives the expert's total. One thread per
// expert. Call from the whole block after a barrier; no barrier inside.
template <int NW, int NT>
__device__ __forceinline__ void scan_waves(int* wcnt, int E, int* tot) {
    for (int e = threadIdx.x; e < E; e += NT) {
        int run = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const int c = wcnt[ww * E + e];
            wcnt[ww * E + e] = run;
            run += c;
        }
        if (tot) tot[e] = run;
    }
}

// Row of sorted position pos of expert e ([BIN]/[PAD] Implementation Pattern).
__device__ __forceinline__ int position_row(int layout, int e, int capacity, int offset, int padded_start) {
    if (layout == PEG_BINNED) return offset < capacity ? e * capacity + offset : -1;
    return padded_start + offset;
}

// ---------------------------------------------------------------------------
// Small path: one block of 1024 threads, ITEMS ids per thread.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
// Inputs of 8192 ids and more go to the tiled path: two launches over 32+
// CUs beat one CU from there on (measured 6.7 vs 8.9 us at 8192 ids).
#ifndef PEG_SMALL_MAX_IDS
#define PEG_SMALL_MAX_IDS 8191
#endif
constexpr int64_t kSmallMaxIds = PEG_SMALL_MAX_IDS;
constexpr size_t kSmallMaxTable = 48 * 1024;
constexpr size_t kSmallMaxLds = 64 * 1024 - 512;  // dynamic LDS budget of the small path

// Exclusive scan over experts of `count` (LDS, E <= 1024 entries) by wave 0
// alone: each lane sums a run of consecutive experts, one wave64 scan, then
// the run prefixes. Writes start[e] (and padded starts / bins when asked);
// returns the total through *n_out. Call from wave 0 only.
__device__ __forceinline__ void wave0_bins(const int* count, int E, int pad_multiple, int* start, int* pstart,
                                           int32_t* bins, int32_t* padded_bins, int32_t* tokens_per_expert,
                                           int* n_out) {
    const int lane = lane_id();
    const int per = (E + kWave - 1) / kWave;  // experts per lane
    const int e0 = lane * per;
    int run = 0, prun = 0;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            run += count[e];
            if (padded_bins) prun += ((count[e] + pad_multiple - 1) / pad_multiple) * pad_multiple;
        }
    }
    const int inc = wave_inclusive_scan(run);
    const int pinc = wave_inclusive_scan(prun);
    int pre = inc - run, ppre = pinc - prun;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int c = count[e];
            start[e] = pre;
            bins[e] = pre + c;
            if (tokens_per_expert) tokens_per_expert[e] = c;
            pre += c;
            if (padded_bins) {
                const int r = ((c + pad_multiple - 1) / pad_multiple) * pad_multiple;
                pstart[e] = ppre;
                padded_bins[e] = ppre + r;
                ppre += r;
            }
        }
    }
    if (lane == kWave - 1) *n_out = inc;
}

// STAGE: indices are first scattered into LDS by sorted position, then
// indices and bin_ids are written out with consecutive threads on
// consecutive positions (coalesced), instead of one scattered store per id.
template <int ITEMS, bool STAGE>
__global__ __launch_bounds__(kSmallThreads) void prep_small_kernel(
    const int32_t* __restrict__ top, int64_t total, int32_t E, int32_t nbits, int32_t pad_multiple, int32_t layout,
    int32_t capacity, int32_t* __restrict__ indices, int32_t* __restrict__ bin_ids,
    int32_t* __restrict__ tokens_per_expert, int32_t* __restrict__ bins, int32_t* __restrict__ padded_bins,
    int32_t* __restrict__ slot_row) {
    extern __shared__ int lds[];
    int* wcnt = lds;                       // [kSmallWaves][E] per-wave counts, then wave bases
    int* start = wcnt + kSmallWaves * E;   // [E] first sorted position of each expert
    int* pstart = start + E;               // [E] first padded row of each expert
    int* tot = pstart + E;                 // [E] count of each expert
    int* sidx = tot + E;                   // [total] assignment id by sorted position (STAGE)
    __shared__ int s_n;

    // wave w owns the ids [w * 64 * ITEMS, (w + 1) * 64 * ITEMS); their loads
    // overlap the clearing of the counts
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t wbase = (int64_t)w * (kWave * ITEMS) + lane_id();
    int v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = wbase + j * kWave;
        v[j] = a < total ? top[a] : -1;
    }
    for (int i = threadIdx.x; i < kSmallWaves * E; i += kSmallThreads) wcnt[i] = 0;
    lds_barrier();

    int rank[ITEMS], pre[ITEMS];
    wave_ranks<ITEMS>(v, E, nbits, wcnt + w * E, rank, pre);
    lds_barrier();
    scan_waves<kSmallWaves, kSmallThreads>(wcnt, E, tot);
    lds_barrier();
    if (w == 0) wave0_bins(tot, E, pad_multiple, start, pstart, bins, padded_bins, tokens_per_expert, &s_n);
    lds_barrier();

    const int n = s_n;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = wbase + j * kWave;
        if (a >= total) continue;
        const int e = v[j];
        if (e >= 0) {
            const int pos = start[e] + wcnt[w * E + e] + pre[j] + rank[j];
            if constexpr (STAGE) {
                sidx[pos] = (int)a;
            } else {
                indices[pos] = (int32_t)a;
                bin_ids[pos] = e;
            }
            if (slot_row)
                slot_row[a] = position_row(layout, e, capacity, pos - start[e], padded_bins ? pstart[e] : 0);
        } else if (slot_row) {
            slot_row[a] = -1;
        }
        if constexpr (!STAGE) {
            if (a >= n) {
                indices[a] = -1;
                bin_ids[a] = -1;
            }
        }
    }
    if constexpr (STAGE) {
        lds_barrier();  // the slot_row stores above stay in flight
        int e = 0;  // expert of position p: positions rise with p, so e only moves forward
        for (int64_t p = threadIdx.x; p < total; p += kSmallThreads) {
            if (p < n) {
                while (e + 1 < E && start[e + 1] <= p) ++e;
                indices[p] = sidx[p];
                bin_ids[p] = e;
            } else {
                indices[p] = -1;
                bin_ids[p] = -1;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled path.
// ---------------------------------------------------------------------------

// The expert x tile count table is tile-major: counts[tile * E + e] (a
// tile's counts are one contiguous run, written and read coalesced).
// table_at(k) is the slot of entry k in expert-major order (k = e * ntiles
// + tile), the order in which the sorted positions run.
__device__ __forceinline__ int64_t table_at(int64_t k, int64_t ntiles, int32_t E) {
    const int64_t e = k / ntiles;
    return (k - e * ntiles) * E + e;
}

template <int ITEMS>
__global__ __launch_bounds__(kBlock) void tile_hist_kernel(const int32_t* __restrict__ top, int64_t total,
                                                           int32_t E, int64_t ntiles,
                                                           int32_t* __restrict__ counts) {
    __shared__ int hist[PEG_MAX_EXPERTS];
    const int64_t base = (int64_t)blockIdx.x * (kBlock * ITEMS);
    int v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = base + j * kBlock + threadIdx.x;
        v[j] = a < total ? top[a] : -1;
    }
    for (int e = threadIdx.x; e < E; e += kBlock) hist[e] = 0;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
        if ((unsigned)v[j] < (unsigned)E) atomicAdd(&hist[v[j]], 1);
    lds_barrier();
    for (int e = threadIdx.x; e < E; e += kBlock) counts[(int64_t)blockIdx.x * E + e] = hist[e];
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
            v[i] = (my + i < L) ? counts[table_at(my + i, ntiles, E)] : 0;
            s += v[i];
        }
        int total;
        int run = carry + block_exclusive_scan<kScanThreads>(s, scratch, &total);
#pragma unroll
        for (int i = 0; i < kScanPer; ++i) {
            if (my + i < L) {
                counts[table_at(my + i, ntiles, E)] = run;  // first sorted position of (expert, tile)
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
        end_e = (e + 1 < E) ? counts[e + 1] : carry;  // (tile 0, expert e + 1)
        end_prev = e > 0 ? counts[e] : 0;
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


// Placement of one tile. With bases_ready (after tile_scan_kernel), `counts`
// holds the first sorted position of every (expert, tile) and bins /
// padded_bins are final. Otherwise `counts` holds the tile histograms and
// every block derives its own bases from them (the whole table is small:
// at most kMergedMaxTable ints); block 0 also writes tokens_per_expert,
// bins and padded_bins.
// SB: table loads each placement thread keeps in flight while summing the
// table (1, 4 or 32: about the tiles one thread sums; 64 at once measured
// 16.2 against 14.4 us at T8192 K8 E256). V4: E is a multiple of 4 and a
// thread reads 4 consecutive experts of a tile row in one 16-byte load
// (SB of them in flight: 1, 4 or 16), so that a thread sums a quarter of
// the tiles it would otherwise; at T32768 K8 E64 and T8192 K8 E256 a thread
// then sums 16 tiles in one round of loads instead of 64 in two.
template <int ITEMS, int SB, bool V4>
__global__ __launch_bounds__(kBlock) void tile_place_kernel(
    const int32_t* __restrict__ top, int64_t total, int32_t E, int32_t nbits, const int32_t* __restrict__ counts,
    int64_t ntiles, int32_t bases_ready, int32_t pad_multiple, int32_t layout, int32_t capacity,
    int32_t* __restrict__ indices, int32_t* __restrict__ bin_ids, int32_t* __restrict__ tokens_per_expert,
    int32_t* __restrict__ bins, int32_t* __restrict__ padded_bins, int32_t* __restrict__ slot_row) {
    constexpr int NW = kBlock / kWave;
    extern __shared__ int lds[];
    int* wcnt = lds;              // [NW][E] per-wave counts of this tile, then each wave's base
    int* tbase = wcnt + NW * E;   // [E] first sorted position of (e, this tile)
    int* start = tbase + E;       // [E] first sorted position of e
    int* pstart = start + E;      // [E] first padded row of e
    __shared__ int scratch[NW];
    __shared__ int s_n;

    // wave w owns the tile's ids [w * 64 * ITEMS, (w + 1) * 64 * ITEMS)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t wbase = (int64_t)blockIdx.x * (kBlock * ITEMS) + (int64_t)w * (kWave * ITEMS) + lane_id();
    int v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = wbase + j * kWave;
        v[j] = a < total ? top[a] : -1;
    }
    for (int i = threadIdx.x; i < NW * E; i += kBlock) wcnt[i] = 0;
    if (bases_ready) {
        for (int e = threadIdx.x; e < E; e += kBlock) {
            start[e] = e ? bins[e - 1] : 0;
            tbase[e] = counts[(int64_t)blockIdx.x * E + e];
            pstart[e] = (padded_bins && e) ? padded_bins[e - 1] : 0;
        }
        if (threadIdx.x == 0) s_n = bins[E - 1];
    } else {
        // each expert's total and this tile's offset inside it: the whole
        // expert x tile table is summed by all threads at once, in
        // registers, with one LDS atomic per (expert, thread group)
        // (pstart = totals, tbase = offsets); then scans over the experts
        // give the starts
        for (int e = threadIdx.x; e < E; e += kBlock) {
            tbase[e] = 0;
            pstart[e] = 0;
        }
        lds_barrier();
        if constexpr (V4) {
            // threads in groups of min(E / 4, kBlock): thread j of group g
            // sums experts 4j .. 4j+3 over the tiles g, g + groups, ...
            const int E4 = E / 4;
            const int eslots = E4 <= kBlock ? E4 : kBlock;
            const int groups = kBlock / eslots;
            const int g = threadIdx.x / eslots;
            const int4* rows4 = reinterpret_cast<const int4*>(counts);
            if (g < groups) {
                for (int j = threadIdx.x - g * eslots; j < E4; j += eslots) {
                    int run[4] = {0, 0, 0, 0}, run_before[4] = {0, 0, 0, 0};
                    for (int64_t t0 = g; t0 < ntiles; t0 += (int64_t)groups * SB) {
                        int4 cb[SB];
#pragma unroll
                        for (int q = 0; q < SB; ++q) {
                            const int64_t t = t0 + (int64_t)q * groups;
                            cb[q] = t < ntiles ? rows4[t * E4 + j] : make_int4(0, 0, 0, 0);
                        }
#pragma unroll
                        for (int q = 0; q < SB; ++q) {
                            const bool before = t0 + (int64_t)q * groups < (int64_t)blockIdx.x;
                            run[0] += cb[q].x;
                            run[1] += cb[q].y;
                            run[2] += cb[q].z;
                            run[3] += cb[q].w;
                            if (before) {
                                run_before[0] += cb[q].x;
                                run_before[1] += cb[q].y;
                                run_before[2] += cb[q].z;
                                run_before[3] += cb[q].w;
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (run[i]) atomicAdd(&pstart[4 * j + i], run[i]);
                        if (run_before[i]) atomicAdd(&tbase[4 * j + i], run_before[i]);
                    }
                }
            }
        } else {
            // threads in groups of min(E, kBlock): thread e of group g sums
            // expert e over the tiles g, g + groups, ... (SB loads in flight
            // at a time; each load instruction of a wave reads consecutive
            // experts of one tile: contiguous bytes)
            const int eslots = E <= kBlock ? E : kBlock;
            const int groups = kBlock / eslots;
            const int g = threadIdx.x / eslots;
            if (g < groups) {
                for (int e = threadIdx.x - g * eslots; e < E; e += eslots) {
                    int run = 0, run_before = 0;
                    for (int64_t t0 = g; t0 < ntiles; t0 += (int64_t)groups * SB) {
                        int cb[SB];
#pragma unroll
                        for (int q = 0; q < SB; ++q) {
                            const int64_t t = t0 + (int64_t)q * groups;
                            cb[q] = t < ntiles ? counts[t * E + e] : 0;
                        }
#pragma unroll
                        for (int q = 0; q < SB; ++q) {
                            run += cb[q];
                            run_before += t0 + (int64_t)q * groups < (int64_t)blockIdx.x ? cb[q] : 0;
                        }
                    }
                    if (run) atomicAdd(&pstart[e], run);
                    if (run_before) atomicAdd(&tbase[e], run_before);
                }
            }
        }
        lds_barrier();
        int carry = 0, pcarry = 0;
        for (int e0 = 0; e0 < E; e0 += kBlock) {
            const int e = e0 + threadIdx.x;
            int before = 0, count = 0;
            if (e < E) {  // read before the scan's barriers; written back after them
                count = pstart[e];
                before = tbase[e];
            }
            int sum;
            const int pre = carry + block_exclusive_scan<kBlock>(count, scratch, &sum);
            carry += sum;
            const int rounded = padded_bins ? ((count + pad_multiple - 1) / pad_multiple) * pad_multiple : 0;
            int psum;
            const int ppre = pcarry + block_exclusive_scan<kBlock>(rounded, scratch, &psum);
            pcarry += psum;
            if (e < E) {
                start[e] = pre;
                tbase[e] = pre + before;
                pstart[e] = ppre;
                if (blockIdx.x == 0) {
                    bins[e] = pre + count;
                    if (tokens_per_expert) tokens_per_expert[e] = count;
                    if (padded_bins) padded_bins[e] = ppre + rounded;
                }
            }
        }
        if (threadIdx.x == 0) s_n = carry;
    }
    lds_barrier();  // the cleared counts and the bases above, before the ranks and scans below

    int rank[ITEMS], pre[ITEMS];
    wave_ranks<ITEMS>(v, E, nbits, wcnt + w * E, rank, pre);
    lds_barrier();
    scan_waves<NW, kBlock>(wcnt, E, nullptr);
    lds_barrier();

    const int n = s_n;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int64_t a = wbase + j * kWave;
        if (a >= total) continue;
        const int e = v[j];
        if (e >= 0) {
            const int pos = tbase[e] + wcnt[w * E + e] + pre[j] + rank[j];
            indices[pos] = (int32_t)a;
            bin_ids[pos] = e;
            if (slot_row) slot_row[a] = position_row(layout, e, capacity, pos - start[e], pstart[e]);
        } else if (slot_row) {
            slot_row[a] = -1;
        }
        if (a >= n) {  // sorted positions past the last valid one
            indices[a] = -1;
            bin_ids[a] = -1;
        }
    }
}

static int id_bits(int E) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    return nbits;
}

// Tiles whose histogram table (experts x tiles) is at most this many ints
// skip the separate scan launch: each placement block reads the table.
#ifndef PEG_MERGED_MAX_TABLE
#define PEG_MERGED_MAX_TABLE 16384
#endif
constexpr int64_t kMergedMaxTable = PEG_MERGED_MAX_TABLE;
#ifndef PEG_PLACE_V4
#define PEG_PLACE_V4 1
#endif

template <int ITEMS>
static peg_status place_tiles(const int32_t* top, int64_t total, int32_t E, int32_t layout, int32_t capacity,
                              int32_t pad_multiple, int32_t* indices, int32_t* bin_ids, int32_t* tpe, int32_t* bins,
                              int32_t* padded_bins, int32_t* slot_row, int32_t* counts, hipStream_t s) {
    const int64_t ntiles = tiles_of(total, ITEMS);
    const int32_t merged = ntiles * E <= kMergedMaxTable ? 1 : 0;
    if (!merged || ntiles == 0)
        PEG_CHECK(launch(tile_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, ntiles, E, pad_multiple, tpe,
                         bins, padded_bins));
    if (ntiles == 0) return PEG_OK;
    const size_t lds = ((size_t)(kBlock / kWave) * E + 3 * (size_t)E) * sizeof(int);
#define PEG_PLACE_LAUNCH(SB, V4)                                                                                \
    return launch(tile_place_kernel<ITEMS, SB, V4>, dim3((unsigned)ntiles), dim3(kBlock), lds, s, top, total,   \
                  E, id_bits(E), counts, ntiles, merged ? 0 : 1, pad_multiple, layout, capacity, indices, bin_ids,  \
                  tpe, bins, padded_bins, slot_row)
    const int64_t groups = kBlock / (E <= kBlock ? E : kBlock);
    const int64_t per = merged ? (ntiles + groups - 1) / groups : 1;  // tiles one thread sums
    // 16-byte table loads when a thread would sum more than 4 tiles and every
    // tile row starts 16-byte aligned (T32768 K8 E64: route_prep 14.3 ->
    // 12.9 us, T8192 K8 E256: 14.5 -> 12.6; with E = 8, 1-2 tiles per
    // thread, the 4-byte loads stay: 8.5 against 9.2 us for the fused gating
    // at T16384 K2)
    if (per > 4 && PEG_PLACE_V4 && E % 4 == 0 && (reinterpret_cast<uintptr_t>(counts) & 15) == 0) {
        const int64_t groups4 = kBlock / (E / 4 <= kBlock ? E / 4 : kBlock);
        const int64_t per4 = (ntiles + groups4 - 1) / groups4;
        if (per4 <= 1) PEG_PLACE_LAUNCH(1, true);
        if (per4 <= 4) PEG_PLACE_LAUNCH(4, true);
        PEG_PLACE_LAUNCH(16, true);
    }
    if (per <= 1) PEG_PLACE_LAUNCH(1, false);
    if (per <= 4) PEG_PLACE_LAUNCH(4, false);
    PEG_PLACE_LAUNCH(32, false);
#undef PEG_PLACE_LAUNCH
}

template <int ITEMS>
static peg_status prep_tiled(const int32_t* top, int64_t total, int32_t E, int32_t layout, int32_t capacity,
                             int32_t pad_multiple, int32_t* indices, int32_t* bin_ids, int32_t* tpe, int32_t* bins,
                             int32_t* padded_bins, int32_t* slot_row, int32_t* counts, hipStream_t s) {
    const int64_t ntiles = tiles_of(total, ITEMS);
    if (ntiles > 0)
        PEG_CHECK(launch(tile_hist_kernel<ITEMS>, dim3((unsigned)ntiles), dim3(kBlock), 0, s, top, total, E, ntiles,
                         counts));
    return place_tiles<ITEMS>(top, total, E, layout, capacity, pad_multiple, indices, bin_ids, tpe, bins,
                              padded_bins, slot_row, counts, s);
}

template <int ITEMS>
static peg_status prep_small(const int32_t* top, int64_t total, int32_t E, int32_t layout, int32_t capacity,
                             int32_t pad_multiple, int32_t* indices, int32_t* bin_ids, int32_t* tpe, int32_t* bins,
                             int32_t* padded_bins, int32_t* slot_row, hipStream_t s) {
    const size_t base = ((size_t)kSmallWaves * E + 3 * (size_t)E) * sizeof(int);
    const size_t staged = base + (size_t)total * sizeof(int);
    if (staged <= kSmallMaxLds)
        return launch(prep_small_kernel<ITEMS, true>, dim3(1), dim3(kSmallThreads), staged, s, top, total, E,
                      id_bits(E), pad_multiple, layout, capacity, indices, bin_ids, tpe, bins, padded_bins, slot_row);
    return launch(prep_small_kernel<ITEMS, false>, dim3(1), dim3(kSmallThreads), base, s, top, total, E, id_bits(E),
                  pad_multiple, layout, capacity, indices, bin_ids, tpe, bins, padded_bins, slot_row);
}

// Ids per thread of the small path, 0 if it does not apply.
static int small_items(int64_t total, int32_t E) {
    if (total > kSmallMaxIds) return 0;
    int items = 1;
    while ((int64_t)items * kSmallThreads < total) items <<= 1;
    if ((size_t)kSmallWaves * E * sizeof(int) > kSmallMaxTable) return 0;
    return items;
}

// Scratch bytes that prep_dispatch uses for these sizes: none on the
// small path, the (experts x tiles) count table on the tiled path.
static size_t prep_scratch_bytes(int64_t total, int32_t E) {
    if (small_items(total, E)) return 0;
    return (size_t)prep_tiles(total, E) * (size_t)E * sizeof(int32_t);
}

// Everything of peg_route_prep after its argument checks; counts: the
// workspace.
static peg_status prep_dispatch(const int32_t* top_experts, int64_t total, int32_t E, int32_t layout,
                                int32_t capacity, int32_t pad_multiple, int32_t* indices, int32_t* bin_ids,
                                int32_t* tokens_per_expert, int32_t* bins, int32_t* padded_bins, int32_t* slot_row,
                                int32_t* counts, hipStream_t s) {
    switch (small_items(total, E)) {
        case 1: return prep_small<1>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                                     tokens_per_expert, bins, padded_bins, slot_row, s);
        case 2: return prep_small<2>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                                     tokens_per_expert, bins, padded_bins, slot_row, s);
        case 4: return prep_small<4>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                                     tokens_per_expert, bins, padded_bins, slot_row, s);
        case 8: return prep_small<8>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                                     tokens_per_expert, bins, padded_bins, slot_row, s);
        case 16: return prep_small<16>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,
                                       tokens_per_expert, bins, padded_bins, slot_row, s);
        default: break;
    }
    switch (tiled_items(total, E)) {
#define PEG_TILED(I)                                                                                             \
    case I:                                                                                                      \
        return prep_tiled<I>(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids,            \
                             tokens_per_expert, bins, padded_bins, slot_row, counts, s)
        PEG_TILED(16);
        PEG_TILED(8);
        PEG_TILED(4);
        PEG_TILED(2);
        PEG_TILED(1);
#undef PEG_TILED
        default: return PEG_ERR_BAD_SHAPE;
    }
}

peg_status prep_place(const int32_t* top, int64_t total, int32_t E, int32_t layout, int32_t capacity,
                      int32_t pad_multiple, int32_t* indices, int32_t* bin_ids, int32_t* tpe, int32_t* bins,
                      int32_t* padded_bins, int32_t* slot_row, int32_t* counts, int items, hipStream_t s) {
    switch (items) {
#define PEG_PLACE(I)                                                                                             \
    case I:                                                                                                      \
        return place_tiles<I>(top, total, E, layout, capacity, pad_multiple, indices, bin_ids, tpe, bins,        \
                              padded_bins, slot_row, counts, s)
        PEG_PLACE(16);
        PEG_PLACE(8);
        PEG_PLACE(4);
        PEG_PLACE(2);
        PEG_PLACE(1);
#undef PEG_PLACE
        default: return PEG_ERR_BAD_SHAPE;
    }
}

// Rows within caller-given windows: slot_row arrives holding each
// assignment's sorted position (the routing of the padded layout with a
// multiple of 1, whose segments are the real ones), and leaves holding
// row_base[e] + (position - start(e)), or -1 past row_limit[e].
__global__ __launch_bounds__(kBlock) void windows_kernel(const int32_t* __restrict__ top, int64_t total, int32_t E,
                                                         const int32_t* __restrict__ bins,
                                                         const int32_t* __restrict__ row_base,
                                                         const int32_t* __restrict__ row_limit,
                                                         int32_t* __restrict__ slot_row) {
    const int64_t a = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (a >= total) return;
    const int e = top[a];
    const int pos = slot_row[a];
    int row = -1;
    if ((unsigned)e < (unsigned)E && pos >= 0) {
        const int64_t r = (int64_t)row_base[e] + (pos - (e ? bins[e - 1] : 0));
        row = (r >= 0 && r < row_limit[e]) ? (int)r : -1;
    }
    slot_row[a] = row;
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
    return prep_dispatch(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids, tokens_per_expert,
                         bins, padded_bins, slot_row, reinterpret_cast<int32_t*>(ws),
                         reinterpret_cast<hipStream_t>(stream));
}

PEG_API peg_status peg_route_prep_windows(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                                          const int32_t* row_base, const int32_t* row_limit, int32_t* indices,
                                          int32_t* bin_ids, int32_t* tokens_per_expert, int32_t* bins,
                                          int32_t* slot_row, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || K < 1 || E < 1 || E > PEG_MAX_EXPERTS) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / K) return PEG_ERR_BAD_SHAPE;
    const int64_t total = T * (int64_t)K;
    if (!bins || (total > 0 && (!top_experts || !indices || !bin_ids || !slot_row || !row_base || !row_limit)))
        return PEG_ERR_NULL_ARG;
    if (!ws || ws_bytes < ws_need(T, K, E)) return PEG_ERR_WORKSPACE;
    // the padded bins of the multiple-1 routing go first in the workspace,
    // the routing preparation's own scratch after them
    const size_t pb_bytes = ((size_t)E * sizeof(int32_t) + 255) & ~size_t(255);
    int32_t* pb = reinterpret_cast<int32_t*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(ws) + pb_bytes);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PEG_CHECK(prep_dispatch(top_experts, total, E, PEG_PADDED, 0, 1, indices, bin_ids, tokens_per_expert, bins, pb,
                            slot_row, counts, s));
    if (total == 0) return PEG_OK;
    return launch(windows_kernel, dim3((unsigned)((total + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, top_experts,
                  total, E, bins, row_base, row_limit, slot_row);
}

// ---------------------------------------------------------------------------
// Allocation-free routing preparation.
// ---------------------------------------------------------------------------

// The count table of peg_route_prep_noalloc lives in this array: device
// memory of the library, one copy per GPU the library runs on, held until
// the process ends. Host code never uses the array's name as an address (on
// the host it names a stand-in): the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
static __device__ __align__(256) uint8_t scratch[PEG_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (resolved on the first
// call for that device).
peg_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PEG_ERR_LAUNCH;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PEG_ERR_LAUNCH;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PEG_OK;
}
}  // namespace

PEG_API peg_status peg_route_prep_noalloc(const int32_t* top_experts, int64_t T, int32_t K, int32_t E,
                                          int32_t layout, int32_t capacity, int32_t pad_multiple,
                                          int32_t* indices, int32_t* bin_ids, int32_t* tokens_per_expert,
                                          int32_t* bins, int32_t* padded_bins, int32_t* slot_row, void* stream) {
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
    if (prep_scratch_bytes(total, E) > (size_t)PEG_NOALLOC_SCRATCH_BYTES) return PEG_ERR_SCRATCH_LIMIT;
    void* counts = nullptr;
    PEG_CHECK(scratch_address(&counts));
    return prep_dispatch(top_experts, total, E, layout, capacity, pad_multiple, indices, bin_ids, tokens_per_expert,
                         bins, padded_bins, slot_row, reinterpret_cast<int32_t*>(counts),
                         reinterpret_cast<hipStream_t>(stream));
}
