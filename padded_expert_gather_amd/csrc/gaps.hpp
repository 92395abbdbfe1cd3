// gaps.hpp - zeroing of the gap rows of an expert tensor: the unused
// capacity of the binned layout ("Build Triton-Ascend Binned MoE Routing",
// Ascend Guardrails: zero-initialised output) and the padding of the padded
// layout ("Build Triton-Ascend Padded MoE Routing", Ascend Guardrails: zero
// gaps). Only gap rows are written, once; each expert's gap is one contiguous
// byte range.
#pragma once

#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

#ifndef PEG_GAP_UNITS
#define PEG_GAP_UNITS 8192  // target vectors zeroed per gap block
#endif
#ifndef PEG_GAP_MAX
#define PEG_GAP_MAX 8192  // most gap blocks per launch
#endif
#ifndef PEG_ZERO_UNROLL
#define PEG_ZERO_UNROLL 4  // zero stores in flight per thread
#endif
#ifndef PEG_NT_STORE_ZERO
#define PEG_NT_STORE_ZERO PEG_NT_STORE  // the nontemporal hint on the zero stores
#endif
constexpr int kZeroUnroll = PEG_ZERO_UNROLL;
// 1: gap chunks dealt to the gap blocks in turn; 0: one contiguous range of
// the gap space per block. Measured: 1 is 3% faster at T32768 H3584 E64 and
// 20% slower at T8192 H7168 E256 (many short padding gaps), so 0 stays.
#ifndef PEG_GAP_STRIDED
#define PEG_GAP_STRIDED 0
#endif

// Where the gap blocks sit in the grid: 0 = after every token block, 1 =
// spread evenly among them (block i is a gap block when floor((i+1)*nz/n)
// steps past floor(i*nz/n), n = all blocks), 2 = before every token block.
// Measured: 1 costs 6-19% against 0, 2 costs 3-17%.
#ifndef PEG_GAP_INTERLEAVE
#define PEG_GAP_INTERLEAVE 0
#endif

// Role of block i of n blocks, nz of them gap blocks: sets *index to its
// gap-block or token-block index and returns whether it zeroes gaps.
__device__ __forceinline__ bool gap_role(int64_t i, int64_t n, int64_t nz, int64_t* index) {
#if PEG_GAP_INTERLEAVE == 1
    const int64_t before = i * nz / n;  // gap blocks among blocks [0, i)
    const bool gap = (i + 1) * nz / n > before;
    *index = gap ? before : i - before;
    return gap;
#elif PEG_GAP_INTERLEAVE == 2
    *index = i < nz ? i : i - nz;
    return i < nz;
#else
    const int64_t tb = n - nz;
    *index = i < tb ? i : i - tb;
    return i >= tb;
#endif
}

// Gap blocks for a tensor of up to max_gap_rows gap rows of nch vectors.
inline int64_t gap_blocks(int64_t max_gap_rows, int64_t nch) {
    const int64_t units = max_gap_rows * nch;
    int64_t b = (units + PEG_GAP_UNITS - 1) / PEG_GAP_UNITS;
    if (b < 1) b = 1;
    if (b > PEG_GAP_MAX) b = PEG_GAP_MAX;
    return b;
}

// Block zb of nz gap blocks zeroes its share of the gap rows of `out`
// (out_rows rows of nch VEC-byte vectors). Binned: expert e's rows
// [e*C + min(count, C), (e+1)*C); padded: [pstart(e) + count, padded_bins[e]).
// With zero_tail, the rows [R, out_rows) past the layout's R rows (E*C, or
// padded_bins[E-1]) are one more gap. Whole block must call it (contains
// barriers).
template <int VEC, bool NT = PEG_NT_STORE_ZERO>
__device__ __forceinline__ void zero_gap_rows(uint8_t* __restrict__ out, int64_t nch, int64_t out_rows,
                                              int32_t layout, int32_t E, int32_t capacity,
                                              const int32_t* __restrict__ bins,
                                              const int32_t* __restrict__ padded_bins, int64_t zb, int64_t nz,
                                              bool zero_tail = false) {
    using V = typename VecOf<VEC>::T;
    // gap g = rows [gstart[g], gstart[g] + glen[g]) for g < NG (expert gaps,
    // then the tail); gpre = exclusive prefix of glen. Rows at or past
    // out_rows are never touched.
    __shared__ int gpre[PEG_MAX_EXPERTS + 2];
    __shared__ int gstart[PEG_MAX_EXPERTS + 1];
    __shared__ int scratch[kBlock / kWave];
    const int NG = E + (zero_tail ? 1 : 0);
    int carry = 0;
    for (int e0 = 0; e0 < NG; e0 += kBlock) {
        const int e = e0 + threadIdx.x;
        int len = 0, start = 0;
        if (zero_tail && e == E) {  // the tail past the layout's rows
            const int64_t s = layout == PEG_BINNED ? (int64_t)E * capacity : (int64_t)padded_bins[E - 1];
            const int64_t g = (s < 0 || s >= out_rows) ? 0 : out_rows - s;
            len = (int)g;
            start = (int)(g > 0 ? s : 0);
        } else if (e < E) {
            int count = bins[e] - (e ? bins[e - 1] : 0);
            count = count < 0 ? 0 : count;
            int64_t s, g;
            if (layout == PEG_BINNED) {
                const int kept = count < capacity ? count : capacity;
                s = (int64_t)e * capacity + kept;
                g = capacity - kept;
            } else {
                const int64_t ps = e ? padded_bins[e - 1] : 0;
                s = ps + count;
                g = (int64_t)padded_bins[e] - s;
            }
            if (g <= 0 || s < 0 || s >= out_rows) g = 0;   // no gap, or it starts past the buffer
            else if (s + g > out_rows) g = out_rows - s;   // gap cut at the end of the buffer
            len = (int)g;
            start = (int)(g > 0 ? s : 0);
        }
        int total;
        int pre = block_exclusive_scan<kBlock>(len, scratch, &total);
        if (e < NG) {
            gpre[e] = carry + pre;
            gstart[e] = start;
        }
        carry += total;
    }
    if (threadIdx.x == 0) gpre[NG] = carry;
    lds_barrier();

    const int64_t units = (int64_t)carry * nch;
    const V z = zero_vec<VEC>();
#if PEG_GAP_STRIDED
    // Chunks of kBlock * kZeroUnroll vectors dealt to the gap blocks in turn
    // (chunk c to block c % nz), so that the blocks running at one time
    // write neighbouring chunks.
    constexpr int64_t kChunk = (int64_t)kBlock * kZeroUnroll;
    const int64_t nchunks = (units + kChunk - 1) / kChunk;
    int e = 0;  // expert of this thread's current unit: units only grow, so e only moves forward
    for (int64_t c = zb; c < nchunks; c += nz) {
#pragma unroll
        for (int j = 0; j < kZeroUnroll; ++j) {
            const int64_t u = c * kChunk + (int64_t)j * kBlock + threadIdx.x;
            if (u >= units) break;
            while ((int64_t)gpre[e + 1] * nch <= u) ++e;
            const int64_t shift = (int64_t)gstart[e] * nch - (int64_t)gpre[e] * nch;
            stream_store<VEC, NT>(out, shift + u, z);
        }
    }
    return;
#endif
    const int64_t lo = units * zb / nz;
    const int64_t hi = units * (zb + 1) / nz;
    if (lo >= hi) return;
    // first gap holding unit lo: last g with gpre[g] * nch <= lo
    int a = 0, b = NG - 1;
    while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if ((int64_t)gpre[mid] * nch <= lo) a = mid;
        else b = mid - 1;
    }
    // walk this block's range one expert gap (a contiguous byte range) at a
    // time, kZeroUnroll stores in flight per thread
    int64_t u0 = lo;
    for (int e = a; u0 < hi && e < NG; ++e) {
        const int64_t seg_end = (int64_t)gpre[e + 1] * nch < hi ? (int64_t)gpre[e + 1] * nch : hi;
        const int64_t shift = (int64_t)gstart[e] * nch - (int64_t)gpre[e] * nch;  // unit -> output vector
        for (int64_t u = u0 + threadIdx.x; u < seg_end; u += (int64_t)kBlock * kZeroUnroll) {
#pragma unroll
            for (int j = 0; j < kZeroUnroll; ++j) {
                const int64_t uu = u + (int64_t)j * kBlock;
                if (uu < seg_end) stream_store<VEC, NT>(out, shift + uu, z);
            }
        }
        u0 = seg_end > u0 ? seg_end : u0;
    }
}

// Gap rows of a binned tensor by a 2-D grid of their own launch: blockIdx.y
// = expert (E: the rows past E*C when the tensor has more), blockIdx.x = a
// chunk of kBlock * V row vectors of that expert's gap, which is one
// contiguous byte range [e*C + min(count, C), (e+1)*C). Each block writes V
// vectors per thread and the blocks of an expert sweep its gap in address
// order: the access pattern of a plain fill, which HBM takes faster than
// the long-lived gap blocks that share a launch with the token rows (T32768
// H3584 E64 C4096: 1.29 GB of gap rows in 205 us, 6.3 TB/s).
// Block (x, e) of the fill: zeroes its chunk x of expert e's gap (e = E:
// the rows past E*C).
template <int VEC, bool NT>
__device__ __forceinline__ void gap_fill_block(uint8_t* __restrict__ out, int64_t nch, int64_t out_rows, int32_t E,
                                               int32_t capacity, const int32_t* __restrict__ bins, int e,
                                               int64_t x, int v) {
    int64_t s, g;
    if (e >= E) {
        s = (int64_t)E * capacity;
        g = out_rows - s;
    } else {
        int count = bins[e] - (e ? bins[e - 1] : 0);
        count = count < 0 ? 0 : (count > capacity ? capacity : count);
        s = (int64_t)e * capacity + count;
        g = capacity - count;
    }
    if (g <= 0 || s < 0 || s >= out_rows) return;
    if (s + g > out_rows) g = out_rows - s;
    const int64_t units = g * nch;
    const int64_t u0 = x * kBlock * v;
    if (u0 >= units) return;
    uint8_t* dst = out + s * nch * VEC;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t u = u0 + j * kBlock + threadIdx.x;
        if (j < v && u < units) stream_store<VEC, NT>(dst, u, zero_vec<VEC>());
    }
}

template <int VEC, int V, bool NT>
__global__ __launch_bounds__(kBlock) void gap_fill_kernel(uint8_t* __restrict__ out, int64_t nch, int64_t out_rows,
                                                          int32_t E, int32_t capacity,
                                                          const int32_t* __restrict__ bins) {
    gap_fill_block<VEC, NT>(out, nch, out_rows, E, capacity, bins, blockIdx.y, blockIdx.x, V);
}

// Binned tensors of at least this many bytes get their gap rows from
// gap_fill_kernel in a launch of its own before the token rows (measured:
// T32768 H3584 E64 C4096 gather 397 -> 359 us, T16384 H6144 E8 C5120 127 ->
// 122 us; the T512 H250 f32 tensor of 1 MB is faster in one launch). The
// same fill blocks placed at the front of the token kernel's own grid took
// 413 us at T32768 H3584 against 320 for the two launches.
#ifndef PEG_GAP_FILL_MIN_BYTES
#define PEG_GAP_FILL_MIN_BYTES (int64_t(128) << 20)
#endif

inline bool use_gap_fill(int32_t layout, int64_t out_rows, int64_t row_bytes, int32_t E) {
    return layout == PEG_BINNED && out_rows * row_bytes >= PEG_GAP_FILL_MIN_BYTES && E < 65535;
}

// Shape of the fill over a binned tensor of out_rows rows of nch vectors:
// gx chunks per expert, ey experts (E, or E + 1 with rows past E*C), v
// vectors per thread: 1 for rows of at most 512 vectors, else 2 (T32768
// H3584: 205 us at 1 against 219 at 2; T16384 H6144: 42 us at 2 against 52
// at 1).
struct GapFillShape {
    int64_t gx;
    int ey, v;
};
inline GapFillShape gap_fill_shape(int64_t nch, int64_t out_rows, int32_t E, int32_t capacity) {
    const int64_t tail = out_rows - (int64_t)E * capacity;
    const int64_t max_rows = tail > capacity ? tail : capacity;
    const int v = nch <= 512 ? 1 : 2;
    const int64_t gx = (max_rows * nch + (int64_t)kBlock * v - 1) / ((int64_t)kBlock * v);
    return GapFillShape{gx > 0 ? gx : 0, E + (tail > 0 ? 1 : 0), v};
}

// Launches gap_fill_kernel over the binned tensor `out` of out_rows rows
// (nch vectors of VEC bytes each); rows past E*C are zeroed too. Stores
// carry the nontemporal hint (3-5% faster here).
template <int VEC>
inline peg_status launch_gap_fill(uint8_t* out, int64_t nch, int64_t out_rows, int32_t E, int32_t capacity,
                                  const int32_t* bins, hipStream_t s) {
    const GapFillShape f = gap_fill_shape(nch, out_rows, E, capacity);
    const int V = f.v;
    const int64_t gx = f.gx;
    if (gx <= 0) return PEG_OK;
    if (!grid_fits(gx, kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)gx, (unsigned)f.ey);
    if (V == 1) return launch(gap_fill_kernel<VEC, 1, true>, grid, dim3(kBlock), 0, s, out, nch, out_rows, E, capacity, bins);
    return launch(gap_fill_kernel<VEC, 2, true>, grid, dim3(kBlock), 0, s, out, nch, out_rows, E, capacity, bins);
}

inline peg_status launch_gap_fill_vec(int vec, uint8_t* out, int64_t nch, int64_t out_rows, int32_t E,
                                      int32_t capacity, const int32_t* bins, hipStream_t s) {
    switch (vec) {
        case 16: return launch_gap_fill<16>(out, nch, out_rows, E, capacity, bins, s);
        case 8: return launch_gap_fill<8>(out, nch, out_rows, E, capacity, bins, s);
        case 4: return launch_gap_fill<4>(out, nch, out_rows, E, capacity, bins, s);
        default: return launch_gap_fill<2>(out, nch, out_rows, E, capacity, bins, s);
    }
}

}  // namespace peg
