// gather.hip - dispatch of token rows into the expert tensor (binned
// [E, C, H] or padded [padded_bins[E-1], H]) on gfx950.
//
// What is computed ("Build Triton-Ascend Binned MoE Routing": Goal, Workflow
// step 3, Implementation Pattern, Ascend Guardrails; "Build Triton-Ascend
// Padded MoE Routing": Workflow steps 4-5, Implementation Pattern, Ascend
// Guardrails): every kept sorted position copies token indices[i] / TOP_K
// into its row; every other row of the tensor is zero.
//
// How (MI355X design, not the pages' Ascend sub-block buffering):
//   * token-major: the waves of a token read its row once from HBM into
//     VGPRs (16-byte lanes) and store it to each of its <= K rows, so the
//     source is read exactly once however many experts it goes to; each wave
//     owns a contiguous slice of the row;
//   * the rows of a token come from the assignment -> row map (slot_row) by
//     wave-uniform scalar loads, so the row loads issue at once, with no LDS
//     staging or barrier in front of them;
//   * trailing "gap" blocks of the same launch write zeros into the unused
//     capacity / padding rows only (each gap of an expert is one contiguous
//     byte range), so no row is written twice and no memset pass is needed;
//     a large binned tensor gets its gap rows from a fill-shaped launch of
//     their own just before (gap_fill_kernel).
#include "gaps.hpp"
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

// The columns of a token row are split into WPT contiguous slices, one per
// wave; a wave moves its slice in passes of 64 lanes x U vectors.
template <int VEC, int U, int WPT>
__global__ __launch_bounds__(kBlock) void gather_kernel(
    const uint8_t* __restrict__ x, uint8_t* __restrict__ out, int64_t nch, int64_t slice, int32_t K,
    const int32_t* __restrict__ slot_row, int64_t out_rows, int32_t layout, int32_t E, int32_t capacity,
    const int32_t* __restrict__ bins, const int32_t* __restrict__ padded_bins, int64_t T, int64_t token_blocks,
    uint32_t* __restrict__ err_flag, int32_t early) {
    using V = typename VecOf<VEC>::T;
    const int64_t row_bytes = nch * VEC;

    int64_t role_index;
    const int64_t nz = (int64_t)gridDim.x - token_blocks;
    if (!gap_role(blockIdx.x, gridDim.x, nz, &role_index)) {
        // ---------------- token row -> its expert rows ----------------
        // (no barrier in this part: waves run independently)
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        const int64_t gw = xcd_block(role_index, token_blocks) * (kBlock / kWave) + w;  // wave of the launch
        const int64_t t = gw / WPT;
        if (t >= T) return;
        const int lane = lane_id();
        const int64_t c_begin = (gw % WPT) * slice;
        const int64_t c_end = c_begin + slice < nch ? c_begin + slice : nch;
        const int32_t* my_rows = slot_row + t * K;
        const uint8_t* src = x + t * row_bytes;
        // early: the first pass's token-row loads go out before the row
        // indices arrive (they do not depend on them), so the two latencies
        // overlap; otherwise they wait for the indices, and a token whose
        // routes are all dropped is never read
        int64_t c0 = c_begin;
        V v[U];
        if (early) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u * kWave + lane;
                if (c < c_end) v[u] = stream_load<VEC>(src, c);
            }
        }
        // rows of the token: wave-uniform loads (scalar unit), K <= 8 kept in SGPRs
        int r8[kRowsFast];
#pragma unroll
        for (int k = 0; k < kRowsFast; ++k) r8[k] = k < K ? my_rows[k] : -1;
        bool any = false, over = false;
#pragma unroll
        for (int k = 0; k < kRowsFast; ++k) {
            if (r8[k] >= out_rows) over = true;
            any |= r8[k] >= 0 && r8[k] < out_rows;
        }
        for (int k = kRowsFast; k < K; ++k) {
            const int r = my_rows[k];
            if (r >= out_rows) over = true;
            any |= r >= 0 && r < out_rows;
        }
        if (over && err_flag && lane == 0 && gw % WPT == 0) atomicOr(err_flag, PEG_FLAG_OUT_ROWS);
        if (!any) return;  // token fully dropped: nothing is stored
        if (!early) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u * kWave + lane;
                if (c < c_end) v[u] = stream_load<VEC>(src, c);
            }
        }
        for (;;) {
#pragma unroll
            for (int k = 0; k < kRowsFast; ++k) {
                const int r = r8[k];
                if (r < 0 || r >= out_rows) continue;
                uint8_t* dst = out + (int64_t)r * row_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t c = c0 + u * kWave + lane;
                    if (c < c_end) stream_store<VEC>(dst, c, v[u]);
                }
            }
            for (int k = kRowsFast; k < K; ++k) {
                const int r = my_rows[k];
                if (r < 0 || r >= out_rows) continue;
                uint8_t* dst = out + (int64_t)r * row_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t c = c0 + u * kWave + lane;
                    if (c < c_end) stream_store<VEC>(dst, c, v[u]);
                }
            }
            c0 += (int64_t)kWave * U;
            if (c0 >= c_end) break;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u * kWave + lane;
                if (c < c_end) v[u] = stream_load<VEC>(src, c);
            }
        }
        return;
    }

    // ---------------- zero the gap rows ----------------
    zero_gap_rows<VEC>(out, nch, out_rows, layout, E, capacity, bins, padded_bins, role_index, nz);
}

struct GatherArgs {
    const uint8_t* x;
    uint8_t* out;
    int64_t nch, slice;
    int32_t K;
    const int32_t* slot_row;
    int64_t out_rows;
    int32_t layout, E, capacity;
    const int32_t* bins;
    const int32_t* padded_bins;
    int64_t T, token_blocks;
    uint32_t* err_flag;
    int32_t early;
};

template <int VEC, int WPT>
static peg_status gather_launch(int u, dim3 grid, hipStream_t s, const GatherArgs& a) {
#define PEG_GATHER_U(UU)                                                                                        \
    return launch(gather_kernel<VEC, UU, WPT>, grid, dim3(kBlock), 0, s, a.x, a.out, a.nch, a.slice, a.K,   \
                  a.slot_row, a.out_rows, a.layout, a.E, a.capacity, a.bins, a.padded_bins, a.T, a.token_blocks, \
                  a.err_flag, a.early)
    if (u == 1) PEG_GATHER_U(1);
    if (u == 2) PEG_GATHER_U(2);
    PEG_GATHER_U(4);
#undef PEG_GATHER_U
}

template <int WPT>
static peg_status gather_vec(int vec, int u, dim3 grid, hipStream_t s, const GatherArgs& a) {
    switch (vec) {
        case 16: return gather_launch<16, WPT>(u, grid, s, a);
        case 8: return gather_launch<8, WPT>(u, grid, s, a);
        case 4: return gather_launch<4, WPT>(u, grid, s, a);
        default: return gather_launch<2, WPT>(u, grid, s, a);
    }
}

// Waves per token 2, 4 and 8 are built; 16 only when PEG_GATHER_WPT asks for it.
static peg_status gather_dispatch(int wpt, int vec, int u, dim3 grid, hipStream_t s, const GatherArgs& a) {
    if (wpt == 2) return gather_vec<2>(vec, u, grid, s, a);
    if (wpt == 8) return gather_vec<8>(vec, u, grid, s, a);
#if PEG_GATHER_WPT == 16
    if (wpt == 16) return gather_vec<16>(vec, u, grid, s, a);
#endif
    return gather_vec<4>(vec, u, grid, s, a);
}

static peg_status gather_common(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K, int32_t E,
                                int32_t layout, int32_t capacity, const int32_t* indices, const int32_t* bin_ids,
                                const int32_t* bins, const int32_t* padded_bins, const int32_t* slot_row,
                                void* out, int64_t out_rows, uint32_t* err_flag, void* ws, size_t ws_bytes,
                                void* stream) {
    if (!dtype_ok(dtype)) return PEG_ERR_BAD_DTYPE;
    if (T < 0 || H < 1 || K < 1 || E < 1 || E > PEG_MAX_EXPERTS) return PEG_ERR_BAD_SHAPE;
    if (K > PEG_MAX_EXPERTS || T > kMaxAssign / K || out_rows < 0 || out_rows > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    const int eb = elem_bytes(dtype);
    if (H > (int64_t(1) << 40) / eb) return PEG_ERR_BAD_SHAPE;
    if ((!x && T > 0) || (!out && out_rows > 0) || !bins || (layout == PEG_PADDED && !padded_bins))
        return PEG_ERR_NULL_ARG;
    if (!slot_row && T > 0 && (!indices || !bin_ids)) return PEG_ERR_NULL_ARG;
    const int64_t row_bytes = H * eb;
    if (!aligned(x, eb) || !aligned(out, eb)) return PEG_ERR_ALIGNMENT;
    const int vec = pick_vec(row_bytes, eb, x, out);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    const int64_t total = T * (int64_t)K;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!slot_row) {
        if (!ws) return PEG_ERR_WORKSPACE;
        if (ws_bytes < ws_need(T, K, E)) return PEG_ERR_WORKSPACE;
        int32_t* rebuilt = reinterpret_cast<int32_t*>(ws);
        PEG_CHECK(rebuild_slot_row(total, E, layout, capacity, indices, bin_ids, bins, padded_bins, rebuilt, s));
        slot_row = rebuilt;
    }
    const int64_t nch = row_bytes / vec;
    // large binned tensors: the gap rows in a fill-shaped launch of their own
    // first, then token blocks only; otherwise gap blocks after the token
    // blocks of one launch
    const bool fill = use_gap_fill(layout, out_rows, row_bytes, E);
    const int64_t nz = fill ? 0 : gap_blocks(out_rows, nch);
    const int wpt = gather_wpt(nch, K);
    const int64_t tb = token_blocks(T, wpt);
    if (!grid_fits(tb + nz, kBlock)) return PEG_ERR_BAD_SHAPE;
    if (fill) PEG_CHECK(launch_gap_fill_vec(vec, (uint8_t*)out, nch, out_rows, E, capacity, bins, s));
    const dim3 grid((unsigned)(tb + nz));
    const int64_t slice = wave_slice(nch, wpt);
    const int u = lanes_per_pass(slice);
    const GatherArgs a{(const uint8_t*)x, (uint8_t*)out, nch, slice, K, slot_row, out_rows, layout, E, capacity,
                       bins, padded_bins, T, tb, err_flag, gather_early(T, wpt)};
    return gather_dispatch(wpt, vec, u, grid, s, a);
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_gather_binned(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K, int32_t E,
                                     int32_t capacity, const int32_t* indices, const int32_t* bin_ids,
                                     const int32_t* bins, const int32_t* slot_row, void* out, void* ws,
                                     size_t ws_bytes, void* stream) {
    if (capacity < 1 || E < 1 || (int64_t)E * capacity > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    return gather_common(x, dtype, T, H, K, E, PEG_BINNED, capacity, indices, bin_ids, bins, nullptr, slot_row,
                         out, (int64_t)E * capacity, nullptr, ws, ws_bytes, stream);
}

PEG_API peg_status peg_gather_padded(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K, int32_t E,
                                     const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                                     const int32_t* padded_bins, const int32_t* slot_row, void* out,
                                     int64_t out_rows, uint32_t* err_flag, void* ws, size_t ws_bytes,
                                     void* stream) {
    return gather_common(x, dtype, T, H, K, E, PEG_PADDED, 0, indices, bin_ids, bins, padded_bins, slot_row, out,
                         out_rows, err_flag, ws, ws_bytes, stream);
}

PEG_API peg_status peg_gather_rows(const void* x, int32_t dtype, int64_t T, int64_t H, int32_t K,
                                   const int32_t* slot_row, void* out, int64_t out_rows, uint32_t* err_flag,
                                   void* stream) {
    if (!dtype_ok(dtype)) return PEG_ERR_BAD_DTYPE;
    if (T < 0 || H < 1 || K < 1 || K > PEG_MAX_EXPERTS || T > kMaxAssign / K) return PEG_ERR_BAD_SHAPE;
    if (out_rows < 0 || out_rows > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    const int eb = elem_bytes(dtype);
    if (H > (int64_t(1) << 40) / eb) return PEG_ERR_BAD_SHAPE;
    if (T > 0 && (!x || !slot_row || (!out && out_rows > 0))) return PEG_ERR_NULL_ARG;
    if (!aligned(x, eb) || !aligned(out, eb)) return PEG_ERR_ALIGNMENT;
    const int64_t row_bytes = H * eb;
    const int vec = pick_vec(row_bytes, eb, x, out);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    if (T == 0) return PEG_OK;
    const int64_t nch = row_bytes / vec;
    const int wpt = gather_wpt(nch, K);
    const int64_t tb = token_blocks(T, wpt);
    const int64_t slice = wave_slice(nch, wpt);
    const int u = lanes_per_pass(slice);
    // no gap blocks: the grid holds token blocks only, so the gap arguments
    // are never read
    const GatherArgs a{(const uint8_t*)x, (uint8_t*)out, nch, slice, K, slot_row, out_rows, PEG_BINNED, 1, 1,
                       nullptr, nullptr, T, tb, err_flag, gather_early(T, wpt)};
    if (!grid_fits(tb, kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)tb);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return gather_dispatch(wpt, vec, u, grid, s, a);
}

