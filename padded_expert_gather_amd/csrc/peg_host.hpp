// peg_host.hpp - host-side helpers shared by the launchers: argument checks,
// launch wrapper, row-vector width choice, workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "peg.h"

#define PEG_API extern "C" __attribute__((visibility("default")))

namespace peg {

constexpr int kBlock = 256;        // threads per block of the streaming kernels
constexpr int64_t kMaxAssign = (int64_t(1) << 31) - 1;

inline bool dtype_ok(int32_t dt) { return dt == PEG_F32 || dt == PEG_BF16 || dt == PEG_F16; }
inline int elem_bytes(int32_t dt) { return dt == PEG_F32 ? 4 : 2; }
inline bool layout_ok(int32_t l) { return l == PEG_BINNED || l == PEG_PADDED; }

inline bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

// Largest lane width in {16, 8, 4, 2} that divides the row length in bytes
// and the address of every row buffer; 0 if even the element size fails.
inline int pick_vec(int64_t row_bytes, int eb, const void* a, const void* b, const void* c = nullptr) {
    for (int v = 16; v >= eb; v >>= 1) {
        if (row_bytes % v) continue;
        if (!aligned(a, v) || !aligned(b, v) || (c && !aligned(c, v))) continue;
        return v;
    }
    return 0;
}

// The token kernels give each token WPT waves of a 4-wave block, so a block
// holds 4 / WPT tokens (WPT 8 or 16: a token spans 2 or 4 blocks). Measured
// on MI355X: the gather's choice is below; the combine likes 4, wgrad and
// the combine backward 2 (1 when K <= 2; the per-K values sit with those
// kernels).
#ifndef PEG_COMBINE_WPT
#define PEG_COMBINE_WPT 4
#endif
#ifndef PEG_WGRAD_WPT
#define PEG_WGRAD_WPT 2
#endif
#ifndef PEG_GATHER_WPT_SPLIT
#define PEG_GATHER_WPT_SPLIT 512  // rows of at most this many vectors: 2 waves per token
#endif

// Waves per token of the gather: 2 up to PEG_GATHER_WPT_SPLIT vectors per
// row; above it 8 (a token over 2 blocks) when K <= 2, else 4. Measured
// (gather alone, bf16, HIP events, 3 runs of 40 launches): T4096 H4096 K2
// 19.6 us at 2 against 21.7 at 4 and 24.3 at 8; T16384 H6144 K2 126.7 us at
// 4 against 121.9 at 8; T8192 H7168 E256 K8 161-162 us at 4 against 164 at
// 8; T32768 H3584 K8 395 us at 2, 391 at 4, 416 at 8. PEG_GATHER_WPT (2, 4,
// 8 or 16) overrides the rule.
#ifndef PEG_GATHER_WPT
#define PEG_GATHER_WPT 0
#endif
inline int gather_wpt(int64_t nch, int32_t K) {
    if (PEG_GATHER_WPT > 0) return PEG_GATHER_WPT;
    if (nch <= PEG_GATHER_WPT_SPLIT) return 2;
    return K <= 2 ? 8 : 4;
}

// The gather issues a token row's first loads before its row indices arrive
// when the token waves fit in about two rounds of the chip's wave slots
// (T4096 H4096 K2, 8192 waves: 17.0 against 17.8 us); with more rounds the
// indices' latency is hidden by other waves and the early loads slowed the
// write-bound gathers (T16384 H6144 K2, 131072 waves: 127.8 against 122.1
// us; T32768 H3584 K8: 401.8 against 396.5; T8192 H7168 K8: even).
#ifndef PEG_GATHER_EARLY_WAVES
#define PEG_GATHER_EARLY_WAVES 16384
#endif
inline int32_t gather_early(int64_t T, int wpt) { return T * wpt <= PEG_GATHER_EARLY_WAVES ? 1 : 0; }

template <int WPT>
struct TokenMap {
    static_assert(WPT == 1 || WPT == 2 || WPT == 4 || WPT == 8 || WPT == 16, "waves per token: 1 to 16");
    static constexpr int kTokensPerBlock = (kBlock / 64) / WPT;
};

// A row of nch vectors is split over the wpt waves of its token: each wave
// owns a contiguous slice, rounded up to 8 vectors (128 bytes at 16-byte
// vectors) so that every wave starts on a cache-line boundary.
inline int64_t wave_slice(int64_t nch, int wpt) {
    const int64_t q = (nch + wpt - 1) / wpt;
    return (q + 7) & ~int64_t(7);
}

// Vectors per lane per pass (1, 2 or 4) so that one pass covers a slice
// when it can.
inline int lanes_per_pass(int64_t slice) {
    const int64_t p = (slice + 63) / 64;
    return p <= 1 ? 1 : (p <= 2 ? 2 : 4);
}

// Blocks for T tokens at wpt waves per token (wpt > 4: a token spans
// wpt / 4 blocks).
inline int64_t token_blocks(int64_t T, int wpt) {
    const int64_t waves = T * wpt;
    const int64_t per = kBlock / 64;
    return (waves + per - 1) / per;
}

// Tiles of the routing preparation: 256 threads x ITEMS assignments. The
// per-chunk count table of a tile (4 * ITEMS chunks of 64 x E ints) stays
// within 32 KB of LDS.
// Small inputs take fewer ids per thread (down to 1) until they make at least
// PEG_MIN_TILES tiles, so that more CUs share the work.
#ifndef PEG_MIN_TILES
#define PEG_MIN_TILES 64
#endif
// Ids per thread of a tile are capped at PEG_PREP_ITEMS_MAX. Measured (in
// the step): T32768 K8 E64 14.3 us at 4 against 15.1 at 8; T8192 K8 E256 and
// T4096 K2 E8 move by less than 0.1 us.
#ifndef PEG_PREP_ITEMS_MAX
#define PEG_PREP_ITEMS_MAX 4
#endif
inline int prep_items(int32_t E) {
    const int items = E <= 128 ? 16 : (E <= 256 ? 8 : (E <= 512 ? 4 : 2));
    return items < PEG_PREP_ITEMS_MAX ? items : PEG_PREP_ITEMS_MAX;
}
inline int64_t tiles_of(int64_t total, int items) {
    return (total + (int64_t)kBlock * items - 1) / ((int64_t)kBlock * items);
}
inline int tiled_items(int64_t total, int32_t E) {
    int items = prep_items(E);
    while (items > 1 && tiles_of(total, items) < PEG_MIN_TILES) items >>= 1;
    return items;
}
// Tiles of the gating fused with the histogram: about 128 tokens per tile
// (one pass of a 1024-thread block at 8 lanes per token), so that the
// gating is spread over many blocks.
// (Measured: giving the fused gating route_prep's larger tiles instead costs
// 0.3-3 us.)
inline int fused_items(int64_t total, int32_t K, int32_t E) {
    int items = 1;
    while (items * 2 <= K / 2 && items * 2 <= prep_items(E)) items <<= 1;
    return items < tiled_items(total, E) ? items : tiled_items(total, E);
}
inline int64_t prep_tiles(int64_t total, int32_t E) { return tiles_of(total, tiled_items(total, E)); }

// Workspace: every call uses one region starting at offset 0.
inline size_t ws_need(int64_t T, int32_t K, int32_t E) {
    int64_t total = T * (int64_t)K;
    int64_t ntiles = prep_tiles(total, E);
    const int64_t nfused = K > 0 ? tiles_of(total, fused_items(total, K, E)) : 0;
    if (nfused > ntiles) ntiles = nfused;
    // route_prep (plain or fused with the gating); with row windows the
    // padded bins of E experts sit in front of the table
    size_t tile_counts = (size_t)ntiles * (size_t)E * 4 + (((size_t)E * 4 + 255) & ~size_t(255));
    size_t slots = (size_t)total * 4;                                   // slot_row rebuild
    size_t bitmap = (size_t)((total + 31) / 32) * 4 + 64;               // validation
    size_t need = tile_counts;
    if (slots > need) need = slots;
    if (bitmap > need) need = bitmap;
    need = (need + 255) & ~size_t(255);
    return need < 256 ? 256 : need;
}

// A HIP dispatch holds its size in threads as a 32-bit number: a launch of
// `blocks` blocks of `threads` threads must stay within it.
inline bool grid_fits(int64_t blocks, int64_t threads) {
    return blocks >= 0 && blocks <= (int64_t)0xFFFFFFFF / threads;
}

// Launch through hipLaunchKernel so that the status of this very launch is
// returned (no reliance on the thread's sticky last-error state).
template <typename... KArgs, size_t... I>
inline void fill_argv(std::tuple<KArgs...>& t, void** argv, std::index_sequence<I...>) {
    ((argv[I] = (void*)&std::get<I>(t)), ...);
}

template <typename... KArgs, typename... Args>
inline peg_status launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                         Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) return PEG_OK;
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    fill_argv(vals, argv, std::index_sequence_for<KArgs...>{});
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, s);
    return e == hipSuccess ? PEG_OK : PEG_ERR_LAUNCH;
}

// Rebuilds the assignment -> row map from the sorted routing arrays into the
// workspace (internal; shared by the gathers, the combine and wgrad).
// Placement of the routing preparation from per-tile expert counts
// (counts[tile * E + e], tiles of kBlock * items ids, items one of
// 1, 2, 4, 8, 16): writes indices, bin_ids, tokens_per_expert, bins,
// padded_bins (if non-NULL) and slot_row (if non-NULL). Defined in
// route_prep.hip.
peg_status prep_place(const int32_t* top, int64_t total, int32_t E, int32_t layout, int32_t capacity,
                      int32_t pad_multiple, int32_t* indices, int32_t* bin_ids, int32_t* tpe, int32_t* bins,
                      int32_t* padded_bins, int32_t* slot_row, int32_t* counts, int items, hipStream_t s);

peg_status rebuild_slot_row(int64_t total, int32_t E, int32_t layout, int32_t capacity,
                            const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                            const int32_t* padded_bins, int32_t* slot_row, hipStream_t s);

}  // namespace peg

#define PEG_CHECK(x)                        \
    do {                                    \
        peg_status st_ = (x);               \
        if (st_ != PEG_OK) return st_;      \
    } while (0)
