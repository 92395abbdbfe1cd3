// combine.hip - weighted top-k scatter-combine and router-weight gradient
// (wgrad) on gfx950.
//
// What is computed:
//   combine: out[t] = sum over kept k (ascending) of w[t*K+k] * y[row(t*K+k)]
//     ("Build Triton-Ascend Binned MoE Routing", Workflow step 5: load kept
//     rows, scale, reduce the TOP_K slots of a token; "Build Triton-Ascend
//     Padded MoE Routing", Workflow step 6 and Ascend Guardrails: weights
//     indexed by assignment id).
//   wgrad: wgrad[a] = <y[row(a)], grad[a / K]> for kept a, else 0 (Workflow
//     step 6 of both pages; fp32 accumulation per their Ascend Guardrails).
//
//   combine backward: dy[row(a)] = w[a] * dout[a / K] in the expert layout
//     (zero gap rows) and wgrad of dout: in one pass over dout for K <= 2;
//     for larger K a weighted gather of dout into dy, then the wgrad kernel.
//
// How: token-major. The token's rows (and weights) come in by wave-uniform
// scalar loads, and each of the token's waves streams its slice of the H
// columns in 16-byte lanes: every kept expert row is read once, the output
// row (combine) is written once, the gradient row (wgrad) is read once for
// all K dots. Accumulation is fp32 FMA; the wgrad dots finish with a DPP wave
// reduction and a sum over the token's waves in LDS. The kernels are compiled
// for 2 routes per pass (K <= 2: fewer registers, full occupancy) and for 8.
// Rows that are unused capacity, padding or dropped are never read.
#include "gaps.hpp"
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

// The combine loads the vectors of up to PEG_COMBINE_INFLIGHT / U expert
// rows (U vectors per lane each) before it uses them: 16 vectors per lane
// in flight, 4 rows at 4 vectors per lane, 8 rows at 2 (T8192 H7168 K8,
// 2 vectors per lane: 107.0 us at 8 rows against 110.4 at 4; T32768 H3584
// K8, 4 vectors per lane: 155.7 us at 4 rows against 158.7 at 8 rows of 2
// vectors).
#ifndef PEG_COMBINE_INFLIGHT
#define PEG_COMBINE_INFLIGHT 16
#endif
#ifndef PEG_WGRAD_KBATCH
#define PEG_WGRAD_KBATCH 2
#endif
constexpr int kWgradKBatch = PEG_WGRAD_KBATCH;  // the same for wgrad and the combine backward
// Occupancy hint for wgrad / the combine backward (waves per SIMD the
// register allocation must allow); 0 = the compiler's choice.
#ifndef PEG_WGRAD_WAVES
#define PEG_WGRAD_WAVES 0
#endif
#if PEG_WGRAD_WAVES > 0
#define PEG_WGRAD_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PEG_WGRAD_WAVES)))
#else
#define PEG_WGRAD_OCCUPANCY
#endif

// Rows of the expert tensor y; none when y is NULL (a padded tensor of no
// rows), so that no row is read.
__device__ __forceinline__ int64_t expert_rows(const void* y, int64_t static_rows, const int32_t* padded_bins,
                                               int32_t E) {
    if (!y) return 0;
    return padded_bins ? (int64_t)padded_bins[E - 1] : static_rows;
}

// Row of route k of a token, -1 when the route is absent, dropped or outside
// [0, R). Wave-uniform (scalar) loads.
__device__ __forceinline__ int route_row(const int32_t* __restrict__ rows, int k, int K, int64_t R) {
    if (k >= K) return -1;
    const int r = rows[k];
    return (r < 0 || r >= R) ? -1 : r;
}

// The columns of a token row are split into WPT contiguous slices, one per
// wave; a wave covers its slice in passes of 64 lanes x U vectors.
template <int DT, int VEC, int U, int WPT, int KR>
__global__ __launch_bounds__(kBlock) void combine_kernel(const uint8_t* __restrict__ y, uint8_t* __restrict__ out,
                                                         int64_t nch, int64_t slice, int64_t T, int32_t K,
                                                         const int32_t* __restrict__ slot_row,
                                                         const float* __restrict__ weights, int64_t static_rows,
                                                         const int32_t* __restrict__ padded_bins, int32_t E) {
    using L = Lanes<DT, VEC>;
    using V = typename L::V;
    constexpr int N = L::N;
    constexpr int KBU = PEG_COMBINE_INFLIGHT / U > 0 ? PEG_COMBINE_INFLIGHT / U : 1;
    constexpr int KB = KR < KBU ? KR : KBU;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t gw = xcd_block(blockIdx.x, gridDim.x) * (kBlock / kWave) + w;  // wave of the launch
    const int64_t t = gw / WPT;  // WPT 8 or 16: a token spans 2 or 4 blocks
    if (t >= T) return;  // no barrier in this kernel
    const int lane = lane_id();
    const int64_t c_begin = (gw % WPT) * slice;
    const int64_t c_end = c_begin + slice < nch ? c_begin + slice : nch;
    const int64_t R = expert_rows(y, static_rows, padded_bins, E);
    const int32_t* my_rows = slot_row + t * K;
    const float* my_w = weights ? weights + t * K : nullptr;
    int r8[KR];
    float w8[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        r8[k] = route_row(my_rows, k, K, R);
        w8[k] = (my_w && k < K) ? my_w[k] : 1.0f;
    }
    const int64_t row_bytes = nch * VEC;
    uint8_t* dst = out + t * row_bytes;

    for (int64_t c0 = c_begin; c0 < c_end; c0 += (int64_t)kWave * U) {
        float acc[U][N];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < N; ++i) acc[u][i] = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KR; kb += KB) {
            V v[KB][U];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int r = r8[kb + kk];
                if (r < 0) continue;
                const uint8_t* src = y + (int64_t)r * row_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t c = c0 + u * kWave + lane;
                    if (c < c_end) v[kk][u] = stream_load<VEC>(src, c);
                }
            }
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                if (r8[kb + kk] < 0) continue;
                const float wk = w8[kb + kk];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (c0 + u * kWave + lane < c_end) {
                        float f[N];
                        L::unpack(v[kk][u], f);
#pragma unroll
                        for (int i = 0; i < N; ++i) acc[u][i] = fmaf(wk, f[i], acc[u][i]);
                    }
                }
            }
        }
        for (int k = KR; k < K; ++k) {  // routes beyond the first 8, one at a time
            const int r = route_row(my_rows, k, K, R);
            if (r < 0) continue;
            const float wk = my_w ? my_w[k] : 1.0f;
            const uint8_t* src = y + (int64_t)r * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u * kWave + lane;
                if (c < c_end) {
                    float f[N];
                    L::unpack(stream_load<VEC>(src, c), f);
#pragma unroll
                    for (int i = 0; i < N; ++i) acc[u][i] = fmaf(wk, f[i], acc[u][i]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * kWave + lane;
            if (c < c_end) stream_store<VEC, PEG_NT_STORE_COMBINE>(dst, c, L::pack(acc[u]));
        }
    }
}

// wgrad: each wave dots its slice of the token's columns for up to 8 routes
// at a time; partial dots finish with a wave64 butterfly and a sum over the
// token's WPT waves in LDS.
//
// DY != 0 is the backward of the combine fused with wgrad: `grad` is then the
// upstream gradient of the combine output, and while each of its vectors is
// in registers it is also stored into the gradient of the expert tensor, dy,
// at every kept row of the token - scaled by that route's weight (DY == 2)
// or as raw bits (DY == 1). Blocks past token_blocks zero dy's gap rows and
// its rows past the layout's (when dy has more).
template <int DT, int VEC, int U, int WPT, int DY, int KR>
__device__ __forceinline__ void wgrad_body(const uint8_t* __restrict__ y, const uint8_t* __restrict__ grad,
                                           float* __restrict__ wgrad, int64_t nch, int64_t slice, int64_t T,
                                           int32_t K, const int32_t* __restrict__ slot_row, int64_t static_rows,
                                           const int32_t* __restrict__ padded_bins, int32_t E,
                                           const float* __restrict__ weights, uint8_t* __restrict__ dy,
                                           int64_t dy_rows, int32_t layout, int32_t capacity,
                                           const int32_t* __restrict__ bins, int64_t token_blocks) {
    using L = Lanes<DT, VEC>;
    using V = typename L::V;
    constexpr int N = L::N;
    constexpr int NW = kBlock / kWave;
    constexpr int KB = KR < kWgradKBatch ? KR : kWgradKBatch;
    int64_t tblock = blockIdx.x;  // token-block index
    if constexpr (DY != 0) {
        const int64_t nz = (int64_t)gridDim.x - token_blocks;
        int64_t role_index;
        if (gap_role(blockIdx.x, gridDim.x, nz, &role_index)) {
            zero_gap_rows<VEC, PEG_NT_STORE_DY_ZERO>(dy, nch, dy_rows, layout, E, capacity, bins, padded_bins, role_index,
                                                      nz, true);
            return;
        }
        tblock = role_index;
    }
    tblock = xcd_block(tblock, token_blocks);
    __shared__ float red[NW][KR];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int TPB = TokenMap<WPT>::kTokensPerBlock;
    const int64_t t = tblock * TPB + w / WPT;
    const bool active = t < T;  // every wave still takes part in the barriers
    const int lane = lane_id();
    const int64_t c_begin = (w % WPT) * slice;
    const int64_t c_end = c_begin + slice < nch ? c_begin + slice : nch;
    const int64_t R = expert_rows(y, static_rows, padded_bins, E);
    const int32_t* my_rows = slot_row + (active ? t : 0) * K;
    const int64_t row_bytes = nch * VEC;
    const uint8_t* g_row = grad + (active ? t : 0) * row_bytes;

    for (int k0 = 0; k0 < K; k0 += KR) {
        int r8[KR];
        float w8[KR];
        bool any = false;
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            r8[k] = active ? route_row(my_rows, k0 + k, K, R) : -1;
            any |= r8[k] >= 0;
            if constexpr (DY == 2) w8[k] = r8[k] >= 0 ? weights[(active ? t : 0) * K + k0 + k] : 0.0f;
        }
        float acc[KR];
#pragma unroll
        for (int k = 0; k < KR; ++k) acc[k] = 0.0f;
        if (any) {
            for (int64_t c0 = c_begin; c0 < c_end; c0 += (int64_t)kWave * U) {
                V gv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t c = c0 + u * kWave + lane;
                    if (c < c_end) gv[u] = stream_load<VEC>(g_row, c);
                }
#pragma unroll
                for (int kb = 0; kb < KR; kb += KB) {
                    V v[KB][U];
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk) {
                        const int r = r8[kb + kk];
                        if (r < 0) continue;
                        const uint8_t* src = y + (int64_t)r * row_bytes;
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int64_t c = c0 + u * kWave + lane;
                            if (c < c_end) v[kk][u] = stream_load<VEC>(src, c);
                        }
                    }
                    if constexpr (DY != 0) {
                        // dy rows need only dout: they are stored while the
                        // expert rows loaded above are still in flight
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int64_t c = c0 + u * kWave + lane;
                            if (c >= c_end) continue;
                            float g[N];
                            if constexpr (DY == 2) L::unpack(gv[u], g);
#pragma unroll
                            for (int kk = 0; kk < KB; ++kk) {
                                const int r = r8[kb + kk];
                                if (r < 0 || r >= dy_rows) continue;
                                uint8_t* drow = dy + (int64_t)r * row_bytes;
                                if constexpr (DY == 1) {
                                    stream_store<VEC, PEG_NT_STORE_DY>(drow, c, gv[u]);
                                } else {
                                    float o[N];
#pragma unroll
                                    for (int i = 0; i < N; ++i) o[i] = w8[kb + kk] * g[i];
                                    stream_store<VEC, PEG_NT_STORE_DY>(drow, c, L::pack(o));
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int64_t c = c0 + u * kWave + lane;
                        if (c >= c_end) continue;
                        float g[N];
                        L::unpack(gv[u], g);
#pragma unroll
                        for (int kk = 0; kk < KB; ++kk) {
                            if (r8[kb + kk] < 0) continue;
                            float f[N];
                            L::unpack(v[kk][u], f);
#pragma unroll
                            for (int i = 0; i < N; ++i) acc[kb + kk] = fmaf(f[i], g[i], acc[kb + kk]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            if (r8[k] < 0) continue;
            const float s = wave_sum(acc[k]);
            if (lane == 0) red[w][k] = s;
        }
        lds_barrier();
        if (threadIdx.x < TPB * KR) {
            const int tl = threadIdx.x / KR;
            const int k = threadIdx.x % KR;
            const int64_t tt = tblock * TPB + tl;
            if (tt < T && k0 + k < K) {
                float s = 0.0f;
                if (route_row(slot_row + tt * K, k0 + k, K, R) >= 0) {
#pragma unroll
                    for (int i = 0; i < WPT; ++i) s += red[tl * WPT + i][k];
                }
                wgrad[tt * K + k0 + k] = s;  // 0 for dropped or unrouted assignments
            }
        }
        lds_barrier();
    }
}

// Same parameter list for both kernels, so one launcher serves them.
#define PEG_WGRAD_PARAMS                                                                                      \
    const uint8_t *__restrict__ y, const uint8_t *__restrict__ grad, float *__restrict__ wgrad, int64_t nch,  \
        int64_t slice, int64_t T, int32_t K, const int32_t *__restrict__ slot_row, int64_t static_rows,       \
        const int32_t *__restrict__ padded_bins, int32_t E, const float *__restrict__ weights,                \
        uint8_t *__restrict__ dy, int64_t dy_rows, int32_t layout, int32_t capacity,                          \
        const int32_t *__restrict__ bins, int64_t token_blocks
#define PEG_WGRAD_ARGS \
    y, grad, wgrad, nch, slice, T, K, slot_row, static_rows, padded_bins, E, weights, dy, dy_rows, layout, capacity, bins, token_blocks

// KR: routes handled per pass over the row (2 when K <= 2, else 8).
template <int DT, int VEC, int U, int WPT, int KR>
__global__ __launch_bounds__(kBlock) PEG_WGRAD_OCCUPANCY void wgrad_kernel(PEG_WGRAD_PARAMS) {
    wgrad_body<DT, VEC, U, WPT, 0, KR>(PEG_WGRAD_ARGS);
}

// DY: 1 = dy rows are dout rows as bits (no weights), 2 = weighted.
template <int DT, int VEC, int U, int WPT, int DY, int KR>
__global__ __launch_bounds__(kBlock) PEG_WGRAD_OCCUPANCY void combine_backward_kernel(PEG_WGRAD_PARAMS) {
    wgrad_body<DT, VEC, U, WPT, DY, KR>(PEG_WGRAD_ARGS);
}
#undef PEG_WGRAD_PARAMS
#undef PEG_WGRAD_ARGS

// dy of the combine backward as a weighted gather of dout (used for K > 2,
// with wgrad then computed by wgrad_kernel): the WPT waves of a token read
// its dout row once, in slices, and store it into each of its kept rows of
// dy - scaled by the route's weight and rounded once (DY == 2) or as raw
// bits (DY == 1). Blocks past token_blocks zero dy's gap rows and the rows
// past the layout's R.
template <int DT, int VEC, int U, int WPT, int DY>
__global__ __launch_bounds__(kBlock) void dy_gather_kernel(
    const uint8_t* __restrict__ dout, uint8_t* __restrict__ dy, int64_t nch, int64_t slice, int64_t T, int32_t K,
    const int32_t* __restrict__ slot_row, const float* __restrict__ weights, int64_t dy_rows, int32_t layout,
    int32_t E, int32_t capacity, const int32_t* __restrict__ bins, const int32_t* __restrict__ padded_bins,
    int64_t token_blocks) {
    using L = Lanes<DT, VEC>;
    using V = typename L::V;
    constexpr int N = L::N;
    const int64_t nz = (int64_t)gridDim.x - token_blocks;
    int64_t role_index;
    if (gap_role(blockIdx.x, gridDim.x, nz, &role_index)) {
        zero_gap_rows<VEC, PEG_NT_STORE_DY_ZERO>(dy, nch, dy_rows, layout, E, capacity, bins, padded_bins,
                                                  role_index, nz, true);
        return;
    }
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t gw = role_index * (kBlock / kWave) + w;  // wave of the launch
    const int64_t t = gw / WPT;
    if (t >= T) return;  // no barrier in the token part
    const int lane = lane_id();
    const int64_t c_begin = (gw % WPT) * slice;
    const int64_t c_end = c_begin + slice < nch ? c_begin + slice : nch;
    const int32_t* my_rows = slot_row + t * K;
    int r8[kRowsFast];
    float w8[kRowsFast];
    bool any = false;
#pragma unroll
    for (int k = 0; k < kRowsFast; ++k) {
        const int r = k < K ? my_rows[k] : -1;
        r8[k] = (r >= 0 && r < dy_rows) ? r : -1;
        w8[k] = (DY == 2 && r8[k] >= 0) ? weights[t * K + k] : 1.0f;
        any |= r8[k] >= 0;
    }
    for (int k = kRowsFast; k < K; ++k) {
        const int r = my_rows[k];
        any |= r >= 0 && r < dy_rows;
    }
    if (!any) return;  // no kept route: nothing to store
    const int64_t row_bytes = nch * VEC;
    const uint8_t* src = dout + t * row_bytes;
    for (int64_t c0 = c_begin; c0 < c_end; c0 += (int64_t)kWave * U) {
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * kWave + lane;
            if (c < c_end) v[u] = stream_load<VEC>(src, c);
        }
        for (int k = 0; k < K; ++k) {
            int r;
            float wk;
            if (k < kRowsFast) {
                r = r8[k];
                wk = w8[k];
            } else {
                r = my_rows[k];
                r = (r >= 0 && r < dy_rows) ? r : -1;
                wk = (DY == 2 && r >= 0) ? weights[t * K + k] : 1.0f;
            }
            if (r < 0) continue;
            uint8_t* drow = dy + (int64_t)r * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u * kWave + lane;
                if (c >= c_end) continue;
                if constexpr (DY == 1) {
                    stream_store<VEC>(drow, c, v[u]);
                } else {
                    float f[N];
                    L::unpack(v[u], f);
#pragma unroll
                    for (int i = 0; i < N; ++i) f[i] = wk * f[i];
                    stream_store<VEC>(drow, c, L::pack(f));
                }
            }
        }
    }
}

struct RowArgs {
    int64_t static_rows;
    const int32_t* padded_bins;
};

static peg_status check_common(int32_t dtype, int32_t layout, int64_t T, int64_t H, int32_t K, int32_t E,
                               int32_t capacity, const int32_t* padded_bins) {
    if (!dtype_ok(dtype) || !layout_ok(layout)) return PEG_ERR_BAD_DTYPE;
    if (T < 0 || H < 1 || K < 1 || E < 1 || E > PEG_MAX_EXPERTS || K > PEG_MAX_EXPERTS) return PEG_ERR_BAD_SHAPE;
    if (T > kMaxAssign / K) return PEG_ERR_BAD_SHAPE;
    if (H > (int64_t(1) << 40) / elem_bytes(dtype)) return PEG_ERR_BAD_SHAPE;
    if (layout == PEG_BINNED && (capacity < 1 || (int64_t)E * capacity > kMaxAssign)) return PEG_ERR_BAD_SHAPE;
    if (layout == PEG_PADDED && !padded_bins) return PEG_ERR_NULL_ARG;
    return PEG_OK;
}

static peg_status ensure_slots(int64_t T, int32_t K, int32_t E, int32_t layout, int32_t capacity,
                               const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                               const int32_t* padded_bins, const int32_t** slot_row, void* ws, size_t ws_bytes,
                               hipStream_t s) {
    if (*slot_row || T == 0) return PEG_OK;
    if (!indices || !bin_ids || !bins) return PEG_ERR_NULL_ARG;
    if (!ws || ws_bytes < ws_need(T, K, E)) return PEG_ERR_WORKSPACE;
    int32_t* rebuilt = reinterpret_cast<int32_t*>(ws);
    PEG_CHECK(rebuild_slot_row(T * (int64_t)K, E, layout, capacity, indices, bin_ids, bins, padded_bins, rebuilt, s));
    *slot_row = rebuilt;
    return PEG_OK;
}

// Waves per token (WPT) and most vectors per lane per pass (UMAX) of the
// combine and of wgrad / the combine backward, for K <= 2 (the _K2 values)
// and for larger K; measured on the workloads.
#ifndef PEG_COMBINE_UMAX
#define PEG_COMBINE_UMAX 4
#endif
#ifndef PEG_COMBINE_WPT_K2
#define PEG_COMBINE_WPT_K2 PEG_COMBINE_WPT
#endif
#ifndef PEG_COMBINE_UMAX_K2
#define PEG_COMBINE_UMAX_K2 PEG_COMBINE_UMAX
#endif
// K > 2 with rows of at most PEG_COMBINE_SPLIT vectors: PEG_COMBINE_WPT_SHORT
// waves per token, so that a wave still covers about 256 vectors in one pass
// (T32768 H3584 K8: 144.5 us at 2 waves against 150.4 at 4; T8192 H7168
// K8 keeps 4: 104.9 us against 110.9 at 2).
#ifndef PEG_COMBINE_SPLIT
#define PEG_COMBINE_SPLIT 512
#endif
#ifndef PEG_COMBINE_WPT_SHORT
#define PEG_COMBINE_WPT_SHORT 2
#endif
// ... and above it PEG_COMBINE_WPT_LONG (T8192 H7168 K8: 102.8 us at 8 waves,
// a token over two blocks, against 104.9 at 4).
#ifndef PEG_COMBINE_WPT_LONG
#define PEG_COMBINE_WPT_LONG 8
#endif
#ifndef PEG_WGRAD_UMAX
#define PEG_WGRAD_UMAX 2
#endif
// K <= 2 with rows of at most PEG_WGRAD_SPLIT vectors: 4 waves per token
// (T4096 H4096 K2, inside the step: wgrad 15.5 us against 18.4 at 1, the
// combine backward 33.1 against 34.4; with the caches flushed first both
// within 1%).
#ifndef PEG_WGRAD_WPT_K2
#define PEG_WGRAD_WPT_K2 4
#endif
#ifndef PEG_WGRAD_UMAX_K2
#define PEG_WGRAD_UMAX_K2 4
#endif

struct RowShape {
    int wpt, umax;
};
static RowShape combine_shape(int32_t K, int64_t nch) {
    if (K <= 2) return RowShape{PEG_COMBINE_WPT_K2, PEG_COMBINE_UMAX_K2};
    return RowShape{nch <= PEG_COMBINE_SPLIT ? PEG_COMBINE_WPT_SHORT : PEG_COMBINE_WPT_LONG, PEG_COMBINE_UMAX};
}
// K > 2 with rows above PEG_WGRAD_SPLIT vectors: PEG_WGRAD_WPT_LONG waves
// per token (T8192 H7168 K8: wgrad 90.5 us at 4 waves against 94.9 at 2,
// the one-pass combine backward 271.6 against 283.7; T32768 H3584 K8 keeps
// 2: wgrad 121.5 us against 131.5 at 4).
#ifndef PEG_WGRAD_SPLIT
#define PEG_WGRAD_SPLIT 512
#endif
#ifndef PEG_WGRAD_WPT_LONG
#define PEG_WGRAD_WPT_LONG 4
#endif
// The same for K <= 2 above PEG_WGRAD_SPLIT vectors: 2 waves (T16384 H6144
// K2: wgrad 66.5 us against 67.5 at 1, the combine backward 177.1 against
// 181.6).
#ifndef PEG_WGRAD_WPT_K2_LONG
#define PEG_WGRAD_WPT_K2_LONG 2
#endif
static RowShape wgrad_shape(int32_t K, int64_t nch) {
    const bool long_rows = nch > PEG_WGRAD_SPLIT;
    if (K <= 2) return RowShape{long_rows ? PEG_WGRAD_WPT_K2_LONG : PEG_WGRAD_WPT_K2, PEG_WGRAD_UMAX_K2};
    return RowShape{long_rows ? PEG_WGRAD_WPT_LONG : PEG_WGRAD_WPT, PEG_WGRAD_UMAX};
}
#ifndef PEG_BACKWARD_WPT_K2
#define PEG_BACKWARD_WPT_K2 PEG_WGRAD_WPT_K2
#endif
#ifndef PEG_BACKWARD_UMAX_K2
#define PEG_BACKWARD_UMAX_K2 PEG_WGRAD_UMAX_K2
#endif
#ifndef PEG_BACKWARD_WPT
#define PEG_BACKWARD_WPT PEG_WGRAD_WPT
#endif
// The one-pass combine backward with K > 2 (which runs only when
// PEG_BACKWARD_SPLIT_K is raised above 2) keeps 4 vectors per lane per pass
// (T8192 H7168 K8: 250.8 us against 262.2 at 2; T32768 H3584 K8 509.9
// against 511.1).
#ifndef PEG_BACKWARD_UMAX
#define PEG_BACKWARD_UMAX 4
#endif
#ifndef PEG_BACKWARD_WPT_LONG
#define PEG_BACKWARD_WPT_LONG PEG_WGRAD_WPT_LONG
#endif
#ifndef PEG_BACKWARD_WPT_K2_LONG
#define PEG_BACKWARD_WPT_K2_LONG PEG_WGRAD_WPT_K2_LONG
#endif
static RowShape backward_shape(int32_t K, int64_t nch) {
    const bool long_rows = nch > PEG_WGRAD_SPLIT;
    if (K <= 2) return RowShape{long_rows ? PEG_BACKWARD_WPT_K2_LONG : PEG_BACKWARD_WPT_K2, PEG_BACKWARD_UMAX_K2};
    return RowShape{long_rows ? PEG_BACKWARD_WPT_LONG : PEG_BACKWARD_WPT, PEG_BACKWARD_UMAX};
}

// Vectors per lane per pass: 1, 2 or 4, capped.
static int pass_vectors(int64_t slice, int cap) {
    const int u = lanes_per_pass(slice);
    return u < cap ? u : cap;
}

template <int DT, int VEC, int U>
static peg_status combine_go(int wpt, dim3 grid, hipStream_t s, const uint8_t* y, uint8_t* out, int64_t nch,
                             int64_t q, int64_t T, int32_t K, const int32_t* slot_row, const float* w, RowArgs ra,
                             int32_t E) {
#define PEG_COMBINE_LAUNCH(WPT, KR)                                                                            \
    return launch(combine_kernel<DT, VEC, U, WPT, KR>, grid, dim3(kBlock), 0, s, y, out, nch, q, T, K, slot_row, \
                  w, ra.static_rows, ra.padded_bins, E)
    if (K <= 2) PEG_COMBINE_LAUNCH(PEG_COMBINE_WPT_K2, 2);
    if (wpt == PEG_COMBINE_WPT_SHORT) PEG_COMBINE_LAUNCH(PEG_COMBINE_WPT_SHORT, kRowsFast);
    PEG_COMBINE_LAUNCH(PEG_COMBINE_WPT_LONG, kRowsFast);
#undef PEG_COMBINE_LAUNCH
}

template <int DT, int VEC>
static peg_status combine_vec(int wpt, int u, dim3 grid, hipStream_t s, const uint8_t* y, uint8_t* out,
                              int64_t nch, int64_t q, int64_t T, int32_t K, const int32_t* slot_row, const float* w,
                              RowArgs ra, int32_t E) {
    if (u == 1) return combine_go<DT, VEC, 1>(wpt, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
    if (u == 2) return combine_go<DT, VEC, 2>(wpt, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
    return combine_go<DT, VEC, 4>(wpt, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
}

template <int DT>
static peg_status combine_dispatch(int vec, hipStream_t s, const uint8_t* y, uint8_t* out, int64_t nch, int64_t T,
                                   int32_t K, const int32_t* slot_row, const float* w, RowArgs ra, int32_t E) {
    const RowShape sh = combine_shape(K, nch);
    const int64_t q = wave_slice(nch, sh.wpt);
    const int u = pass_vectors(q, sh.umax);
    if (!grid_fits(token_blocks(T, sh.wpt), kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)token_blocks(T, sh.wpt));
    switch (vec) {
        case 16: return combine_vec<DT, 16>(sh.wpt, u, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
        case 8: return combine_vec<DT, 8>(sh.wpt, u, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
        case 4: return combine_vec<DT, 4>(sh.wpt, u, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
        default:
            if constexpr (Elem<DT>::bytes == 2)
                return combine_vec<DT, 2>(sh.wpt, u, grid, s, y, out, nch, q, T, K, slot_row, w, ra, E);
            return PEG_ERR_ALIGNMENT;
    }
}

// Arguments of the wgrad / fused-backward launch.
struct WgradArgs {
    const uint8_t* y;
    const uint8_t* g;
    float* wg;
    int64_t nch, slice, T;
    int32_t K;
    const int32_t* slot_row;
    RowArgs ra;
    int32_t E;
    const float* weights;
    uint8_t* dy;
    int64_t dy_rows;
    int32_t layout, capacity;
    const int32_t* bins;
    int64_t token_blocks;
    int wpt;  // waves per token of the launch
};

template <int DT, int VEC, int U, int DY>
static peg_status wgrad_go(dim3 grid, hipStream_t s, const WgradArgs& a) {
#define PEG_WGRAD_LAUNCH(KERNEL)                                                                                 \
    return launch(KERNEL, grid, dim3(kBlock), 0, s, a.y, a.g, a.wg, a.nch, a.slice, a.T, a.K, a.slot_row,        \
                  a.ra.static_rows, a.ra.padded_bins, a.E, a.weights, a.dy, a.dy_rows, a.layout, a.capacity, a.bins, \
                  a.token_blocks)
    if (a.K <= 2) {
        if constexpr (DY == 0) {
#if PEG_WGRAD_WPT_K2_LONG != PEG_WGRAD_WPT_K2
            if (a.wpt == PEG_WGRAD_WPT_K2_LONG) PEG_WGRAD_LAUNCH((wgrad_kernel<DT, VEC, U, PEG_WGRAD_WPT_K2_LONG, 2>));
#endif
            PEG_WGRAD_LAUNCH((wgrad_kernel<DT, VEC, U, PEG_WGRAD_WPT_K2, 2>));
        } else {
#if PEG_BACKWARD_WPT_K2_LONG != PEG_BACKWARD_WPT_K2
            if (a.wpt == PEG_BACKWARD_WPT_K2_LONG)
                PEG_WGRAD_LAUNCH((combine_backward_kernel<DT, VEC, U, PEG_BACKWARD_WPT_K2_LONG, DY, 2>));
#endif
            PEG_WGRAD_LAUNCH((combine_backward_kernel<DT, VEC, U, PEG_BACKWARD_WPT_K2, DY, 2>));
        }
    }
    if constexpr (DY == 0) {
#if PEG_WGRAD_WPT_LONG != PEG_WGRAD_WPT
        if (a.wpt == PEG_WGRAD_WPT_LONG) PEG_WGRAD_LAUNCH((wgrad_kernel<DT, VEC, U, PEG_WGRAD_WPT_LONG, kRowsFast>));
#endif
        PEG_WGRAD_LAUNCH((wgrad_kernel<DT, VEC, U, PEG_WGRAD_WPT, kRowsFast>));
    } else {
#if PEG_BACKWARD_WPT_LONG != PEG_BACKWARD_WPT
        if (a.wpt == PEG_BACKWARD_WPT_LONG)
            PEG_WGRAD_LAUNCH((combine_backward_kernel<DT, VEC, U, PEG_BACKWARD_WPT_LONG, DY, kRowsFast>));
#endif
        PEG_WGRAD_LAUNCH((combine_backward_kernel<DT, VEC, U, PEG_BACKWARD_WPT, DY, kRowsFast>));
    }
#undef PEG_WGRAD_LAUNCH
}

template <int DT, int VEC, int DY>
static peg_status wgrad_u(int u, dim3 grid, hipStream_t s, const WgradArgs& a) {
    if (u == 1) return wgrad_go<DT, VEC, 1, DY>(grid, s, a);
    if (u == 2) return wgrad_go<DT, VEC, 2, DY>(grid, s, a);
    return wgrad_go<DT, VEC, 4, DY>(grid, s, a);
}

template <int DT, int DY>
static peg_status wgrad_dispatch(int vec, int u, dim3 grid, hipStream_t s, const WgradArgs& a) {
    switch (vec) {
        case 16: return wgrad_u<DT, 16, DY>(u, grid, s, a);
        case 8: return wgrad_u<DT, 8, DY>(u, grid, s, a);
        case 4: return wgrad_u<DT, 4, DY>(u, grid, s, a);
        default:
            if constexpr (Elem<DT>::bytes == 2) return wgrad_u<DT, 2, DY>(u, grid, s, a);
            return PEG_ERR_ALIGNMENT;
    }
}

template <int DY>
static peg_status wgrad_by_dtype(int32_t dtype, int vec, int u, dim3 grid, hipStream_t s, const WgradArgs& a) {
    if (dtype == PEG_F32) return wgrad_dispatch<PEG_F32, DY>(vec, u, grid, s, a);
    if (dtype == PEG_BF16) return wgrad_dispatch<PEG_BF16, DY>(vec, u, grid, s, a);
    return wgrad_dispatch<PEG_F16, DY>(vec, u, grid, s, a);
}

// wgrad_kernel over a valid row map (the launch of peg_wgrad after its
// checks); vec: the row-vector width of y and grad.
static peg_status wgrad_launch(const void* y, const void* grad, int32_t dtype, int vec, int32_t layout, int64_t T,
                               int64_t H, int32_t K, int32_t E, int32_t capacity, const int32_t* bins,
                               const int32_t* padded_bins, const int32_t* slot_row, float* wgrad, hipStream_t s) {
    const RowArgs ra{layout == PEG_BINNED ? (int64_t)E * capacity : 0,
                     layout == PEG_PADDED ? padded_bins : nullptr};
    const int64_t nch = H * elem_bytes(dtype) / vec;
    const RowShape sh = wgrad_shape(K, nch);
    const int64_t q = wave_slice(nch, sh.wpt);
    const int u = pass_vectors(q, sh.umax);
    const int64_t tb = token_blocks(T, sh.wpt);
    const WgradArgs a{(const uint8_t*)y, (const uint8_t*)grad, wgrad, nch, q, T, K, slot_row, ra, E, nullptr,
                      nullptr, 0, layout, capacity, bins, tb, sh.wpt};
    if (!grid_fits(tb, kBlock)) return PEG_ERR_BAD_SHAPE;
    return wgrad_by_dtype<0>(dtype, vec, u, dim3((unsigned)tb), s, a);
}

// Arguments of the dy gather launch.
struct DyArgs {
    const uint8_t* dout;
    uint8_t* dy;
    int64_t nch, slice, T;
    int32_t K;
    const int32_t* slot_row;
    const float* weights;
    int64_t dy_rows;
    int32_t layout, E, capacity;
    const int32_t* bins;
    const int32_t* padded_bins;
    int64_t token_blocks;
};

template <int DT, int VEC, int DY>
static peg_status dy_gather_go(int wpt, int u, dim3 grid, hipStream_t s, const DyArgs& a) {
#define PEG_DY_LAUNCH(WPT, UU)                                                                                  \
    return launch(dy_gather_kernel<DT, VEC, UU, WPT, DY>, grid, dim3(kBlock), 0, s, a.dout, a.dy, a.nch, a.slice, \
                  a.T, a.K, a.slot_row, a.weights, a.dy_rows, a.layout, a.E, a.capacity, a.bins, a.padded_bins,   \
                  a.token_blocks)
    if (wpt == 2) {
        if (u == 1) PEG_DY_LAUNCH(2, 1);
        if (u == 2) PEG_DY_LAUNCH(2, 2);
        PEG_DY_LAUNCH(2, 4);
    }
    if (u == 1) PEG_DY_LAUNCH(4, 1);
    if (u == 2) PEG_DY_LAUNCH(4, 2);
    PEG_DY_LAUNCH(4, 4);
#undef PEG_DY_LAUNCH
}

template <int DT, int DY>
static peg_status dy_gather_vec(int vec, int wpt, int u, dim3 grid, hipStream_t s, const DyArgs& a) {
    switch (vec) {
        case 16: return dy_gather_go<DT, 16, DY>(wpt, u, grid, s, a);
        case 8: return dy_gather_go<DT, 8, DY>(wpt, u, grid, s, a);
        case 4: return dy_gather_go<DT, 4, DY>(wpt, u, grid, s, a);
        default:
            if constexpr (Elem<DT>::bytes == 2) return dy_gather_go<DT, 2, DY>(wpt, u, grid, s, a);
            return PEG_ERR_ALIGNMENT;
    }
}

// dy of the combine backward by dy_gather_kernel, its gap rows zeroed as the
// gather zeroes its own (a fill-shaped launch first for a binned dy of 128 MB
// and more, else trailing gap blocks).
static peg_status dy_gather(const void* dout, const float* weights, int32_t dtype, int vec, int32_t layout,
                            int64_t T, int64_t H, int32_t K, int32_t E, int32_t capacity, const int32_t* bins,
                            const int32_t* padded_bins, const int32_t* slot_row, void* dy, int64_t dy_rows,
                            hipStream_t s) {
    const int64_t row_bytes = H * elem_bytes(dtype);
    const int64_t nch = row_bytes / vec;
    const bool fill = dy_rows > 0 && use_gap_fill(layout, dy_rows, row_bytes, E);
    const int64_t nz = fill ? 0 : gap_blocks(dy_rows, nch);
    const int wpt = nch <= 512 ? 2 : 4;  // waves per token: the gather's for K > 2
    const int64_t tb = token_blocks(T, wpt);
    if (!grid_fits(tb + nz, kBlock)) return PEG_ERR_BAD_SHAPE;
    if (fill) PEG_CHECK(launch_gap_fill_vec(vec, (uint8_t*)dy, nch, dy_rows, E, capacity, bins, s));
    const int64_t slice = wave_slice(nch, wpt);
    const int u = lanes_per_pass(slice);
    const DyArgs a{(const uint8_t*)dout, (uint8_t*)dy, nch, slice, T, K, slot_row, weights, dy_rows, layout, E,
                   capacity, bins, padded_bins, tb};
    const dim3 grid((unsigned)(tb + nz));
    if (weights) {
        if (dtype == PEG_F32) return dy_gather_vec<PEG_F32, 2>(vec, wpt, u, grid, s, a);
        if (dtype == PEG_BF16) return dy_gather_vec<PEG_BF16, 2>(vec, wpt, u, grid, s, a);
        return dy_gather_vec<PEG_F16, 2>(vec, wpt, u, grid, s, a);
    }
    return dy_gather_vec<PEG_BF16, 1>(vec, wpt, u, grid, s, a);  // raw bits: the type plays no part
}

// K above this: the combine backward runs as dy_gather_kernel then
// wgrad_kernel instead of one fused pass.
#ifndef PEG_BACKWARD_SPLIT_K
#define PEG_BACKWARD_SPLIT_K 2
#endif

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_scatter_combine(const void* y, int32_t dtype, int32_t layout, int64_t T, int64_t H,
                                       int32_t K, int32_t E, int32_t capacity, const int32_t* indices,
                                       const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
                                       const int32_t* slot_row, const float* weights, void* out, void* ws,
                                       size_t ws_bytes, void* stream) {
    PEG_CHECK(check_common(dtype, layout, T, H, K, E, capacity, padded_bins));
    if (T > 0 && ((!y && layout == PEG_BINNED) || !out)) return PEG_ERR_NULL_ARG;
    const int eb = elem_bytes(dtype);
    if (!aligned(y, eb) || !aligned(out, eb) || (weights && !aligned(weights, 4))) return PEG_ERR_ALIGNMENT;
    const int vec = pick_vec(H * eb, eb, y, out);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PEG_CHECK(ensure_slots(T, K, E, layout, capacity, indices, bin_ids, bins, padded_bins, &slot_row, ws, ws_bytes, s));
    const RowArgs ra{layout == PEG_BINNED ? (int64_t)E * capacity : 0,
                     layout == PEG_PADDED ? padded_bins : nullptr};
    const int64_t nch = H * eb / vec;
    const uint8_t* yb = (const uint8_t*)y;
    uint8_t* ob = (uint8_t*)out;
    if (dtype == PEG_F32) return combine_dispatch<PEG_F32>(vec, s, yb, ob, nch, T, K, slot_row, weights, ra, E);
    if (dtype == PEG_BF16) return combine_dispatch<PEG_BF16>(vec, s, yb, ob, nch, T, K, slot_row, weights, ra, E);
    return combine_dispatch<PEG_F16>(vec, s, yb, ob, nch, T, K, slot_row, weights, ra, E);
}

PEG_API peg_status peg_wgrad(const void* y, const void* grad, int32_t dtype, int32_t layout, int64_t T, int64_t H,
                             int32_t K, int32_t E, int32_t capacity, const int32_t* indices, const int32_t* bin_ids,
                             const int32_t* bins, const int32_t* padded_bins, const int32_t* slot_row,
                             float* wgrad, void* ws, size_t ws_bytes, void* stream) {
    PEG_CHECK(check_common(dtype, layout, T, H, K, E, capacity, padded_bins));
    if (T > 0 && ((!y && layout == PEG_BINNED) || !grad || !wgrad)) return PEG_ERR_NULL_ARG;
    const int eb = elem_bytes(dtype);
    if (!aligned(y, eb) || !aligned(grad, eb) || !aligned(wgrad, 4)) return PEG_ERR_ALIGNMENT;
    const int vec = pick_vec(H * eb, eb, y, grad);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PEG_CHECK(ensure_slots(T, K, E, layout, capacity, indices, bin_ids, bins, padded_bins, &slot_row, ws, ws_bytes, s));
    return wgrad_launch(y, grad, dtype, vec, layout, T, H, K, E, capacity, bins, padded_bins, slot_row, wgrad, s);
}

PEG_API peg_status peg_combine_backward(const void* y, const void* dout, const float* weights, int32_t dtype,
                                        int32_t layout, int64_t T, int64_t H, int32_t K, int32_t E, int32_t capacity,
                                        const int32_t* indices, const int32_t* bin_ids, const int32_t* bins,
                                        const int32_t* padded_bins, const int32_t* slot_row, void* dy,
                                        int64_t dy_rows, float* wgrad, void* ws, size_t ws_bytes, void* stream) {
    PEG_CHECK(check_common(dtype, layout, T, H, K, E, capacity, padded_bins));
    if (dy_rows < 0 || dy_rows > kMaxAssign) return PEG_ERR_BAD_SHAPE;
    if (!bins || (T > 0 && ((!y && layout == PEG_BINNED) || !dout || !wgrad)) || (dy_rows > 0 && !dy))
        return PEG_ERR_NULL_ARG;
    const int eb = elem_bytes(dtype);
    if (!aligned(y, eb) || !aligned(dout, eb) || !aligned(dy, eb) || !aligned(wgrad, 4) ||
        (weights && !aligned(weights, 4)))
        return PEG_ERR_ALIGNMENT;
    const int vec = pick_vec(H * eb, eb, y, dout, dy);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PEG_CHECK(ensure_slots(T, K, E, layout, capacity, indices, bin_ids, bins, padded_bins, &slot_row, ws, ws_bytes, s));
    if (K > PEG_BACKWARD_SPLIT_K) {
        // both launches' sizes checked before the first is queued
        if (!grid_fits(token_blocks(T, wgrad_shape(K, H * eb / vec).wpt), kBlock)) return PEG_ERR_BAD_SHAPE;
        PEG_CHECK(dy_gather(dout, weights, dtype, vec, layout, T, H, K, E, capacity, bins, padded_bins, slot_row, dy,
                            dy_rows, s));
        return wgrad_launch(y, dout, dtype, vec, layout, T, H, K, E, capacity, bins, padded_bins, slot_row, wgrad,
                            s);
    }
    const RowArgs ra{layout == PEG_BINNED ? (int64_t)E * capacity : 0,
                     layout == PEG_PADDED ? padded_bins : nullptr};
    const int64_t nch = H * eb / vec;
    const RowShape sh = backward_shape(K, nch);
    const int64_t q = wave_slice(nch, sh.wpt);
    const int u = pass_vectors(q, sh.umax);
    const int64_t tb = token_blocks(T, sh.wpt);
    // a large binned dy gets its gap rows (and rows past E*C) from a
    // fill-shaped launch of its own first; otherwise gap blocks follow the
    // token blocks in one launch
    const bool fill = dy_rows > 0 && use_gap_fill(layout, dy_rows, H * eb, E);
    const int64_t nzb = fill ? 0 : gap_blocks(dy_rows, nch);
    if (!grid_fits(tb + nzb, kBlock)) return PEG_ERR_BAD_SHAPE;
    const dim3 grid((unsigned)(tb + nzb));
    if (fill) PEG_CHECK(launch_gap_fill_vec(vec, (uint8_t*)dy, nch, dy_rows, E, capacity, bins, s));
    const WgradArgs a{(const uint8_t*)y, (const uint8_t*)dout, wgrad, nch, q, T, K, slot_row, ra, E, weights,
                      (uint8_t*)dy, dy_rows, layout, capacity, bins, tb, sh.wpt};
    if (weights) return wgrad_by_dtype<2>(dtype, vec, u, grid, s, a);
    return wgrad_by_dtype<1>(dtype, vec, u, grid, s, a);
}
