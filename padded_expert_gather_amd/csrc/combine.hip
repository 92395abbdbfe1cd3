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
// How: token-major. One block per token stages the token's kept rows (and
// weights) in LDS, then streams its H columns in 16-byte lanes: every kept
// expert row is read once, the output row (combine) is written once, the
// gradient row (wgrad) is read once for all K dots. Accumulation is fp32
// FMA; the wgrad dots finish with a wave64 butterfly and a 4-wave LDS sum.
// Rows that are unused capacity, padding or dropped are never read.
#include "peg_device.hpp"
#include "peg_host.hpp"

namespace peg {

constexpr int kCombUnroll = 2;  // column vectors per thread per pass
constexpr int kKBatch = 4;      // expert rows loaded together before use

// Stage the kept (row, weight, k) of token t in LDS, in k order. Returns the
// number kept. Rows outside [0, R) are treated as not kept.
__device__ __forceinline__ int stage_token(int64_t t, int32_t K, const int32_t* __restrict__ slot_row,
                                           const float* __restrict__ weights, int64_t R, int* srow, float* sw,
                                           int* sk, int* s_nv) {
    for (int k = threadIdx.x; k < K; k += kBlock) {
        int r = slot_row[t * K + k];
        if (r < 0 || r >= R) r = -1;
        srow[k] = r;
        if (sw) sw[k] = weights ? weights[t * K + k] : 1.0f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int nv = 0;
        for (int k = 0; k < K; ++k) {
            const int r = srow[k];
            if (r >= 0) {
                srow[nv] = r;
                if (sw) sw[nv] = sw[k];
                if (sk) sk[nv] = k;
                ++nv;
            }
        }
        *s_nv = nv;
    }
    __syncthreads();
    return *s_nv;
}

__device__ __forceinline__ int64_t expert_rows(int64_t static_rows, const int32_t* padded_bins, int32_t E) {
    return padded_bins ? (int64_t)padded_bins[E - 1] : static_rows;
}

template <int DT, int VEC>
__global__ __launch_bounds__(kBlock) void combine_kernel(const uint8_t* __restrict__ y, uint8_t* __restrict__ out,
                                                         int64_t nch, int32_t K, const int32_t* __restrict__ slot_row,
                                                         const float* __restrict__ weights, int64_t static_rows,
                                                         const int32_t* __restrict__ padded_bins, int32_t E) {
    using L = Lanes<DT, VEC>;
    using V = typename L::V;
    constexpr int N = L::N;
    __shared__ int srow[PEG_MAX_EXPERTS];
    __shared__ float sw[PEG_MAX_EXPERTS];
    __shared__ int s_nv;
    const int64_t t = blockIdx.x;
    const int64_t R = expert_rows(static_rows, padded_bins, E);
    const int nv = stage_token(t, K, slot_row, weights, R, srow, sw, nullptr, &s_nv);
    const int64_t row_bytes = nch * VEC;
    uint8_t* dst = out + t * row_bytes;

    for (int64_t c0 = threadIdx.x; c0 < nch; c0 += (int64_t)kBlock * kCombUnroll) {
        float acc[kCombUnroll][N];
#pragma unroll
        for (int u = 0; u < kCombUnroll; ++u)
#pragma unroll
            for (int i = 0; i < N; ++i) acc[u][i] = 0.0f;
        for (int k0 = 0; k0 < nv; k0 += kKBatch) {
            V v[kKBatch][kCombUnroll];
#pragma unroll
            for (int kk = 0; kk < kKBatch; ++kk) {
                if (k0 + kk < nv) {
                    const uint8_t* src = y + (int64_t)srow[k0 + kk] * row_bytes;
#pragma unroll
                    for (int u = 0; u < kCombUnroll; ++u) {
                        const int64_t c = c0 + (int64_t)u * kBlock;
                        if (c < nch) v[kk][u] = load_vec<VEC>(src, c);
                    }
                }
            }
#pragma unroll
            for (int kk = 0; kk < kKBatch; ++kk) {
                if (k0 + kk < nv) {
                    const float w = sw[k0 + kk];
#pragma unroll
                    for (int u = 0; u < kCombUnroll; ++u) {
                        if (c0 + (int64_t)u * kBlock < nch) {
                            float f[N];
                            L::unpack(v[kk][u], f);
#pragma unroll
                            for (int i = 0; i < N; ++i) acc[u][i] = fmaf(w, f[i], acc[u][i]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kCombUnroll; ++u) {
            const int64_t c = c0 + (int64_t)u * kBlock;
            if (c < nch) store_vec<VEC>(dst, c, L::pack(acc[u]));
        }
    }
}

constexpr int kWgBatch = 8;  // dots accumulated per pass over the gradient row

template <int DT, int VEC>
__global__ __launch_bounds__(kBlock) void wgrad_kernel(const uint8_t* __restrict__ y, const uint8_t* __restrict__ grad,
                                                       float* __restrict__ wgrad, int64_t nch, int32_t K,
                                                       const int32_t* __restrict__ slot_row, int64_t static_rows,
                                                       const int32_t* __restrict__ padded_bins, int32_t E) {
    using L = Lanes<DT, VEC>;
    using V = typename L::V;
    constexpr int N = L::N;
    constexpr int NW = kBlock / kWave;
    __shared__ int srow[PEG_MAX_EXPERTS];
    __shared__ int sk[PEG_MAX_EXPERTS];
    __shared__ float red[NW][kWgBatch];
    __shared__ int s_nv;
    const int64_t t = blockIdx.x;
    const int64_t R = expert_rows(static_rows, padded_bins, E);
    // every output of the token starts at 0 (dropped / unrouted stay 0)
    for (int k = threadIdx.x; k < K; k += kBlock) wgrad[t * K + k] = 0.0f;
    const int nv = stage_token(t, K, slot_row, nullptr, R, srow, nullptr, sk, &s_nv);
    if (nv == 0) return;
    const int64_t row_bytes = nch * VEC;
    const uint8_t* g_row = grad + t * row_bytes;
    const int w = threadIdx.x / kWave;

    for (int k0 = 0; k0 < nv; k0 += kWgBatch) {
        float acc[kWgBatch];
#pragma unroll
        for (int kk = 0; kk < kWgBatch; ++kk) acc[kk] = 0.0f;
        for (int64_t c = threadIdx.x; c < nch; c += kBlock) {
            float g[N];
            L::unpack(load_vec<VEC>(g_row, c), g);
            V v[kWgBatch];
#pragma unroll
            for (int kk = 0; kk < kWgBatch; ++kk)
                if (k0 + kk < nv) v[kk] = load_vec<VEC>(y + (int64_t)srow[k0 + kk] * row_bytes, c);
#pragma unroll
            for (int kk = 0; kk < kWgBatch; ++kk) {
                if (k0 + kk < nv) {
                    float f[N];
                    L::unpack(v[kk], f);
#pragma unroll
                    for (int i = 0; i < N; ++i) acc[kk] = fmaf(f[i], g[i], acc[kk]);
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < kWgBatch; ++kk) {
            const float s = wave_sum(acc[kk]);
            if (lane_id() == 0) red[w][kk] = s;
        }
        __syncthreads();
        if (threadIdx.x < kWgBatch && k0 + (int)threadIdx.x < nv) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < NW; ++i) s += red[i][threadIdx.x];
            wgrad[t * K + sk[k0 + threadIdx.x]] = s;
        }
        __syncthreads();
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

template <int DT>
static peg_status combine_dispatch(int vec, dim3 grid, hipStream_t s, const uint8_t* y, uint8_t* out, int64_t nch,
                                   int32_t K, const int32_t* slot_row, const float* w, RowArgs ra, int32_t E) {
    switch (vec) {
        case 16:
            return launch(combine_kernel<DT, 16>, grid, dim3(kBlock), 0, s, y, out, nch, K, slot_row, w,
                          ra.static_rows, ra.padded_bins, E);
        case 8:
            return launch(combine_kernel<DT, 8>, grid, dim3(kBlock), 0, s, y, out, nch, K, slot_row, w,
                          ra.static_rows, ra.padded_bins, E);
        case 4:
            return launch(combine_kernel<DT, 4>, grid, dim3(kBlock), 0, s, y, out, nch, K, slot_row, w,
                          ra.static_rows, ra.padded_bins, E);
        default:
            if constexpr (Elem<DT>::bytes == 2)
                return launch(combine_kernel<DT, 2>, grid, dim3(kBlock), 0, s, y, out, nch, K, slot_row, w,
                              ra.static_rows, ra.padded_bins, E);
            return PEG_ERR_ALIGNMENT;
    }
}

template <int DT>
static peg_status wgrad_dispatch(int vec, dim3 grid, hipStream_t s, const uint8_t* y, const uint8_t* g, float* wg,
                                 int64_t nch, int32_t K, const int32_t* slot_row, RowArgs ra, int32_t E) {
    switch (vec) {
        case 16:
            return launch(wgrad_kernel<DT, 16>, grid, dim3(kBlock), 0, s, y, g, wg, nch, K, slot_row,
                          ra.static_rows, ra.padded_bins, E);
        case 8:
            return launch(wgrad_kernel<DT, 8>, grid, dim3(kBlock), 0, s, y, g, wg, nch, K, slot_row,
                          ra.static_rows, ra.padded_bins, E);
        case 4:
            return launch(wgrad_kernel<DT, 4>, grid, dim3(kBlock), 0, s, y, g, wg, nch, K, slot_row,
                          ra.static_rows, ra.padded_bins, E);
        default:
            if constexpr (Elem<DT>::bytes == 2)
                return launch(wgrad_kernel<DT, 2>, grid, dim3(kBlock), 0, s, y, g, wg, nch, K, slot_row,
                              ra.static_rows, ra.padded_bins, E);
            return PEG_ERR_ALIGNMENT;
    }
}

}  // namespace peg

using namespace peg;

PEG_API peg_status peg_scatter_combine(const void* y, int32_t dtype, int32_t layout, int64_t T, int64_t H,
                                       int32_t K, int32_t E, int32_t capacity, const int32_t* indices,
                                       const int32_t* bin_ids, const int32_t* bins, const int32_t* padded_bins,
                                       const int32_t* slot_row, const float* weights, void* out, void* ws,
                                       size_t ws_bytes, void* stream) {
    PEG_CHECK(check_common(dtype, layout, T, H, K, E, capacity, padded_bins));
    if (T > 0 && (!y || !out)) return PEG_ERR_NULL_ARG;
    const int eb = elem_bytes(dtype);
    if (!aligned(y, eb) || !aligned(out, eb) || (weights && !aligned(weights, 4))) return PEG_ERR_ALIGNMENT;
    const int vec = pick_vec(H * eb, eb, y, out);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PEG_CHECK(ensure_slots(T, K, E, layout, capacity, indices, bin_ids, bins, padded_bins, &slot_row, ws, ws_bytes, s));
    const RowArgs ra{layout == PEG_BINNED ? (int64_t)E * capacity : 0,
                     layout == PEG_PADDED ? padded_bins : nullptr};
    const int64_t nch = H * eb / vec;
    const dim3 grid((unsigned)T);
    const uint8_t* yb = (const uint8_t*)y;
    uint8_t* ob = (uint8_t*)out;
    if (dtype == PEG_F32) return combine_dispatch<PEG_F32>(vec, grid, s, yb, ob, nch, K, slot_row, weights, ra, E);
    if (dtype == PEG_BF16) return combine_dispatch<PEG_BF16>(vec, grid, s, yb, ob, nch, K, slot_row, weights, ra, E);
    return combine_dispatch<PEG_F16>(vec, grid, s, yb, ob, nch, K, slot_row, weights, ra, E);
}

PEG_API peg_status peg_wgrad(const void* y, const void* grad, int32_t dtype, int32_t layout, int64_t T, int64_t H,
                             int32_t K, int32_t E, int32_t capacity, const int32_t* indices, const int32_t* bin_ids,
                             const int32_t* bins, const int32_t* padded_bins, const int32_t* slot_row,
                             float* wgrad, void* ws, size_t ws_bytes, void* stream) {
    PEG_CHECK(check_common(dtype, layout, T, H, K, E, capacity, padded_bins));
    if (T > 0 && (!y || !grad || !wgrad)) return PEG_ERR_NULL_ARG;
    const int eb = elem_bytes(dtype);
    if (!aligned(y, eb) || !aligned(grad, eb) || !aligned(wgrad, 4)) return PEG_ERR_ALIGNMENT;
    const int vec = pick_vec(H * eb, eb, y, grad);
    if (vec == 0) return PEG_ERR_ALIGNMENT;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    PEG_CHECK(ensure_slots(T, K, E, layout, capacity, indices, bin_ids, bins, padded_bins, &slot_row, ws, ws_bytes, s));
    const RowArgs ra{layout == PEG_BINNED ? (int64_t)E * capacity : 0,
                     layout == PEG_PADDED ? padded_bins : nullptr};
    const int64_t nch = H * eb / vec;
    const dim3 grid((unsigned)T);
    const uint8_t* yb = (const uint8_t*)y;
    const uint8_t* gb = (const uint8_t*)grad;
    if (dtype == PEG_F32) return wgrad_dispatch<PEG_F32>(vec, grid, s, yb, gb, wgrad, nch, K, slot_row, ra, E);
    if (dtype == PEG_BF16) return wgrad_dispatch<PEG_BF16>(vec, grid, s, yb, gb, wgrad, nch, K, slot_row, ra, E);
    return wgrad_dispatch<PEG_F16>(vec, grid, s, yb, gb, wgrad, nch, K, slot_row, ra, E);
}
