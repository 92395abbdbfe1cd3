// peg_device.hpp - device-side building blocks of the gfx950 kernels:
// element codecs, 16/8/4/2-byte row vectors, wave64 scans and reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "peg.h"

namespace peg {

constexpr int kWave = 64;
constexpr int kRowsFast = 8;  // routes per token held in scalar registers (more are looped)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A row is moved as VEC-byte lanes: 16 (dwordx4), 8, 4 or 2 bytes.
template <int VEC> struct VecOf;
template <> struct VecOf<16> { using T = u32x4; };
template <> struct VecOf<8> { using T = u32x2; };
template <> struct VecOf<4> { using T = uint32_t; };
template <> struct VecOf<2> { using T = uint16_t; };

// Build-time tuning knobs (defaults are the measured best on MI355X):
//   PEG_NT_LOAD  - streamed row loads carry the nontemporal hint (+4-6% on
//                  every row kernel);
//   PEG_NT_STORE - the gathers' row stores carry it too (off: it costs the
//                  write-bound gathers up to 17%);
//   PEG_NT_STORE_COMBINE - the combine's output stores carry it (+7-9%);
//   PEG_NT_STORE_DY - the combine backward's dy row stores carry it (2-8%
//                  faster on the four model-shaped batches); its zero stores
//                  of dy's gap rows do not (PEG_NT_STORE_DY_ZERO: up to 10%
//                  slower with it).
#ifndef PEG_NT_LOAD
#define PEG_NT_LOAD 1
#endif
#ifndef PEG_NT_STORE
#define PEG_NT_STORE 0
#endif
#ifndef PEG_NT_STORE_COMBINE
#define PEG_NT_STORE_COMBINE 1
#endif
#ifndef PEG_NT_STORE_DY
#define PEG_NT_STORE_DY 1
#endif
#ifndef PEG_NT_STORE_DY_ZERO
#define PEG_NT_STORE_DY_ZERO PEG_NT_STORE
#endif

template <int VEC>
__device__ __forceinline__ typename VecOf<VEC>::T load_vec(const uint8_t* base, int64_t unit) {
    return reinterpret_cast<const typename VecOf<VEC>::T*>(base)[unit];
}

template <int VEC>
__device__ __forceinline__ void store_vec(uint8_t* base, int64_t unit, typename VecOf<VEC>::T v) {
    reinterpret_cast<typename VecOf<VEC>::T*>(base)[unit] = v;
}

// Row streaming: data touched once per launch (token rows, expert rows,
// gradient rows, outputs).
template <int VEC>
__device__ __forceinline__ typename VecOf<VEC>::T stream_load(const uint8_t* base, int64_t unit) {
#if PEG_NT_LOAD
    return __builtin_nontemporal_load(reinterpret_cast<const typename VecOf<VEC>::T*>(base) + unit);
#else
    return load_vec<VEC>(base, unit);
#endif
}

template <int VEC, bool NT = PEG_NT_STORE>
__device__ __forceinline__ void stream_store(uint8_t* base, int64_t unit, typename VecOf<VEC>::T v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<typename VecOf<VEC>::T*>(base) + unit);
    else store_vec<VEC>(base, unit, v);
}

template <int VEC>
__device__ __forceinline__ typename VecOf<VEC>::T zero_vec() {
    return typename VecOf<VEC>::T(0);
}

// ---------------------------------------------------------------------------
// Element codecs. Widening is exact; narrowing rounds to nearest even.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays a quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                 // ties to even
    return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t h16) {
    uint16_t b = (uint16_t)h16;
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}

__device__ __forceinline__ uint32_t float_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;  // hardware conversion, round to nearest even
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

template <int DT> struct Elem;
template <> struct Elem<PEG_F32> {
    static constexpr int bytes = 4;
};
template <> struct Elem<PEG_BF16> {
    static constexpr int bytes = 2;
};
template <> struct Elem<PEG_F16> {
    static constexpr int bytes = 2;
};

template <int DT>
__device__ __forceinline__ float decode(uint32_t bits) {
    if constexpr (DT == PEG_F32) return __uint_as_float(bits);
    else if constexpr (DT == PEG_BF16) return bf16_bits_to_float(bits);
    else return f16_bits_to_float(bits);
}

template <int DT>
__device__ __forceinline__ uint32_t encode(float v) {
    if constexpr (DT == PEG_F32) return __float_as_uint(v);
    else if constexpr (DT == PEG_BF16) return float_to_bf16_bits(v);
    else return float_to_f16_bits(v);
}

// Unpack a VEC-byte vector into its N = VEC / element-bytes elements (as
// float), and pack them back.
template <int DT, int VEC>
struct Lanes {
    static constexpr int EB = Elem<DT>::bytes;
    static constexpr int N = VEC / EB;
    using V = typename VecOf<VEC>::T;

    __device__ static __forceinline__ void unpack(const V& v, float (&f)[N]) {
        if constexpr (VEC == 2) {
            f[0] = decode<DT>((uint32_t)v);
        } else {
            constexpr int W = VEC / 4;
            uint32_t w[W];
            __builtin_memcpy(w, &v, VEC);
            if constexpr (EB == 4) {
#pragma unroll
                for (int i = 0; i < W; ++i) f[i] = decode<DT>(w[i]);
            } else {
#pragma unroll
                for (int i = 0; i < W; ++i) {
                    f[2 * i] = decode<DT>(w[i] & 0xffffu);
                    f[2 * i + 1] = decode<DT>(w[i] >> 16);
                }
            }
        }
    }

    __device__ static __forceinline__ V pack(const float (&f)[N]) {
        V v;
        if constexpr (VEC == 2) {
            v = (uint16_t)encode<DT>(f[0]);
        } else {
            constexpr int W = VEC / 4;
            uint32_t w[W];
            if constexpr (EB == 4) {
#pragma unroll
                for (int i = 0; i < W; ++i) w[i] = encode<DT>(f[i]);
            } else {
#pragma unroll
                for (int i = 0; i < W; ++i) w[i] = encode<DT>(f[2 * i]) | (encode<DT>(f[2 * i + 1]) << 16);
            }
            __builtin_memcpy(&v, w, VEC);
        }
        return v;
    }
};

// ---------------------------------------------------------------------------
// Wave64 / block primitives.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Block barrier that orders LDS accesses only: global stores issued before it
// stay in flight (__syncthreads would wait for them to complete). For
// barriers that protect LDS data; global data shared between the threads of
// a block still needs __syncthreads.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// popcount(mask & lanes below this one), in two instructions.
__device__ __forceinline__ int rank_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t lanes_below() {
    return (uint64_t(1) << lane_id()) - 1;  // lane 0 -> 0
}

// DPP lane moves (VALU operations, no LDS crossbar). Lanes whose source is
// outside the pattern, or whose row is not in ROW_MASK, read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_read(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_read_f(float v) {
    return __int_as_float(dpp_read<CTRL>(__float_as_int(v)));
}

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShr = 0x110;     // + n: lane i <- lane i-n of its 16-lane row
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i of its 8 lanes
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15-i of its row
constexpr int kDppBcast15 = 0x142;    // rows 1..3 <- last lane of the row before
constexpr int kDppBcast31 = 0x143;    // rows 2..3 <- lane 31

// Sum over the wave, the same value in every lane: a butterfly inside each
// 16-lane row (each step adds a pair of partial sums that the two lanes hold
// in swapped order, so the row's lanes agree), then the four row sums read
// as scalars and added in row order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_read_f<kDppQuadXor1>(v);
    v += dpp_read_f<kDppQuadXor2>(v);
    v += dpp_read_f<kDppHalfMirror>(v);
    v += dpp_read_f<kDppRowMirror>(v);
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return ((r0 + r1) + r2) + r3;
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside each row by
// DPP row shifts, then the row totals carried forward by the two row
// broadcasts). The last lane holds the wave total.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += dpp_read<kDppRowShr + 1>(v);
    v += dpp_read<kDppRowShr + 2>(v);
    v += dpp_read<kDppRowShr + 4>(v);
    v += dpp_read<kDppRowShr + 8>(v);
    v += dpp_read<kDppBcast15, 0xA>(v);
    v += dpp_read<kDppBcast31, 0xC>(v);
    return v;
}

// Blocks of a launch go to the 8 XCDs in turn (block b to XCD b % 8). With
// PEG_XCD_REMAP the token kernels give XCD x one contiguous run of their n
// token blocks instead of every 8th, so that each XCD's L2 and address
// translation see 1/8 of the rows. xcd_block(b, n) is a bijection on [0, n).
// Measured and left off: it costs 1-10% at T4096 H4096 and up to 2x at
// T32768 H3584 (a contiguous run of rows per XCD concentrates the
// concurrent accesses on fewer memory channels).
#ifndef PEG_XCD_REMAP
#define PEG_XCD_REMAP 0
#endif
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t n) {
#if PEG_XCD_REMAP
    const int64_t x = b & 7, i = b >> 3, base = n >> 3, rem = n & 7;
    return x * base + (x < rem ? x : rem) + i;
#else
    (void)n;
    return b;
#endif
}

// Value of lane 63 in every lane.
__device__ __forceinline__ int last_lane(int v) { return __builtin_amdgcn_readlane(v, kWave - 1); }

// Exclusive prefix sum over the NT threads of a block (NT a multiple of 64).
// `scratch` holds NT/64 ints of LDS. Returns the prefix of this thread's
// value; *total receives the block-wide sum. Contains barriers: every
// thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    constexpr int NW = NT / kWave;
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[w] = inc;
    lds_barrier();
    if (w == 0) {
        int t = lane < NW ? scratch[lane] : 0;
        t = wave_inclusive_scan(t);
        if (lane < NW) scratch[lane] = t;
    }
    lds_barrier();
    int prefix = (w ? scratch[w - 1] : 0) + inc - v;
    *total = scratch[NW - 1];
    lds_barrier();
    return prefix;
}

}  // namespace peg
