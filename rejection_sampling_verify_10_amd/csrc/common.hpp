// Device helpers shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTopkMax = 64;

// Row flags written by the statistics / selection kernels.
constexpr uint32_t kFlagInvalid = 1u;   // E1 / E3 / E4 for the row

// bfloat16 halves of a 32-bit word, widened exactly to float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT> struct Elem;          // DT: 0 = float32, 1 = bfloat16 (spec_dtype_t)
template <> struct Elem<0> {
    static constexpr int kPerVec = 4;   // elements per 16-byte vector
    static constexpr int kBytes = 4;
    __device__ static __forceinline__ float get(const u32x4& v, int e) { return __uint_as_float(v[e]); }
    __device__ static __forceinline__ float scalar(const void* row, long i) {
        return static_cast<const float*>(row)[i];
    }
};
template <> struct Elem<1> {
    static constexpr int kPerVec = 8;
    static constexpr int kBytes = 2;
    __device__ static __forceinline__ float get(const u32x4& v, int e) {
        return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
    }
    __device__ static __forceinline__ float scalar(const void* row, long i) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[i]) << 16);
    }
};

__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Relaxed 64-bit accesses at device (agent) scope.  They carry the
// device-coherence bit: a store is written through the XCD's L2, and a load
// does not return a stale copy from another XCD's write.  Aligned 8-byte
// accesses are single-copy atomic, so a word carrying its own valid bit can be
// handed between workgroups of one launch without any cache write-back.
__device__ __forceinline__ void st_agent64(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent64(const unsigned long long* p) {
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Value of lane (lane ^ j) for j in {1, 2, 4, 8, 16, 32}, on the VALU: DPP quad
// permutes (1, 2), row shifts (4), a row rotate (8) and the gfx950 lane-swap
// instructions (16, 32).  All 64 lanes must be active.  j must fold to a
// constant (the networks below are fully unrolled).
__device__ __forceinline__ int xshfl_i(int v, int j) {
    const int lane = threadIdx.x & 63;
    switch (j) {
        case 1: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);     // quad_perm [1,0,3,2]
        case 2: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);     // quad_perm [2,3,0,1]
        case 4: {
            const int up = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0xF, false);  // row_shl:4
            const int dn = __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, false);  // row_shr:4
            return (lane & 4) ? dn : up;
        }
        case 8: return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);    // row_ror:8
        case 16: {
            const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            return (lane & 16) ? static_cast<int>(r[0]) : static_cast<int>(r[1]);
        }
        default: {
            const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            return (lane & 32) ? static_cast<int>(r[0]) : static_cast<int>(r[1]);
        }
    }
}
__device__ __forceinline__ unsigned xshfl(unsigned v, int j) { return static_cast<unsigned>(xshfl_i(static_cast<int>(v), j)); }
__device__ __forceinline__ int xshfl(int v, int j) { return xshfl_i(v, j); }
__device__ __forceinline__ float xshfl(float v, int j) { return __int_as_float(xshfl_i(__float_as_int(v), j)); }
__device__ __forceinline__ double xshfl(double v, int j) {
    const long long b = __double_as_longlong(v);
    const int lo = xshfl_i(static_cast<int>(b), j);
    const int hi = xshfl_i(static_cast<int>(b >> 32), j);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
typedef unsigned long long pkey_t;     // (value, index) sort key, see below
__device__ __forceinline__ pkey_t xshfl(pkey_t v, int j) {
    const int lo = xshfl_i(static_cast<int>(v), j);
    const int hi = xshfl_i(static_cast<int>(v >> 32), j);
    return (static_cast<pkey_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Value of lane 63 - lane (the wave reversed): xor 63 composed of the steps above.
template <typename T> __device__ __forceinline__ T xrev(T v) {
#pragma unroll
    for (int j = 1; j < 64; j <<= 1) v = xshfl(v, j);
    return v;
}
// Value of lane `src` (any lane, per lane) through the LDS crossbar.
__device__ __forceinline__ uint32_t lane_gather(uint32_t v, int src) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(v)));
}
__device__ __forceinline__ unsigned long long lane_gather(unsigned long long v, int src) {
    const uint32_t lo = lane_gather(static_cast<uint32_t>(v), src);
    const uint32_t hi = lane_gather(static_cast<uint32_t>(v >> 32), src);
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ float lane_gather(float v, int src) {
    return __uint_as_float(lane_gather(__float_as_uint(v), src));
}
__device__ __forceinline__ double lane_gather(double v, int src) {
    return __longlong_as_double(static_cast<long long>(lane_gather(static_cast<unsigned long long>(__double_as_longlong(v)), src)));
}
// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value:
// branches on it then compile to scalar branches instead of exec-mask regions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave); }
// Broadcast from a wave-uniform lane (v_readlane).
__device__ __forceinline__ int bcast(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float bcast(float v, int lane) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane)); }
__device__ __forceinline__ double bcast(double v, int lane) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// Wave-wide reductions (all lanes receive the result).
template <typename T> __device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += xshfl(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, xshfl(v, o));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, xshfl(v, o));
    return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, xshfl(v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, xshfl(v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, xshfl(v, o));
    return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, xshfl(v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= xshfl(v, o);
    return v;
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Inclusive prefix sum across the wave in fp32: row-local steps of 1, 2, 4 and 8
// lanes (DPP row shifts, lanes shifted in from outside the row read 0), then the
// totals of the rows below (lanes 15, 31, 47) added in.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    const int lane = threadIdx.x & (kWave - 1);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));   // row_shr:1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));   // row_shr:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));   // row_shr:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));   // row_shr:8
    const float r0 = bcast(v, 15), r1 = bcast(v, 31), r2 = bcast(v, 47);
    const int row = lane >> 4;
    const float below = row == 0 ? 0.f : (row == 1 ? r0 : (row == 2 ? r0 + r1 : (r0 + r1) + r2));
    return v + below;
}

// (value desc, index asc) ordering: true when (va, ia) comes first.
__device__ __forceinline__ bool precedes(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Arg-max reduction across the wave with the lowest index winning ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float ov = xshfl(v, o);
        int oi = xshfl(i, o);
        if (precedes(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

}  // namespace sv

namespace sv {

// ---- bitonic networks over one 32-bit key per lane ----

// Keeps in this lane the larger (keep_large) or the smaller of {mine, lane^j's}.
__device__ __forceinline__ uint32_t cx_u32(uint32_t k, int j, bool keep_large) {
    const uint32_t o = xshfl(k, j);
    return ((o > k) == keep_large) ? o : k;
}
// Sorts the wave's 64 keys, largest first.
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t k) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int s = 2; s <= kWave; s <<= 1) {
#pragma unroll
        for (int j = s >> 1; j > 0; j >>= 1) {
            const bool up = (lane & s) == 0 || s == kWave;
            k = cx_u32(k, j, ((lane & j) == 0) == up);
        }
    }
    return k;
}
// Sorts a bitonic sequence of 64 keys, largest first (desc) or smallest first.
__device__ __forceinline__ uint32_t wave_bitonic_clean(uint32_t k, bool desc) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int j = kWave >> 1; j > 0; j >>= 1) k = cx_u32(k, j, ((lane & j) == 0) == desc);
    return k;
}

// ---- wave-level bitonic networks over (value, index) pairs, one pair per lane ----
//
// Order: larger value first, lower index on equal values (a strict total order
// for distinct indices).  A pair travels as one 64-bit key whose unsigned order
// is that order: the order-preserving bits of the value above the complement of
// the index, so a compare-exchange is one 64-bit compare and two selects.
// Empty slots hold (-inf, kNoIndex) and sort after every real entry.

constexpr int kNoIndex = 0x7fffffff;

__device__ __forceinline__ float maximum3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);   // NaN-propagating
}
__device__ __forceinline__ float minimum3(float a, float b, float c) {
    return __builtin_elementwise_minimum(__builtin_elementwise_minimum(a, b), c);
}

// Order-preserving unsigned key of a float: NaN lowest, -0 folded onto +0.
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 0u;
    if (v == 0.f) v = 0.f;
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ pkey_t pair_key(float v, int i) {
    return (static_cast<pkey_t>(order_key(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(i));
}
__device__ __forceinline__ float key_val(pkey_t k) { return order_value(static_cast<uint32_t>(k >> 32)); }
__device__ __forceinline__ int key_idx(pkey_t k) { return static_cast<int>(0xffffffffu - static_cast<uint32_t>(k)); }
__device__ __forceinline__ pkey_t empty_key() { return pair_key(-INFINITY, kNoIndex); }

// Keeps in this lane the larger (keep_first) or the smaller of {mine, lane^j's}.
// Written as one compare and a select (no branch): take the partner's key when it
// is larger and the larger is kept, or not larger and the smaller is kept (equal
// keys make either choice the same).
__device__ __forceinline__ void cx_key(pkey_t& k, int j, bool keep_first) {
    const pkey_t o = xshfl(k, j);
    const bool take = (o > k) == keep_first;
    k = take ? o : k;
}

// Full sort of the 64 keys of the wave (lane 0 = first).
__device__ __forceinline__ void wave_sort_keys(pkey_t& k) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int s = 2; s <= kWave; s <<= 1) {
#pragma unroll
        for (int j = s >> 1; j > 0; j >>= 1) {
            const bool up = (lane & s) == 0 || s == kWave;
            cx_key(k, j, ((lane & j) == 0) == up);
        }
    }
}

// a and b each sorted (lane 0 first): leaves in a the first 64 of their union,
// sorted.  Pairing lane l of one list with lane 63-l of the other gives a bitonic
// sequence holding the 64 winners; a bitonic merge sorts it.
__device__ __forceinline__ void wave_merge_keys(pkey_t& a, pkey_t b) {
    const int lane = threadIdx.x & (kWave - 1);
    const pkey_t rb = lane_gather(b, kWave - 1 - lane);     // b reversed
    a = a > rb ? a : rb;
#pragma unroll
    for (int j = kWave >> 1; j > 0; j >>= 1) cx_key(a, j, (lane & j) == 0);
}

}  // namespace sv
