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

// Wave-wide reductions (all lanes receive the result).
template <typename T> __device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
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

// (value desc, index asc) ordering: true when (va, ia) comes first.
__device__ __forceinline__ bool precedes(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Arg-max reduction across the wave with the lowest index winning ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(v, o, kWave);
        int oi = __shfl_xor(i, o, kWave);
        if (precedes(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// Sorts one value per lane in descending order (bitonic network over the wave).
__device__ __forceinline__ float wave_sort_desc(float v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            float o = __shfl_xor(v, j, kWave);
            // descending overall: block direction flips with (lane & k)
            bool up = ((lane & k) == 0);
            bool lower = ((lane & j) == 0);
            bool take_max = (up == lower);
            v = take_max ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return v;
}

}  // namespace sv
