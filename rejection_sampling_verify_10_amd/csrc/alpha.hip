// Acceptance rate of dense rows in one pass over each row's bytes.
//
// "064 · 投机解码", section 二: one drafted token survives with probability
// alpha = sum_i min(p'(i), q'(i)), the overlap of the target distribution
// p' = softmax(z/T) and the draft distribution q' (q as given at T = 1, else
// q^(1/T) renormalised).  p' needs the row's maximum and normaliser before any
// term is known, so a one-pass kernel keeps the whole logit row in registers:
// one workgroup of 1024 threads per (b, k) loads its row once (16 vectors of
// 16 bytes per thread: up to 131072 bf16 or 65536 fp32 logits), reduces the
// maximum and the normaliser, and then streams the draft row once, each thread
// reading the draft entries of the logits it holds (two adjacent vectors per
// bf16 vector), so that every byte of both rows crosses HBM once.  A
// transformed draft (T != 1) needs its own normaliser first and is streamed
// twice.  Rows that do not fit take the two-kernel route (row statistics, then
// alpha_dense_kernel).
//
// Sums: fp32 exponentials and terms within a thread (at most 128 terms), fp64
// across threads; alpha agrees with the fp64 definition to ~1e-7.

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kAlphaThreads = 1024;
constexpr int kAlphaVecs = 16;          // 16-byte vectors of the logit row per thread
constexpr int kAlphaWaves = kAlphaThreads / kWave;

template <typename T, typename F>
__device__ __forceinline__ T block_reduce(T v, T* red, F op) {
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    T r = red[0];
#pragma unroll
    for (int w = 1; w < kAlphaWaves; ++w) r = op(r, red[w]);
    __syncthreads();                    // red is reused by the next reduction
    return r;
}

// Draft entries i0 .. i0+EPV-1 (the logits of one target vector) as EPV/4 vectors.
template <int EPV>
__device__ __forceinline__ void load_draft(const float* qrow, long i0, u32x4 (&d)[EPV / 4]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(qrow + i0);
#pragma unroll
    for (int c = 0; c < EPV / 4; ++c) d[c] = load_stream(p + c);
}

template <int DT, bool TRANSFORMED>
__global__ __launch_bounds__(kAlphaThreads, 1) void alpha_row_kernel(AlphaArgs a) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    __shared__ float red_f[kAlphaWaves];
    __shared__ double red_d[kAlphaWaves];
    __shared__ uint32_t red_u[kAlphaWaves];
    const int r = blockIdx.x;                         // b*K + k
    const int b = r / a.K, k = r - b * a.K;
    const int tid = threadIdx.x;
    const long zrow = static_cast<long>(b) * (a.K + 1) + k;
    const u32x4* zv = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.logits) + zrow * a.V * E::kBytes);
    const float* qrow = a.q + static_cast<long>(r) * a.V;
    const int nvec = a.V / EPV;

    u32x4 v[kAlphaVecs];
#pragma unroll
    for (int s = 0; s < kAlphaVecs; ++s) {
        const int g = s * kAlphaThreads + tid;
        v[s] = g < nvec ? load_stream(zv + g) : u32x4{0u, 0u, 0u, 0u};
    }
    // maximum; NaN or +inf anywhere makes the row unusable (E1)
    float m = -INFINITY;
    uint32_t bad = 0;
#pragma unroll
    for (int s = 0; s < kAlphaVecs; ++s) {
        if (s * kAlphaThreads + tid < nvec) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float z = E::get(v[s], e);
                bad |= !(z < INFINITY);               // NaN or +inf
                m = fmaxf(m, z);
            }
        }
    }
    const float M = block_reduce(wave_max(m), red_f, [](float x, float y) { return fmaxf(x, y); });
    const float sc = a.scale;
    float part = 0.f;
    if (M > -INFINITY) {
#pragma unroll
        for (int s = 0; s < kAlphaVecs; ++s)
            if (s * kAlphaThreads + tid < nvec)
#pragma unroll
                for (int e = 0; e < EPV; ++e) part += __builtin_amdgcn_exp2f((E::get(v[s], e) - M) * sc);
    }
    const double Z = block_reduce(wave_sum(static_cast<double>(part)), red_d, [](double x, double y) { return x + y; });
    const float invZ = static_cast<float>(1.0 / Z);

    // transformed draft: its normaliser sum q^(1/T) over the row first
    float invQ = 1.f;
    if (TRANSFORMED) {
        float qs = 0.f;
#pragma unroll
        for (int s = 0; s < kAlphaVecs; ++s) {
            const int g = s * kAlphaThreads + tid;
            if (g < nvec) {
                u32x4 d[EPV / 4];
                load_draft<EPV>(qrow, static_cast<long>(g) * EPV, d);
#pragma unroll
                for (int c = 0; c < EPV / 4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float q = __uint_as_float(d[c][e]);
                        qs += q > 0.f ? __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(q) * a.invT) : 0.f;
                    }
            }
        }
        const double S = block_reduce(wave_sum(static_cast<double>(qs)), red_d,
                                      [](double x, double y) { return x + y; });
        bad |= !(S > 0.0);                           // E4 (also NaN sums)
        invQ = static_cast<float>(1.0 / S);
    }

    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < kAlphaVecs; ++s) {
        const int g = s * kAlphaThreads + tid;
        if (g < nvec) {
            u32x4 d[EPV / 4];
            load_draft<EPV>(qrow, static_cast<long>(g) * EPV, d);
#pragma unroll
            for (int c = 0; c < EPV / 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float q = __uint_as_float(d[c][e]);
                    bad |= !q_ok(q);                  // E3
                    const float p = __builtin_amdgcn_exp2f((E::get(v[s], c * 4 + e) - M) * sc) * invZ;
                    float qq = q;
                    if (TRANSFORMED) qq = q > 0.f ? __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(q) * a.invT) * invQ : 0.f;
                    acc += fminf(p, qq);
                }
        }
    }
    const double alpha = block_reduce(wave_sum(static_cast<double>(acc)), red_d,
                                      [](double x, double y) { return x + y; });
    bad = block_reduce(wave_or(bad), red_u, [](uint32_t x, uint32_t y) { return x | y; });
    if (tid == 0) {
        const bool ok = !bad && M > -INFINITY && Z >= 1.0 && Z < INFINITY;
        a.out_alpha[r] = ok ? static_cast<float>(alpha) : NAN;
    }
}

}  // namespace

bool alpha_rows_fit(const AlphaArgs& a) {
    const int esz = a.dtype ? 2 : 4;
    return vec_ok(a.logits, a.V, esz) && vec_ok(a.q, a.V, 4) &&
           static_cast<long>(a.V) * esz <= static_cast<long>(kAlphaVecs) * kAlphaThreads * 16;
}

hipError_t launch_alpha_rows(const AlphaArgs& a, hipStream_t s, Timing t) {
    const dim3 grid(a.B * a.K), block(kAlphaThreads);
    if (a.dtype == 1) {
        if (a.transformed) launch_timed(t, alpha_row_kernel<1, true>, grid, block, 0, s, a);
        else launch_timed(t, alpha_row_kernel<1, false>, grid, block, 0, s, a);
    } else {
        if (a.transformed) launch_timed(t, alpha_row_kernel<0, true>, grid, block, 0, s, a);
        else launch_timed(t, alpha_row_kernel<0, false>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sv
