// Row statistics over the vocabulary: one pass over each logit row.
//
// Softmax mode gives the row maximum m and Z = sum_i exp((z_i - m)/T), the
// normaliser of the target distribution p' = softmax(z/T) ("064 · 投机解码",
// section 二: p must carry the temperature).  Argmax mode gives the lowest
// index of the maximum, the greedy rule of "投机解码与 EAGLE", section 二.
//
// The rows are HBM-bound: each is read once with 16-byte non-temporal loads,
// four vectors in flight per thread.  Inside a thread the sum is accumulated
// in fp32 against a running maximum (rescaled once per tile of 4 vectors);
// the 256 per-thread partials are combined in fp64 with exact per-thread
// rescaling, so Z carries the accuracy of the fp32 exponentials.

#include "common.hpp"
#include "internal.hpp"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ u32x4 neg_inf_vec(int dt) {
    const uint32_t w = dt ? 0xff80ff80u : 0xff800000u;
    return u32x4{w, w, w, w};
}

template <int DT>
__device__ __forceinline__ void softmax_row_vec(const char* row, int V, float scale, float& m, float& s) {
    using E = Elem<DT>;
    const u32x4* rv = reinterpret_cast<const u32x4*>(row);
    const int nvec = V / E::kPerVec;
    float acc[kUnroll] = {0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    // Tile t+1 is loaded while tile t is summed (two register buffers), so each
    // thread keeps 8 vectors in flight instead of 4.  Full tiles load without a
    // bounds check (the surplus load at the end re-reads the last full tile and
    // is dropped), so that no load sits behind a branch and waiting for one
    // buffer does not also wait for the other; the partial last tile comes after.
    auto load_tile = [&](int base, u32x4 (&v)[kUnroll]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = base + u * kThreads + threadIdx.x;
            v[u] = (i < nvec) ? load_stream(rv + i) : neg_inf_vec(DT);
        }
    };
    auto load_full = [&](int base, u32x4 (&v)[kUnroll]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load_stream(rv + base + u * kThreads + threadIdx.x);
    };
    auto sum_tile = [&](const u32x4 (&v)[kUnroll]) {
        float tmax = m;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < E::kPerVec; ++e) tmax = fmaxf(tmax, E::get(v[u], e));
        if (tmax > m) {
            const float f = __builtin_amdgcn_exp2f((m - tmax) * scale);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc[u] *= f;
            m = tmax;
        }
        if (m != -INFINITY) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int e = 0; e < E::kPerVec; ++e)
                    acc[u] += __builtin_amdgcn_exp2f((E::get(v[u], e) - m) * scale);
        } else {
            // Everything seen so far is -inf (or padding); only a NaN may matter.
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int e = 0; e < E::kPerVec; ++e)
                    if (E::get(v[u], e) != E::get(v[u], e)) acc[0] = NAN;
        }
    };
    constexpr int kTile = kThreads * kUnroll;
    const int nfull = nvec / kTile;
    u32x4 va[kUnroll], vb[kUnroll];
    int t = 0;
    if (nfull > 0) {
        load_full(0, va);
        for (; t + 1 < nfull; t += 2) {
            load_full((t + 1) * kTile, vb);
            sum_tile(va);
            load_full(min(t + 2, nfull - 1) * kTile, va);
            sum_tile(vb);
        }
        if (t < nfull) sum_tile(va);
    }
    if (nfull * kTile < nvec) {
        load_tile(nfull * kTile, va);
        sum_tile(va);
    }
    s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <int DT>
__device__ __forceinline__ void softmax_row_scalar(const char* row, int V, float scale, float& m, float& s) {
    m = -INFINITY;
    s = 0.f;
    for (int i = threadIdx.x; i < V; i += kThreads) {
        const float z = Elem<DT>::scalar(row, i);
        if (z > m) {
            s *= __builtin_amdgcn_exp2f((m - z) * scale);
            m = z;
        }
        if (m != -INFINITY) s += __builtin_amdgcn_exp2f((z - m) * scale);
        else if (z != z) s = NAN;
    }
}

template <int DT, bool VEC>
__device__ __forceinline__ void argmax_row(const char* row, int V, float& best, int& bi, uint32_t& nan) {
    using E = Elem<DT>;
    best = -INFINITY;
    bi = 0x7fffffff;
    nan = 0;
    if (VEC) {
        const u32x4* rv = reinterpret_cast<const u32x4*>(row);
        const int nvec = V / E::kPerVec;
        for (int base = 0; base < nvec; base += kThreads * kUnroll) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = base + u * kThreads + threadIdx.x;
                v[u] = (i < nvec) ? load_stream(rv + i) : neg_inf_vec(DT);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i0 = (base + u * kThreads + threadIdx.x) * E::kPerVec;
#pragma unroll
                for (int e = 0; e < E::kPerVec; ++e) {
                    const float z = E::get(v[u], e);
                    nan |= (z != z);
                    if (z > best) { best = z; bi = i0 + e; }
                }
            }
        }
    } else {
        for (int i = threadIdx.x; i < V; i += kThreads) {
            const float z = E::scalar(row, i);
            nan |= (z != z);
            if (z > best) { best = z; bi = i; }
        }
    }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void rowstats_kernel(RowStatsArgs a) {
    __shared__ float s_m[kThreads / kWave];
    __shared__ double s_z[kThreads / kWave];
    __shared__ int s_i[kThreads / kWave];
    __shared__ uint32_t s_f[kThreads / kWave];

    const int r = blockIdx.x;
    const int b = r / a.rows_per_batch;
    const int k = r - b * a.rows_per_batch;
    const long mem_row = static_cast<long>(b) * a.batch_stride + k;
    const char* row = static_cast<const char*>(a.base) + mem_row * a.V * Elem<DT>::kBytes;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = wave_id();

    if (a.argmax_mode) {
        float best;
        int bi;
        uint32_t nan;
        argmax_row<DT, VEC>(row, a.V, best, bi, nan);
        wave_argmax(best, bi);
        nan = wave_or(nan);
        if (lane == 0) { s_m[wid] = best; s_i[wid] = bi; s_f[wid] = nan; }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < kThreads / kWave; ++w) {
                if (precedes(s_m[w], s_i[w], best, bi)) { best = s_m[w]; bi = s_i[w]; }
                nan |= s_f[w];
            }
            // Every element was -inf: the lowest index, 0, is the argmax.
            if (bi == 0x7fffffff) bi = 0;
            a.out.m[r] = best;
            a.out.arg[r] = bi;
            a.out.flags[r] = nan ? kFlagInvalid : 0u;
        }
        return;
    }

    float m, s;
    if (VEC) softmax_row_vec<DT>(row, a.V, a.scale, m, s);
    else softmax_row_scalar<DT>(row, a.V, a.scale, m, s);

    float M = wave_max(m);
    if (lane == 0) s_m[wid] = M;
    __syncthreads();
    M = s_m[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) M = fmaxf(M, s_m[w]);
    // Rescale each thread's partial to the row maximum in fp64.
    double c = static_cast<double>(s) * exp((static_cast<double>(m) - static_cast<double>(M)) * a.invT);
    c = wave_sum(c);
    if (lane == 0) s_z[wid] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        double Z = 0.0;
        for (int w = 0; w < kThreads / kWave; ++w) Z += s_z[w];
        a.out.m[r] = M;
        a.out.Z[r] = Z;
        a.out.flags[r] = (Z >= 1.0 && Z < INFINITY) ? 0u : kFlagInvalid;
        if (a.out.zx) {
            float zx = NAN;
            if (a.gather_tokens && k < a.gather_K) {
                const int x = a.gather_tokens[static_cast<long>(b) * a.gather_K + k];
                if (x >= 0 && x < a.V) zx = Elem<DT>::scalar(row, x);
            }
            a.out.zx[r] = zx;
        }
    }
}

// sum_i q_i^(1/T) of a draft-probability row, plus validity (E3, E4).
// Sum of q^(1/T) (fp32 terms, 64-term fp32 groups added in fp64) and the E3 check
// of one draft row.  VEC: the row is read as 16-byte vectors, two tiles of four
// per thread in flight (the next tile loaded while this one is summed).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void power_sums_kernel(PowerSumArgs a) {
    __shared__ double s_z[kThreads / kWave];
    __shared__ uint32_t s_f[kThreads / kWave];
    const float* row = a.q + static_cast<long>(blockIdx.x) * a.V;
    double acc = 0.0;
    uint32_t bad = 0;
    auto term = [&](float v) -> float {
        bad |= !(v >= 0.f && v < INFINITY);
        return (v > 0.f) ? __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(v) * a.invT) : 0.f;
    };
    if constexpr (VEC) {
        const u32x4* rv = reinterpret_cast<const u32x4*>(row);
        const int nvec = a.V / 4;
        constexpr int kTileV = kThreads * kUnroll;
        // vectors past the row load the row's last vector and count as zero
        auto load = [&](int base, u32x4 (&v)[kUnroll]) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = base + u * kThreads + static_cast<int>(threadIdx.x);
                v[u] = load_stream(rv + (i < nvec ? i : nvec - 1));
            }
        };
        auto sum = [&](int base, const u32x4 (&v)[kUnroll]) {
            float part = 0.f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool in = base + u * kThreads + static_cast<int>(threadIdx.x) < nvec;
#pragma unroll
                for (int e = 0; e < 4; ++e) part += in ? term(__uint_as_float(v[u][e])) : 0.f;
            }
            acc += part;
        };
        u32x4 va[kUnroll], vb[kUnroll];
        load(0, va);
#pragma unroll 1
        for (int base = 0; base < nvec; base += 2 * kTileV) {
            load(base + kTileV, vb);
            __builtin_amdgcn_sched_barrier(0);
            sum(base, va);
            load(base + 2 * kTileV, va);
            __builtin_amdgcn_sched_barrier(0);
            if (base + kTileV < nvec) sum(base + kTileV, vb);
        }
    } else {
        float part = 0.f;
        int n = 0;
        for (int i = threadIdx.x; i < a.V; i += kThreads) {
            part += term(row[i]);
            if (++n == 64) { acc += part; part = 0.f; n = 0; }
        }
        acc += part;
    }
    acc = wave_sum(acc);
    bad = wave_or(bad);
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    if (lane == 0) { s_z[wid] = acc; s_f[wid] = bad; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double S = 0.0;
        uint32_t f = 0;
        for (int w = 0; w < kThreads / kWave; ++w) { S += s_z[w]; f |= s_f[w]; }
        a.S[blockIdx.x] = S;
        a.flags[blockIdx.x] = (f || !(S > 0.0)) ? kFlagInvalid : 0u;
    }
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        __builtin_nontemporal_store(load_stream(src + i), dst + i);
}

// Read-only streaming probe: every 16-byte vector once, non-temporal.  Each
// workgroup reads runs of 4 x 256 consecutive vectors (16 KiB), striding over
// the buffer by the grid.  The xor of the data decides a store that practically
// never happens, so the loads cannot be dropped.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n,
                                                         uint32_t* __restrict__ sink) {
    constexpr int kU = 4;
    const size_t stride = static_cast<size_t>(gridDim.x) * 256 * kU;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (size_t base = static_cast<size_t>(blockIdx.x) * 256 * kU; base < n; base += stride) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const size_t i = base + static_cast<size_t>(u) * 256 + threadIdx.x;
            v[u] = i < n ? load_stream(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u];
    }
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9e3779b9u) sink[0] = x;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* __restrict__ dst, size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = 0u;
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, void* sink, hipStream_t s) {
    const size_t n = bytes / 16;
    size_t blocks = (n + 1023) / 1024;
    if (blocks > 2048) blocks = 2048;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), n, static_cast<uint32_t*>(sink));
    return hipGetLastError();
}

hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 4;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<uint32_t*>(dst), n);
    return hipGetLastError();
}

hipError_t launch_rowstats(const RowStatsArgs& a, hipStream_t s, Timing t) {
    const bool vec = vec_ok(a.base, a.V, a.dtype ? 2 : 4);
    dim3 grid(a.R), block(kThreads);
    if (a.dtype == 1) {
        if (vec) launch_timed(t, rowstats_kernel<1, true>, grid, block, 0, s, a);
        else launch_timed(t, rowstats_kernel<1, false>, grid, block, 0, s, a);
    } else {
        if (vec) launch_timed(t, rowstats_kernel<0, true>, grid, block, 0, s, a);
        else launch_timed(t, rowstats_kernel<0, false>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_power_sums(const PowerSumArgs& a, hipStream_t s) {
    if (vec_ok(a.q, a.V, 4)) hipLaunchKernelGGL(power_sums_kernel<true>, dim3(a.R), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(power_sums_kernel<false>, dim3(a.R), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 16;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

}  // namespace sv
