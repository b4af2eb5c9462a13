// Exact top-k of logit rows and draft-probability rows.
//
// The sampling transforms must be applied to both distributions before the
// ratio test ("064 · 投机解码", section 二).  Top-k keeps exactly k entries,
// larger value first and lower index on ties.  Both transforms are monotone
// (z/T for logits, q^(1/T) for probabilities), so the kept set is selected on
// the raw values and only the k survivors are ever exponentiated.
//
// Stage 1 (topk_chunk_kernel): each workgroup owns one <= 64 KiB chunk of a
// row and holds it in registers (16 x 16-byte vectors per thread).
//   - Every thread keeps the maximum of each of its vectors.
//   - tau = the smallest, over the 4 waves, of each wave's ceil(k/4)-th
//     largest thread maximum.  At least k distinct elements (those maxima) are
//     >= tau, so every element of the chunk's top-k is >= tau.
//   - Elements >= tau (typically ~1.5k of 16-32k) go to an LDS list; each
//     candidate's rank is the number of candidates that precede it, which
//     writes the chunk's top-k already sorted.  A list that overflows the LDS
//     capacity (heavy ties, -inf rows) takes an exact bisection on the value
//     order plus an index-ordered scan of the tied values instead.
// Stage 2 (topk_rows_kernel): one workgroup per row merges its chunks' sorted
// lists by rank (binary search in the other lists), applies the transform to
// the k survivors in fp64 and writes (index, probability) sorted by index.

#include "common.hpp"
#include "internal.hpp"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kSlots = 16;
constexpr int kCap = 1024;

struct ChunkSmem {
    float cv[kCap];
    int32_t ci[kCap];
    float tau[kWaves];
    int32_t red[kWaves];
    int32_t cnt;
    uint32_t flags;
};

__device__ __forceinline__ uint32_t ordered_key(float v) {
    if (v != v) return 0u;                 // NaN never selected
    if (v == 0.f) v = 0.f;                 // -0 and +0 are equal values
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int block_sum(int v, ChunkSmem& sm) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) sm.red[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += sm.red[w];
    return t;
}

// Exclusive prefix of v over the threads of the block; returns the block total in *total.
__device__ __forceinline__ int block_exclusive(int v, ChunkSmem& sm, int* total) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == kWave - 1) sm.red[wid] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wid) before += sm.red[w];
        all += sm.red[w];
    }
    *total = all;
    return before + incl - v;
}

template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_slot(const char* row, long e0, long end) {
    using E = Elem<DT>;
    if (VEC) return load_stream(reinterpret_cast<const u32x4*>(row + e0 * E::kBytes));
    u32x4 v;
    if (DT == 1) {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = (e0 + 2 * w < end) ? h[e0 + 2 * w] : 0xff80u;
            const uint32_t hi = (e0 + 2 * w + 1 < end) ? h[e0 + 2 * w + 1] : 0xff80u;
            v[w] = lo | (hi << 16);
        }
    } else {
        const uint32_t* f = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = (e0 + w < end) ? f[e0 + w] : 0xff800000u;
    }
    return v;
}

__device__ __forceinline__ float load_elem(const char* row, int dt, long i) {
    return dt ? Elem<1>::scalar(row, i) : Elem<0>::scalar(row, i);
}

// Exact top-k candidates of a chunk when the tau filter lets too many through
// (heavy ties, -inf rows): bisection for the k-th largest value in the total
// order, then every larger element plus the lowest-index elements equal to it.
// Re-reads the chunk from memory; leaves the candidates in sm and returns
// their number (<= top_k).
__device__ __noinline__ int chunk_exact(const char* row, int dt, long start, int len, int top_k, ChunkSmem& sm) {
    const int tid = threadIdx.x;
    uint32_t lo = 0u, hi = 0xffffffffu;
    while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;
        int c = 0;
        for (int i = tid; i < len; i += kThreads) c += ordered_key(load_elem(row, dt, start + i)) >= mid;
        if (block_sum(c, sm) >= top_k) lo = mid;
        else hi = mid - 1u;
    }
    const uint32_t kappa = lo;
    __syncthreads();
    if (tid == 0) sm.cnt = 0;
    __syncthreads();
    int gt = 0;
    for (int i = tid; i < len; i += kThreads) {
        const float v = load_elem(row, dt, start + i);
        if (ordered_key(v) > kappa) {
            const int p = atomicAdd(&sm.cnt, 1);
            sm.cv[p] = v;
            sm.ci[p] = static_cast<int32_t>(start + i);
            ++gt;
        }
    }
    const int need = top_k - block_sum(gt, sm);
    int prior = 0;
    for (int base = 0; base < len && prior < need; base += kThreads) {
        const int i = base + tid;
        float v = 0.f;
        int tie = 0;
        if (i < len) {
            v = load_elem(row, dt, start + i);
            tie = ordered_key(v) == kappa;
        }
        int total;
        const int rank = prior + block_exclusive(tie, sm, &total);
        if (tie && rank < need) {
            const int p = atomicAdd(&sm.cnt, 1);
            sm.cv[p] = v;
            sm.ci[p] = static_cast<int32_t>(start + i);
        }
        prior += total;
    }
    __syncthreads();
    return sm.cnt;
}

// Selects the chunk's top-k; writes the sorted list to (ov, oi) and returns the count.
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_topk(const char* row, long start, int len, int top_k, bool is_draft, float* ov,
                           int32_t* oi, int32_t* ocnt, uint32_t* oflag, ChunkSmem& sm) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const long end = start + len;

    // Vector vi (= s*256 + tid) of the chunk holds elements [vi*EPV, vi*EPV + EPV).
    const u32x4* vbase = reinterpret_cast<const u32x4*>(row + start * E::kBytes);
    const int nvec = (len + EPV - 1) / EPV;
    u32x4 d[kSlots];
    float gmax[kSlots];
    float tmax = -INFINITY;
    uint32_t bad = 0;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int vi = s * kThreads + tid;
        const bool valid = vi < nvec;
        if (VEC) d[s] = valid ? load_stream(vbase + vi) : u32x4{0u, 0u, 0u, 0u};
        else d[s] = valid ? load_slot<DT, false>(row, start + static_cast<long>(vi) * EPV, end) : u32x4{0u, 0u, 0u, 0u};
        float g = -INFINITY;
        if (valid) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float v = E::get(d[s], e);
                g = fmaxf(g, v);
                bad |= (v != v);
                if (is_draft) bad |= (v < 0.f) & (VEC || vi * EPV + e < len);
            }
        }
        gmax[s] = g;
        tmax = fmaxf(tmax, g);
    }

    // Lower bound on the chunk's k-th largest value.
    const int kw = (top_k + kWaves - 1) / kWaves;
    const float sorted = wave_sort_desc(tmax);
    const float tw = __shfl(sorted, kw - 1, kWave);
    bad = wave_or(bad);
    if (tid == 0) { sm.cnt = 0; sm.flags = 0; }
    if (lane == 0) sm.tau[wid] = tw;
    __syncthreads();
    if (lane == 0 && bad) atomicOr(&sm.flags, kFlagInvalid);
    float tau = sm.tau[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tau = fminf(tau, sm.tau[w]);

#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        if (gmax[s] >= tau) {
            const int i0 = (s * kThreads + tid) * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float v = E::get(d[s], e);
                if (v >= tau && i0 + e < len) {
                    const int p = atomicAdd(&sm.cnt, 1);
                    if (p < kCap) { sm.cv[p] = v; sm.ci[p] = static_cast<int32_t>(start) + i0 + e; }
                }
            }
        }
    }
    __syncthreads();
    int n = sm.cnt;
    if (n > kCap) n = chunk_exact(row, DT, start, len, top_k, sm);

    // Rank selection: position = number of candidates that precede this one.
    for (int c = tid; c < n; c += kThreads) {
        const float v = sm.cv[c];
        const int i = sm.ci[c];
        int rank = 0;
        for (int j = 0; j < n; ++j) rank += precedes(sm.cv[j], sm.ci[j], v, i);
        if (rank < top_k) { ov[rank] = v; oi[rank] = i; }
    }
    if (tid == 0) {
        *ocnt = n < top_k ? n : top_k;
        *oflag = sm.flags;
    }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(TopkChunkArgs a) {
    __shared__ ChunkSmem sm;
    const int unit = blockIdx.x;
    const int Ut = a.Rt * a.Ct;
    float* ov = a.vals + static_cast<long>(unit) * kTopkMax;
    int32_t* oi = a.idx + static_cast<long>(unit) * kTopkMax;
    if (unit < Ut) {
        const int rt = unit / a.Ct, c = unit - rt * a.Ct;
        const int b = rt / a.target_rows_per_batch, k = rt - b * a.target_rows_per_batch;
        const long mem_row = static_cast<long>(b) * a.target_batch_stride + k;
        const char* row = static_cast<const char*>(a.target) + mem_row * a.V * Elem<DT>::kBytes;
        const long start = static_cast<long>(c) * a.chunk_t;
        const int len = static_cast<int>(min(static_cast<long>(a.chunk_t), a.V - start));
        chunk_topk<DT, VEC>(row, start, len, a.top_k, false, ov, oi, a.cnt + unit, a.flags + unit, sm);
    } else {
        const int u = unit - Ut;
        const int rd = u / a.Cd, c = u - rd * a.Cd;
        const char* row = reinterpret_cast<const char*>(a.draft + static_cast<long>(rd) * a.V);
        const long start = static_cast<long>(c) * a.chunk_d;
        const int len = static_cast<int>(min(static_cast<long>(a.chunk_d), a.V - start));
        chunk_topk<0, VEC>(row, start, len, a.top_k, true, ov, oi, a.cnt + unit, a.flags + unit, sm);
    }
}

constexpr int kMaxChunks = 16;

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(TopkRowsArgs a) {
    __shared__ float lv[kMaxChunks * kTopkMax];
    __shared__ int32_t li[kMaxChunks * kTopkMax];
    __shared__ int32_t lcnt[kMaxChunks], loff[kMaxChunks + 1];
    __shared__ float sel_v[kTopkMax];
    __shared__ int32_t sel_i[kTopkMax];
    __shared__ uint32_t s_flags;

    const int r = blockIdx.x;
    const bool draft = r >= a.Rt;
    const int C = draft ? a.Cd : a.Ct;
    const long unit0 = draft ? static_cast<long>(a.Rt) * a.Ct + static_cast<long>(r - a.Rt) * a.Cd
                             : static_cast<long>(r) * a.Ct;
    const int tid = threadIdx.x;
    if (tid == 0) {
        uint32_t f = 0;
        int off = 0;
        for (int c = 0; c < C; ++c) {
            lcnt[c] = a.chunk_cnt[unit0 + c];
            loff[c] = off;
            off += lcnt[c];
            f |= a.chunk_flags[unit0 + c];
        }
        loff[C] = off;
        s_flags = f;
    }
    __syncthreads();
    const int n = loff[C];
    for (int t = tid; t < C * kTopkMax; t += kThreads) {
        const int c = t / kTopkMax, p = t - c * kTopkMax;
        if (p < lcnt[c]) {
            lv[loff[c] + p] = a.chunk_vals[(unit0 + c) * kTopkMax + p];
            li[loff[c] + p] = a.chunk_idx[(unit0 + c) * kTopkMax + p];
        }
    }
    __syncthreads();
    // Merge by rank: own position plus, in every other list, the number of
    // entries that precede this one (lists are sorted, so binary search).
    for (int t = tid; t < n; t += kThreads) {
        int c = 0;
        while (t >= loff[c + 1]) ++c;
        const float v = lv[t];
        const int i = li[t];
        int rank = t - loff[c];
        for (int o = 0; o < C; ++o) {
            if (o == c) continue;
            int lo = loff[o], hi = loff[o + 1];
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (precedes(lv[mid], li[mid], v, i)) lo = mid + 1;
                else hi = mid;
            }
            rank += lo - loff[o];
        }
        if (rank < a.top_k) { sel_v[rank] = v; sel_i[rank] = i; }
    }
    __syncthreads();
    if (tid >= kWave) return;
    const int kk = n < a.top_k ? n : a.top_k;
    const int l = tid;
    const bool have = l < kk;
    const float v = have ? sel_v[l] : 0.f;
    const int idx = have ? sel_i[l] : 0x7fffffff;
    const float v0 = sel_v[0];
    uint32_t flags = s_flags;
    double w = 0.0;
    if (!draft) {
        if (kk == 0 || !(v0 > -INFINITY && v0 < INFINITY)) flags |= kFlagInvalid;
        if (have) w = exp((static_cast<double>(v) - static_cast<double>(v0)) * a.invT);
    } else {
        if (kk == 0 || v0 == INFINITY) flags |= kFlagInvalid;
        if (have && v > 0.f) w = a.draft_identity ? static_cast<double>(v) : pow(static_cast<double>(v), a.invT);
    }
    const double Z = wave_sum(w);
    if (!(Z > 0.0 && Z < INFINITY)) flags |= kFlagInvalid;
    const double p = w / Z;
    // Order by token index for the inverse-CDF draw.
    int pos = 0;
    for (int t = 0; t < kk; ++t) pos += sel_i[t] < idx;
    if (have) {
        a.row_idx[static_cast<long>(r) * kTopkMax + pos] = idx;
        a.row_p[static_cast<long>(r) * kTopkMax + pos] = p;
    }
    if (l == 0) {
        a.row_cnt[r] = kk;
        a.row_flags[r] = flags;
    }
}

}  // namespace

hipError_t launch_topk_chunks(const TopkChunkArgs& a, hipStream_t s) {
    const int esz = a.dtype ? 2 : 4;
    const bool vec = vec_ok(a.target, a.V, esz) && (a.Rd == 0 || vec_ok(a.draft, a.V, 4));
    const unsigned units = static_cast<unsigned>(a.Rt * a.Ct + a.Rd * a.Cd);
    if (units == 0) return hipSuccess;
    if (a.dtype == 1) {
        if (vec) hipLaunchKernelGGL((topk_chunk_kernel<1, true>), dim3(units), dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((topk_chunk_kernel<1, false>), dim3(units), dim3(kThreads), 0, s, a);
    } else {
        if (vec) hipLaunchKernelGGL((topk_chunk_kernel<0, true>), dim3(units), dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((topk_chunk_kernel<0, false>), dim3(units), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_topk_rows(const TopkRowsArgs& a, hipStream_t s) {
    const unsigned rows = static_cast<unsigned>(a.Rt + a.Rd);
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sv
