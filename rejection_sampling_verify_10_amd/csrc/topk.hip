// Exact top-k of logit rows and draft-probability rows: per-chunk selection.
//
// The sampling transforms must be applied to both distributions before the
// ratio test ("064 · 投机解码", section 二).  Top-k keeps exactly k entries,
// larger value first and lower index on ties.  Both transforms are monotone
// (z/T for logits, q^(1/T) for probabilities), so the kept set is selected on
// the raw values and only the k survivors are ever exponentiated.
//
// topk_chunk_kernel: one workgroup per <= 112 KiB chunk of a target or draft row,
// held in registers (28 x 16-byte non-temporal vectors per thread; three
// workgroups per CU).  Per chunk:
//   - Per vector, a NaN-propagating maximum (v_maximum3_f32): 1.5 VALU ops per
//     bf16 element, 0.5 per fp32 element; the thread maximum carries NaN.
//   - tau = the exact k-th largest of the 256 thread maxima (each wave sorts
//     its 64 maxima; every wave merges the four sorted lists).  At least k
//     distinct elements (those maxima) are >= tau, so the chunk's top-k are.
//   - Elements >= tau (about k + 10 of 16-32k) go to LDS; one wave sorts them
//     with a bitonic network, 64 at a time, merging blocks if there are more.
//     A list that overflows LDS (heavy ties, -inf rows) switches to an exact
//     bisection on the value order plus an index-ordered scan of the ties.
// Chunk lists go to the workspace, units ordered by batch row and position
// (position k: Ct target chunks, then Cd draft chunks when k has a draft row),
// and the verification kernels merge them.  No workgroup waits for another.

#include "chain_finish.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kSlots = 28;           // 16-byte vectors per thread: a chunk of up to 112 KiB
constexpr int kCap = 1024;

constexpr int kStage = kWave;             // staged (lane, vector) pairs per wave
static_assert(kSlots * kThreads * 16 >= kChunkBytes, "a chunk fits the registers of one workgroup");
static_assert(kWaves == kFinishWaves, "a finisher workgroup has the selection's block size");

struct ChunkSmem {
    float cv[kCap];                      // candidates of the chunk
    int32_t ci[kCap];
    uint32_t tkey[kThreads];             // ordered keys of the thread maxima
    u32x4 stage[kWaves][kStage];         // vectors whose maximum reaches tau
    int32_t stage_vi[kWaves][kStage];
    int32_t red[kWaves];
    int32_t cnt;
    uint32_t flags, overflow;
};

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

// Exclusive prefix of v over the threads of the block; the block total in *total.
__device__ __forceinline__ int block_exclusive(int v, ChunkSmem& sm, int* total) {
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
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

__device__ __forceinline__ float load_elem(const char* row, int dt, long i) {
    return dt ? Elem<1>::scalar(row, i) : Elem<0>::scalar(row, i);
}

// Exact candidates when the tau filter lets too many through: bisection for the
// k-th largest value in the total order, then every larger element plus the
// lowest-index elements equal to it.  Re-reads the chunk; leaves the candidates
// in sm and returns their number (<= top_k).
__device__ __noinline__ int chunk_exact(const char* row, int dt, long start, int len, int top_k, ChunkSmem& sm) {
    const int tid = threadIdx.x;
    uint32_t lo = 0u, hi = 0xffffffffu;
    while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;
        int c = 0;
        for (int i = tid; i < len; i += kThreads) c += order_key(load_elem(row, dt, start + i)) >= mid;
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
        if (order_key(v) > kappa) {
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
            tie = order_key(v) == kappa;
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

// Maximum (NaN-propagating) of one 16-byte vector.
template <int DT>
__device__ __forceinline__ float vec_max(const u32x4& d) {
    if (DT == 1) {
        const float a = bf16_lo(d[0]), b = bf16_hi(d[0]), c = bf16_lo(d[1]), e = bf16_hi(d[1]);
        const float f = bf16_lo(d[2]), g = bf16_hi(d[2]), h = bf16_lo(d[3]), k = bf16_hi(d[3]);
        return maximum3(maximum3(a, b, c), maximum3(e, f, g), __builtin_elementwise_maximum(h, k));
    }
    return maximum3(__uint_as_float(d[0]), __uint_as_float(d[1]),
                    __builtin_elementwise_maximum(__uint_as_float(d[2]), __uint_as_float(d[3])));
}
__device__ __forceinline__ float vec_min_f32(const u32x4& d) {
    return minimum3(__uint_as_float(d[0]), __uint_as_float(d[1]),
                    __builtin_elementwise_minimum(__uint_as_float(d[2]), __uint_as_float(d[3])));
}

// Loads one chunk (len elements from `start`) into registers: vector vi = s*256 + tid.
template <int DT, bool VEC>
__device__ __forceinline__ void load_chunk(const char* row, long start, int len, u32x4 (&d)[kSlots]) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    const u32x4* vbase = reinterpret_cast<const u32x4*>(row + start * E::kBytes);
    const int nvec = (len + EPV - 1) / EPV;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int vi = s * kThreads + static_cast<int>(threadIdx.x);
        d[s] = u32x4{0u, 0u, 0u, 0u};
        if (vi < nvec)
            d[s] = VEC ? load_stream(vbase + vi)
                       : load_slot<DT, false>(row, start + static_cast<long>(vi) * EPV, start + len);
    }
}

// Top-k of one register-resident chunk, left sorted in list slot `slot`: as
// (ov, oi, ocnt, oflag), or (WORDS) as 64 list words for a finisher workgroup
// of the same launch (chain_finish.hpp), stored at device scope.
template <int DT, bool VEC, bool WORDS>
__device__ __forceinline__ void select_chunk(u32x4 (&d)[kSlots], const char* row, long start, int len, int top_k,
                                             bool is_draft, float* ov, int32_t* oi, int32_t* ocnt,
                                             uint32_t* oflag, unsigned long long* ow, uint32_t tag,
                                             ChunkSmem& sm) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = wave_id();
    const int nvec = (len + EPV - 1) / EPV;
    float gmax[kSlots];
    float tmax = -INFINITY, tmin = INFINITY;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int vi = s * kThreads + tid;
        gmax[s] = -INFINITY;
        if (vi < nvec) {
            gmax[s] = vec_max<DT>(d[s]);
            if (is_draft) {
                // the -inf padding of a partial vector must not enter the minimum
                if (VEC || (vi + 1) * EPV <= len) {
                    tmin = __builtin_elementwise_minimum(tmin, vec_min_f32(d[s]));
                } else {
                    for (int e = 0; e < EPV; ++e)
                        if (vi * EPV + e < len) tmin = __builtin_elementwise_minimum(tmin, E::get(d[s], e));
                }
            }
        }
        tmax = __builtin_elementwise_maximum(tmax, gmax[s]);
    }
    // The widened values are cheaper to recompute for the few candidate vectors
    // than to keep live: hide the raw registers' provenance from the compiler.
#pragma unroll
    for (int s = 0; s < kSlots; ++s) asm volatile("" : "+v"(d[s]));
    // NaN anywhere (E1/E3) or a negative draft probability (E3) flags the chunk.
    uint32_t bad = (tmax != tmax) || (is_draft && !(tmin >= 0.f));
    bad = wave_or(bad);
    if (tmax != tmax) tmax = -INFINITY;

    // tau: the top_k-th largest of the 256 thread maxima.  Each wave sorts its 64
    // ordered keys; after one barrier every wave merges the four sorted lists
    // itself (two bitonic merges, then one more), so no second barrier is needed.
    sm.tkey[tid] = wave_sort_desc(order_key(tmax));
    if (tid == 0) { sm.cnt = 0; sm.flags = 0; sm.overflow = 0; }
    __syncthreads();
    if (lane == 0 && bad) atomicOr(&sm.flags, kFlagInvalid);
    uint32_t m01 = wave_bitonic_clean(max(sm.tkey[lane], sm.tkey[127 - lane]), true);
    const uint32_t m23 = wave_bitonic_clean(max(sm.tkey[128 + lane], sm.tkey[255 - lane]), false);
    m01 = wave_bitonic_clean(max(m01, m23), true);
    const uint32_t kth = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(m01), top_k - 1));
    const float tau = kth == 0u ? -INFINITY : order_value(kth);

    // Stage the vectors whose maximum reaches tau (about k + 10 per chunk) in
    // wave-private LDS, then let each lane check one staged vector's elements.
    int staged = 0;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const bool pass = gmax[s] >= tau;
        const unsigned long long bal = __ballot(pass);
        if (bal) {
            const int p = staged + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                             __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
            if (pass && p < kStage) {
                sm.stage[wid][p] = d[s];
                sm.stage_vi[wid][p] = s * kThreads + tid;
            }
            staged += __popcll(bal);
        }
    }
    if (staged > kStage) {
        if (lane == 0) sm.overflow = 1;
    } else if (staged > 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const bool mine = lane < staged;
        u32x4 w = u32x4{0u, 0u, 0u, 0u};
        int vi = 0;
        if (mine) {
            w = sm.stage[wid][lane];
            vi = sm.stage_vi[wid][lane];
        }
        int base = 0;
        int total = 0;
        bool take[EPV];
        unsigned long long tb[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float v = E::get(w, e);
            take[e] = mine && v >= tau && vi * EPV + e < len;
            tb[e] = __ballot(take[e]);
            total += __popcll(tb[e]);
        }
        if (lane == 0) base = atomicAdd(&sm.cnt, total);
        base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const int p = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(tb[e] >> 32),
                                                           __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(tb[e]), 0u));
            if (take[e] && p < kCap) {
                sm.cv[p] = E::get(w, e);
                sm.ci[p] = static_cast<int32_t>(start) + vi * EPV + e;
            }
            base += __popcll(tb[e]);
        }
    }
    __syncthreads();
    int n = sm.cnt;
    if (n > kCap || sm.overflow) n = chunk_exact(row, DT, start, len, top_k, sm);
    if (wid != 0) return;

    // One wave: sort 64 candidates at a time and merge the blocks.
    pkey_t key = lane < n ? pair_key(sm.cv[lane], sm.ci[lane]) : empty_key();
    wave_sort_keys(key);
    for (int base = kWave; base < n; base += kWave) {
        pkey_t w = base + lane < n ? pair_key(sm.cv[base + lane], sm.ci[base + lane]) : empty_key();
        wave_sort_keys(w);
        wave_merge_keys(key, w);
    }
    const int kk = n < top_k ? n : top_k;
    if constexpr (WORDS) {
        st_agent64(ow + lane, list_word(lane < kk ? key : empty_key(), sm.flags != 0u, tag));
    } else {
        ov[lane] = key_val(key);            // every slot: past kk the entries are ignored
        oi[lane] = key_idx(key);
        if (lane == 0) {
            *ocnt = kk;
            *oflag = sm.flags;
        }
    }
}

// FIN: a chain call; the grid holds B*Ub selection units followed by one
// finisher workgroup per batch row (chain_finish.hpp).
template <int DT, bool VEC, bool FIN>
__global__ __launch_bounds__(kThreads, 3) void topk_chunk_kernel(TopkChainArgs fa) {
    __shared__ union {
        ChunkSmem sel;
        FinishSmem fin;
    } smu;
    ChunkSmem& sm = smu.sel;
    const TopkChunkArgs& a = fa.sel;
    const long unit = blockIdx.x;
    if constexpr (FIN) {
        const long units = static_cast<long>(a.B) * a.l.Ub;
        if (unit >= units) {
            const int G = finish_groups(a.K);
            const int f = static_cast<int>(unit - units);
            chain_finish_group(fa.ch, f / G, f - (f / G) * G, smu.fin);
            return;
        }
    }
    const TopkLists& t = a.l;
    const int b = static_cast<int>(unit / t.Ub);
    const long local = unit - static_cast<long>(b) * t.Ub;
    const int PB = t.Ct + t.Cd;
    int k = static_cast<int>(local / PB);
    if (k > a.K) k = a.K;
    const int within = static_cast<int>(local - static_cast<long>(k) * PB);
    float* ov = t.vals + unit * kTopkMax;
    int32_t* oi = t.idx + unit * kTopkMax;
    u32x4 d[kSlots];
    if (within < t.Ct) {
        // no target logits: the target rows' lists were written before the launch
        // (the LM-head fusion), only the draft rows are selected here
        if (a.target == nullptr) return;
        const char* row = static_cast<const char*>(a.target) + (static_cast<long>(b) * (a.K + 1) + k) * a.V * Elem<DT>::kBytes;
        const long start = static_cast<long>(within) * t.chunk_t;
        const int len = static_cast<int>(min(static_cast<long>(t.chunk_t), a.V - start));
        load_chunk<DT, VEC>(row, start, len, d);
        select_chunk<DT, VEC, FIN>(d, row, start, len, t.top_k, false, ov, oi, t.cnt + unit, t.flags + unit,
                                   t.words + unit * kTopkMax, t.tag, sm);
    } else {
        const int c = within - t.Ct;
        const char* row = reinterpret_cast<const char*>(a.draft + (static_cast<long>(b) * a.K + k) * a.V);
        const long start = static_cast<long>(c) * t.chunk_d;
        const int len = static_cast<int>(min(static_cast<long>(t.chunk_d), a.V - start));
        load_chunk<0, VEC>(row, start, len, d);
        select_chunk<0, VEC, FIN>(d, row, start, len, t.top_k, true, ov, oi, t.cnt + unit, t.flags + unit,
                                  t.words + unit * kTopkMax, t.tag, sm);
    }
}

}  // namespace

template <bool FIN>
hipError_t launch_selection(const TopkChainArgs& fa, hipStream_t s, Timing t) {
    const TopkChunkArgs& a = fa.sel;
    const int esz = a.dtype ? 2 : 4;
    const bool vec = vec_ok(a.target, a.V, esz) && vec_ok(a.draft, a.V, 4);
    const unsigned units =
        static_cast<unsigned>(static_cast<long>(a.B) * a.l.Ub + (FIN ? static_cast<long>(a.B) * finish_groups(a.K) : 0));
    if (units == 0) return hipSuccess;
    if (a.dtype == 1) {
        if (vec) launch_timed(t, topk_chunk_kernel<1, true, FIN>, dim3(units), dim3(kThreads), 0, s, fa);
        else launch_timed(t, topk_chunk_kernel<1, false, FIN>, dim3(units), dim3(kThreads), 0, s, fa);
    } else {
        if (vec) launch_timed(t, topk_chunk_kernel<0, true, FIN>, dim3(units), dim3(kThreads), 0, s, fa);
        else launch_timed(t, topk_chunk_kernel<0, false, FIN>, dim3(units), dim3(kThreads), 0, s, fa);
    }
    return hipGetLastError();
}

hipError_t launch_topk_chunks(const TopkChunkArgs& a, hipStream_t s, Timing t) {
    TopkChainArgs fa{};
    fa.sel = a;
    return launch_selection<false>(fa, s, t);
}

hipError_t launch_chain_topk(const TopkChainArgs& a, hipStream_t s, Timing t) { return launch_selection<true>(a, s, t); }

}  // namespace sv
