// Wave-level operations on the sorted per-chunk top-k lists: merge a row's
// chunk lists, turn the kept values into the transformed distribution, look
// tokens up and draw by inverse CDF in index order.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace sv {

__device__ __forceinline__ bool u_ok(float u) { return u >= 0.f && u < 1.f; }
__device__ __forceinline__ bool q_ok(float v) { return v >= 0.f && v < INFINITY; }

constexpr int kMergeBatch = 8;

// Merges the C (<= 64) sorted chunk lists of a row (workspace units unit0 ..
// unit0+C-1): lane l ends with the l-th ranked (value, index) of their union.
// Up to kMergeBatch lists are loaded at once, every load issued before any is
// used (a list owns all kTopkMax slots), and merged by a pairwise tree whose
// merges within a level are independent.  Returns the total number of entries;
// flags collects the chunks' flags.
__device__ __forceinline__ int merge_global_lists(const TopkLists& t, long unit0, int C, float& v, int& i,
                                                  uint32_t& flags) {
    const int lane = threadIdx.x & (kWave - 1);
    int nl = 0;
    uint32_t fl = 0u;
    if (lane < C) {
        nl = t.cnt[unit0 + lane];
        fl = t.flags[unit0 + lane];
    }
    pkey_t acc = empty_key();
#pragma unroll 1
    for (int base = 0; base < C; base += kMergeBatch) {
        float w[kMergeBatch];
        int wi[kMergeBatch];
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c) {
            if (base + c < C) {
                const long u = unit0 + base + c;
                w[c] = t.vals[u * kTopkMax + lane];
                wi[c] = t.idx[u * kTopkMax + lane];
            }
        }
        if (base == 0) nl = min(max(nl, 0), kTopkMax);
        pkey_t k[kMergeBatch];
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c)
            if (base + c < C) k[c] = lane < bcast(nl, base + c) ? pair_key(w[c], wi[c]) : empty_key();
#pragma unroll
        for (int step = 1; step < kMergeBatch; step <<= 1) {
#pragma unroll
            for (int c = 0; c + step < kMergeBatch; c += 2 * step)
                if (base + c + step < C) wave_merge_keys(k[c], k[c + step]);
        }
        if (base == 0) acc = k[0];
        else wave_merge_keys(acc, k[0]);
    }
    flags |= wave_or(fl);
    v = key_val(acc);
    i = key_idx(acc);
    return wave_sum(nl);
}

// Sorts the wave's indices ascending (empty lanes carry kNoIndex and end up
// last): a bitonic network on 32-bit keys (index << 6 | lane, indices < 2^26).
// Returns for each lane the lane its index came from, to gather payloads with.
__device__ __forceinline__ int wave_sort_indices(int& i) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr uint32_t kEmpty = 0xffffffc0u;
    uint32_t key = i == kNoIndex ? (kEmpty | lane) : ((static_cast<uint32_t>(i) << 6) | lane);
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t o = xshfl(key, j);
            const bool up = (lane & k) == 0 || k == kWave;
            const bool keep_small = ((lane & j) == 0) == up;
            key = ((o < key) == keep_small) ? o : key;      // a select, no branch
        }
    }
    i = key >= kEmpty ? kNoIndex : static_cast<int>(key >> 6);
    return static_cast<int>(key & 63u);
}

// (index, probability) pairs sorted by index ascending.
template <typename P>
__device__ __forceinline__ void wave_sort_by_index(int& i, P& p) {
    p = lane_gather(p, wave_sort_indices(i));
}

// From a row's ranked top entries (lane l = l-th, kk kept) to its transformed
// distribution in index order: p' = softmax(z/T) over the kept logits (target)
// or q' = q^(1/T) renormalised over the kept probabilities (draft).  Returns
// false when the row is unusable (E1 / E3 / E4).
__device__ __forceinline__ bool kept_distribution(float v, int idx_in, int kk, bool valid, bool draft,
                                                  double invT, bool identity, int& idx, double& p) {
    const int lane = threadIdx.x & (kWave - 1);
    const float v0 = bcast(v, 0);
    const bool have = lane < kk;
    double w = 0.0;
    bool ok = valid && kk > 0;
    if (!draft) {
        ok = ok && v0 > -INFINITY && v0 < INFINITY;
        if (have) w = exp((static_cast<double>(v) - static_cast<double>(v0)) * invT);
    } else {
        ok = ok && v0 < INFINITY;
        if (have && v > 0.f) w = identity ? static_cast<double>(v) : pow(static_cast<double>(v), invT);
    }
    const double Z = wave_sum(w);
    ok = ok && Z > 0.0 && Z < INFINITY;
    p = have ? w / Z : 0.0;
    idx = have ? idx_in : kNoIndex;
    wave_sort_by_index(idx, p);
    return ok;
}

// Probability of token x in a list held one entry per lane (0 if absent).
template <typename P>
__device__ __forceinline__ P lane_lookup(int idx, P p, int x) {
    const unsigned long long m = __ballot(idx == x);
    if (!m) return P(0);
    return bcast(p, __ffsll(static_cast<long long>(m)) - 1);
}

// Probability of token x in an index-sorted LDS list of n entries (0 if absent).
__device__ __forceinline__ double lds_lookup(const int* sidx, const double* sp, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sidx[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return (lo < n && sidx[lo] == x) ? sp[lo] : 0.0;
}

// Inverse-CDF draw over an index-sorted list of weights r (one per lane), C their
// inclusive prefix, with target u*S: first lane whose prefix exceeds the target;
// rounding fallback = last lane with a positive weight.  Returns the lane.
template <typename P>
__device__ __forceinline__ int lane_draw_scanned(P r, P C, bool have, P target) {
    const unsigned long long hit = __ballot(have && r > P(0) && target < C);
    if (hit) return __ffsll(static_cast<long long>(hit)) - 1;
    const unsigned long long pos = __ballot(have && r > P(0));
    return pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
}

// Kept distribution of row (b, k) of a chain or acceptance-rate call: target
// row (draft = false) or draft row; one wave.  Returns false when the row is
// unusable.
__device__ __forceinline__ bool position_row(const TopkLists& t, int b, int k, bool draft, int& idx, double& p,
                                             int& kk) {
    const long unit0 = t.unit_base(b, k) + (draft ? t.Ct : 0);
    float v;
    int i;
    uint32_t flags = 0;
    const int tot = merge_global_lists(t, unit0, draft ? t.Cd : t.Ct, v, i, flags);
    kk = tot < t.top_k ? tot : t.top_k;
    return kept_distribution(v, i, kk, flags == 0u, draft, t.invT, draft && t.draft_identity, idx, p);
}

}  // namespace sv
