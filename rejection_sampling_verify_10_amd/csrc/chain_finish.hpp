// Finish of a top-k chain inside the selection launch (topk.hip).
//
// The loop follows "064 · 投机解码", section 三: for positions k = 0, 1, ...
// accept x_k iff u_k < min(1, p'_k(x_k) / q'_k(x_k)) (acceptance a(x) of
// section 二); at the first rejection j draw one token from
// r = max(0, p'_j - q'_j) normalised (zero mass: from p'_j, as the residual
// routine of "Việc giải mã giả định và EAGLE-3", step 2, does); if nothing is
// rejected draw the bonus token from p'_K.  The draw is an inverse CDF over
// token indices in ascending order driven by u_K.
//
// Hand-over without waiting on the producer side: a selection workgroup stores
// its chunk list as 64 self-validating words (bit 0 set) with device-scope
// stores and retires at once.  One finisher workgroup per batch row, placed
// after every selection unit in the grid (so dispatched after all of them on
// its XCD), polls the words of each position until all are valid, merges them,
// clears them back to zero for the next call, runs test k and draws the token
// that would be emitted if k were the first rejection.  Its waves then pick
// the first rejection from the position records in LDS and write the row's
// outputs.  The polls are bounded: a row whose lists never complete is
// reported as failed instead of hanging the launch.
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

// ---- list words: (value, index, chunk flag, valid) in 64 bits ----
// bits 63..32: order_key(value); bits 31..2: index; bit 1: the chunk's invalid
// flag; bit 0: valid.  Zero = not yet written in this call.
constexpr uint32_t kWordNoIndex = 0x3fffffffu;
__device__ __forceinline__ unsigned long long list_word(pkey_t key, bool flagged) {
    const int i = key_idx(key);
    const uint32_t idx = (i < 0 || i >= static_cast<int>(kWordNoIndex)) ? kWordNoIndex : static_cast<uint32_t>(i);
    return (key & 0xffffffff00000000ull) | (static_cast<unsigned long long>(idx) << 2) |
           (flagged ? 2ull : 0ull) | 1ull;
}
__device__ __forceinline__ pkey_t word_key(unsigned long long w) {
    const uint32_t idx = static_cast<uint32_t>(w) >> 2;
    const int i = idx == kWordNoIndex ? kNoIndex : static_cast<int>(idx);
    return (w & 0xffffffff00000000ull) | (0xffffffffu - static_cast<uint32_t>(i));
}

// Polls per list batch before a row is given up (each poll sleeps ~256 cycles
// and waits for a load): about 0.1 s, thousands of times the time between a
// finisher's dispatch and the completion of the last selection unit.
constexpr int kSpinLimit = 1 << 16;

// Merges the C (<= 16) chunk lists of a row from their words (units unit0 ..
// unit0+C-1), polling until every word is valid, then clears them.  Lane l
// ends with the l-th ranked key of the union; returns false on a poll timeout.
// flagged: some chunk flagged the row.
__device__ __forceinline__ bool merge_words(unsigned long long* words, long unit0, int C, pkey_t& out,
                                            bool& flagged) {
    const int lane = threadIdx.x & (kWave - 1);
    pkey_t acc = empty_key();
    bool ok = true;
    flagged = false;
#pragma unroll 1
    for (int base = 0; base < C; base += kMergeBatch) {
        unsigned long long w[kMergeBatch];
        unsigned long long* p = words + (unit0 + base) * kTopkMax + lane;
        int tries = 0;
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c)
            if (base + c < C) w[c] = ld_agent64(p + c * kTopkMax);
#pragma unroll 1
        for (;; ++tries) {
            bool missing = false;
#pragma unroll
            for (int c = 0; c < kMergeBatch; ++c)
                if (base + c < C) missing |= (w[c] & 1ull) == 0ull;
            if (!__ballot(missing)) break;
            if (tries >= kSpinLimit) { ok = false; break; }
            __builtin_amdgcn_s_sleep(4);
#pragma unroll
            for (int c = 0; c < kMergeBatch; ++c)
                if (base + c < C && (w[c] & 1ull) == 0ull) w[c] = ld_agent64(p + c * kTopkMax);
        }
        bool fl = false;
        pkey_t k[kMergeBatch];
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c) {
            if (base + c < C) {
                fl |= (w[c] & 2ull) != 0ull;
                k[c] = (w[c] & 1ull) ? word_key(w[c]) : empty_key();
                st_agent64(p + c * kTopkMax, 0ull);          // ready for the next call
            }
        }
        flagged |= __ballot(fl) != 0ull;
#pragma unroll
        for (int step = 1; step < kMergeBatch; step <<= 1) {
#pragma unroll
            for (int c = 0; c + step < kMergeBatch; c += 2 * step)
                if (base + c + step < C) wave_merge_keys(k[c], k[c + step]);
        }
        if (base == 0) acc = k[0];
        else wave_merge_keys(acc, k[0]);
    }
    out = acc;
    return ok;
}

// Kept distribution of row (b, k) from the list words; one wave.
__device__ __forceinline__ bool word_row(const TopkLists& t, int b, int k, bool draft, int& idx, double& p,
                                         int& kk) {
    const long unit0 = t.unit_base(b, k) + (draft ? t.Ct : 0);
    pkey_t key;
    bool flagged;
    const bool done = merge_words(t.words, unit0, draft ? t.Cd : t.Ct, key, flagged);
    // Real (non-empty) entries of the merged list; top_k of them are kept.
    const int real = static_cast<int>(__popcll(__ballot(key_idx(key) != kNoIndex)));
    kk = real < t.top_k ? real : t.top_k;
    return kept_distribution(key_val(key), key_idx(key), kk, done && !flagged, draft, t.invT,
                             draft && t.draft_identity, idx, p) &&
           done;
}

// ---- position records: kRecWords words per position (payload in bits 63..32,
// bit 0 valid): y with accept (bit 2), rows unusable (bit 1: E1 / E3 / E4,
// they count only if the walk reaches the position) and inputs invalid (bit 3:
// E2 / E5, they always count); then p'_k(x_k), q'_k(x_k), the draw's mass S
// and the drawn token's probability.  Zero between calls.
static_assert(kRecWords == 5, "record layout");

// Target wave of position (b, k): test k and the token to emit if k is the
// first rejection (residual draw, or from p'_k when the residual has no mass;
// bonus draw for k = K).  (it, pt, kt): the target's kept distribution in index
// order, one entry per lane; (sidx, sp, kd): the draft's, in LDS.  Stores the
// position's record words.
// (uk, uK, x): u_k, u_K and x_k (x unused for k = K), loaded by the caller
// ahead of the list merges.
__device__ __forceinline__ void position_test_draw(const ChainArgs& a, int b, int k, int it, double pt, int kt,
                                                   bool ok, const int32_t* sidx, const double* sp, int kd,
                                                   float uk, float uK, int x) {
    const int K = a.K, V = a.V;
    const int lane = threadIdx.x & (kWave - 1);
    const long rbase = static_cast<long>(b) * (K + 1);
    const bool inputs_ok = u_ok(uk) && u_ok(uK) && (k == K || (x >= 0 && x < V));
    double r = pt, px = 0.0, qx = 0.0;
    bool accept = false;
    if (k < K) {
        px = lane_lookup(it, pt, x);
        qx = lds_lookup(sidx, sp, kd, x);
        double ratio;
        if (qx > 0.0) ratio = px / qx;
        else ratio = px > 0.0 ? INFINITY : 0.0;
        const double thr = ratio < 1.0 ? ratio : 1.0;
        accept = static_cast<double>(uk) < thr;
        const double q = lane < kt ? lds_lookup(sidx, sp, kd, it) : 0.0;
        r = lane < kt ? fmax(pt - q, 0.0) : 0.0;
    }
    double S = wave_sum(r);
    if (!(S > 0.0)) {                       // zero residual: draw from p'_k
        r = pt;
        S = wave_sum(pt);
    }
    const int src = lane_draw(r, lane < kt, static_cast<double>(uK) * S);
    const int y = bcast(it, src);
    const double ry = bcast(r, src);
    if (lane < kRecWords) {
        uint32_t hi;
        uint32_t lo = 1u;
        if (lane == 0) {
            hi = static_cast<uint32_t>(y);
            lo |= (accept ? 4u : 0u) | (ok ? 0u : 2u) | (inputs_ok ? 0u : 8u);
        } else if (lane == 1) {
            hi = __float_as_uint(static_cast<float>(px));
        } else if (lane == 2) {
            hi = __float_as_uint(static_cast<float>(qx));
        } else if (lane == 3) {
            hi = __float_as_uint(static_cast<float>(S));
        } else {
            hi = __float_as_uint(static_cast<float>(ry / S));
        }
        st_agent64(a.recw + (rbase + k) * kRecWords + lane, (static_cast<unsigned long long>(hi) << 32) | lo);
    }
}

// One wave: batch row b from the K+1 position records (lane k = position k,
// K <= 63), polled until complete and then cleared: first rejection j, emitted
// tokens x_0..x_{j-1}, y_j, accept_len = j.
__device__ __forceinline__ void chain_combine(const ChainArgs& a, int b) {
    const int K = a.K;
    const int lane = threadIdx.x & (kWave - 1);
    const long rb = static_cast<long>(b) * (K + 1);
    const bool have = lane <= K;
    unsigned long long* pw = a.recw + (rb + (have ? lane : 0)) * kRecWords;
    unsigned long long w[kRecWords];
#pragma unroll
    for (int i = 0; i < kRecWords; ++i) w[i] = have ? ld_agent64(pw + i) : 1ull;
    bool timeout = false;
#pragma unroll 1
    for (int tries = 0;; ++tries) {
        bool missing = false;
#pragma unroll
        for (int i = 0; i < kRecWords; ++i) missing |= (w[i] & 1ull) == 0ull;
        if (!__ballot(missing)) break;
        if (tries >= kSpinLimit) { timeout = true; break; }
        __builtin_amdgcn_s_sleep(4);
#pragma unroll
        for (int i = 0; i < kRecWords; ++i)
            if ((w[i] & 1ull) == 0ull) w[i] = ld_agent64(pw + i);
    }
    if (have) {
#pragma unroll
        for (int i = 0; i < kRecWords; ++i) st_agent64(pw + i, 0ull);      // ready for the next call
    }
    const int y = static_cast<int>(w[0] >> 32);
    const bool acc = (w[0] & 4ull) != 0ull;
    const bool bad = (w[0] & 2ull) != 0ull;
    const bool inputs_bad = (w[0] & 8ull) != 0ull;
    const float pk = __uint_as_float(static_cast<uint32_t>(w[1] >> 32));
    const float qk = __uint_as_float(static_cast<uint32_t>(w[2] >> 32));
    const float S = __uint_as_float(static_cast<uint32_t>(w[3] >> 32));
    const float py = __uint_as_float(static_cast<uint32_t>(w[4] >> 32));
    // The walk stops at the first position whose rows are unusable (an error) or
    // whose draft token is rejected; invalid tokens or uniforms count anywhere.
    const unsigned long long stop = __ballot(have && (bad || (lane < K && !acc)));
    const int j = stop ? __ffsll(static_cast<long long>(stop)) - 1 : K;
    const bool err = timeout || __ballot(have && inputs_bad) != 0ull || (stop && bcast(static_cast<int>(bad), j));
    const int yj = bcast(y, j);
    const float Sj = bcast(S, j), pyj = bcast(py, j);
    if (have) {
        int tok = -1;
        if (!err) tok = lane < j ? a.x[static_cast<long>(b) * K + lane] : (lane == j ? yj : -1);
        a.out_tokens[rb + lane] = tok;
    }
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    if (diag && lane < K) {
        diag[lane] = (err || lane > j) ? NAN : pk;
        diag[K + lane] = (err || lane > j) ? NAN : qk;
    }
    if (lane == 0) {
        a.out_accept_len[b] = err ? -1 : j;
        if (diag) {
            diag[2 * K] = err ? NAN : Sj;
            diag[2 * K + 1] = err ? NAN : pyj;
        }
    }
}

constexpr int kFinishWaves = 4;
constexpr int kGroupPositions = kFinishWaves / 2;

// Finisher workgroups per batch row: two positions each.
__host__ __device__ inline int finish_groups(int K) { return (K + 1 + kGroupPositions - 1) / kGroupPositions; }

struct FinishSmem {
    int32_t sidx[kGroupPositions][kWave];     // the draft rows' kept entries, index order
    double sp[kGroupPositions][kWave];
    int32_t skd[kGroupPositions], sok[kGroupPositions];
};

// Finisher workgroup g of batch row b: positions k = 2g + p (p = 0, 1), wave
// 2p merging target row k, wave 2p+1 draft row k.  The row's last group then
// combines the row.
__device__ __forceinline__ void chain_finish_group(const ChainArgs& a, int b, int g, FinishSmem& fs) {
    const int K = a.K;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int p = wid >> 1;
    const bool draft_wave = (wid & 1) != 0;
    const int k = kGroupPositions * g + p;
    const TopkLists& t = a.tk;
    // The finish is the launch's critical path once the selection units run
    // out: its waves take precedence over co-resident selection waves.
    __builtin_amdgcn_s_setprio(3);
    int it = kNoIndex, kt = 0;
    double pt = 0.0;
    bool ok = false;
    float uk = 0.f, uK = 0.f;
    int x = 0;
    if (k <= K && !draft_wave) {            // issued before the merges
        const long rbase = static_cast<long>(b) * (K + 1);
        uk = a.u[rbase + k];
        uK = a.u[rbase + K];
        if (k < K) x = a.x[static_cast<long>(b) * K + k];
    }
    if (k <= K) {
        if (!draft_wave) {
            ok = word_row(t, b, k, false, it, pt, kt);
        } else if (k < K) {
            int id, kd;
            double pd;
            const bool okd = word_row(t, b, k, true, id, pd, kd);
            fs.sidx[p][lane] = id;
            fs.sp[p][lane] = pd;
            if (lane == 0) { fs.skd[p] = kd; fs.sok[p] = okd; }
        } else if (lane == 0) {
            fs.skd[p] = 0;
            fs.sok[p] = 1;
        }
    }
    __syncthreads();
    if (k <= K && !draft_wave)
        position_test_draw(a, b, k, it, pt, kt, ok && fs.sok[p] != 0, fs.sidx[p], fs.sp[p], fs.skd[p], uk, uK, x);
    if (g == finish_groups(K) - 1 && wid == 0) chain_combine(a, b);
}

}  // namespace sv
