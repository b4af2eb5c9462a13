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
// stores and retires at once.  One finisher workgroup per position (b, k),
// placed after every selection unit in the grid (so dispatched after all of
// them on its XCD), polls the position's words until all are valid, merges
// them, runs test k and draws the token that would be emitted if k were the
// first rejection, stores the position's record words and clears the list
// words for the next call.  Wave 3 of position K's finisher polls the K+1
// records, picks the first rejection and writes the row's outputs.  Every poll
// is bounded: a row whose words never complete is reported as failed instead
// of hanging the launch.
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

// ---- list words: (value, index, chunk flag, call tag, valid) in 64 bits ----
// bits 63..32: order_key(value); bits 31..23: the call's tag; bits 22..2: index
// (V <= 2^20, so 21 bits hold every index and the no-index code); bit 1: the
// chunk's invalid flag; bit 0: valid.  A word counts only with the valid bit
// and this call's tag: a word a late selection unit of an earlier call stored
// after that call's finisher gave up and cleared its slot is ignored.
constexpr uint32_t kWordNoIndex = 0x1fffffu;
constexpr int kTagShift = 23;
constexpr uint32_t kTagMask = 0x1ffu;
static_assert(kMaxV <= static_cast<int>(kWordNoIndex), "word index field");
__device__ __forceinline__ unsigned long long list_word(pkey_t key, bool flagged, uint32_t tag) {
    const int i = key_idx(key);
    const uint32_t idx = (i < 0 || i >= static_cast<int>(kWordNoIndex)) ? kWordNoIndex : static_cast<uint32_t>(i);
    return (key & 0xffffffff00000000ull) | (static_cast<unsigned long long>(tag & kTagMask) << kTagShift) |
           (static_cast<unsigned long long>(idx) << 2) | (flagged ? 2ull : 0ull) | 1ull;
}
__device__ __forceinline__ pkey_t word_key(unsigned long long w) {
    const uint32_t idx = (static_cast<uint32_t>(w) >> 2) & kWordNoIndex;
    const int i = idx == kWordNoIndex ? kNoIndex : static_cast<int>(idx);
    return (w & 0xffffffff00000000ull) | (0xffffffffu - static_cast<uint32_t>(i));
}
// A list or record word written by this call (valid bit and tag).
__device__ __forceinline__ bool word_here(unsigned long long w, uint32_t tag) {
    return (w & 1ull) != 0ull && ((static_cast<uint32_t>(w) >> kTagShift) & kTagMask) == (tag & kTagMask);
}

// Polls per list batch before a row is given up (each poll sleeps ~256 cycles
// and waits for a load): about 0.1 s by default (TopkLists::spin_limit),
// thousands of times the time between a finisher's dispatch and the completion
// of the last selection unit.

// Merges the C (<= 64) chunk lists of a row from their words (units unit0 ..
// unit0+C-1), polling until every word is valid.  Lane l ends with the l-th
// ranked key of the union; returns false on a poll timeout.  flagged: some
// chunk flagged the row.  The caller clears the words (clear_words) once it has
// no more loads to wait for: the vector memory counter retires in order, so a
// load issued after these stores would wait for their write-through.
__device__ __forceinline__ bool merge_words(unsigned long long* words, long unit0, int C, pkey_t& out,
                                            bool& flagged, uint32_t tag, int spin_limit) {
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
                if (base + c < C) missing |= !word_here(w[c], tag);
            if (!__ballot(missing)) break;
            if (tries >= spin_limit) { ok = false; break; }
            __builtin_amdgcn_s_sleep(4);
#pragma unroll
            for (int c = 0; c < kMergeBatch; ++c)
                if (base + c < C && !word_here(w[c], tag)) w[c] = ld_agent64(p + c * kTopkMax);
        }
        bool fl = false;
        pkey_t k[kMergeBatch];
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c) {
            if (base + c < C) {
                const bool here = word_here(w[c], tag);
                fl |= here && (w[c] & 2ull) != 0ull;
                k[c] = here ? word_key(w[c]) : empty_key();
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

// Zeroes the words of C lists (units unit0 ..), ready for the next call.
__device__ __forceinline__ void clear_words(unsigned long long* words, long unit0, int C) {
    unsigned long long* p = words + unit0 * kTopkMax + (threadIdx.x & (kWave - 1));
#pragma unroll 1
    for (int c = 0; c < C; ++c) st_agent64(p + c * kTopkMax, 0ull);
}

// Kept distribution of a merged row in fp32, one wave: lane l holds the l-th
// ranked (value v, index) of the row, kk of them kept.  Target rows (draft =
// false): w_l = exp((v_l - v_0)/T) = 2^((v_l - v_0) * k1), k1 = log2(e)/T.
// Draft rows: w_l = (v_l / v_0)^(1/T) (v_l / v_0 when T = 1), the same
// distribution as q^(1/T) renormalised, with every weight in [0, 1].  p_l =
// w_l / sum w.  Returns false when the row is unusable (E1 / E3 / E4).  fp32
// keeps the probabilities within a few units in the seventh digit of the fp64
// values, far inside the 1e-5 agreement the test and draw decisions need.
__device__ __forceinline__ bool kept_dist32(float v, int idx_in, int kk, bool valid, bool draft, float k1,
                                            float invT, bool identity, int& idx, float& p) {
    const int lane = threadIdx.x & (kWave - 1);
    const float v0 = bcast(v, 0);
    const bool have = lane < kk;
    float w = 0.f;
    bool ok = valid && kk > 0;
    if (!draft) {
        ok = ok && v0 > -INFINITY && v0 < INFINITY;
        if (have) w = exp2f((v - v0) * k1);
    } else {
        ok = ok && v0 < INFINITY;
        if (have && v > 0.f) {
            const float r = v / v0;
            w = identity ? r : exp2f(log2f(r) * invT);
        }
    }
    const float Z = wave_sum(w);
    ok = ok && Z > 0.f && Z < INFINITY;
    p = have ? w / Z : 0.f;
    idx = have ? idx_in : kNoIndex;
    return ok;
}

// Nucleus cut of a row's kept entries (lane l = l-th largest, kk kept): the
// length of the shortest prefix whose mass reaches top_p, the probabilities
// taken in fp64 (exp((v - v0)/T) for the target, q^(1/T) for the draft) so that
// the cut is decided on the same numbers to ~1e-16.  The nucleus keeps the
// tokens whose preceding mass is below top_p (and whose probability is not 0).
__device__ __forceinline__ int nucleus_count(float v, int kk, bool draft, double invT, bool identity, float top_p) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool have = lane < kk;
    const double v0 = static_cast<double>(bcast(v, 0));
    double w = 0.0;
    if (have) {
        if (!draft) w = exp((static_cast<double>(v) - v0) * invT);
        else if (v > 0.f) w = identity ? static_cast<double>(v) : pow(static_cast<double>(v), invT);
    }
    const double Z = wave_sum(w);
    const double p = Z > 0.0 ? w / Z : 0.0;
    const double incl = wave_inclusive_scan(p);
    const bool keep = have && p > 0.0 && (incl - p) < static_cast<double>(top_p);
    return static_cast<int>(__popcll(__ballot(keep)));
}

// ---- position records: kRecWords words per position (payload in bits 63..32,
// the call's tag in bits 31..23 as in the list words, bit 0 valid): y with
// accept (bit 2), rows unusable (bit 1: E1 / E3 / E4, they count only if the
// walk reaches the position) and inputs invalid (bit 3: E2 / E5, they always
// count); then p'_k(x_k), q'_k(x_k), the draw's mass S and the drawn token's
// probability.  Zero between calls.
static_assert(kRecWords == 5, "record layout");

constexpr int kFinishWaves = 4;

struct FinishSmem {
    pkey_t dkey[kWave];            // wave 2's half of the draft merge
    int32_t didx[kWave];           // the draft's kept entries, value order
    float dq[kWave];
    int32_t tidx[kWave];           // the target's kept indices, value order
    float qpart[kFinishWaves][kWave];   // q'_k at those indices, from wave w's draft entries
    int32_t dkd, dok, dbad;
    int32_t dlate, dlate1;         // lists of wave 2's draft half, of either half, did not arrive
};

// Wave 0 of position (b, k)'s finisher: test k and the token to emit if k is
// the first rejection (residual draw, or from p'_k when the residual has no
// mass; bonus draw for k = K).  (it, pt, kt): the target's kept distribution in
// index order, one entry per lane; the draft's kept entries and the draft
// probability at each target entry (fs.qpart, one part per wave) are in LDS.
// Stores the position's record words.  (uk, uK, x): u_k, u_K and x_k (x unused
// for k = K).
__device__ __forceinline__ void position_test_draw(const ChainArgs& a, int b, int k, int it, float pt, int kt,
                                                   bool ok, bool late, const FinishSmem& fs, float uk, float uK,
                                                   int x) {
    const int K = a.K, V = a.V;
    const int lane = threadIdx.x & (kWave - 1);
    const long rbase = static_cast<long>(b) * (K + 1);
    const bool inputs_ok = u_ok(uk) && u_ok(uK) && (k == K || (x >= 0 && x < V));
    float r = pt, px = 0.f, qx = 0.f;
    bool accept = false;
    if (k < K) {
        const int kd = fs.dkd;
        const int di = lane < kd ? fs.didx[lane] : kNoIndex;
        const float dq = lane < kd ? fs.dq[lane] : 0.f;
        px = lane_lookup(it, pt, x);
        qx = lane_lookup(di, dq, x);
        float ratio;
        if (qx > 0.f) ratio = px / qx;
        else ratio = px > 0.f ? INFINITY : 0.f;
        accept = uk < fminf(ratio, 1.f);
        const float q = fmaxf(fmaxf(fs.qpart[0][lane], fs.qpart[1][lane]), fmaxf(fs.qpart[2][lane], fs.qpart[3][lane]));
        r = lane < kt ? fmaxf(pt - q, 0.f) : 0.f;
    }
    // inverse CDF in index order: S is the last inclusive prefix
    float C = wave_inclusive_scan(r);
    float S = bcast(C, kWave - 1);
    if (!(S > 0.f)) {                       // zero residual: draw from p'_k
        r = pt;
        C = wave_inclusive_scan(r);
        S = bcast(C, kWave - 1);
    }
    const int src = lane_draw_scanned(r, C, lane < kt, uK * S);
    const int y = bcast(it, src);
    const float ry = bcast(r, src);
    if (lane < kRecWords) {
        uint32_t hi;
        uint32_t lo = 1u | ((a.tk.tag & kTagMask) << kTagShift);
        if (lane == 0) {
            hi = static_cast<uint32_t>(y);
            lo |= (accept ? 4u : 0u) | (ok ? 0u : 2u) | (inputs_ok ? 0u : 8u) | (late ? 16u : 0u);
        } else if (lane == 1) {
            hi = __float_as_uint(px);
        } else if (lane == 2) {
            hi = __float_as_uint(qx);
        } else if (lane == 3) {
            hi = __float_as_uint(S);
        } else {
            hi = __float_as_uint(ry / S);
        }
        st_agent64(a.recw + (rbase + k) * kRecWords + lane, (static_cast<unsigned long long>(hi) << 32) | lo);
    }
}

// One wave: batch row b from the K+1 position records (lane k = position k,
// K <= 63), polled until complete and then cleared: first rejection j, emitted
// tokens x_0..x_{j-1}, y_j, accept_len = j.  A row whose records (or, through a
// finisher's flag, whose lists) did not arrive within the poll limit gets
// accept_len = kTimedOut and -1 tokens.
__device__ __forceinline__ void chain_combine(const ChainArgs& a, int b) {
    const int K = a.K;
    const int lane = threadIdx.x & (kWave - 1);
    const long rb = static_cast<long>(b) * (K + 1);
    const bool have = lane <= K;
    unsigned long long* pw = a.recw + (rb + (have ? lane : 0)) * kRecWords;
    // the draft tokens, loaded before any store of this wave (see merge_words)
    const int xl = lane < K ? a.x[static_cast<long>(b) * K + lane] : -1;
    unsigned long long w[kRecWords];
    const uint32_t tag = a.tk.tag;
    const unsigned long long filler = 1ull | (static_cast<unsigned long long>(tag & kTagMask) << kTagShift);
#pragma unroll
    for (int i = 0; i < kRecWords; ++i) w[i] = have ? ld_agent64(pw + i) : filler;
    bool timeout = false;
#pragma unroll 1
    for (int tries = 0;; ++tries) {
        bool missing = false;
#pragma unroll
        for (int i = 0; i < kRecWords; ++i) missing |= !word_here(w[i], tag);
        if (!__ballot(missing)) break;
        if (tries >= a.tk.spin_limit) { timeout = true; break; }
        __builtin_amdgcn_s_sleep(4);
#pragma unroll
        for (int i = 0; i < kRecWords; ++i)
            if (!word_here(w[i], tag)) w[i] = ld_agent64(pw + i);
    }
    const int y = static_cast<int>(w[0] >> 32);
    const bool acc = (w[0] & 4ull) != 0ull;
    const bool bad = (w[0] & 2ull) != 0ull;
    const bool inputs_bad = (w[0] & 8ull) != 0ull;
    const bool late = (w[0] & 16ull) != 0ull;       // a finisher gave up on its lists
    const float pk = __uint_as_float(static_cast<uint32_t>(w[1] >> 32));
    const float qk = __uint_as_float(static_cast<uint32_t>(w[2] >> 32));
    const float S = __uint_as_float(static_cast<uint32_t>(w[3] >> 32));
    const float py = __uint_as_float(static_cast<uint32_t>(w[4] >> 32));
    // The walk stops at the first position whose rows are unusable (an error) or
    // whose draft token is rejected; invalid tokens or uniforms count anywhere.
    const unsigned long long stop = __ballot(have && (bad || (lane < K && !acc)));
    const int j = stop ? __ffsll(static_cast<long long>(stop)) - 1 : K;
    // a position whose lists never arrived is unusable wherever it lies: the row
    // cannot be decided, and it is reported as timed out rather than as bad data
    const bool timed_out = timeout || __ballot(have && late) != 0ull;
    const bool err = timed_out || __ballot(have && inputs_bad) != 0ull || (stop && bcast(static_cast<int>(bad), j));
    const int yj = bcast(y, j);
    const float Sj = bcast(S, j), pyj = bcast(py, j);
    if (have) {
        int tok = -1;
        if (!err) tok = lane < j ? xl : (lane == j ? yj : -1);
        a.out_tokens[rb + lane] = tok;
    }
    float* diag = a.out_diag ? a.out_diag + static_cast<long>(b) * (2 * K + 2) : nullptr;
    if (diag && lane < K) {
        diag[lane] = (err || lane > j) ? NAN : pk;
        diag[K + lane] = (err || lane > j) ? NAN : qk;
    }
    if (lane == 0) {
        a.out_accept_len[b] = timed_out ? kTimedOut : (err ? -1 : j);
        if (diag) {
            diag[2 * K] = err ? NAN : Sj;
            diag[2 * K + 1] = err ? NAN : pyj;
        }
    }
    if (have) {
#pragma unroll
        for (int i = 0; i < kRecWords; ++i) st_agent64(pw + i, 0ull);      // ready for the next call
    }
}

// Finisher workgroups per batch row: one per position.
__host__ __device__ inline int finish_groups(int K) { return K + 1; }

// Finisher workgroup of position (b, k).  Wave 0 merges the target row's chunk
// lists and forms p'_k; waves 1 and 2 merge the two halves of the draft row's
// lists (k < K), wave 2 handing its half to wave 1, which forms q'_k.  All four
// waves then look q'_k up at p'_k's indices, a quarter of the draft entries each,
// and wave 0 tests x_k, draws, and stores the position's record; wave 3 of
// position K's workgroup combines the row.
__device__ __forceinline__ void chain_finish_group(const ChainArgs& a, int b, int k, FinishSmem& fs) {
    const int K = a.K;
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    const TopkLists& t = a.tk;
    // The finish is the launch's critical path once the selection units run
    // out: its waves take precedence over co-resident selection waves.
    __builtin_amdgcn_s_setprio(3);
    const long unit0 = t.unit_base(b, k);
    const int half = (t.Cd + 1) >> 1;
    float uk = 0.f, uK = 0.f;
    int x = 0;
    pkey_t key = empty_key();
    bool flagged = false, done = true;
    if (wid == 0) {
        const long rbase = static_cast<long>(b) * (K + 1);
        uk = a.u[rbase + k];                 // issued before the merges
        uK = a.u[rbase + K];
        if (k < K) x = a.x[static_cast<long>(b) * K + k];
        done = merge_words(t.words, unit0, t.Ct, key, flagged, t.tag, t.spin_limit);
    } else if (wid <= 2 && k < K) {
        const int c0 = wid == 1 ? 0 : half;
        const int cn = wid == 1 ? half : t.Cd - half;
        if (cn > 0) done = merge_words(t.words, unit0 + t.Ct + c0, cn, key, flagged, t.tag, t.spin_limit);
        if (wid == 2) {
            fs.dkey[lane] = key;
            if (lane == 0) { fs.dbad = flagged || !done; fs.dlate = !done; }
        }
    }
    __syncthreads();
    int it = kNoIndex, kt = 0;
    float pt = 0.f;
    bool ok = false;
    if (wid == 0) {
        // real (non-empty) entries of the merged list; top_k of them are kept
        const int real = static_cast<int>(__popcll(__ballot(key_idx(key) != kNoIndex)));
        kt = real < t.top_k ? real : t.top_k;
        if (t.top_p < 1.f) kt = nucleus_count(key_val(key), kt, false, t.invT, false, t.top_p);
        ok = kept_dist32(key_val(key), key_idx(key), kt, done && !flagged, false,
                         static_cast<float>(1.4426950408889634 * t.invT), 0.f, false, it, pt) && done;
        pt = lane_gather(pt, wave_sort_indices(it));     // index order
        fs.tidx[lane] = it;
    } else if (wid == 1 && k < K) {
        wave_merge_keys(key, fs.dkey[lane]);
        const int real = static_cast<int>(__popcll(__ballot(key_idx(key) != kNoIndex)));
        int kd = real < t.top_k ? real : t.top_k;
        if (t.top_p < 1.f) kd = nucleus_count(key_val(key), kd, true, t.invT, t.draft_identity != 0, t.top_p);
        int di;
        float dq;
        const bool okd = kept_dist32(key_val(key), key_idx(key), kd, done && !flagged && !fs.dbad, true, 0.f,
                                     static_cast<float>(t.invT), t.draft_identity != 0, di, dq);
        if (lane == 0) fs.dlate1 = !done || fs.dlate;
        fs.didx[lane] = di;
        fs.dq[lane] = dq;
        if (lane == 0) { fs.dkd = kd; fs.dok = okd; }
    }
    __syncthreads();
    if (k < K) {
        // q'_k at each kept target index: wave w matches draft entries 16w .. 16w+15
        // (past kd they are (kNoIndex, 0) and match nothing that is kept)
        const int ti = fs.tidx[lane];
        const int m0 = wid * 16;
        float q = 0.f;
        if (m0 < fs.dkd) {
            const int di = fs.didx[m0 + (lane & 15)];
            const float dq = fs.dq[m0 + (lane & 15)];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int dm = __builtin_amdgcn_readlane(di, e);
                const float qm = bcast(dq, e);
                q = ti == dm ? qm : q;
            }
        }
        fs.qpart[wid][lane] = q;
        __syncthreads();
    }
    if (wid == 0) {
        const bool late = !done || (k < K && fs.dlate1 != 0);
        position_test_draw(a, b, k, it, pt, kt, ok && (k == K || fs.dok != 0), late, fs, uk, uK, x);
        clear_words(t.words, unit0, t.Ct);
    } else if (wid <= 2 && k < K) {
        const int c0 = wid == 1 ? 0 : half;
        const int cn = wid == 1 ? half : t.Cd - half;
        clear_words(t.words, unit0 + t.Ct + c0, cn);
    }
    if (k == K && wid == 3) chain_combine(a, b);
}

}  // namespace sv
