// The LM head fused with the verification's selection: the target pass that
// yields p[1..gamma+1] ("064 · 投机解码", section 三) computed as logits =
// hidden @ W^T on the matrix cores, with the verification's selection in the
// GEMM's epilogue, so that the [B, K+1, V] logits never reach HBM ("Việc giải
// mã giả định và EAGLE-3": decoding is bound by memory bandwidth; verifying
// K+1 positions takes one forward pass of the target).
//
// GEMM: C[r][v] = sum_h A[r][h] * W[v][h], A = hidden states [R][H], W = head
// [V][H], both bfloat16 and contiguous along h, fp32 accumulation with the
// gfx950 v_mfma_f32_32x32x16_bf16 instruction.  A lane's operand fragment is 8
// consecutive h of one row (16 bytes).  A workgroup of 4 waves computes a 128 x
// 256 tile; each wave a 64 x 128 sub-tile, 2 x 4 blocks of 32 x 32.  The
// workgroup stages 64 h of its 128 hidden rows and 256 head rows at a time in
// LDS (the next step's global loads in flight during this step's 32 MFMAs per
// wave), and every wave reads its fragments from there.  The
// M tiles that share one N tile of W are dispatched back to back on the same
// XCD, so that they read that slice of W through one L2.  Every 32 x 32 block
// accumulates k = 0, 16, 32, ... in order from zero, and a row's results do not
// depend on the other rows of its block: recomputing a block gives the same
// bits (the fixup below relies on it).
//
// Epilogue, per (row, unit of 128 columns = one wave's column span): top-k mode
// keeps the unit's 4 largest (value, column) pairs, larger value first and the
// lower column among equals; greedy mode keeps the largest.  A NaN logit flags
// the unit.
//
// Merge, per row: the exact top_k (<= 64) of the row from its units'
// candidates.  A unit whose 4th candidate is not below the row's top_k-th key
// may hold more of the top_k than it kept: its 128 logits are recomputed (same
// blocks, same order, same bits) and merged.  The result goes, as one list,
// into the hand-over words of a top-k chain launch whose selection covers the
// draft rows only (topk.hip, chain_finish.hpp), or, greedy, into the row's
// argmax for the greedy chain.

#include "chain_finish.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "lists.hpp"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLmThreads = 256;          // 4 waves: 2 over rows x 2 over columns
constexpr int kTileM = 128, kTileN = 256;
constexpr int kMB = 2, kNB = 4;          // a wave's blocks of 32 x 32: 64 rows x 128 columns
constexpr int kUnit = 128;               // columns of one candidate unit
constexpr int kCand = 4;                 // candidates per (row, unit), top-k mode
constexpr int kLdsStride = kUnit + 1;    // floats per staged row (odd: conflict-free row reads)

__device__ __forceinline__ bf16x8 frag_load(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// acc[mb][nb] = A(rows arow[mb]) x W(rows wrow[nb])^T over h = 0..H-1, 16 at a
// time in increasing order, starting from zero.  arow / wrow: this lane's row
// of each block (lane % 32 within the block, clamped into range by the caller);
// the lane's 8 values of h come from offset (lane / 32) * 8 of each 16.
template <int MB, int NB>
__device__ __forceinline__ void mma_blocks(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                           const int (&arow)[MB], const int (&wrow)[NB], int H,
                                           f32x16 (&acc)[MB][NB]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int koff = (lane >> 5) * 8;
    const uint16_t* pa[MB];
    const uint16_t* pw[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) pa[i] = A + static_cast<long>(arow[i]) * H + koff;
#pragma unroll
    for (int j = 0; j < NB; ++j) pw[j] = W + static_cast<long>(wrow[j]) * H + koff;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[MB], fw[NB], na[MB], nw[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[i] = frag_load(pa[i]);
#pragma unroll
    for (int j = 0; j < NB; ++j) fw[j] = frag_load(pw[j]);
    for (int k0 = 0; k0 < H; k0 += 16) {
        // the next step's fragments are in flight while this step multiplies
        const int kn = k0 + 16 < H ? k0 + 16 : k0;
#pragma unroll
        for (int i = 0; i < MB; ++i) na[i] = frag_load(pa[i] + kn);
#pragma unroll
        for (int j = 0; j < NB; ++j) nw[j] = frag_load(pw[j] + kn);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fw[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[i] = na[i];
#pragma unroll
        for (int j = 0; j < NB; ++j) fw[j] = nw[j];
    }
}

// Row (within its 32-row block) of accumulator register r of this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Inserts key x into the descending list k[0..3] (the 4 largest kept).
__device__ __forceinline__ void top4_insert(pkey_t (&k)[kCand], pkey_t x) {
    const pkey_t k0 = k[0], k1 = k[1], k2 = k[2];
    k[3] = max(k[3], min(k2, x));
    k[2] = max(k2, min(k1, x));
    k[1] = max(k1, min(k0, x));
    k[0] = max(k0, x);
}

// Tile mapping: the M tiles of one N tile on the same XCD, back to back.
struct TileId {
    int m, n;
};
__device__ __forceinline__ TileId tile_of(int block, int mtiles) {
    const int xcd = block & 7, slot = block >> 3;
    TileId t;
    t.m = slot % mtiles;
    t.n = (slot / mtiles) * 8 + xcd;
    return t;
}

// The workgroup's operands per step of 64 h: rows of 64 bf16 (128 bytes, 8
// chunks of 16) padded to 144 bytes, so that consecutive rows of a fragment
// read start 36 banks apart and 16 of them hit 16 different groups of 4 banks.
// One LDS buffer (two workgroups per CU fit); the next step waits in registers.
constexpr int kKS = 64;                          // h per staged step (four MFMA steps)
constexpr int kRowC = 9;                         // 16-byte chunks per staged row (8 + 1 of padding)
struct GemmStage {
    u32x4 a[kTileM * kRowC];                     // hidden-state rows
    u32x4 b[kTileN * kRowC];                     // head rows
};
union TileSmem {
    GemmStage g;
    float stage[4][32 * kLdsStride];             // the epilogue's per-wave slabs
};

template <bool GREEDY>
__global__ __launch_bounds__(kLmThreads, 2) void lmhead_tile_kernel(LMHeadArgs a) {
    __shared__ TileSmem sm;
    const int mtiles = (a.R + kTileM - 1) / kTileM;
    const TileId t = tile_of(blockIdx.x, mtiles);
    if (t.n * kTileN >= a.V) return;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = wave_id();
    const int wm = wid >> 1, wn = wid & 1;
    const int m0 = t.m * kTileM + wm * 64, n0 = t.n * kTileN + wn * kUnit;
    const int H = a.H;

    // global -> LDS copy of one step: thread t moves chunk (t % 8) of rows t / 8 + 32 i,
    // 4 rows of hidden states and 8 of the head
    constexpr int kRA = kTileM / 32, kRB = kTileN / 32;
    const int part = tid & 7, r0 = tid >> 3;
    int oa[kRA], ob[kRB];
#pragma unroll
    for (int i = 0; i < kRA; ++i) oa[i] = min(t.m * kTileM + r0 + 32 * i, a.R - 1) * H + part * 8;
#pragma unroll
    for (int i = 0; i < kRB; ++i) ob[i] = min(t.n * kTileN + r0 + 32 * i, a.V - 1) * H + part * 8;
    u32x4 ra[kRA], rb[kRB];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kRA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a.hidden + static_cast<long>(oa[i]) + k0);
#pragma unroll
        for (int i = 0; i < kRB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(a.weight + static_cast<long>(ob[i]) + k0);
    };
    const int ls = r0 * kRowC + part;
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < kRA; ++i) sm.g.a[ls + 32 * kRowC * i] = ra[i];
#pragma unroll
        for (int i = 0; i < kRB; ++i) sm.g.b[ls + 32 * kRowC * i] = rb[i];
    };
    // this lane's fragment chunks within a staged step: chunk 2*ks + lane/32 of its row
    const int fa0 = (wm * 64 + (lane & 31)) * kRowC + (lane >> 5);
    const int fb0 = (wn * kUnit + (lane & 31)) * kRowC + (lane >> 5);

    f32x16 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x16{};
    const int steps = H / kKS;
    fetch(0);
    stash();
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const bool more = s + 1 < steps;
        if (more) fetch((s + 1) * kKS);           // the next step's operands in flight
#pragma unroll
        for (int ks = 0; ks < kKS / 16; ++ks) {
            bf16x8 xa[kMB], xb[kNB];
#pragma unroll
            for (int i = 0; i < kMB; ++i) xa[i] = __builtin_bit_cast(bf16x8, sm.g.a[fa0 + 32 * kRowC * i + 2 * ks]);
#pragma unroll
            for (int j = 0; j < kNB; ++j) xb[j] = __builtin_bit_cast(bf16x8, sm.g.b[fb0 + 32 * kRowC * j + 2 * ks]);
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            __syncthreads();                      // every wave is done with this step
            stash();
        }
        __syncthreads();
    }

    // Epilogue: one 32-row block at a time through this wave's LDS slab; lane l
    // then scans half of row l % 32 (64 columns) and the two halves combine.
    float* slab = sm.stage[wid];
    const int unit = n0 / kUnit;
    const int rr = lane & 31, half = lane >> 5;
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) slab[acc_row(r, lane) * kLdsStride + 32 * j + (lane & 31)] = acc[i][j][r];
        __syncthreads();
        const int row = m0 + 32 * i + rr;
        const float* src = slab + rr * kLdsStride + half * 64;
        const int c0 = n0 + half * 64;
        uint32_t nan = 0;
        if (GREEDY) {
            pkey_t best = empty_key();
#pragma unroll 8
            for (int c = 0; c < 64; ++c) {
                const float v = src[c];
                const bool in = c0 + c < a.V;
                nan |= in && (v != v);
                const pkey_t kx = in ? pair_key(v, c0 + c) : empty_key();
                best = max(best, kx);
            }
            const pkey_t o = __shfl_xor(best, 32, kWave);
            best = max(best, o);
            nan |= __shfl_xor(nan, 32, kWave);
            if (half == 0 && row < a.R && unit < a.units) {
                a.cand[static_cast<long>(row) * a.units + unit] = best;
                a.cflag[static_cast<long>(row) * a.units + unit] = nan;
            }
        } else {
            pkey_t k[kCand] = {empty_key(), empty_key(), empty_key(), empty_key()};
#pragma unroll 8
            for (int c = 0; c < 64; ++c) {
                const float v = src[c];
                const bool in = c0 + c < a.V;
                nan |= in && (v != v);
                const pkey_t kx = in ? pair_key(v, c0 + c) : empty_key();
                if (kx > k[3]) top4_insert(k, kx);
            }
            // the other half's four, then this lane holds the unit's four
            pkey_t o[kCand];
#pragma unroll
            for (int q = 0; q < kCand; ++q) o[q] = __shfl_xor(k[q], 32, kWave);
#pragma unroll
            for (int q = 0; q < kCand; ++q) top4_insert(k, o[q]);
            nan |= __shfl_xor(nan, 32, kWave);
            if (half == 0 && row < a.R && unit < a.units) {
                pkey_t* out = a.cand + (static_cast<long>(row) * a.units + unit) * kCand;
#pragma unroll
                for (int q = 0; q < kCand; ++q) out[q] = k[q];
                a.cflag[static_cast<long>(row) * a.units + unit] = nan;
            }
        }
        __syncthreads();
    }
}

// The 128 logits of unit u for row r, recomputed exactly as the tile kernel
// computed them (the same 32 x 32 blocks, the same order), as keys, one wave:
// lane l returns the keys of columns u*128 + 32*j + l % 32 for j = 0..3 in
// out[j] when it holds row r (lanes of the right half), else empty keys.
__device__ __forceinline__ void unit_recompute(const LMHeadArgs& a, int r, int u, pkey_t (&out)[kNB],
                                               uint32_t& nan) {
    const int lane = threadIdx.x & (kWave - 1);
    const int mblk = r & ~31, rho = r & 31;
    int arow[1] = {min(mblk + (lane & 31), a.R - 1)};
    int wrow[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) wrow[j] = min(u * kUnit + 32 * j + (lane & 31), a.V - 1);
    f32x16 acc[1][kNB];
    mma_blocks<1, kNB>(a.hidden, a.weight, arow, wrow, a.H, acc);
    // row rho sits in register 4*(rho/8) + rho%4 of the lanes with lane/32 = (rho/4)%2
    const int reg = 4 * (rho >> 3) + (rho & 3);
    const bool mine = (lane >> 5) == ((rho >> 2) & 1);
    nan = 0;
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) v = q == reg ? acc[0][j][q] : v;
        const int col = u * kUnit + 32 * j + (lane & 31);
        const bool in = mine && col < a.V;
        nan |= in && (v != v);
        out[j] = in ? pair_key(v, col) : empty_key();
    }
}

// One workgroup (4 waves) per row: the row's exact top_k as one sorted list
// (top-k mode), or its argmax (greedy: one candidate per unit, already exact).
__global__ __launch_bounds__(kLmThreads) void lmhead_merge_kernel(LMHeadArgs a) {
    __shared__ pkey_t part[4][kWave];
    __shared__ int sat[kWave];
    __shared__ int nsat;
    __shared__ uint32_t sflag;
    const int r = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wid = wave_id();
    const bool greedy = a.greedy_arg != nullptr;
    const int ncand = greedy ? 1 : kCand;
    const pkey_t* cand = a.cand + static_cast<long>(r) * a.units * ncand;
    const uint32_t* cf = a.cflag + static_cast<long>(r) * a.units;
    if (threadIdx.x == 0) { nsat = 0; sflag = 0; }
    __syncthreads();
    // every wave merges 64 candidates at a time into its running top 64
    pkey_t acc = empty_key();
    uint32_t nan = 0;
    const long total = static_cast<long>(a.units) * ncand;
    for (long base = static_cast<long>(wid) * kWave; base < total; base += 4 * kWave) {
        pkey_t k = base + lane < total ? cand[base + lane] : empty_key();
        // a batch with nothing above the running 64th key changes nothing
        if (__ballot(k > __shfl(acc, kWave - 1, kWave)) == 0ull) continue;
        wave_sort_keys(k);
        wave_merge_keys(acc, k);
    }
    for (int u = threadIdx.x; u < a.units; u += kLmThreads) nan |= cf[u];
    nan = wave_or(nan);
    part[wid][lane] = acc;
    __syncthreads();
    if (lane == 0 && nan) atomicOr(&sflag, 1u);
    if (wid == 0) {
#pragma unroll
        for (int w = 1; w < 4; ++w) wave_merge_keys(acc, part[w][lane]);
        part[0][lane] = acc;
    }
    __syncthreads();
    acc = part[0][lane];
    const int kk = greedy ? 1 : a.top_k;
    const pkey_t tau = __shfl(acc, kk - 1, kWave);
    // An element of the row's top kk missing from the candidates lies in a unit
    // whose 4 kept keys all exceed it, hence exceed tau (the kk-th largest
    // candidate is at most the row's kk-th largest): only such units need a look.
    if (!greedy) {
        for (int u = threadIdx.x; u < a.units; u += kLmThreads) {
            const pkey_t fourth = cand[static_cast<long>(u) * kCand + kCand - 1];
            if (fourth > tau && key_idx(fourth) != kNoIndex) {
                const int s = atomicAdd(&nsat, 1);
                if (s < kWave) sat[s] = u;
            }
        }
    }
    __syncthreads();
    const int ns = nsat;
    if (wid == 0 && ns > 0) {
        // (rare) recompute those units and merge all but their 4 kept keys
        for (int s = 0; s < ns; ++s) {
            const int u = s < kWave ? sat[s] : 0;
            pkey_t keys[kNB];
            uint32_t nn;
            unit_recompute(a, r, u, keys, nn);
            nan |= wave_or(nn);
            // 128 keys over 64 lanes (only one half of the lanes holds the row):
            // gather them into two sorted batches of 64
            pkey_t b0 = empty_key(), b1 = empty_key();
            const int holder = ((r & 31) >> 2) & 1;
#pragma unroll
            for (int j = 0; j < kNB; ++j) {
                const pkey_t v = __shfl(keys[j], holder * 32 + (lane & 31), kWave);
                if ((j >> 1) == (lane >> 5)) {
                    if (j & 1) b1 = v;
                    else b0 = v;
                }
            }
            // lanes 0..31 hold columns of blocks 0 (b0) and 1 (b1); lanes 32..63 of 2 and 3
            wave_sort_keys(b0);
            wave_sort_keys(b1);
            wave_merge_keys(b0, b1);             // the unit's keys, largest 64, sorted
            // its first four are the candidates already merged
            b0 = lane + kCand < kWave ? __shfl(b0, lane + kCand, kWave) : empty_key();
            wave_merge_keys(acc, b0);
        }
        if (ns > kWave) nan = 1;                 // more than 64 such units: the row is flagged
    }
    if (wid == 0) {
        const bool flagged = nan != 0 || sflag != 0;
        if (a.greedy_arg) {
            if (lane == 0) {
                a.greedy_arg[r] = key_idx(acc);
                a.greedy_flags[r] = flagged ? kFlagInvalid : 0u;
            }
        } else {
            const int b = r / (a.K + 1), k = r - b * (a.K + 1);
            unsigned long long* w = a.words + a.tk.unit_base(b, k) * kTopkMax;
            st_agent64(w + lane, list_word(lane < kk ? acc : empty_key(), flagged, a.tk.tag));
        }
    }
}

}  // namespace

hipError_t launch_lmhead(const LMHeadArgs& a, hipStream_t s, Timing t) {
    const int mtiles = (a.R + kTileM - 1) / kTileM;
    const int ntiles = (a.V + kTileN - 1) / kTileN;
    const int groups = (ntiles + 7) / 8;
    const unsigned blocks = static_cast<unsigned>(8L * groups * mtiles);
    if (a.greedy_arg) launch_timed(t, lmhead_tile_kernel<true>, dim3(blocks), dim3(kLmThreads), 0, s, a);
    else launch_timed(t, lmhead_tile_kernel<false>, dim3(blocks), dim3(kLmThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3(a.R), dim3(kLmThreads), 0, s, a);
    return hipGetLastError();
}

int lmhead_units(int V) { return (V + kUnit - 1) / kUnit; }

}  // namespace sv
