// KV commit after a tree verification ("Việc giải mã giả định và EAGLE-3", KV
// cache rollback: the draft's entries are written to scratch and committed on
// acceptance).  The verifier appended the N tree nodes' rows at positions
// prefix[b] + n; the accepted path root..n* (path[b][0..d]) moves to positions
// prefix[b] + 0..d in every plane (layer x K/V), and the logical length becomes
// prefix[b] + d + 1.  A batch row whose path or prefix is malformed, or whose
// last path node lies past the cache's capacity, moves nothing.
//
// One workgroup per (plane, batch row).  The path increases and path[t] >= t,
// so a destination row prefix + t can only be the source of an earlier move
// (path[t'] = t, t' < t): reading every moving row of the plane before writing
// any is enough.  Every wave reads the path itself (lane t holds path[t]) and
// checks it with a ballot, so the loads start without a barrier; the moving
// rows are staged in registers (up to kStageVecs 16-byte vectors per thread)
// and, past that, moved one row after another with a barrier between rows.
// Rows whose layout is not 16-byte aligned move with 4-byte or byte accesses.

#include "common.hpp"
#include "internal.hpp"

namespace sv {

namespace {

// Two waves per block and eight waves per SIMD: the whole grid of a 64-plane,
// 64-row commit is resident at once, each block one round trip to memory (256
// threads x 4 vectors and 64 x 16 measured 10% and 4% slower).
constexpr int kKvThreads = 128;
constexpr int kStageVecs = 8;

template <int MODE>   // 0: 16-byte vectors, 1: 4-byte words, 2: bytes
__global__ __launch_bounds__(kKvThreads, 8) void kv_commit_kernel(KVCommitArgs a) {
    const int pl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & (kWave - 1);
    // the row's path, checked by every wave: node 0, then increasing nodes below N
    const int d = a.accept_len[b];
    const long pre = a.prefix[b];
    const int32_t* pb = a.path + static_cast<long>(b) * a.path_stride;
    const int pt = lane < a.path_stride ? pb[lane] : -1;
    const int prev = __shfl_up(pt, 1, kWave);
    const bool lane_bad = lane <= d && (lane == 0 ? pt != 0 : (pt <= prev || pt >= a.N));
    // the path increases, so its last node is the farthest row read (every row
    // written lies below it): that row must exist in the cache
    const long last = pre + __shfl(pt, d >= 0 && d < kWave ? d : 0, kWave);
    const bool ok = d >= 0 && d < a.path_stride && d < a.N && pre >= 0 && last < a.capacity &&
                    __ballot(lane_bad) == 0ull;
    if (!ok) {
        if (pl == 0 && tid == 0) a.new_len[b] = -1;
        return;
    }
    uint8_t* base = a.kv + static_cast<long>(pl) * a.plane_stride + static_cast<long>(b) * a.batch_stride;
    if (MODE == 0) {
        const int rv = a.row_bytes / 16;                 // vectors per row
        if (static_cast<long>(d) * rv <= kStageVecs * kKvThreads) {
            // every read first, then every write; indices fit 32 bits here
            const int nv = d * rv;                       // vectors that move (rows 1..d)
            // (a row already in place, path[t] == t, is neither read nor written)
            u32x4 v[kStageVecs];
#pragma unroll
            for (int k = 0; k < kStageVecs; ++k) {
                const int j = k * kKvThreads + tid;
                const int t = j < nv ? 1 + j / rv : 0;
                const int src = __shfl(pt, t, kWave);
                if (j < nv && src != t)
                    v[k] = reinterpret_cast<const u32x4*>(base + (pre + src) * a.pos_stride)[j - (t - 1) * rv];
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kStageVecs; ++k) {
                const int j = k * kKvThreads + tid;
                const int t = j < nv ? 1 + j / rv : 0;
                const int src = __shfl(pt, t, kWave);
                if (j < nv && src != t)
                    reinterpret_cast<u32x4*>(base + (pre + t) * a.pos_stride)[j - (t - 1) * rv] = v[k];
            }
        } else {
            for (int t = 1; t <= d; ++t) {
                const int src = __shfl(pt, t, kWave);
                const u32x4* s = reinterpret_cast<const u32x4*>(base + (pre + src) * a.pos_stride);
                u32x4* o = reinterpret_cast<u32x4*>(base + (pre + t) * a.pos_stride);
                if (src != t)
                    for (int c = tid; c < rv; c += kKvThreads) o[c] = s[c];
                __syncthreads();
            }
        }
    } else {
        const int esz = MODE == 1 ? 4 : 1;
        const int re = a.row_bytes / esz;
        for (int t = 1; t <= d; ++t) {
            const int src = __shfl(pt, t, kWave);
            const uint8_t* s = base + (pre + src) * a.pos_stride;
            uint8_t* o = base + (pre + t) * a.pos_stride;
            if (src != t) {
                for (int c = tid; c < re; c += kKvThreads) {
                    if (MODE == 1) reinterpret_cast<uint32_t*>(o)[c] = reinterpret_cast<const uint32_t*>(s)[c];
                    else o[c] = s[c];
                }
            }
            __syncthreads();
        }
    }
    if (pl == 0 && tid == 0) a.new_len[b] = static_cast<int32_t>(pre + d + 1);
}

}  // namespace

hipError_t launch_kv_commit(const KVCommitArgs& a, hipStream_t s, Timing t) {
    if (a.path_stride < 1 || a.path_stride > kWave) return hipErrorInvalidValue;   // lane t holds path[t]
    const auto al = [](long long v, long long m) { return v % m == 0; };
    const long long p = static_cast<long long>(reinterpret_cast<uintptr_t>(a.kv));
    const bool v16 = al(p, 16) && al(a.plane_stride, 16) && al(a.batch_stride, 16) && al(a.pos_stride, 16) &&
                     al(a.row_bytes, 16);
    const bool v4 = al(p, 4) && al(a.plane_stride, 4) && al(a.batch_stride, 4) && al(a.pos_stride, 4) &&
                    al(a.row_bytes, 4);
    const dim3 grid(a.planes, a.B);
    if (v16) launch_timed(t, kv_commit_kernel<0>, grid, dim3(kKvThreads), 0, s, a);
    else if (v4) launch_timed(t, kv_commit_kernel<1>, grid, dim3(kKvThreads), 0, s, a);
    else launch_timed(t, kv_commit_kernel<2>, grid, dim3(kKvThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sv
