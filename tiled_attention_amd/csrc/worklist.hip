// worklist.hip -- the work list of a packed (varlen) forward: every live
// query tile of every segment, longest causal work first.
//
// The segments of a packed batch are known only from cu_seqlens, which live
// on the device. Rather than launching a grid padded to max_seqlen_q for every
// segment (most of whose work groups would find no rows), one small work
// group walks cu_seqlens on the device -- no host synchronisation (the
// mxflashattn 1.4.0 page's api.py keeps device syncs out of the call path) --
// and writes the (segment, q tile) pairs into the caller's workspace, ordered
// by the number of key tiles each q tile streams, most first (the work-group
// order of the kernelbot amd-mixed-mla submission 588924 page's program ids
// over qo_indptr / kv_indptr, sorted so that long items start first and short
// ones fill the tail).
//
// Workspace layout (int32): [0] item count E, [1..3] unused, [4 .. 4 + batch]
// the exclusive prefix sum of the q-tile counts of the segments, then E
// (segment, q tile) pairs. The prefix sums are recomputed on every call, so
// nothing in the workspace needs clearing beforehand.
#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBuckets = 1024;   // work is bucketed as min(kBuckets - 1, tiles >> shift)
constexpr int kLdsBatch = 2048;  // up to this many segments, their lengths and prefix sums stay in LDS

// Key tiles of width bn that q tile t (rows [t*bm, t*bm + bm)) of a segment
// with sq queries and sk keys streams; 0 when no row sees a key.
MXFA_DEV int tile_work(int t, int sq, int sk, int bm, int bn, int causal, int wl, int wr) {
    const int off = sk - sq;
    const int row0 = t * bm;
    const int row_last = min(row0 + bm, sq) - 1;
    const int lo = visible_range(row0 + off, sk, causal, wl, wr).lo;
    const int hi = visible_range(row_last + off, sk, causal, wl, wr).hi;
    if (lo > hi) return 0;
    return (hi - (lo & ~(bn - 1))) / bn + 1;
}

// Segment of item i: the last b with prefix[b] <= i (prefix non-decreasing,
// prefix[0] = 0 <= i < prefix[batch]).
template <typename Ptr>
MXFA_DEV int find_segment(Ptr prefix, int batch, int i) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Inclusive sum over the work group of one value per thread: a scan inside
// each wave (lane shuffles), then over the 16 wave totals; *total gets the
// sum over all threads. swave: kWaves ints of LDS.
MXFA_DEV int block_inclusive_scan(int x, int* swave, int* total) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) swave[w] = x;
    __syncthreads();
    if (w == 0) {
        int v = lane < kWaves ? swave[lane] : 0;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const int y = __shfl_up(v, d, 64);
            if (lane >= d) v += y;
        }
        if (lane < kWaves) swave[lane] = v;
    }
    __syncthreads();
    const int r = x + (w > 0 ? swave[w - 1] : 0);
    *total = swave[kWaves - 1];
    __syncthreads();  // swave is reused by the next scan
    return r;
}

// kLds: the segments' lengths and prefix sums in LDS (batch <= kLdsBatch);
// otherwise read from global memory.
template <bool kLds>
__global__ __launch_bounds__(kThreads) void varlen_worklist_kernel(const WorkListParams p) {
    __shared__ int swave[kWaves];
    __shared__ int hist[kBuckets];
    __shared__ int s_prefix[kLds ? kLdsBatch + 1 : 1];
    __shared__ int s_sq[kLds ? kLdsBatch : 1];
    __shared__ int s_sk[kLds ? kLdsBatch : 1];
    const int tid = threadIdx.x;
    int* const ws = p.ws;
    int* const prefix = ws + 4;
    int2* const items = reinterpret_cast<int2*>(ws + 4 + ((p.batch + 2) & ~1));

    // q-tile counts of the segments -> exclusive prefix sums.
    int running = 0;
    if (tid == 0) {
        prefix[0] = 0;
        if constexpr (kLds) s_prefix[0] = 0;
    }
    for (int b0 = 0; b0 < p.batch; b0 += kThreads) {
        const int b = b0 + tid;
        int nt = 0;
        if (b < p.batch) {
            const int sq = p.cu_q[b + 1] - p.cu_q[b];
            nt = (sq + p.bm - 1) / p.bm;
            if constexpr (kLds) {
                s_sq[b] = sq;
                s_sk[b] = p.cu_k[b + 1] - p.cu_k[b];
            }
        }
        int chunk = 0;
        const int incl = block_inclusive_scan(nt, swave, &chunk);
        if (b < p.batch) {
            prefix[b + 1] = running + incl;
            if constexpr (kLds) s_prefix[b + 1] = running + incl;
        }
        running += chunk;
    }
    const int total = running;
    for (int i = tid; i < kBuckets; i += kThreads) hist[i] = 0;
    if constexpr (!kLds) {
        // prefix[] lives in global memory and is read back by every thread
        // below: a device-scope fence (write back, then invalidate this CU's
        // L1) before the barrier, so no stale cached line is read.
        __threadfence();
    }
    __syncthreads();

    auto item_work = [&](int i, int& b, int& t) {
        if constexpr (kLds) {
            b = find_segment(s_prefix, p.batch, i);
            t = i - s_prefix[b];
            return tile_work(t, s_sq[b], s_sk[b], p.bm, p.bn, p.causal, p.window_left, p.window_right);
        } else {
            b = find_segment(prefix, p.batch, i);
            t = i - prefix[b];
            const int sq = p.cu_q[b + 1] - p.cu_q[b];
            const int sk = p.cu_k[b + 1] - p.cu_k[b];
            return tile_work(t, sq, sk, p.bm, p.bn, p.causal, p.window_left, p.window_right);
        }
    };

    // Histogram of the items' work.
    for (int i = tid; i < total; i += kThreads) {
        int b, t;
        const int w = item_work(i, b, t);
        atomicAdd(&hist[min(kBuckets - 1, w >> p.shift)], 1);
    }
    __syncthreads();

    // Start of each bucket, the heaviest bucket first.
    const int hb = hist[kBuckets - 1 - tid];
    int all = 0;
    const int incl = block_inclusive_scan(hb, swave, &all);
    hist[kBuckets - 1 - tid] = incl - hb;
    __syncthreads();

    // Scatter (segment, q tile) into its bucket's range (order inside a bucket
    // is arbitrary: every item is computed independently of where it runs).
    for (int i = tid; i < total; i += kThreads) {
        int b, t;
        const int w = item_work(i, b, t);
        const int pos = atomicAdd(&hist[min(kBuckets - 1, w >> p.shift)], 1);
        // Only a segment longer than the max_seqlen_q the list was sized
        // for makes more items than the workspace holds: the lightest are
        // dropped (their rows are not computed) and nothing is written past
        // the workspace.
        if (pos < p.list_max) items[pos] = int2{b, t};
    }
    if (tid == 0) ws[0] = (int)min((long long)total, p.list_max);
}

}  // namespace

size_t worklist_bytes(int batch, long long max_items) {
    return (size_t)(4 + ((batch + 2) & ~1)) * sizeof(int) + (size_t)max_items * 2 * sizeof(int);
}

hipError_t launch_varlen_worklist(const WorkListParams& args, hipStream_t stream) {
    WorkListParams p = args;
    // Bucket shift: the largest work (key tiles per q tile) maps below kBuckets.
    const long long max_w = ((long long)p.max_seqlen_k + p.bn - 1) / p.bn + 1;
    int shift = 0;
    while ((max_w >> shift) >= kBuckets) ++shift;
    p.shift = shift;
    if (p.batch <= kLdsBatch)
        hipLaunchKernelGGL(varlen_worklist_kernel<true>, dim3(1), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(varlen_worklist_kernel<false>, dim3(1), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mxfa
