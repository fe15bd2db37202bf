// fwd_f32.hip -- fp32 attention forward (dense and packed), fp32 throughout.
//
// The same tiled online softmax as the bf16 kernel (oxillama-runtime 0.1.0
// page, src/flash_attention.rs, flash_attention), on the vector ALU in fp32 so
// that fp32 inputs keep fp32 products. Work group: 32 query rows, L lanes per
// row (L = 16 at d = 64, 8 at d = 128); the L lanes of a row each take every
// L-th key of a tile and keep their own running (max, sum, accumulator); the
// L partial states of a row are merged with the max/sum correction at the end
// (the split combine of the kernelbot amd-mixed-mla submission 588924 page,
// _reduce_splitk, within a row). K/V tiles are staged in LDS with padded
// rows, so the different keys a wave reads at once fall on different banks.
#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int BM = kFwdF32Rows;  // 32 query rows per work group

// Lanes per query row: 16 at d = 64 (512 threads; each lane's dependent FMA
// chain over a tile is half as long), 8 at d = 128 (256 threads), where the
// row's q and accumulator already take 256 registers per lane.
template <int D>
constexpr int lanes_per_row() {
    return D == 64 ? 16 : 8;
}
template <int D>
constexpr int threads_of() {
    return BM * lanes_per_row<D>();
}

// Keys per tile: 128 at d = 64 (70 KB of LDS; the key range of a 128-token
// problem is then one load round trip instead of four), 32 at d = 128, where
// the row's q and accumulator already take 256 registers.
template <int D>
constexpr int tile_keys() {
    return D == 64 ? 128 : kFwdF32Keys;
}

template <int D, bool kCap>
__global__ __launch_bounds__(threads_of<D>()) void fwd_f32_kernel(const FwdParams p) {
    constexpr int LPR = lanes_per_row<D>();
    constexpr int NTHREADS = threads_of<D>();
    constexpr int BN = tile_keys<D>();
    constexpr int RS = D + 4;  // padded LDS row (floats)
    __shared__ __attribute__((aligned(16))) float sK[BN * RS];
    __shared__ __attribute__((aligned(16))) float sV[BN * RS];

    const WorkItem item = p.worklist ? map_listed(blockIdx.x, p.worklist, p.batch, p.heads_kv, p.group, p.list_max)
                                     : map_workgroup(blockIdx.x, p.batch, p.heads_kv, p.group, p.n_qtiles);
    if (item.b < 0) return;
    const int b = item.b;
    const int h = item.h;
    const int kvh = h / p.group;
    int q_start, sq, k_start, sk;
    if (p.cu_q) {
        q_start = p.cu_q[b];
        sq = p.cu_q[b + 1] - q_start;
        k_start = p.cu_k[b];
        sk = p.cu_k[b + 1] - k_start;
    } else {
        q_start = b * p.seqlen_q;
        sq = p.seqlen_q;
        k_start = b * p.seqlen_k;
        sk = p.seqlen_k;
    }
    const int tile_row0 = item.qtile * BM;
    if (tile_row0 >= sq) return;

    const int tid = threadIdx.x;
    const int t = tid % LPR;  // this lane's key phase
    const int off = sk - sq;
    const long long q_tok = (long long)p.heads_q * D;
    const long long kv_tok = (long long)p.heads_kv * D;
    const float* __restrict__ Q = static_cast<const float*>(p.q);
    const float* __restrict__ K = static_cast<const float*>(p.k);
    const float* __restrict__ V = static_cast<const float*>(p.v);

    const int row_last = min(tile_row0 + BM, sq) - 1;
    const int kv_lo = visible_range(tile_row0 + off, sk, p.causal, p.window_left, p.window_right).lo;
    const int kv_hi = visible_range(row_last + off, sk, p.causal, p.window_left, p.window_right).hi;

    const int qi = tile_row0 + tid / LPR;
    const bool q_valid = qi < sq;
    const KeyRange mine = visible_range(qi + off, sk, p.causal, p.window_left, p.window_right);

    float q[D];
    float acc[D];
    {
        const float* qp = Q + (long long)(q_start + (q_valid ? qi : 0)) * q_tok + (long long)h * D;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            f32x4_t v = {0.f, 0.f, 0.f, 0.f};
            if (q_valid) v = *reinterpret_cast<const f32x4_t*>(qp + c);
            q[c] = v[0];
            q[c + 1] = v[1];
            q[c + 2] = v[2];
            q[c + 3] = v[3];
        }
    }
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = 0.0f;
    float m_run = -INFINITY;  // log2 units
    float l_run = 0.0f;

    if (kv_lo <= kv_hi) {
        for (int kt = kv_lo & ~(BN - 1); kt <= kv_hi; kt += BN) {
            __syncthreads();
            // Every 16-byte chunk of the tile's K and V rows: all loads of
            // this thread are issued before its first LDS write, so the tile
            // costs one memory round trip.
            constexpr int NLD = BN * D / 4 / NTHREADS;
            static_assert(NLD * NTHREADS * 4 == BN * D, "whole chunks per thread");
            f32x4_t kk[NLD], vv[NLD];
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int c = n * NTHREADS + tid;
                const int key = kt + c / (D / 4);
                kk[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                vv[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if (key < sk) {
                    const long long g = (long long)(k_start + key) * kv_tok + (long long)kvh * D + (c % (D / 4)) * 4;
                    kk[n] = *reinterpret_cast<const f32x4_t*>(K + g);
                    vv[n] = *reinterpret_cast<const f32x4_t*>(V + g);
                }
            }
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int c = n * NTHREADS + tid;
                const int r = c / (D / 4);
                const int ch = c % (D / 4);
                *reinterpret_cast<f32x4_t*>(&sK[r * RS + ch * 4]) = kk[n];
                *reinterpret_cast<f32x4_t*>(&sV[r * RS + ch * 4]) = vv[n];
            }
            __syncthreads();

            float x[BN / LPR];
            float mt = -INFINITY;
#pragma unroll
            for (int jj = 0; jj < BN / LPR; ++jj) {
                const int j = jj * LPR + t;
                float s = 0.0f;
#pragma unroll
                for (int c = 0; c < D; c += 4) {
                    const f32x4_t kv4 = *reinterpret_cast<const f32x4_t*>(&sK[j * RS + c]);
                    s = fmaf(q[c], kv4[0], s);
                    s = fmaf(q[c + 1], kv4[1], s);
                    s = fmaf(q[c + 2], kv4[2], s);
                    s = fmaf(q[c + 3], kv4[3], s);
                }
                float lg = score_to_logit<kCap>(s, p.x_mul, p.cap_mul, p.cap_out);
                const int key = kt + j;
                if (key < mine.lo || key > mine.hi) lg = -INFINITY;
                x[jj] = lg;
                mt = fmaxf(mt, lg);
            }
            if (mt > m_run) {
                const float alpha = fast_exp2(m_run - mt);  // m_run = -inf -> 0
                m_run = mt;
                l_run *= alpha;
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] *= alpha;
            }
            const float base = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
            for (int jj = 0; jj < BN / LPR; ++jj) {
                const int j = jj * LPR + t;
                const float pj = fast_exp2(x[jj] - base);
                l_run += pj;
#pragma unroll
                for (int c = 0; c < D; c += 4) {
                    const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(&sV[j * RS + c]);
                    acc[c] = fmaf(pj, v4[0], acc[c]);
                    acc[c + 1] = fmaf(pj, v4[1], acc[c + 1]);
                    acc[c + 2] = fmaf(pj, v4[2], acc[c + 2]);
                    acc[c + 3] = fmaf(pj, v4[3], acc[c + 3]);
                }
            }
        }
    }

    // Merge the 8 lanes of the row: M = max m_t, w_t = exp2(m_t - M),
    // l = sum w_t l_t, acc = sum w_t acc_t.
    float M = m_run;
#pragma unroll
    for (int s = 1; s < LPR; s <<= 1) M = fmaxf(M, __shfl_xor(M, s));
    const float w = (M == -INFINITY) ? 0.0f : fast_exp2(m_run - M);
    float l = l_run * w;
#pragma unroll
    for (int s = 1; s < LPR; s <<= 1) l += __shfl_xor(l, s);
#pragma unroll
    for (int c = 0; c < D; ++c) {
        float a = acc[c] * w;
#pragma unroll
        for (int s = 1; s < LPR; s <<= 1) a += __shfl_xor(a, s);
        acc[c] = a;
    }
    if (!q_valid) return;
    const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
    float* O = static_cast<float*>(p.o) + (long long)(q_start + qi) * q_tok + (long long)h * D;
    // Lane t of the row writes channels [t*D/8, (t+1)*D/8).
#pragma unroll
    for (int c = 0; c < D; c += 4) {
        if (c / (D / LPR) == t) {
            const f32x4_t v = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
            *reinterpret_cast<f32x4_t*>(O + c) = v;
        }
    }
    if (p.lse && t == 0) {
        const float lse = (l > 0.0f) ? (M + fast_log2(l)) * kLn2 : -INFINITY;
        const long long idx = p.cu_q ? (long long)h * p.total_q + q_start + qi
                                     : ((long long)b * p.heads_q + h) * sq + qi;
        p.lse[idx] = lse;
    }
}

template <int D>
hipError_t launch_d(const FwdParams& args, hipStream_t stream) {
    FwdParams p = args;
    p.n_qtiles = (p.seqlen_q + BM - 1) / BM;
    const long long grid = p.worklist ? listed_workgroup_count(p.heads_kv, p.group, p.list_max)
                                      : workgroup_count(p.batch, p.heads_kv, p.group, p.n_qtiles);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (p.softcap > 0.0f)
        hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)grid), dim3(threads_of<D>()), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)grid), dim3(threads_of<D>()), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mxfa
