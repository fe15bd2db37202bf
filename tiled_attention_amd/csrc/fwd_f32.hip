// fwd_f32.hip -- fp32 attention forward (dense and packed), fp32 throughout.
//
// The same tiled online softmax as the bf16 kernel (oxillama-runtime 0.1.0
// page, src/flash_attention.rs, flash_attention), computed on the vector ALU
// in fp32 so that fp32 inputs keep fp32 products: one thread per query row,
// 64 rows per work group (one wave), K/V tiles of 32 keys staged in LDS and
// read as broadcasts.
#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int BM = 64;  // query rows per work group (one per lane)
constexpr int BN = 32;  // keys per tile

template <int D, bool kCap>
__global__ __launch_bounds__(BM) void fwd_f32_kernel(const FwdParams p) {
    __shared__ __attribute__((aligned(16))) float sK[BN * D];
    __shared__ __attribute__((aligned(16))) float sV[BN * D];

    const WorkItem item = map_workgroup(blockIdx.x, p.units, p.units_per_xcd, p.n_qtiles);
    if (item.unit < 0) return;
    const int b = item.unit / p.heads_q;
    const int h = item.unit % p.heads_q;
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
    const int off = sk - sq;
    const long long q_tok = (long long)p.heads_q * D;
    const long long kv_tok = (long long)p.heads_kv * D;
    const float* __restrict__ Q = static_cast<const float*>(p.q);
    const float* __restrict__ K = static_cast<const float*>(p.k);
    const float* __restrict__ V = static_cast<const float*>(p.v);

    const int row_last = min(tile_row0 + BM, sq) - 1;
    const int kv_lo = visible_range(tile_row0 + off, sk, p.causal, p.window_left, p.window_right).lo;
    const int kv_hi = visible_range(row_last + off, sk, p.causal, p.window_left, p.window_right).hi;

    const int qi = tile_row0 + tid;
    const bool q_valid = qi < sq;
    const KeyRange mine = visible_range(qi + off, sk, p.causal, p.window_left, p.window_right);

    float q[D];
    float acc[D];
    {
        const float* qp = Q + (long long)(q_start + qi) * q_tok + (long long)h * D;
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
    float m_run = -INFINITY;
    float l_run = 0.0f;

    if (kv_lo <= kv_hi) {
        for (int kt = kv_lo & ~(BN - 1); kt <= kv_hi; kt += BN) {
            __syncthreads();
            for (int c = tid; c < BN * D / 4; c += BM) {
                const int r = c / (D / 4);
                const int ch = c % (D / 4);
                const int key = kt + r;
                f32x4_t kk = {0.f, 0.f, 0.f, 0.f};
                f32x4_t vv = {0.f, 0.f, 0.f, 0.f};
                if (key < sk) {
                    const long long g = (long long)(k_start + key) * kv_tok + (long long)kvh * D + ch * 4;
                    kk = *reinterpret_cast<const f32x4_t*>(K + g);
                    vv = *reinterpret_cast<const f32x4_t*>(V + g);
                }
                *reinterpret_cast<f32x4_t*>(&sK[r * D + ch * 4]) = kk;
                *reinterpret_cast<f32x4_t*>(&sV[r * D + ch * 4]) = vv;
            }
            __syncthreads();
            if (!q_valid) continue;

            float x[BN];
            float mt = -INFINITY;
#pragma unroll
            for (int j = 0; j < BN; ++j) {
                float s = 0.0f;
#pragma unroll
                for (int c = 0; c < D; ++c) s = fmaf(q[c], sK[j * D + c], s);
                float t = score_to_logit<kCap>(s, p.x_mul, p.cap_mul, p.cap_out);
                const int key = kt + j;
                if (key < mine.lo || key > mine.hi) t = -INFINITY;
                x[j] = t;
                mt = fmaxf(mt, t);
            }
            const float m_new = fmaxf(m_run, mt);
            const float base = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m_run - base);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
            for (int j = 0; j < BN; ++j) {
                const float pj = fast_exp2(x[j] - base);
                l_run += pj;
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] = fmaf(pj, sV[j * D + c], acc[c]);
            }
        }
    }

    if (!q_valid) return;
    const float inv = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    float* O = static_cast<float*>(p.o) + (long long)(q_start + qi) * q_tok + (long long)h * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
        const f32x4_t v = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
        *reinterpret_cast<f32x4_t*>(O + c) = v;
    }
    if (p.lse) {
        const float lse = (l_run > 0.0f) ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
        const long long idx = p.cu_q ? (long long)h * p.total_q + q_start + qi
                                     : ((long long)b * p.heads_q + h) * sq + qi;
        p.lse[idx] = lse;
    }
}

template <int D>
hipError_t launch_d(const FwdParams& args, hipStream_t stream) {
    FwdParams p = args;
    p.n_qtiles = (p.seqlen_q + BM - 1) / BM;
    p.units = p.batch * p.heads_q;
    p.units_per_xcd = (p.units + kXcds - 1) / kXcds;
    const long long grid = (long long)kXcds * p.n_qtiles * p.units_per_xcd;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (p.softcap > 0.0f)
        hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)grid), dim3(BM), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)grid), dim3(BM), 0, stream, p);
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
