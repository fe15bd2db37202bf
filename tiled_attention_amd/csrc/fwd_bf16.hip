// fwd_bf16.hip -- bf16 attention forward on gfx950 MFMA (dense and packed).
//
// Tiled online-softmax forward as on the oxillama-runtime 0.1.0 page
// (src/flash_attention.rs, flash_attention: running row max, running sum,
// rescale of the accumulator, final normalisation), in the exp2 domain with
// the scale folded into one multiply after the QK^T contraction (kernelbot
// amd-mixed-mla submission 588924, _flash_fused; scale applied in fp32 after
// the MMA as in the AstrAI v1.3.9 page's attn_mma_utils.cuh), with causal and
// window tiles skipped at tile granularity (flash_attention's causal tile skip,
// extended to the window's lower edge).
//
// Work group: 4 waves, 128 query rows (32 per wave), one (batch, head) unit.
// Each wave computes S^T = K Q^T for a 64-key tile with
// v_mfma_f32_32x32x16_bf16, so lane l owns query row l % 32 and 32 of the 64
// keys: the row max and row sum are in-register reductions plus one exchange
// between the two lane halves. P^T stays in registers as the B operand of
// O^T = V^T P^T (the accumulator layout of S^T is the operand layout of P^T),
// and O^T keeps one query per lane so the online-softmax rescale is one
// multiplier per lane.
#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int BM = 128;       // query rows per work group
constexpr int BN = 64;        // keys per tile
constexpr int NTHREADS = 256; // 4 waves

template <int D, bool kCap>
__global__ __launch_bounds__(NTHREADS) void fwd_bf16_kernel(const FwdParams p) {
    static_assert(D % 32 == 0, "head dim must be a multiple of 32");
    constexpr int KSTEPS = D / 16;  // QK^T contraction steps
    constexpr int DBLK = D / 32;    // 32-wide output blocks
    constexpr int CPR = D / 8;      // 16-byte chunks per K/V row

    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[BN * D];

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
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int lh = lane >> 5;
    const int off = sk - sq;  // bottom-right alignment
    const long long q_tok = (long long)p.heads_q * D;
    const long long kv_tok = (long long)p.heads_kv * D;

    const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(p.q);
    const uint16_t* __restrict__ K = static_cast<const uint16_t*>(p.k);
    const uint16_t* __restrict__ V = static_cast<const uint16_t*>(p.v);

    // Key range of the whole group: lo/hi of a row are non-decreasing in the row.
    const int row_last = min(tile_row0 + BM, sq) - 1;
    const int kv_lo = visible_range(tile_row0 + off, sk, p.causal, p.window_left, p.window_right).lo;
    const int kv_hi = visible_range(row_last + off, sk, p.causal, p.window_left, p.window_right).hi;

    // This wave's rows and their key range.
    const int wrow0 = tile_row0 + wave * 32;
    const int wrow_last = min(wrow0 + 31, sq - 1);
    const bool wave_has_rows = wrow0 < sq;
    const KeyRange wfirst = visible_range(wrow0 + off, sk, p.causal, p.window_left, p.window_right);
    const KeyRange wlast = visible_range(wrow_last + off, sk, p.causal, p.window_left, p.window_right);

    // This lane's query row and its visible keys.
    const int qi = wrow0 + lr;
    const bool q_valid = qi < sq;
    const KeyRange mine = visible_range(qi + off, sk, p.causal, p.window_left, p.window_right);

    // Q^T as the B operand: lane holds row qi, contraction chunk ks*16 + lh*8.
    bf16x8_t qreg[KSTEPS];
    {
        const uint16_t* qp = Q + (long long)(q_start + qi) * q_tok + (long long)h * D + lh * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (q_valid) v = load_u32x4(qp + ks * 16);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    f32x16_t acc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) acc[i] = f32x16_t{};
    float m_run = -INFINITY;  // running max of this row, log2 units
    float l_part = 0.0f;      // running sum over this lane's keys

    if (kv_lo <= kv_hi) {
        for (int kt = kv_lo & ~(BN - 1); kt <= kv_hi; kt += BN) {
            __syncthreads();
            for (int c = tid; c < BN * CPR; c += NTHREADS) {
                const int r = c / CPR;
                const int ch = c % CPR;
                const int key = kt + r;
                u32x4_t kk = {0u, 0u, 0u, 0u};
                u32x4_t vv = {0u, 0u, 0u, 0u};
                if (key < sk) {
                    const long long g = (long long)(k_start + key) * kv_tok + (long long)kvh * D + ch * 8;
                    kk = load_u32x4(K + g);
                    vv = load_u32x4(V + g);
                }
                store_u32x4(&sK[r * D + ch * 8], kk);
                store_u32x4(&sV[r * D + ch * 8], vv);
            }
            __syncthreads();

            // Wave-uniform: does any row of this wave see a key of this tile?
            const int t_last = kt + BN - 1;
            if (!wave_has_rows || kt > wlast.hi || t_last < wfirst.lo) continue;
            // Does every row of this wave see every key of this tile?
            const bool full = t_last < sk && kt >= wlast.lo && t_last <= wfirst.hi;

            f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8_t a = __builtin_bit_cast(
                        bf16x8_t, load_u32x4(&sK[(kb * 32 + lr) * D + ks * 16 + lh * 8]));
                    s[kb] = mfma32x32x16(a, qreg[ks], s[kb]);
                }
            }

            // Logits (log2 units), mask, tile row max.
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = score_to_logit<kCap>(s[kb][r], p.x_mul, p.cap_mul, p.cap_out);
                    if (!full) {
                        const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        if (key < mine.lo || key > mine.hi) x = -INFINITY;
                    }
                    s[kb][r] = x;
                    mt = fmaxf(mt, x);
                }
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            const float base = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m_run - base);
            m_run = m_new;

            float psum = 0.0f;
            uint32_t pk[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(s[kb][r] - base);
                    const float p1 = fast_exp2(s[kb][r + 1] - base);
                    psum += p0 + p1;
                    pk[kb][r >> 1] = pack_bf16x2(p0, p1);
                }
            }
            l_part = l_part * alpha + psum;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;

            // O^T += V^T P^T. P^T operand (kb, half): registers 8*half..8*half+7 of
            // S^T block kb, i.e. keys kb*32 + half*16 + {4*lh + 0..3, 8 + 4*lh + 0..3}.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const u32x4_t pv = {pk[kb][half * 4 + 0], pk[kb][half * 4 + 1],
                                        pk[kb][half * 4 + 2], pk[kb][half * 4 + 3]};
                    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
                    const int key0 = kb * 32 + half * 16 + 4 * lh;
#pragma unroll
                    for (int db = 0; db < DBLK; ++db) {
                        const int col = db * 32 + lr;
                        uint16_t e[8];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            e[t] = sV[(key0 + t) * D + col];
                            e[4 + t] = sV[(key0 + 8 + t) * D + col];
                        }
                        const u32x4_t av = {e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                                            e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
                        acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pb, acc[db]);
                    }
                }
            }
        }
    }

    // Epilogue: combine the two lane halves' sums, normalise, store.
    const float l_row = l_part + __shfl_xor(l_part, 32);
    if (!q_valid) return;
    const float inv = (l_row > 0.0f) ? 1.0f / l_row : 0.0f;
    uint16_t* O = static_cast<uint16_t*>(p.o) + (long long)(q_start + qi) * q_tok + (long long)h * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = db * 32 + 8 * rg + 4 * lh;
            const u32x2_t v = {pack_bf16x2(acc[db][4 * rg + 0] * inv, acc[db][4 * rg + 1] * inv),
                               pack_bf16x2(acc[db][4 * rg + 2] * inv, acc[db][4 * rg + 3] * inv)};
            store_u32x2(O + d, v);
        }
    }
    if (p.lse && lh == 0) {
        const float lse = (l_row > 0.0f) ? (m_run + fast_log2(l_row)) * kLn2 : -INFINITY;
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
        hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mxfa
