// decode_mla.hip -- split-KV decode over a shared latent KV (qk 576 / v 512).
//
// The scheme of the kernelbot amd-mixed-mla submission 588924 page
// (_flash_splitk writes per-split un-normalised acc, row max and row sum;
// _reduce_splitk rescales every split by exp2(m_s - M) and divides by the
// combined sum) and of the AstrAI v1.3.9 page (attn_decode_split_kv_mma.cuh:
// query heads of one kv head packed into the MMA row tile; a separate
// combine kernel). Keys are whole kv rows; values are their first 512 channels,
// read from the same LDS tile.
//
// Split kernel work group: 4 waves, 64 rows = (query token, head of the kv
// group) pairs of one sequence, one key split. Per 64-key tile:
//   QK: wave w computes the S^T block (keys 32*(w/2).., rows 32*(w%2)..) with
//       36 steps of v_mfma_f32_32x32x16_bf16 (Q^T lives in registers);
//   softmax: the two waves of a row block exchange their row maxima in LDS,
//       write P (bf16) and the rescale factor of each row to LDS;
//   PV: wave w owns 128 of the 512 output channels for all 64 rows and
//       accumulates O^T = V^T P^T, one row per lane column.
// Combine kernel: one work group per 64 rows merges the splits.
#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int BN = 64;             // keys per tile
constexpr int ROWS = kDecodeRows;  // 64
constexpr int KSTR = DQK + 8;      // padded LDS row stride (elements): conflict-free 16-byte reads
constexpr int PSTR = BN + 8;       // padded P row stride
constexpr int NTHREADS = 256;
constexpr int KSTEPS = DQK / 16;   // 36

template <bool kCap>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel(const DecodeParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sKV[BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t sP[ROWS * PSTR];
    __shared__ float sMax[2][ROWS];
    __shared__ float sAlpha[ROWS];
    __shared__ float sSum[2][ROWS];

    int id = blockIdx.x;
    const int sp = id % p.splits;
    id /= p.splits;
    const int mg = id % p.m_groups;
    id /= p.m_groups;
    const int g = id % p.heads_kv;
    const int b = id / p.heads_kv;
    const int G = p.group;

    const int q_start = p.cu_q[b];
    const int sq = p.cu_q[b + 1] - q_start;
    const int k_start = p.cu_k[b];
    const int sk = p.cu_k[b + 1] - k_start;
    const int row0 = mg * ROWS;
    const int nrows = sq * G;
    if (row0 >= nrows) return;
    const int off = sk - sq;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int lh = lane >> 5;
    const int kb = w >> 1;  // key block of this wave's S^T block
    const int rb = w & 1;   // row block of this wave's S^T block

    // Keys any row of the group can see, cut to this split.
    const int tok_first = row0 / G;
    const int tok_last = min(row0 + ROWS - 1, nrows - 1) / G;
    const KeyRange first = visible_range(tok_first + off, sk, p.causal, p.window_left, p.window_right);
    const KeyRange last = visible_range(tok_last + off, sk, p.causal, p.window_left, p.window_right);
    const int ntiles = (sk + BN - 1) / BN;
    const int tiles_per_split = (ntiles + p.splits - 1) / p.splits;
    const int s_lo = sp * tiles_per_split * BN;
    const int s_hi = min(sk, (sp + 1) * tiles_per_split * BN) - 1;
    const int lo = max(first.lo, s_lo);
    const int hi = min(last.hi, s_hi);

    // This lane's S^T column: row rb*32 + lr of the group.
    const int my_row = row0 + rb * 32 + lr;
    const int my_tok = my_row / G;
    const bool row_valid = my_row < nrows;
    const int my_head = g * G + my_row % G;
    const KeyRange mine = visible_range(my_tok + off, sk, p.causal, p.window_left, p.window_right);

    const long long q_tok_stride = (long long)p.heads_q * DQK;
    const long long kv_tok_stride = (long long)p.heads_kv * DQK;
    const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(p.q);
    const uint16_t* __restrict__ KV = static_cast<const uint16_t*>(p.kv);

    bf16x8_t qreg[KSTEPS];
    {
        const uint16_t* qp = Q + (long long)(q_start + my_tok) * q_tok_stride + (long long)my_head * DQK + lh * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row_valid) v = load_u32x4(qp + ks * 16);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // O^T accumulators: channel block db (32 channels at w*128 + db*32), row block rr.
    f32x16_t acc[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        acc[db][0] = f32x16_t{};
        acc[db][1] = f32x16_t{};
    }
    float m_run = -INFINITY;  // running max of row my_row (log2 units)
    float l_part = 0.0f;      // running sum over this lane's keys

    if (lo <= hi) {
        for (int kt = lo & ~(BN - 1); kt <= hi; kt += BN) {
            __syncthreads();
            // KV tile -> LDS (rows past the sequence are zero).
            for (int c = tid; c < BN * (DQK / 8); c += NTHREADS) {
                const int r = c / (DQK / 8);
                const int ch = c % (DQK / 8);
                const int key = kt + r;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (key < sk)
                    v = load_u32x4(KV + (long long)(k_start + key) * kv_tok_stride + (long long)g * DQK + ch * 8);
                store_u32x4(&sKV[r * KSTR + ch * 8], v);
            }
            __syncthreads();

            const bool full = kt >= last.lo && kt + BN - 1 <= first.hi && kt + BN - 1 <= hi;

            f32x16_t s = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8_t a =
                    __builtin_bit_cast(bf16x8_t, load_u32x4(&sKV[(kb * 32 + lr) * KSTR + ks * 16 + lh * 8]));
                s = mfma32x32x16(a, qreg[ks], s);
            }
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = score_to_logit<kCap>(s[r], p.x_mul, p.cap_mul, p.cap_out);
                if (!full) {
                    const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    if (key < mine.lo || key > mine.hi || key < lo || key > hi) x = -INFINITY;
                }
                s[r] = x;
                mt = fmaxf(mt, x);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            if (lh == 0) sMax[kb][rb * 32 + lr] = mt;
            __syncthreads();
            mt = fmaxf(sMax[0][rb * 32 + lr], sMax[1][rb * 32 + lr]);
            const float m_new = fmaxf(m_run, mt);
            const float base = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m_run - base);
            m_run = m_new;
            float psum = 0.0f;
            uint16_t* prow = &sP[(rb * 32 + lr) * PSTR + kb * 32 + 4 * lh];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const float p0 = fast_exp2(s[4 * rg + 0] - base);
                const float p1 = fast_exp2(s[4 * rg + 1] - base);
                const float p2 = fast_exp2(s[4 * rg + 2] - base);
                const float p3 = fast_exp2(s[4 * rg + 3] - base);
                psum += (p0 + p1) + (p2 + p3);
                const u32x2_t pk = {pack_bf16x2(p0, p1), pack_bf16x2(p2, p3)};
                store_u32x2(prow + 8 * rg, pk);
            }
            l_part = l_part * alpha + psum;
            if (kb == 0 && lh == 0) sAlpha[rb * 32 + lr] = alpha;
            __syncthreads();

            // O^T += V^T P^T over the tile's 64 keys (4 steps of 16).
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const float a = sAlpha[rr * 32 + lr];
#pragma unroll
                for (int db = 0; db < 4; ++db) acc[db][rr] *= a;
            }
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                bf16x8_t pb[2];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
                    pb[rr] = __builtin_bit_cast(bf16x8_t, load_u32x4(&sP[(rr * 32 + lr) * PSTR + k4 * 16 + lh * 8]));
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int col = w * 128 + db * 32 + lr;
                    const int key0 = k4 * 16 + lh * 8;
                    uint32_t e[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        e[t] = (uint32_t)sKV[(key0 + 2 * t) * KSTR + col] |
                               ((uint32_t)sKV[(key0 + 2 * t + 1) * KSTR + col] << 16);
                    const u32x4_t av = {e[0], e[1], e[2], e[3]};
                    const bf16x8_t va = __builtin_bit_cast(bf16x8_t, av);
                    acc[db][0] = mfma32x32x16(va, pb[0], acc[db][0]);
                    acc[db][1] = mfma32x32x16(va, pb[1], acc[db][1]);
                }
            }
        }
    }

    // Partial (m, l, acc) of this split.
    const float l_wave = l_part + __shfl_xor(l_part, 32);
    __syncthreads();
    if (lh == 0) sSum[kb][rb * 32 + lr] = l_wave;
    if (kb == 0 && lh == 0) sMax[0][rb * 32 + lr] = m_run;
    __syncthreads();
    const long long pidx = (((long long)b * p.heads_kv + g) * p.m_groups + mg) * p.splits + sp;
    float* pacc = p.part_acc + pidx * ROWS * DV;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = rr * 32 + lr;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = w * 128 + db * 32 + 8 * rg + 4 * lh;
                const f32x4_t v = {acc[db][rr][4 * rg], acc[db][rr][4 * rg + 1], acc[db][rr][4 * rg + 2],
                                   acc[db][rr][4 * rg + 3]};
                *reinterpret_cast<f32x4_t*>(pacc + (long long)row * DV + d) = v;
            }
        }
    }
    if (tid < ROWS) {
        float* pml = p.part_ml + pidx * 2 * ROWS;
        pml[tid] = sMax[0][tid];
        pml[ROWS + tid] = sSum[0][tid] + sSum[1][tid];
    }
}

// Merge the splits of 64 rows: M = max_s m_s, w_s = exp2(m_s - M),
// O = sum_s w_s acc_s / sum_s w_s l_s, LSE = ln2 * (M + log2 sum_s w_s l_s).
__global__ __launch_bounds__(NTHREADS) void decode_combine_kernel(const DecodeParams p) {
    int id = blockIdx.x;
    const int mg = id % p.m_groups;
    id /= p.m_groups;
    const int g = id % p.heads_kv;
    const int b = id / p.heads_kv;
    const int G = p.group;
    const int q_start = p.cu_q[b];
    const int sq = p.cu_q[b + 1] - q_start;
    const int row0 = mg * ROWS;
    const int nrows = sq * G;
    if (row0 >= nrows) return;
    const long long pidx0 = (((long long)b * p.heads_kv + g) * p.m_groups + mg) * p.splits;
    const int d = threadIdx.x * 2;
    uint16_t* O = static_cast<uint16_t*>(p.o);
    for (int row = 0; row < ROWS && row0 + row < nrows; ++row) {
        const int r = row0 + row;
        const int tok = r / G;
        const int h = g * G + r % G;
        float M = -INFINITY;
        for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_ml[(pidx0 + s) * 2 * ROWS + row]);
        float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
        if (M != -INFINITY) {
            for (int s = 0; s < p.splits; ++s) {
                const float* pml = p.part_ml + (pidx0 + s) * 2 * ROWS;
                const float ws = fast_exp2(pml[row] - M);
                L += ws * pml[ROWS + row];
                const f32x2_t a = *reinterpret_cast<const f32x2_t*>(p.part_acc + ((pidx0 + s) * ROWS + row) * DV + d);
                o0 += ws * a[0];
                o1 += ws * a[1];
            }
        }
        const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
        *reinterpret_cast<uint32_t*>(O + ((long long)(q_start + tok) * p.heads_q + h) * DV + d) =
            pack_bf16x2(o0 * inv, o1 * inv);
        if (p.lse && threadIdx.x == 0)
            p.lse[(long long)h * p.total_q + q_start + tok] = (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream) {
    const long long units = (long long)p.batch * p.heads_kv * p.m_groups;
    if (units <= 0) return hipSuccess;
    const long long grid_split = units * p.splits;
    if (grid_split > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (p.softcap > 0.0f)
        hipLaunchKernelGGL((decode_split_kernel<true>), dim3((unsigned)grid_split), dim3(NTHREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<false>), dim3((unsigned)grid_split), dim3(NTHREADS), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)units), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mxfa
