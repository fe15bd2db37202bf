// decode_mla.hip -- split-KV decode over a shared latent KV (qk 576 / v 512).
//
// The scheme of the kernelbot amd-mixed-mla submission 588924 page
// (_flash_splitk writes per-split un-normalised acc, row max and row sum;
// _reduce_splitk rescales every split by exp2(m_s - M) and divides by the
// combined sum) and of the AstrAI v1.3.9 page (attn_decode_split_kv_mma.cuh:
// query heads of one kv head packed into the MMA row tile; a separate
// combine kernel). Keys are whole kv rows; values are their first 512
// channels, read from the same LDS tile.
//
// Split kernel: one work group (4 waves, one per SIMD, one group per CU)
// owns 64 rows = (query token, head of the kv group) pairs of one sequence
// and one key split. Latent tiles of 64 keys x 576 channels (72 KB) are
// double-buffered in LDS and filled by buffer loads that write LDS directly,
// so the next tile streams in while the current one is computed. Per tile:
//   QK: wave w computes the S^T block (keys 32*(w/2).., rows 32*(w%2)..) with
//       36 steps of v_mfma_f32_32x32x16_bf16 (Q^T lives in registers);
//   softmax: the two waves of a row block exchange their row maxima in LDS
//       and write P (bf16) and each row's rescale factor to LDS;
//   PV: wave w owns 128 of the 512 output channels for all 64 rows and
//       accumulates O^T = V^T P^T with the V^T operand read by
//       ds_read_b64_tr_b16; the rescale is skipped when no row max grew.
// Combine kernel: one thread per (row, 16 channels) merges the splits.
#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int BN = 64;                   // keys per tile
constexpr int ROWS = kDecodeRows;        // 64
constexpr int NTHREADS = 256;
constexpr int KSTEPS = DQK / 16;         // 36
constexpr int ROWB = DQK * 2;            // 1152 bytes per latent row
constexpr int CPR = DQK / 8;             // 72 chunks of 16 bytes per row
constexpr int TILEB = BN * ROWB;         // 73728 bytes per tile
constexpr int LOADS = BN * CPR / NTHREADS;  // 18 chunks per thread per tile
constexpr int PSTR = BN + 8;             // padded P row (elements): 144 bytes, conflict-free 16-byte reads
constexpr float kLazyRescale = 8.0f;

// 1152-byte rows put consecutive rows 8 chunks apart in the 16-chunk bank
// line; this XOR (< 8, so it stays inside a row's aligned 8-chunk groups)
// makes 16 consecutive rows x one chunk, and 4 consecutive rows x an aligned
// group of 4 chunks, fall on distinct banks.
MXFA_DEV int swz(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

// One 16-key step (keys K4*16 + 8*lh + 0..7 of the tile) of O^T += V^T P^T for
// this wave's 128 channels and both 32-row blocks.
template <int K4>
MXFA_DEV void pv_k4(f32x16_t (&acc)[4][2], const uint32_t (&va)[8], const uint16_t* sP, int lr, int lh) {
    const bf16x8_t p0 = __builtin_bit_cast(bf16x8_t, load_u32x4(sP + lr * PSTR + K4 * 16 + lh * 8));
    const bf16x8_t p1 = __builtin_bit_cast(bf16x8_t, load_u32x4(sP + (32 + lr) * PSTR + K4 * 16 + lh * 8));
    u32x2_t r[8];
    lds_read_tr16_x8<K4 * 16 * ROWB>(r, va);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const u32x4_t av = {r[2 * db][0], r[2 * db][1], r[2 * db + 1][0], r[2 * db + 1][1]};
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
        acc[db][0] = mfma32x32x16(a, p0, acc[db][0]);
        acc[db][1] = mfma32x32x16(a, p1, acc[db][1]);
    }
}

template <bool kCap>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel(const DecodeParams p) {
    extern __shared__ __attribute__((aligned(1024))) char dsmem[];
    char* sKV = dsmem;                                        // [2][TILEB]
    uint16_t* sP = reinterpret_cast<uint16_t*>(dsmem + 2 * TILEB);  // [ROWS][PSTR]
    float* sMax = reinterpret_cast<float*>(dsmem + 2 * TILEB + ROWS * PSTR * 2);  // [2][ROWS]
    float* sAlpha = sMax + 2 * ROWS;                          // [ROWS]
    float* sSum = sAlpha + ROWS;                              // [2][ROWS]

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

    // Keys any row of the group can see, cut to this split (splits are tile aligned).
    const int tok_first = row0 / G;
    const int tok_last = min(row0 + ROWS - 1, nrows - 1) / G;
    const KeyRange first = visible_range(tok_first + off, sk, p.causal, p.window_left, p.window_right);
    const KeyRange last = visible_range(tok_last + off, sk, p.causal, p.window_left, p.window_right);
    const int ntiles_all = (sk + BN - 1) / BN;
    const int tiles_per_split = (ntiles_all + p.splits - 1) / p.splits;
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

    bf16x8_t qreg[KSTEPS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (long long)(q_start + my_tok) * q_tok_stride +
                             (long long)my_head * DQK + lh * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row_valid) v = load_u32x4(qp + ks * 16);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // K operand reads: row kb*32 + lr, chunk ks*2 + lh -> byte offset
    // row*ROWB + (ks/4)*128 + kx[ks%4].
    const int f_lr = swz(lr & 15);
    uint32_t kx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kx[j] = (uint32_t)((kb * 32 + lr) * ROWB + (((j * 2 + lh) ^ f_lr) << 4));
    // V^T operand (transposing reads): 16-lane group gq, lane i reads key row
    // 8*(gq/2) + 4*hi + i/4 of a 16-key step, channels w*128 + db*32 + (gq%2)*16 + 4*(i%4).
    uint32_t vx[2][2];
    {
        const int gq = lane >> 4;
        const int i = lane & 15;
        const int cl = (gq & 1) * 2 + ((i & 3) >> 1);
#pragma unroll
        for (int hi2 = 0; hi2 < 2; ++hi2) {
            const int rowl = 8 * (gq >> 1) + 4 * hi2 + (i >> 2);
            const int fw = swz(rowl);
#pragma unroll
            for (int d1 = 0; d1 < 2; ++d1)
                vx[hi2][d1] = (uint32_t)(rowl * ROWB + ((w * 16 + ((d1 * 4 + cl) ^ fw)) << 4) + (i & 1) * 8);
        }
    }
    // Global -> LDS: chunk position P = n*256 + tid of the tile.
    uint32_t goff[LOADS];
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
        const int P = n * NTHREADS + tid;
        const int row = P / CPR;
        const int c = (P % CPR) ^ swz(row & 15);
        goff[n] = (uint32_t)(((long long)row * kv_tok_stride + c * 8) * 2);
    }
    const uint16_t* KVseg = static_cast<const uint16_t*>(p.kv) + (long long)k_start * kv_tok_stride + (long long)g * DQK;
    auto issue_tile = [&](int kt, int buf) {
        long long bytes = (long long)(sk - kt - 1) * kv_tok_stride * 2 + DQK * 2;
        if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(KVseg + (long long)kt * kv_tok_stride, (uint32_t)bytes);
#pragma unroll
        for (int n = 0; n < LOADS; ++n) buffer_load_lds16(r, sKV + buf * TILEB + (n * NTHREADS + w * 64) * 16, goff[n]);
    };

    // O^T accumulators: channel block db (32 channels at w*128 + db*32), row block rr.
    f32x16_t acc[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        acc[db][0] = f32x16_t{};
        acc[db][1] = f32x16_t{};
    }
    float m_run = -INFINITY;  // running max of row my_row, log2 units (may trail the true max by <= 8)
    float l_part = 0.0f;      // running sum over this lane's keys
    const float c_exp = kCap ? 1.0f : p.x_mul;

    if (lo <= hi) {
        const int kt0 = lo & ~(BN - 1);
        const int ntiles = (hi - kt0) / BN + 1;
        issue_tile(kt0, 0);
        wait_vmem();
        __syncthreads();
        for (int it = 0; it < ntiles; ++it) {
            const int kt = kt0 + it * BN;
            const int buf = it & 1;
            if (it + 1 < ntiles) issue_tile(kt + BN, buf ^ 1);
            const char* tile = sKV + buf * TILEB;
            const bool full = kt >= last.lo && kt + BN - 1 <= first.hi && kt + BN - 1 <= hi && kt >= lo;

            // S^T block (32 keys x 32 rows).
            f32x16_t s = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, load_u32x4(tile + (ks >> 2) * 128 + kx[ks & 3]));
                s = mfma32x32x16(a, qreg[ks], s);
            }
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[r];
                if constexpr (kCap) x = score_to_logit<true>(x, p.x_mul, p.cap_mul, p.cap_out);
                if (!full) {
                    const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    if (key < mine.lo || key > mine.hi || key < lo || key > hi) x = -INFINITY;
                }
                s[r] = x;
                mt = fmaxf(mt, x);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            if (lh == 0) sMax[kb * ROWS + rb * 32 + lr] = mt;
            lds_barrier();
            mt = fmaxf(sMax[rb * 32 + lr], sMax[ROWS + rb * 32 + lr]);
            if constexpr (!kCap) mt *= c_exp;
            const bool grow = mt > m_run + kLazyRescale;
            const float m_new = grow ? mt : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
            m_run = m_new;
            l_part *= alpha;
            const float nb = (m_run == -INFINITY) ? 0.0f : -m_run;
            float psum = 0.0f;
            uint16_t* prow = &sP[(rb * 32 + lr) * PSTR + kb * 32 + 4 * lh];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const float p0 = fast_exp2(fmaf(s[4 * rg + 0], c_exp, nb));
                const float p1 = fast_exp2(fmaf(s[4 * rg + 1], c_exp, nb));
                const float p2 = fast_exp2(fmaf(s[4 * rg + 2], c_exp, nb));
                const float p3 = fast_exp2(fmaf(s[4 * rg + 3], c_exp, nb));
                psum += (p0 + p1) + (p2 + p3);
                const u32x2_t pk = {pack_bf16x2(p0, p1), pack_bf16x2(p2, p3)};
                store_u32x2(prow + 8 * rg, pk);
            }
            l_part += psum;
            if (kb == 0 && lh == 0) sAlpha[rb * 32 + lr] = alpha;
            lds_barrier();

            // O^T += V^T P^T over the tile's 64 keys (4 steps of 16).
            {
                const float a0 = sAlpha[lr];
                const float a1 = sAlpha[32 + lr];
                if (wave_any(a0 != 1.0f || a1 != 1.0f)) {
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        acc[db][0] *= a0;
                        acc[db][1] *= a1;
                    }
                }
            }
            const uint32_t tbase = lds_addr(tile);
            uint32_t va[8];
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                va[2 * db] = tbase + vx[0][db & 1] + (db >> 1) * 128;
                va[2 * db + 1] = tbase + vx[1][db & 1] + (db >> 1) * 128;
            }
            pv_k4<0>(acc, va, sP, lr, lh);
            pv_k4<1>(acc, va, sP, lr, lh);
            pv_k4<2>(acc, va, sP, lr, lh);
            pv_k4<3>(acc, va, sP, lr, lh);
            wait_vmem();
            __syncthreads();
        }
    }

    // Partial (m, l, acc) of this split.
    const float l_wave = l_part + __shfl_xor(l_part, 32);
    __syncthreads();
    if (lh == 0) sSum[kb * ROWS + rb * 32 + lr] = l_wave;
    if (kb == 0 && lh == 0) sMax[rb * 32 + lr] = m_run;
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
        pml[tid] = sMax[tid];
        pml[ROWS + tid] = sSum[tid] + sSum[ROWS + tid];
    }
}

// Merge the splits: M = max_s m_s, w_s = exp2(m_s - M),
// O = sum_s w_s acc_s / sum_s w_s l_s, LSE = ln2 * (M + log2 sum_s w_s l_s).
// One thread per (row, 16 channels); 8 rows per work group.
constexpr int CROWS = NTHREADS / 32;

__global__ __launch_bounds__(NTHREADS) void decode_combine_kernel(const DecodeParams p) {
    int id = blockIdx.x;
    const int rgrp = id % (ROWS / CROWS);
    id /= ROWS / CROWS;
    const int mg = id % p.m_groups;
    id /= p.m_groups;
    const int g = id % p.heads_kv;
    const int b = id / p.heads_kv;
    const int G = p.group;
    const int q_start = p.cu_q[b];
    const int sq = p.cu_q[b + 1] - q_start;
    const int row = rgrp * CROWS + (threadIdx.x >> 5);
    const int r = mg * ROWS + row;
    if (r >= sq * G) return;
    const int d0 = (threadIdx.x & 31) * 16;
    const int tok = r / G;
    const int h = g * G + r % G;
    const long long pidx0 = (((long long)b * p.heads_kv + g) * p.m_groups + mg) * p.splits;
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_ml[(pidx0 + s) * 2 * ROWS + row]);
    float L = 0.0f;
    float o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < p.splits; ++s) {
            const float* pml = p.part_ml + (pidx0 + s) * 2 * ROWS;
            const float ws = fast_exp2(pml[row] - M);
            L += ws * pml[ROWS + row];
            const f32x4_t* a = reinterpret_cast<const f32x4_t*>(p.part_acc + ((pidx0 + s) * ROWS + row) * DV + d0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4_t v = a[j];
                o[4 * j + 0] += ws * v[0];
                o[4 * j + 1] += ws * v[1];
                o[4 * j + 2] += ws * v[2];
                o[4 * j + 3] += ws * v[3];
            }
        }
    }
    const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
    uint16_t* O = static_cast<uint16_t*>(p.o) + ((long long)(q_start + tok) * p.heads_q + h) * DV + d0;
    u32x4_t v0, v1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v0[j] = pack_bf16x2(o[2 * j] * inv, o[2 * j + 1] * inv);
        v1[j] = pack_bf16x2(o[8 + 2 * j] * inv, o[8 + 2 * j + 1] * inv);
    }
    store_u32x4(O, v0);
    store_u32x4(O + 8, v1);
    if (p.lse && d0 == 0)
        p.lse[(long long)h * p.total_q + q_start + tok] = (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

}  // namespace

size_t decode_split_lds_bytes() { return 2 * TILEB + ROWS * PSTR * 2 + 5 * ROWS * sizeof(float); }

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream) {
    const long long units = (long long)p.batch * p.heads_kv * p.m_groups;
    if (units <= 0) return hipSuccess;
    const long long grid_split = units * p.splits;
    if (grid_split > 0x7fffffffLL || units * (ROWS / CROWS) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const size_t lds = decode_split_lds_bytes();
    // Opt in to more than 64 KB of dynamic LDS (once per kernel instance).
    static const hipError_t attr_cap = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_split_kernel<true>), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    static const hipError_t attr_plain = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_split_kernel<false>), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (p.softcap > 0.0f) {
        if (attr_cap != hipSuccess) return attr_cap;
        hipLaunchKernelGGL((decode_split_kernel<true>), dim3((unsigned)grid_split), dim3(NTHREADS), lds, stream, p);
    } else {
        if (attr_plain != hipSuccess) return attr_plain;
        hipLaunchKernelGGL((decode_split_kernel<false>), dim3((unsigned)grid_split), dim3(NTHREADS), lds, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(units * (ROWS / CROWS))), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mxfa
