// decode_gqa.hip -- split-KV decode for standard attention heads (separate K
// and V, head dim 64 or 128) with few query rows per kv head.
//
// The split / combine scheme of the kernelbot amd-mixed-mla submission 588924
// page (_flash_splitk: per split an un-normalised accumulator, row max and row
// sum; _reduce_splitk: rescale every split by exp2(m_s - M), divide by the
// combined sum) and the head packing of the AstrAI v1.3.9 page's split-KV MMA
// decode (the query heads that share one kv head are packed into the rows of
// one MMA tile, so the kv head's keys are read once for all of them).
//
// Split kernel: one work group (2 waves) owns 32 rows = (query token, head of
// the kv group) pairs of one sequence and one kv head, and one key split.
// K and V stream from HBM through a two-stage LDS ring of 64-key tiles,
// filled by buffer loads that write LDS directly (keys past the end read as
// zero). Wave w takes keys 32w..32w+31 of every tile for all 32 rows:
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (lane l: row l % 32, 16 keys),
//   mask, row max (one lane exchange), lazy rescale, exp2,
//   O^T += V^T P^T (P^T is the S^T accumulator packed to bf16; the V^T
//   operand comes from ds_read_b64_tr_b16 in the matching key order).
// Each wave keeps its own running (max, sum, accumulator); at the end the two
// are merged through LDS. With one split the work group writes O and the LSE
// itself; otherwise it writes the split's partial and a combine kernel (one
// thread per row and 4 channels) merges the splits.
//
// The rows hold at most 32 valid (token, head) pairs and usually 8 (one token,
// a group of 8): the MFMAs do up to 4x more work than needed, which costs
// nothing here -- the kernel is bound by the K/V bytes it streams.
#include <type_traits>

#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int ROWS = kGqaRows;   // 32 rows per work group
constexpr int TK = kGqaTile;     // 64 keys per tile, 32 per wave
constexpr int NT = 128;          // 2 waves
constexpr float kLazyRescale = 8.0f;

// Chunk swizzle of an LDS row of 16-byte chunks (physical = logical ^ swz),
// the same pattern as the prefill tiles: 16 rows x one chunk (K operand
// reads) and 4 rows x 4 chunks (transposing V reads) hit distinct banks.
template <int D>
MXFA_DEV int gswz(int row);
template <>
MXFA_DEV int gswz<128>(int row) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
}
template <>
MXFA_DEV int gswz<64>(int row) {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D, bool kCap>
__global__ __launch_bounds__(NT) void decode_gqa_split_kernel(const GqaDecodeParams p) {
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    constexpr int KSTEPS = D / 16;                 // QK^T contraction steps
    constexpr int DBLK = D / 32;                   // 32-channel output blocks
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int ROWB = D * 2;                    // bytes per K/V row
    constexpr int TILEB = TK * ROWB;               // bytes per K or V tile
    constexpr int LOADS = TILEB / (16 * NT);       // loads per thread per K (or V) tile
    constexpr int RPL = NT / CPR;                  // rows per load
    constexpr int SWP = RPL >= 16 ? 1 : 16 / RPL;  // loads per swizzle period
    static_assert(LOADS * 16 * NT == TILEB && LOADS % SWP == 0, "tile must split into whole loads");
    static_assert(ROWS * D * 4 <= TILEB, "the merge buffer reuses one K tile");

    // Separate LDS objects per stage and operand: reads of one never wait for
    // the loads streaming into another.
    __shared__ __attribute__((aligned(TILEB))) char sK0[TILEB];
    __shared__ __attribute__((aligned(TILEB))) char sK1[TILEB];
    __shared__ __attribute__((aligned(TILEB))) char sV0[TILEB];
    __shared__ __attribute__((aligned(TILEB))) char sV1[TILEB];
    __shared__ float sML[2][3][ROWS];  // per wave: row max, row sum (fp32), row sum of the bf16 weights

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
    const int off = sk - sq;  // bottom-right alignment

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int lh = lane >> 5;

    // Keys any row of the group can see, cut to this split (splits are tile aligned).
    const int last_row = min(row0 + ROWS, nrows) - 1;
    const KeyRange first = visible_range(row0 / G + off, sk, p.causal, p.window_left, p.window_right);
    const KeyRange last = visible_range(last_row / G + off, sk, p.causal, p.window_left, p.window_right);
    const int ntiles_all = (sk + TK - 1) / TK;
    const int tiles_per_split = (ntiles_all + p.splits - 1) / p.splits;
    const int s_lo = sp * tiles_per_split * TK;
    const int s_hi = min(sk, (sp + 1) * tiles_per_split * TK) - 1;
    const int lo = max(first.lo, s_lo);
    const int hi = min(last.hi, s_hi);

    // This lane's row.
    const int my_row = row0 + lr;
    const bool row_valid = my_row < nrows;
    const int my_tok = my_row / G;
    const int my_head = g * G + my_row % G;
    const KeyRange mine = visible_range(my_tok + off, sk, p.causal, p.window_left, p.window_right);
    // Keys this lane's row may use, as key_lo + [0, key_span] (an empty range
    // becomes one that no key reaches).
    int key_lo = max(mine.lo, lo);
    int key_span = min(mine.hi, hi) - key_lo;
    if (!row_valid || key_span < 0) {
        key_lo = 0x40000000;
        key_span = 0;
    }

    const long long q_tok = (long long)p.heads_q * D;
    const long long kv_tok = (long long)p.heads_kv * D;

    // Q^T as the B operand: lane holds row my_row, channels 16*ks + 8*lh .. +7.
    bf16x8_t qreg[KSTEPS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (long long)(q_start + (row_valid ? my_tok : 0)) * q_tok +
                             (long long)my_head * D + lh * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row_valid) v = load_u32x4(qp + ks * 16);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // K operand: key 32w + lr of the tile, logical chunk 2*ks + lh.
    const uint32_t kx = (uint32_t)((32 * w + lr) * ROWB) | (uint32_t)((lh ^ gswz<D>(lr & 15)) << 4);
    // V^T operand via transposing reads: 16-lane group gq, lane i reads key
    // 8*which + 4*(gq/2) + i/4 of a 16-key step, channels
    // 32*db + 16*(gq%2) + 4*(i%4) .. +3, i.e. logical chunk 4*db + cl.
    uint32_t vx[2];
    {
        const int gq = lane >> 4;
        const int i = lane & 15;
        const int cl = (gq & 1) * 2 + ((i & 3) >> 1);
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const int rowl = which * 8 + 4 * (gq >> 1) + (i >> 2);
            vx[which] = (uint32_t)((32 * w + rowl) * ROWB) | (uint32_t)((cl ^ gswz<D>(rowl)) << 4) |
                        (uint32_t)((i & 1) * 8);
        }
    }
    // Global -> LDS: chunk position P = n*NT + tid of a tile is row P / CPR,
    // physical chunk tid % CPR, which holds logical chunk (tid % CPR) ^ swz(row).
    uint32_t goff[SWP];
#pragma unroll
    for (int n = 0; n < SWP; ++n) {
        const int row = n * RPL + tid / CPR;
        goff[n] = (uint32_t)(((long long)row * kv_tok + (((tid % CPR) ^ gswz<D>(row & 15)) * 8)) * 2);
    }
    const uint16_t* Kseg = static_cast<const uint16_t*>(p.k) + (long long)k_start * kv_tok + (long long)g * D;
    const uint16_t* Vseg = static_cast<const uint16_t*>(p.v) + (long long)k_start * kv_tok + (long long)g * D;
    // Tiles past the split's last key are issued too, as loads of zero bytes,
    // so the count of loads behind every wait is fixed.
    auto issue_tile = [&](int kt, char* sK, char* sV) __attribute__((always_inline)) {
        long long bytes = (long long)(sk - kt - 1) * kv_tok * 2 + D * 2;
        if (kt > hi) bytes = 0;
        if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(bytes ? Kseg + (long long)kt * kv_tok : Kseg, (uint32_t)bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(bytes ? Vseg + (long long)kt * kv_tok : Vseg, (uint32_t)bytes);
#pragma unroll
        for (int n = 0; n < LOADS; ++n)
            buffer_load_lds16(rk, sK + (n * NT + w * 64) * 16, goff[n % SWP],
                              (uint32_t)((n / SWP) * SWP * RPL * kv_tok * 2));
#pragma unroll
        for (int n = 0; n < LOADS; ++n)
            buffer_load_lds16(rv, sV + (n * NT + w * 64) * 16, goff[n % SWP],
                              (uint32_t)((n / SWP) * SWP * RPL * kv_tok * 2));
    };

    f32x16_t acc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc[db] = f32x16_t{};
    float m_run = -INFINITY;  // running max of this row, log2 units (may trail the true max by <= 8)
    float l_part = 0.0f;      // running sum of p over this lane's keys (fp32; for the LSE)
    float lb_part = 0.0f;     // running sum of bf16(p), the weights the P V MFMAs use (normalises O)

    // One tile: scores, softmax, P V for this wave's 32 keys.
    auto tile_step = [&](const char* sK, const char* sV, int kt) __attribute__((always_inline)) {
        uint32_t kxl = kx;
        asm volatile("" : "+v"(kxl));
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_read16(sK + (kxl ^ (uint32_t)(ks << 5))));
            s = mfma32x32x16(a, qreg[ks], s);
        }
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = kCap ? score_to_logit<true>(s[r], p.x_mul, p.cap_mul, p.cap_out) : s[r] * p.x_mul;
            const int key = kt + 32 * w + 8 * (r >> 2) + 4 * lh + (r & 3);
            x = ((unsigned)(key - key_lo) <= (unsigned)key_span) ? x : -INFINITY;
            s[r] = x;
            mt = fmaxf(mt, x);
        }
        mt = half_max(mt);
        const bool grow = mt > m_run + kLazyRescale;
        if (wave_any(grow)) {
            const float m_new = grow ? mt : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
            m_run = m_new;
            l_part *= alpha;
            lb_part *= alpha;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
        }
        const float nb = (m_run == -INFINITY) ? 0.0f : -m_run;
        uint32_t pk[8];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(s[r] + nb);
            const float p1 = fast_exp2(s[r + 1] + nb);
            psum += p0 + p1;
            pk[r >> 1] = pack_bf16x2(p0, p1);
            lb_part = add_bf16x2(pk[r >> 1], lb_part);
        }
        l_part += psum;
        uint32_t vxl[2] = {vx[0], vx[1]};
        asm volatile("" : "+v"(vxl[0]), "+v"(vxl[1]));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t pv = {pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
            const char* base = sV + 16 * ROWB * h;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const u32x2_t r0 = lds_read_tr16(base + (vxl[0] ^ (uint32_t)(db << 6)));
                const u32x2_t r1 = lds_read_tr16(base + (vxl[1] ^ (uint32_t)(db << 6)));
                const u32x4_t av = {r0[0], r0[1], r1[0], r1[1]};
                acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pb, acc[db]);
            }
        }
    };

    if (lo <= hi) {
        const int kt0 = lo & ~(TK - 1);
        const int ntiles = (hi - kt0) / TK + 1;
        issue_tile(kt0, sK0, sV0);
        issue_tile(kt0 + TK, sK1, sV1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * LOADS) : "memory");  // Q and this thread's loads of tile 0
        // Q was loaded before the tiles, so the wait above covers it; saying
        // so keeps the compiler from draining every load before the loop.
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" : "+v"(qreg[ks]));
        lds_barrier();
        // Step j: P V of tile j from its stage; barrier (stage free); tile
        // j+2 into it; wait for this thread's loads of tile j+1; barrier.
        auto step = [&](auto stage_tag, int j) __attribute__((always_inline)) {
            constexpr int S = decltype(stage_tag)::value;
            char* const sK = S == 0 ? sK0 : sK1;
            char* const sV = S == 0 ? sV0 : sV1;
            tile_step(sK, sV, kt0 + j * TK);
            lds_barrier();
            issue_tile(kt0 + (j + 2) * TK, sK, sV);
            asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * LOADS) : "memory");
            lds_barrier();
        };
        using st0 = std::integral_constant<int, 0>;
        using st1 = std::integral_constant<int, 1>;
        int j = 0;
        for (; j + 2 <= ntiles; j += 2) {
            step(st0{}, j);
            step(st1{}, j + 1);
        }
        if (j < ntiles) step(st0{}, j);
    }
    // Drain the look-ahead loads (zero-byte loads still write LDS) before the
    // stages are reused for the merge.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Merge the two waves: M = max of the waves' maxima, each accumulator
    // scaled by exp2(m_w - M), L (fp32 sums) and Lb (sums of the bf16
    // weights) the scaled row sums.
    const float l_row = half_sum(l_part);
    const float lb_row = half_sum(lb_part);
    if (lh == 0) {
        sML[w][0][lr] = m_run;
        sML[w][1][lr] = l_row;
        sML[w][2][lr] = lb_row;
    }
    lds_barrier();
    const float m0 = sML[0][0][lr], m1 = sML[1][0][lr];
    const float M = fmaxf(m0, m1);
    float L = 0.0f, Lb = 0.0f, f_mine = 0.0f;
    if (M != -INFINITY) {
        const float f0 = fast_exp2(m0 - M), f1 = fast_exp2(m1 - M);
        L = sML[0][1][lr] * f0 + sML[1][1][lr] * f1;
        Lb = sML[0][2][lr] * f0 + sML[1][2][lr] * f1;
        f_mine = fast_exp2(m_run - M);
    }
    f32x4_t* const xbuf = reinterpret_cast<f32x4_t*>(sK0);  // [DBLK][4][64] float4
    if (w == 1) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                xbuf[(db * 4 + q4) * 64 + lane] = f32x4_t{acc[db][4 * q4] * f_mine, acc[db][4 * q4 + 1] * f_mine,
                                                          acc[db][4 * q4 + 2] * f_mine, acc[db][4 * q4 + 3] * f_mine};
    }
    lds_barrier();
    if (w == 1 || !row_valid) return;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t o = xbuf[(db * 4 + q4) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] = acc[db][4 * q4 + e] * f_mine + o[e];
        }

    // Lane lr holds row my_row, channels 32*db + 8*q4 + 4*lh .. +3.
    if (p.splits == 1) {
        // O over the sum of the bf16 weights the P V MFMAs used; the LSE from the fp32 sum.
        const float inv = (Lb > 0.0f) ? 1.0f / Lb : 0.0f;
        uint16_t* O = static_cast<uint16_t*>(p.o) + ((long long)(q_start + my_tok) * p.heads_q + my_head) * D + 4 * lh;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                store_u32x2(O + 32 * db + 8 * q4,
                            u32x2_t{pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                                    pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv)});
        if (p.lse && lh == 0)
            p.lse[(long long)my_head * p.total_q + q_start + my_tok] =
                (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : -INFINITY;
        return;
    }
    const long long pidx = (((long long)b * p.heads_kv + g) * p.m_groups + mg) * p.splits + sp;
    float* pacc = p.part_acc + (pidx * ROWS + lr) * D + 4 * lh;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4_t*>(pacc + 32 * db + 8 * q4) =
                f32x4_t{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
    if (lh == 0) {
        float* pml = p.part_ml + pidx * 3 * ROWS;
        pml[lr] = M;
        pml[ROWS + lr] = L;
        pml[2 * ROWS + lr] = Lb;
    }
}

// Merge the splits of one (sequence, kv head, row group): M = max_s m_s,
// w_s = exp2(m_s - M), O = sum_s w_s acc_s / sum_s w_s lb_s (lb: sums of the
// bf16 weights), LSE = ln2 * (M + log2 sum_s w_s l_s) (l: fp32 sums). One thread per (row, 4 channels).
// The splits are read in chunks of 8 whose loads are all issued before any
// is used (one memory round trip per chunk), merged with a running max.
constexpr int kCombineThreads = 64;  // small groups spread the few valid rows over many CUs

template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_gqa_combine_kernel(const GqaDecodeParams p) {
    constexpr int TPR = D / 4;                     // threads per row
    constexpr int RPB = kCombineThreads / TPR;     // rows per work group
    constexpr int CH = 8;             // splits per chunk
    int id = blockIdx.x;
    const int rgrp = id % (ROWS / RPB);
    id /= ROWS / RPB;
    const int mg = id % p.m_groups;
    id /= p.m_groups;
    const int g = id % p.heads_kv;
    const int b = id / p.heads_kv;
    const int G = p.group;
    const int q_start = p.cu_q[b];
    const int sq = p.cu_q[b + 1] - q_start;
    const int row = rgrp * RPB + (int)threadIdx.x / TPR;
    const int r = mg * ROWS + row;
    if (r >= sq * G) return;
    const int d0 = ((int)threadIdx.x % TPR) * 4;
    const int tok = r / G;
    const int h = g * G + r % G;
    const long long pidx0 = (((long long)b * p.heads_kv + g) * p.m_groups + mg) * p.splits;
    float M = -INFINITY, L = 0.0f, Lb = 0.0f;
    f32x4_t o = f32x4_t{};
    for (int s0 = 0; s0 < p.splits; s0 += CH) {
        float ms[CH], ls[CH], lbs[CH];
        f32x4_t as[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const bool in = s0 + j < p.splits;
            const long long pi = pidx0 + (in ? s0 + j : 0);
            ms[j] = in ? p.part_ml[pi * 3 * ROWS + row] : -INFINITY;
            ls[j] = p.part_ml[pi * 3 * ROWS + ROWS + row];
            lbs[j] = p.part_ml[pi * 3 * ROWS + 2 * ROWS + row];
            as[j] = *reinterpret_cast<const f32x4_t*>(p.part_acc + (pi * ROWS + row) * D + d0);
        }
        float mc = M;
#pragma unroll
        for (int j = 0; j < CH; ++j) mc = fmaxf(mc, ms[j]);
        if (mc == -INFINITY) continue;  // nothing visible so far
        const float a = fast_exp2(M - mc);  // 0 while M is -inf
        L *= a;
        Lb *= a;
        o *= a;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float ws = fast_exp2(ms[j] - mc);  // 0 for splits past the end or with no keys
            L += ws * ls[j];
            Lb += ws * lbs[j];
            o += ws * as[j];
        }
        M = mc;
    }
    const float inv = (Lb > 0.0f) ? 1.0f / Lb : 0.0f;
    uint16_t* O = static_cast<uint16_t*>(p.o) + ((long long)(q_start + tok) * p.heads_q + h) * D + d0;
    store_u32x2(O, u32x2_t{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)});
    if (p.lse && d0 == 0)
        p.lse[(long long)h * p.total_q + q_start + tok] = (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_gqa(const GqaDecodeParams& p, hipStream_t stream) {
    const long long units = (long long)p.batch * p.heads_kv * p.m_groups;
    if (units <= 0) return hipSuccess;
    const long long grid_split = units * p.splits;
    constexpr int RPB = kCombineThreads / (D / 4);
    const long long grid_comb = units * (ROWS / RPB);
    if (grid_split > 0x7fffffffLL || grid_comb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (p.softcap > 0.0f)
        hipLaunchKernelGGL((decode_gqa_split_kernel<D, true>), dim3((unsigned)grid_split), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_gqa_split_kernel<D, false>), dim3((unsigned)grid_split), dim3(NT), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL((decode_gqa_combine_kernel<D>), dim3((unsigned)grid_comb), dim3(kCombineThreads), 0, stream,
                       p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gqa(const GqaDecodeParams& p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_gqa<64>(p, stream);
        case 128: return launch_gqa<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mxfa
