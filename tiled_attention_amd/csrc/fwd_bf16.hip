// fwd_bf16.hip -- bf16 attention forward on gfx950 MFMA (dense and packed).
//
// Tiled online-softmax forward as on the oxillama-runtime 0.1.0 page
// (src/flash_attention.rs, flash_attention: running row max, running sum,
// rescale of the accumulator, final normalisation), in the exp2 domain with
// the scale folded into the exponent after the QK^T contraction (kernelbot
// amd-mixed-mla submission 588924, _flash_fused; scale applied in fp32 after
// the MMA as in the AstrAI v1.3.9 page's attn_mma_utils.cuh), with causal and
// window tiles skipped at tile granularity (flash_attention's causal tile skip,
// extended to the window's lower edge).
//
// Work group: 4 waves, 128 query rows (32 per wave), one (batch, head) unit,
// two work groups per CU (<= 256 registers per lane, 64 KB LDS each).
//
// Per 64-key tile, each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, so lane l owns query row l % 32 and 32 of the 64
// keys: row max and row sum are in-register reductions plus one exchange
// between the lane halves. P^T stays in registers as the B operand of
// O^T = V^T P^T (the accumulator layout of S^T is the operand layout of
// P^T); the V^T operand comes from LDS through ds_read_b64_tr_b16. O^T keeps
// one query per lane, so the online-softmax rescale is one multiplier per
// lane. P of a tile is computed against the running max of the earlier
// tiles; only when some lane's sum of it exceeds 2^8 (the max grew) is the
// tile's row max taken, the accumulator rescaled and P recomputed.
//
// Software pipeline inside each wave (two S register sets): while the MFMAs
// compute S for tile j+1, the vector ALU turns S of tile j into P; while the
// MFMAs accumulate P V for tile j, the vector ALU masks tile j+1 (and applies
// the scale or the cap in those modes). K therefore runs one tile ahead of V:
// K tiles j+1 (in use) and j+2 (arriving), V tiles j (in use) and j+1
// (arriving) share two buffers each, filled by buffer loads that write LDS
// directly (out-of-range keys read as zero). The 16-byte chunks of a row are
// XOR-swizzled so that the K operand reads (16 rows x one chunk) and the
// transposing V reads (4 rows x 4 chunks per half wave) hit distinct banks.
// Fully visible tiles take a branch without per-element mask tests.
#include <type_traits>

#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int BM = kFwdBf16Rows;  // 128 query rows per work group
constexpr int BN = kFwdBf16Keys;  // 64 keys per tile
constexpr int NTHREADS = 256;  // 4 waves
constexpr float kLazyRescale = 8.0f;  // log2 units: rescale when a row max grows by > 2^8
constexpr float kOptimisticSum = 256.0f;  // a tile's P sum (per lane) up to which no p can exceed 2^8

// Chunk swizzle of an LDS row (16-byte chunks): physical = logical ^ swz(row).
template <int D>
MXFA_DEV int swz(int row);
template <>
MXFA_DEV int swz<128>(int row) {  // 16 chunks per row, one row per 256-byte bank line
    return ((row & 3) << 2) | ((row >> 2) & 3);
}
template <>
MXFA_DEV int swz<64>(int row) {  // 8 chunks per row, two rows per bank line
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// One 16-key step of O^T += V^T P^T: the V^T operands of all output blocks
// (two transposing reads each) and one MFMA per 32-channel block.
template <int D, int KB, int HALF>
MXFA_DEV void pv_step(f32x16_t (&acc)[D / 32], const uint32_t (&pk)[2][8], const uint32_t (&va)[2 * (D / 32)]) {
    constexpr int DBLK = D / 32;
    constexpr int OFF = (KB * 32 + HALF * 16) * D * 2;
    const u32x4_t pv = {pk[KB][HALF * 4 + 0], pk[KB][HALF * 4 + 1], pk[KB][HALF * 4 + 2], pk[KB][HALF * 4 + 3]};
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
    u32x2_t r[2 * DBLK];
    if constexpr (DBLK == 4)
        lds_read_tr16_x8<OFF>(r, va);
    else
        lds_read_tr16_x4<OFF>(r, va);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
        const u32x4_t av = {r[2 * db][0], r[2 * db][1], r[2 * db + 1][0], r[2 * db + 1][1]};
        acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pb, acc[db]);
    }
}

// kMode 0: no softcap, scale > 0 -- the max runs on raw scores and the scale
//          is folded into the exponent's FMA.
// kMode 1: no softcap, any scale -- logits computed explicitly.
// kMode 2: softcap.
template <int D, int kMode>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const FwdParams p) {
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    constexpr int KSTEPS = D / 16;             // QK^T contraction steps
    constexpr int DBLK = D / 32;               // 32-wide output blocks
    constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
    constexpr int ROWB = D * 2;                // bytes per K/V row in LDS
    constexpr int TILEB = BN * ROWB;           // bytes per K or V tile
    constexpr int LOADS = TILEB / (16 * NTHREADS);  // 16-byte loads per thread per tile

    // Four separate LDS objects rather than two arrays of two: reads of one
    // buffer may then proceed while the buffer loads into another are in
    // flight (the compiler waits for in-flight LDS-bound loads only before
    // reads of the object they write).
    __shared__ __attribute__((aligned(TILEB))) char sK0[TILEB];
    __shared__ __attribute__((aligned(TILEB))) char sK1[TILEB];
    __shared__ __attribute__((aligned(TILEB))) char sV0[TILEB];
    __shared__ __attribute__((aligned(TILEB))) char sV1[TILEB];

    const WorkItem item = p.worklist
                              ? map_listed(blockIdx.x, p.worklist, p.batch, p.heads_kv, p.group, p.list_max, p.xcd_cus)
                              : map_workgroup(blockIdx.x, p.batch, p.heads_kv, p.group, p.n_qtiles, p.xcd_cus);
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
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int lh = lane >> 5;
    const int off = sk - sq;  // bottom-right alignment
    const long long q_tok = (long long)p.heads_q * D;
    const long long kv_tok = (long long)p.heads_kv * D;

    // Key range of the whole group (lo/hi of a row are non-decreasing in the row).
    const int row_last = min(tile_row0 + BM, sq) - 1;
    const int kv_lo = visible_range(tile_row0 + off, sk, p.causal, p.window_left, p.window_right).lo;
    const int kv_hi = visible_range(row_last + off, sk, p.causal, p.window_left, p.window_right).hi;

    // This wave's rows and their key range (decides fully visible tiles).
    const int wrow0 = tile_row0 + wave * 32;
    const int wrow_last = max(min(wrow0 + 31, sq - 1), wrow0);
    const KeyRange wfirst = visible_range(wrow0 + off, sk, p.causal, p.window_left, p.window_right);
    const KeyRange wlast = visible_range(wrow_last + off, sk, p.causal, p.window_left, p.window_right);
    const bool wave_rows_valid = wrow0 < sq;

    // This lane's query row and its visible keys.
    const int qi = wrow0 + lr;
    const bool q_valid = qi < sq;
    const KeyRange mine = visible_range(qi + off, sk, p.causal, p.window_left, p.window_right);
    // The row's keys as lo + [0, span] (an empty range becomes one no key
    // reaches), for the masked tiles: key kt + 4*lh + c (c a constant of the
    // register) is visible iff (unsigned)(c - (lo - kt - 4*lh)) <= span.
    int m_lo = mine.lo, m_span = mine.hi - mine.lo;
    if (m_span < 0) {
        m_lo = 0x40000000;
        m_span = 0;
    }

    // Q^T as the B operand: lane holds row qi, contraction chunk ks*16 + lh*8.
    bf16x8_t qreg[KSTEPS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (long long)(q_start + qi) * q_tok +
                             (long long)h * D + lh * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (q_valid) v = load_u32x4(qp + ks * 16);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // LDS read offsets. Tiles are 16 KB aligned (D = 128; 8 KB for D = 64) and
    // the swizzle only moves bits inside a row, so a read address is
    // tile_base + (lane constant XOR step constant).
    // K operand: row kb*32 + lr, chunk (ks*2 + lh) ^ swz(lr) ->
    //   (kx ^ (ks << 5)) + kb*32*ROWB with kx = lr*ROWB | ((lh ^ swz(lr)) << 4).
    const uint32_t kx = (uint32_t)(lr * ROWB) | (uint32_t)((lh ^ swz<D>(lr & 15)) << 4);
    // V^T operand via transposing reads: 16-lane group g, lane i reads row
    // (which*8 + 4*(g/2) + i/4) of a 16-key step, columns db*32 + (g%2)*16 + 4*(i%4):
    //   chunk (db*4 + cl) ^ swz(row) -> vx[which] ^ (db << 6).
    uint32_t vx[2];
    {
        const int g = lane >> 4;
        const int i = lane & 15;
        const int cl = (g & 1) * 2 + ((i & 3) >> 1);
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const int rowl = which * 8 + 4 * (g >> 1) + (i >> 2);
            vx[which] = (uint32_t)(rowl * ROWB) | (uint32_t)((cl ^ swz<D>(rowl)) << 4) | (uint32_t)((i & 1) * 8);
        }
    }
    // Global -> LDS loads: 16-byte chunk position P = n*256 + tid of a tile, i.e.
    // row n*(256/CPR) + tid/CPR, chunk tid%CPR; the swizzle depends on the row
    // only through row % 16, which is the same for every n.
    const int lrow = tid / CPR;
    const uint32_t goff = (uint32_t)(((long long)lrow * kv_tok + (((tid % CPR) ^ swz<D>(lrow & 15)) * 8)) * 2);
    const uint32_t gstep = (uint32_t)((NTHREADS / CPR) * kv_tok * 2);
    const uint16_t* Kseg = static_cast<const uint16_t*>(p.k) + (long long)k_start * kv_tok + (long long)kvh * D;
    const uint16_t* Vseg = static_cast<const uint16_t*>(p.v) + (long long)k_start * kv_tok + (long long)kvh * D;
    // Bytes from key kt on that hold keys < sk (keys past the end read as zero).
    auto tile_bytes = [&](int kt) -> uint32_t {
        long long bytes = (long long)(sk - kt - 1) * kv_tok * 2 + D * 2;
        if (kt >= sk) bytes = 0;  // a tile wholly past the end is a zero-byte load
        return (uint32_t)(bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
    };
    // This wave's part of a tile in LDS as a wave-uniform byte offset: each
    // load's LDS address (M0) is then a scalar sum instead of a lane read.
    const uint32_t woff = __builtin_amdgcn_readfirstlane((uint32_t)(wave * 64 * 16));
    // One tile into LDS: LOADS loads per thread, reading `bytes` from key kt on.
    auto issue_b = [&](const uint16_t* seg, int kt, char* tile, uint32_t bytes) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(seg + (long long)kt * kv_tok, bytes);
#pragma unroll
        for (int n = 0; n < LOADS; ++n) buffer_load_lds16(r, tile + n * NTHREADS * 16 + woff, goff, n * gstep);
    };
    auto issue = [&](const uint16_t* seg, int kt, char* tile) __attribute__((always_inline)) {
        issue_b(seg, kt, tile, tile_bytes(kt));
    };

    f32x16_t acc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) acc[i] = f32x16_t{};
    float m_run = -INFINITY;  // running max of this row, log2 units (may trail the true max by <= 8)
    float l_part = 0.0f;      // running sum of p over this lane's keys (fp32; for the LSE)
    float lb_part = 0.0f;     // running sum of bf16(p), the weights the P V MFMAs use (normalises O)
    const float c_exp = (kMode == 0) ? p.x_mul : 1.0f;

    // ---- pipeline pieces
    // S^T = K Q^T for one tile.
    auto qk = [&](f32x16_t (&s)[2], const char* kt_lds) __attribute__((always_inline)) {
        s[0] = f32x16_t{};
        s[1] = f32x16_t{};
        // Recompute the per-step offsets in each tile instead of keeping all
        // of them live across the loop (registers are the scarce resource).
        uint32_t kxl = kx;
        asm volatile("" : "+v"(kxl));
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const char* a0 = kt_lds + (kxl ^ (uint32_t)(ks << 5));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_read16(a0 + kb * 32 * ROWB));
                s[kb] = mfma32x32x16(a, qreg[ks], s[kb]);
            }
        }
    };
    // Logits (raw scores in mode 0), mask, and the tile's row max in log2 units.
    auto logits_max = [&](auto masked_tag, f32x16_t (&s)[2], int kt) -> float {
        // 0: every key visible; 1: keys below the tile are all visible, test
        // the upper bound only; 2: test both bounds.
        constexpr int kMask = decltype(masked_tag)::value;
        const int hiT = mine.hi - kt - 4 * lh;
        const int loT = m_lo - kt - 4 * lh;
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[kb][r];
                if constexpr (kMode == 1) x = x * p.x_mul;
                if constexpr (kMode == 2) x = score_to_logit<true>(x, p.x_mul, p.cap_mul, p.cap_out);
                const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
                if constexpr (kMask == 1) x = (c <= hiT) ? x : -INFINITY;
                if constexpr (kMask == 2) x = ((unsigned)(c - loT) <= (unsigned)m_span) ? x : -INFINITY;
                s[kb][r] = x;
                m = fmaxf(m, x);
            }
        }
        m = half_max(m);
        if constexpr (kMode == 0) m *= c_exp;
        return m;
    };
    // Every row of this wave sees all keys below kt (its lower bounds are
    // non-decreasing in the row, so the last row's decides), and no row's
    // range is empty.
    auto lows_visible = [&](int kt) { return wave_rows_valid && wlast.lo <= kt && wfirst.lo <= wfirst.hi; };
    auto tile_full = [&](int kt) {
        const int t_last = kt + BN - 1;
        return wave_rows_valid && t_last < sk && kt >= wlast.lo && t_last <= wfirst.hi;
    };
    // Lazy max update: rescale only when some row's max grew by more than 2^8.
    auto update_max = [&](float mt) {
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
    };
    // P = exp2(logit - max) as bf16 pairs; P^T operand (kb, half) = registers
    // 8*half..8*half+7 of S^T block kb. Returns the fp32 sum of p; psb gets
    // the sum of the rounded values.
    auto exp_tile = [&](f32x16_t (&s)[2], uint32_t (&pk)[2][8], float& psb) {
        const float nb = (m_run == -INFINITY) ? 0.0f : -m_run;
        float psum = 0.0f;
        psb = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(s[kb][r], c_exp, nb));
                const float p1 = fast_exp2(fmaf(s[kb][r + 1], c_exp, nb));
                psum += p0 + p1;
                pk[kb][r >> 1] = pack_bf16x2(p0, p1);
                psb = add_bf16x2(pk[kb][r >> 1], psb);
            }
        }
        return psum;
    };
    // Optimistic max: P of a tile is first computed against the running max
    // of the earlier tiles. If every lane's sum of it stays <= 2^8, every p
    // is <= 2^8 -- the bound the lazy rescale keeps -- and the tile is done
    // without its row max. Otherwise (the max grew, or no key was seen yet)
    // take the tile's max, rescale and recompute P.
    auto settle = [&](f32x16_t (&s)[2], uint32_t (&pk)[2][8], float psum, float psb) __attribute__((always_inline)) {
        if (wave_any(m_run == -INFINITY || psum > kOptimisticSum)) {
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
            mt = half_max(mt);
            if constexpr (kMode == 0) mt *= c_exp;
            const float m_new = fmaxf(m_run, mt);
            const float alpha = (m_new == m_run) ? 1.0f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_part *= alpha;
            lb_part *= alpha;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
            psum = exp_tile(s, pk, psb);
        }
        l_part += psum;
        lb_part += psb;
    };
    // O^T += V^T P^T for one tile.
    auto pv = [&](const uint32_t (&pk)[2][8], const char* vt_lds) __attribute__((always_inline)) {
        uint32_t va[2 * DBLK];
        const uint32_t v0 = lds_addr(vt_lds) + vx[0];
        const uint32_t v1 = lds_addr(vt_lds) + vx[1];
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            va[2 * db] = v0 ^ (uint32_t)(db << 6);
            va[2 * db + 1] = v1 ^ (uint32_t)(db << 6);
        }
        pv_step<D, 0, 0>(acc, pk, va);
        pv_step<D, 0, 1>(acc, pk, va);
        pv_step<D, 1, 0>(acc, pk, va);
        pv_step<D, 1, 1>(acc, pk, va);
    };

    // Phase A, fused: S_{j+1} = K_{j+1} Q^T on the MFMAs while the vector
    // ALU turns S_j into P_j. After each MFMA one slice of the exponentials
    // (two elements), fenced so that the compiler keeps the interleave; the K
    // operand reads run AHEAD MFMAs ahead. `issue_v` (the next V tile's
    // loads) goes out after MFMA kIssueV.
    auto qk_exp = [&](f32x16_t (&sn)[2], const char* kt_lds, f32x16_t (&sc)[2], uint32_t (&pk)[2][8],
                      float& psb, auto&& issue_v) __attribute__((always_inline)) {
        constexpr int kIssueV = 4;
        constexpr int NM = 2 * KSTEPS;  // MFMAs: m = 2*ks + kb
        constexpr int EPS = 32 / NM;    // exponentials per slice
        constexpr int AHEAD = 4;
        sn[0] = f32x16_t{};
        sn[1] = f32x16_t{};
        uint32_t kxl = kx;
        asm volatile("" : "+v"(kxl));
        auto rd = [&](int m) __attribute__((always_inline)) {
            return __builtin_bit_cast(bf16x8_t,
                                      lds_read16(kt_lds + (kxl ^ (uint32_t)((m >> 1) << 5)) + (m & 1) * 32 * ROWB));
        };
        bf16x8_t a[NM];
#pragma unroll
        for (int m = 0; m < AHEAD; ++m) a[m] = rd(m);
        const float nb = (m_run == -INFINITY) ? 0.0f : -m_run;
        float psum = 0.0f;
        psb = 0.0f;
        // Raised issue priority for this phase: where the two waves sharing a
        // SIMD (one from each work group) are both ready, the one in its
        // exponential phase goes first, and its vector work then fills the
        // other wave's MFMA time (3-4% faster on the causal and chunked
        // prefill workloads).
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + AHEAD < NM) a[m + AHEAD] = rd(m + AHEAD);
            sn[m & 1] = mfma32x32x16(a[m], qreg[m >> 1], sn[m & 1]);
            if (m == kIssueV) issue_v();
#pragma unroll
            for (int e = 0; e < EPS; e += 2) {
                const int idx = m * EPS + e;
                const int kb = idx >> 4;
                const int r = idx & 15;
                const float p0 = fast_exp2(fmaf(sc[kb][r], c_exp, nb));
                const float p1 = fast_exp2(fmaf(sc[kb][r + 1], c_exp, nb));
                pk[kb][r >> 1] = pack_bf16x2(p0, p1);
                psum += p0 + p1;
                psb = add_bf16x2(pk[kb][r >> 1], psb);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        return psum;
    };
    // Phase B, fused: O += V_j P_j on the MFMAs while the vector ALU takes
    // the logits and the mask of S_{j+1}, a slice after each MFMA; the
    // transposing V reads run AHEAD MFMAs ahead.
    auto pv_mask = [&](auto masked_tag, const uint32_t (&pk)[2][8], const char* vt_lds, f32x16_t (&sn)[2],
                       int kt) __attribute__((always_inline)) {
        constexpr int kMask = decltype(masked_tag)::value;  // as for logits_max
        const int hiT = mine.hi - kt - 4 * lh;
        const int loT = m_lo - kt - 4 * lh;
        constexpr int NP = 4 * DBLK;  // MFMAs: n = DBLK*step + db, step = 2*kb + half (16 keys each)
        constexpr int EPS = 32 / NP;  // score elements per slice
        constexpr int AHEAD = 4;
        uint32_t vxl[2] = {vx[0], vx[1]};
        asm volatile("" : "+v"(vxl[0]), "+v"(vxl[1]));
        auto rd = [&](int n, int which) __attribute__((always_inline)) {
            const int st = n / DBLK;
            const int db = n % DBLK;
            return lds_read_tr16(vt_lds + st * 16 * ROWB + (vxl[which] ^ (uint32_t)(db << 6)));
        };
        u32x2_t r0[NP], r1[NP];
#pragma unroll
        for (int n = 0; n < AHEAD; ++n) {
            r0[n] = rd(n, 0);
            r1[n] = rd(n, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            if (n + AHEAD < NP) {
                r0[n + AHEAD] = rd(n + AHEAD, 0);
                r1[n + AHEAD] = rd(n + AHEAD, 1);
            }
            const int st = n / DBLK;
            const int db = n % DBLK;
            const int kb = st >> 1;
            const int half = st & 1;
            const u32x4_t av = {r0[n][0], r0[n][1], r1[n][0], r1[n][1]};
            const u32x4_t pv4 = {pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2], pk[kb][4 * half + 3]};
            acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, pv4), acc[db]);
#pragma unroll
            for (int e = 0; e < EPS; ++e) {
                const int idx = n * EPS + e;
                const int skb = idx >> 4;
                const int r = idx & 15;
                float x = sn[skb][r];
                if constexpr (kMode == 1) x = x * p.x_mul;
                if constexpr (kMode == 2) x = score_to_logit<true>(x, p.x_mul, p.cap_mul, p.cap_out);
                const int c = skb * 32 + 8 * (r >> 2) + (r & 3);
                if constexpr (kMask == 1) x = (c <= hiT) ? x : -INFINITY;
                if constexpr (kMask == 2) x = ((unsigned)(c - loT) <= (unsigned)m_span) ? x : -INFINITY;
                sn[skb][r] = x;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (kv_lo <= kv_hi) {
        const int kt0 = kv_lo & ~(BN - 1);
        const int ntiles = (kv_hi - kt0) / BN + 1;
        // The loop's loads read one tile's span, or for the last tile up to the
        // segment's end (rows past it read as zero); both are set here, so
        // the per-step issue is a compare, a select and scalar adds (the
        // 64-bit range arithmetic per tile took ~2% of the prefill's time).
        const long long span64 = (long long)(BN - 1) * kv_tok * 2 + D * 2;
        const uint32_t span = (uint32_t)(span64 > 0x7fffffffLL ? 0x7fffffffLL : span64);
        const int kt_last = kt0 + (ntiles - 1) * BN;
        const uint32_t last_bytes = min(span, tile_bytes(kt_last));
        auto loop_bytes = [&](int kt) __attribute__((always_inline)) { return kt == kt_last ? last_bytes : span; };
        // Prologue: K0, V0, K1 in flight; S and row max of tile 0.
        issue(Kseg, kt0, sK0);
        issue(Vseg, kt0, sV0);
        issue(Kseg, kt0 + BN, sK1);  // zero-byte past the end
        // Q and K0 are all tile 0's scores need (V0 and K1 may still run).
        asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * LOADS) : "memory");
        lds_barrier();
        f32x16_t sa[2], sb[2];
        float mt_a = -INFINITY;
        qk(sa, sK0);
        using mask0 = std::integral_constant<int, 0>;
        using mask1 = std::integral_constant<int, 1>;
        using mask2 = std::integral_constant<int, 2>;
        mt_a = tile_full(kt0)      ? logits_max(mask0{}, sa, kt0)
               : lows_visible(kt0) ? logits_max(mask1{}, sa, kt0)
                                   : logits_max(mask2{}, sa, kt0);
        update_max(mt_a);  // later tiles start from this max (optimistic)
        // The first step reads K1 and V0. Each of them is loaded by all four
        // waves, and a wave's own wait covers only its own part: wait for all
        // of this wave's loads, then the barrier covers the other waves'
        // parts (and ends every wave's use of K0 before K2 overwrites it).
        wait_vmem();
        lds_barrier();

        // Tile j (parity P = j % 2): S_j in s_cur (masked); K(j+1)
        // in sK[1-P] and V(j) in sV[P] are resident; K(j+2) goes to sK[P] and
        // V(j+1) to sV[1-P].
        auto step = [&](auto has_next_tag, auto parity_tag, int j, f32x16_t (&s_cur)[2], f32x16_t (&s_next)[2]) {
            constexpr bool kNext = decltype(has_next_tag)::value;
            constexpr int P = decltype(parity_tag)::value;
            char* const k_fill = P ? sK1 : sK0;
            const char* const k_use = P ? sK0 : sK1;
            char* const v_fill = P ? sV0 : sV1;
            const char* const v_use = P ? sV1 : sV0;
            const int kt = kt0 + j * BN;
            // K(j+2) goes out at the start of the step and V(j+1) a few MFMAs
            // into phase A (their buffers were released by the previous
            // step's barrier): splitting the group's 32 KB burst of loads
            // shortens each wave's issue stall (~1%), and V(j+1) is not read
            // before the next step's phase B.
            if (j + 2 < ntiles) issue_b(Kseg, kt + 2 * BN, k_fill, loop_bytes(kt + 2 * BN));
            auto issue_v = [&]() __attribute__((always_inline)) {
                if (j + 1 < ntiles) issue_b(Vseg, kt + BN, v_fill, loop_bytes(kt + BN));
            };
            uint32_t pk[2][8];
            if constexpr (kNext) {
                // Phase A: S_{j+1} = K_{j+1} Q^T on the MFMAs, P_j on the vector ALU.
                float psb;
                const float psum = qk_exp(s_next, k_use, s_cur, pk, psb, issue_v);
                settle(s_cur, pk, psum, psb);
                // Phase B: O += V_j P_j on the MFMAs, mask + max of S_{j+1} on the vector ALU.
                if (tile_full(kt + BN))
                    pv_mask(mask0{}, pk, v_use, s_next, kt + BN);
                else if (lows_visible(kt + BN))
                    pv_mask(mask1{}, pk, v_use, s_next, kt + BN);
                else
                    pv_mask(mask2{}, pk, v_use, s_next, kt + BN);
            } else {
                issue_v();  // (no next tile: nothing to load)
                float psb;
                const float psum = exp_tile(s_cur, pk, psb);
                settle(s_cur, pk, psum, psb);
                pv(pk, v_use);
            }
            wait_vmem();
            __syncthreads();
        };
        using even = std::integral_constant<int, 0>;
        using odd = std::integral_constant<int, 1>;

        int j = 0;
        for (; j + 2 < ntiles; j += 2) {
            step(std::true_type{}, even{}, j, sa, sb);
            step(std::true_type{}, odd{}, j + 1, sb, sa);
        }
        if (j + 1 < ntiles) {
            step(std::true_type{}, even{}, j, sa, sb);
            step(std::false_type{}, odd{}, j + 1, sb, sa);
        } else {
            step(std::false_type{}, even{}, j, sa, sb);
        }
    }

    // Epilogue: combine the two lane halves' sums, normalise, store. O is
    // divided by the sum of the bf16 weights the P V MFMAs multiplied (so
    // the weights of a row sum to one), the LSE takes the fp32 sum. O goes
    // through this wave's own part of the K/V buffers (free after the last
    // step's barrier; chunks XOR-swizzled by row), so that every global store
    // writes whole rows: 64 lanes x 16 bytes = 4 rows of 256 bytes (d = 128)
    // or 8 of 128 (d = 64), instead of 16 bytes of each of 32 rows.
    const float l_row = half_sum(l_part);
    const float lb_row = half_sum(lb_part);
    const float inv = (lb_row > 0.0f) ? 1.0f / lb_row : 0.0f;
    {
        typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
        typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
        constexpr int OCH = D / 8;      // 16-byte chunks per O row
        constexpr int RPI = 64 / OCH;   // rows per store instruction
        char* const ost = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = db * 4 + rg;  // channels 8c .. 8c+7; this lane holds 8c + 4*lh .. +3
                const u32x2_t v = {pack_bf16x2(acc[db][4 * rg + 0] * inv, acc[db][4 * rg + 1] * inv),
                                   pack_bf16x2(acc[db][4 * rg + 2] * inv, acc[db][4 * rg + 3] * inv)};
                *(lds_u32x2*)to_lds(ost + lr * ROWB + ((c ^ (lr % OCH)) << 4) + lh * 8) = v;
            }
        }
        const int rsub = lane / OCH;
        const int c = lane % OCH;
        uint16_t* const Ow = static_cast<uint16_t*>(p.o) + (long long)(q_start + wrow0) * q_tok + (long long)h * D;
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int r = it * RPI + rsub;  // row of this wave's 32
            const u32x4_t v = *(const lds_u32x4*)to_lds(ost + r * ROWB + ((c ^ (r % OCH)) << 4));
            if (wrow0 + r < sq) store_u32x4(Ow + (long long)r * q_tok + c * 8, v);
        }
    }
    if (p.lse && lh == 0 && q_valid) {
        const float lse = (l_row > 0.0f) ? (m_run + fast_log2(l_row)) * kLn2 : -INFINITY;
        const long long idx = p.cu_q ? (long long)h * p.total_q + q_start + qi
                                     : ((long long)b * p.heads_q + h) * sq + qi;
        p.lse[idx] = lse;
    }
}

template <int D, int kMode>
void launch_mode(const FwdParams& p, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, kMode>), dim3(grid), dim3(NTHREADS), 0, stream, p);
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
        launch_mode<D, 2>(p, (unsigned)grid, stream);
    else if (p.scale > 0.0f)
        launch_mode<D, 0>(p, (unsigned)grid, stream);
    else
        launch_mode<D, 1>(p, (unsigned)grid, stream);
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
