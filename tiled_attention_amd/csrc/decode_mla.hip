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
// and one key split. The latent rows stream from HBM through four 36 KB LDS
// stages (32-key tiles) filled by buffer loads that write LDS directly; each
// wave waits only for the tile it needs (vmcnt with the count of later
// loads). The steps are software pipelined: while tile j's P V runs, tile
// j+1 is read for its scores and tiles j+2 and j+3 stream in. An fp8 cache
// takes three stages instead, filled from registers (see the fp8 path).
// Wave w = (rb, ch) with rb = w % 2 (rows 32*rb..+31) and ch = w / 2:
//   QK: the partial S^T (32 keys x 32 rows) over channels 288*ch..+287 with
//       18 v_mfma_f32_32x32x16_bf16 (its Q^T slice lives in accumulation
//       registers); the two waves of a row block swap partials through LDS
//       and both add them (same operands, same order: the same S^T);
//   softmax: logits and mask, then exp2 against the running max of the
//       earlier tiles; only when some lane's sum of P exceeds 2^8 is the
//       tile's row max taken (one lane exchange) and P recomputed; done
//       identically by both waves of the row block;
//   PV: O^T (channels 256*ch..+255 x 32 rows) += V^T P^T with 16 MFMAs;
//       P^T is the S^T accumulator re-packed to bf16 in place and the V^T
//       operand comes from ds_read_b64_tr_b16 in the matching key order.
// Splitting the contraction keeps the 32x32x16 MFMA shape (twice the rate of
// 16x16x32 on this chip) and halves the LDS bytes each wave reads per tile.
// Combine kernel: one thread per (row, 16 channels) merges the splits.
#include <type_traits>

#include "mxfa_device.h"

namespace mxfa {
namespace {

constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int BN = kDecodeTile;          // 32 keys per tile
constexpr int ROWS = kDecodeRows;        // 64 rows per work group
constexpr int NTHREADS = 256;
constexpr int STAGES = 4;                // LDS tiles; STAGES - 1 in flight
constexpr int KSTEPS = DQK / 16 / 2;     // 18 contraction steps of 16 channels per wave
constexpr int CBLK = DV / 32 / 2;        // 8 blocks of 32 output channels per wave
constexpr int ROWB = DQK * 2;            // 1152 bytes per latent row
constexpr int CPR = DQK / 8;             // 72 chunks of 16 bytes per row
constexpr int TILEB = BN * ROWB;         // 36864 bytes per tile
constexpr int LOADS = TILEB / (16 * NTHREADS);  // 9 loads per thread per tile
static_assert(LOADS * 16 * NTHREADS == TILEB, "tile must split into whole loads");

// Chunk swizzle of a 1152-byte row (physical chunk = logical ^ swz(row)).
// Rows alternate between the two halves of the 16-chunk bank line; the XOR
// (< 8, so a chunk stays in its aligned group of 8 and inside the row)
// spreads 16 consecutive rows x one chunk over all 16 bank slots (K operand
// reads) and 4 consecutive rows x an aligned group of 4 chunks likewise
// (transposing V reads).
MXFA_DEV int swz(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

// fp8 latent rows: 16-byte chunks per row, chunks per thread per tile.
constexpr int CPR8 = DQK / 16;                                // 36
constexpr int LOADS8 = (BN * CPR8 + NTHREADS - 1) / NTHREADS;  // 5 (the last for half the threads)

template <bool kCap, bool kPaged, bool kFp8>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel(const DecodeParams p) {
    static_assert(!(kPaged && kFp8), "the fp8 cache is contiguous");
    constexpr int ESZ = kFp8 ? 1 : 2;  // bytes per stored kv element
    // Five LDS objects: a reader of one stage then never waits for the loads
    // streaming into the others.
    __shared__ __attribute__((aligned(1024))) char sT0[TILEB];
    __shared__ __attribute__((aligned(1024))) char sT1[TILEB];
    __shared__ __attribute__((aligned(1024))) char sT2[TILEB];
    __shared__ __attribute__((aligned(1024))) char sT3[TILEB];
    __shared__ __attribute__((aligned(1024))) f32x4_t sS[4][4][64];  // partial S^T per wave: [wave][r/4][lane]
    // fp8: a second exchange buffer (tiles alternate between the two), which
    // the three-stage fp8 pipeline leaves room for.
    __shared__ __attribute__((aligned(1024))) f32x4_t sS1[4][4][64];
    typedef f32x4_t Exchange[4][4][64];

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
    // Paged cache: sequence b's keys sit in pages block_table[b][*] of
    // page_size rows each; its length is capped at what its table row holds.
    const int k_start = kPaged ? 0 : p.cu_k[b];
    const int sk = kPaged ? max(0, min(p.seqlens_k[b], p.max_pages * p.page_size)) : p.cu_k[b + 1] - k_start;
    const int row0 = mg * ROWS;
    const int nrows = sq * G;
    if (row0 >= nrows) return;
    const int off = sk - sq;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int rb = w & 1;
    const int ch = w >> 1;
    const int lane = tid & 63;
    const int lr = lane & 31;  // S^T / O^T column: row 32*rb + lr of the group
    const int lh = lane >> 5;

    // Keys any row of the group can see, cut to this split (splits are tile aligned).
    const int last_row = min(row0 + ROWS, nrows) - 1;
    const KeyRange first = visible_range(row0 / G + off, sk, p.causal, p.window_left, p.window_right);
    const KeyRange last = visible_range(last_row / G + off, sk, p.causal, p.window_left, p.window_right);
    const int ntiles_all = (sk + BN - 1) / BN;
    const int tiles_per_split = (ntiles_all + p.splits - 1) / p.splits;
    const int s_lo = sp * tiles_per_split * BN;
    const int s_hi = min(sk, (sp + 1) * tiles_per_split * BN) - 1;
    const int lo = max(first.lo, s_lo);
    const int hi = min(last.hi, s_hi);

    // This wave's row block and this lane's row.
    const int brow0 = row0 + 32 * rb;
    const int my_row = brow0 + lr;
    const bool row_valid = my_row < nrows;
    const int my_tok = my_row / G;
    const int my_head = g * G + my_row % G;
    KeyRange mine = visible_range(my_tok + off, sk, p.causal, p.window_left, p.window_right);
    if (!row_valid) {
        mine.lo = 1;
        mine.hi = 0;
    }

    const long long q_tok_stride = (long long)p.heads_q * DQK;
    const long long kv_tok_stride = (long long)p.heads_kv * DQK;

    // Q^T slice as the B operand: lane holds row my_row, channels
    // 288*ch + 16*ks + 8*lh .. +7. Kept in accumulation registers: the MFMAs
    // read their B operand from there directly, which leaves the vector
    // registers to the accumulators and to LDS reads in flight.
    bf16x8_t qreg[KSTEPS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(p.q) + (long long)(q_start + (row_valid ? my_tok : 0)) * q_tok_stride +
                             (long long)my_head * DQK + 288 * ch + lh * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row_valid) v = load_u32x4(qp + ks * 16);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
        // Moved to accumulation registers only after every load is issued: a
        // move right after each load made each load wait for the one before.
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" : "+a"(qreg[ks]));
    }

    // K operand (A of S^T = K Q^T): key lr, logical chunk 36*ch + 2*ks + lh,
    // at byte kx[ks % 4] + 128*(ks / 4) (adding 8 to a chunk index commutes
    // with the swizzle, which only touches its low three bits).
    uint32_t kx[4];
    {
        const int f = swz(lr);
#pragma unroll
        for (int m = 0; m < 4; ++m) kx[m] = (uint32_t)(lr * ROWB + (((36 * ch + 2 * m + lh) ^ f) << 4));
    }
    // V^T operand (A of O^T = V^T P^T), two transposing reads per 32 channels
    // and 16 keys: 16-lane group gq, lane i reads key 8*which + 4*(gq/2) + i/4
    // of the 16-key step, channels 256*ch + 32*cb + 16*(gq%2) + 4*(i%4) .. +3,
    // i.e. logical chunk 32*ch + 4*cb + 2*(gq%2) + (i%4)/2, at byte
    // vx[which][cb % 2] + 128*(cb / 2) + 16*ROWB*h for key step h.
    uint32_t vx[2][2];
    {
        const int gq = lane >> 4;
        const int i = lane & 15;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const int key = 8 * which + 4 * (gq >> 1) + (i >> 2);
            const int f = swz(key);
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
                vx[which][c2] = (uint32_t)(key * ROWB + (((32 * ch + 4 * c2 + 2 * (gq & 1) + ((i & 3) >> 1)) ^ f) << 4) +
                                           (i & 1) * 8);
        }
    }
    // Global -> LDS: 16-byte chunk P = n*256 + tid of a tile is row P/72,
    // physical chunk P%72, which holds logical chunk (P%72) ^ swz(row).
    auto goff = [&](int n) __attribute__((always_inline)) -> uint32_t {
        const int P = n * NTHREADS + tid;
        const int row = P / CPR;
        const int c = (P % CPR) ^ swz(row);
        return (uint32_t)(row * (int)(kv_tok_stride * 2) + c * 16);
    };
    const char* KVseg = static_cast<const char*>(p.kv) + ((long long)k_start * kv_tok_stride + (long long)g * DQK) * ESZ;
    // Paged cache: physical page of a tile (a tile never straddles a page,
    // pages holding a multiple of BN keys) and the tile's first row in it;
    // page 0 for tiles past the keys, which are never read. Read one step
    // before its use. The table is read through the constant address space:
    // it is not written while the kernel runs, and so the read becomes a
    // scalar load, kept out of the vector-memory count that the stage waits
    // rely on. Tiles are looked up once each, in key order, so a cursor
    // (table index, row in the page) advanced by BN replaces a division by
    // the page size per tile.
    using ConstI32 = const __attribute__((address_space(4))) int32_t;
    struct PageRef {
        int phys;  // physical page
        int off;   // the tile's first row within it
    };
    int pc_idx = 0, pc_off = 0;  // cursor: the next tile to look up
    auto page_cursor_at = [&](int kt) __attribute__((always_inline)) {
        if constexpr (kPaged) {
            pc_idx = kt / p.page_size;
            pc_off = kt - pc_idx * p.page_size;
        }
    };
    auto next_page = [&](int kt) __attribute__((always_inline)) -> PageRef {
        PageRef r{0, pc_off};
        if constexpr (kPaged) {
            if (kt <= hi) {
                const ConstI32* tab = (const ConstI32*)p.block_table;
                r.phys = tab[(long long)b * p.max_pages + pc_idx];
            }
            pc_off += BN;
            if (pc_off == p.page_size) {
                pc_off = 0;
                ++pc_idx;
            }
        }
        return r;
    };
    // Buffer resource over the tile at key kt: its rows up to the last key
    // (rows past it read as zeros). Tiles past the split's last key, and
    // tiles whose page number lies outside the cache, get a resource of zero
    // bytes: their loads return zeros without touching memory.
    auto tile_rsrc = [&](int kt, PageRef pr) __attribute__((always_inline)) -> __amdgpu_buffer_rsrc_t {
        long long bytes = ((long long)(sk - kt - 1) * kv_tok_stride + DQK) * ESZ;
        const char* base = KVseg + (long long)kt * kv_tok_stride * ESZ;
        if (kPaged) {
            if ((unsigned)pr.phys >= (unsigned)p.num_pages) bytes = 0;
            else
                base = static_cast<const char*>(p.kv) +
                       (((long long)pr.phys * p.page_size + pr.off) * kv_tok_stride + (long long)g * DQK) * ESZ;
        }
        if (kt > hi) bytes = 0;
        if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
        return make_rsrc(bytes ? base : KVseg, (uint32_t)bytes);
    };
    // Tiles past the key range are issued too, as loads of zero bytes, so
    // every step has the same number of loads in flight behind it. A tile's
    // loads may be issued in parts (loads [n0, n1)).
    auto issue_part = [&](const __amdgpu_buffer_rsrc_t& r, char* stage, int n0, int n1) __attribute__((always_inline)) {
#pragma unroll
        for (int n = n0; n < n1; ++n) buffer_load_lds16(r, stage + (n * NTHREADS + w * 64) * 16, goff(n));
    };
    auto issue_tile = [&](int kt, char* stage) __attribute__((always_inline)) {
        issue_part(tile_rsrc(kt, next_page(kt)), stage, 0, LOADS);
    };
    // fp8 rows take another way into LDS: 16-byte chunks (16 values) are
    // loaded into registers three tiles ahead, converted to bf16 (exact: every
    // e4m3 value is a bf16 value) and written into the same swizzled bf16
    // stages. Chunk P = n*256 + tid of a tile is row P / 36, chunk P % 36,
    // whose values are the bf16 logical chunks 2c and 2c + 1 of the row (at
    // LDS offsets lo8[n] and lo8[n] ^ 16: the swizzle keeps the pair in one
    // aligned 32-byte slot). Positions past the tile (n = 4, tid >= 128)
    // reload chunk tid and are not written.
    uint32_t go8[LOADS8], lo8[LOADS8];
    if constexpr (kFp8) {
#pragma unroll
        for (int n = 0; n < LOADS8; ++n) {
            int P = n * NTHREADS + tid;
            if (P >= BN * CPR8) P = tid;
            const int row = P / CPR8;
            const int c = P % CPR8;
            go8[n] = (uint32_t)(row * (int)kv_tok_stride + c * 16);
            lo8[n] = (uint32_t)(row * ROWB + (((2 * c) ^ swz(row)) << 4));
        }
    }
    struct Raw8 {
        u32x4_t v[LOADS8];
    };
    auto load8 = [&](int kt, Raw8& r) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(kt, PageRef{0, 0});
#pragma unroll
        for (int n = 0; n < LOADS8; ++n) r.v[n] = buffer_load16(rs, go8[n], 0);
    };
    auto load8_part = [&](const __amdgpu_buffer_rsrc_t& rs, Raw8& r, int n0, int n1) __attribute__((always_inline)) {
#pragma unroll
        for (int n = n0; n < n1; ++n) r.v[n] = buffer_load16(rs, go8[n], 0);
    };
    auto store8 = [&](const Raw8& r, char* stage) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < LOADS8; ++n) {
            if (n == LOADS8 - 1 && tid >= BN * CPR8 - (LOADS8 - 1) * NTHREADS) break;
            uint32_t h[8];
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                // Two e4m3 codes (bytes 0-1, then 2-3) to two bf16 each, scale 1:
                // every e4m3 value is exact in bf16.
                h[2 * wd] = __builtin_bit_cast(uint32_t,
                                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.v[n][wd], 1.0f, false));
                h[2 * wd + 1] = __builtin_bit_cast(uint32_t,
                                                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.v[n][wd], 1.0f, true));
            }
            typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
            *(lds_u32x4*)to_lds(stage + lo8[n]) = u32x4_t{h[0], h[1], h[2], h[3]};
            *(lds_u32x4*)to_lds(stage + (lo8[n] ^ 16u)) = u32x4_t{h[4], h[5], h[6], h[7]};
        }
    };

    // O^T accumulators: channel block cb (channels 256*ch + 32*cb + ...), column lr.
    f32x16_t acc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) acc[cb] = f32x16_t{};
    float m_run = -INFINITY;  // running max of row my_row, log2 units (may trail the true max by <= 8)
    float l_part = 0.0f;      // running sum of p over this lane's keys (fp32; for the LSE)
    float lb_part = 0.0f;     // running sum of bf16(p), the weights the P V MFMAs use (normalises O)

    // Partial S^T over this wave's channel half.
    auto qk_tile = [&](const char* tile) __attribute__((always_inline)) -> f32x16_t {
        uint32_t kxl[4] = {kx[0], kx[1], kx[2], kx[3]};
        asm volatile("" : "+v"(kxl[0]), "+v"(kxl[1]), "+v"(kxl[2]), "+v"(kxl[3]));
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_read16(tile + kxl[ks & 3] + 128 * (ks >> 2)));
            s = mfma32x32x16(a, qreg[ks], s);
        }
        // Schedule: the LDS reads run KQ_AHEAD steps ahead of the MFMAs, and
        // up to 6 vector-ALU instructions (the softmax of the previous tile)
        // follow each MFMA.
        constexpr int KQ_AHEAD = 6;
        __builtin_amdgcn_sched_group_barrier(0x100, KQ_AHEAD, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS - KQ_AHEAD; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
#pragma unroll
        for (int ks = 0; ks < KQ_AHEAD; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
        return s;
    };
    // Keys this lane's row may use: its own visible range cut to the split,
    // as key_lo + [0, key_span] (an empty range becomes one no key reaches).
    int key_lo = max(mine.lo, lo);
    int key_span = min(mine.hi, hi) - key_lo;
    if (key_span < 0) {
        key_lo = 0x40000000;
        key_span = 0;
    }
    // The partial scores of the next tile (MFMAs) interleaved with the
    // softmax of the current one (vector ALU): after each MFMA one slice of
    // the softmax, fenced so that the compiler keeps the interleave (the
    // MFMA runs while the slice issues). s_cur: this wave's partial scores of
    // the current tile; the partner's are added here. Same arithmetic as
    // softmax_tile.
    auto qk_softmax = [&](const char* tile, const f32x16_t& s_cur, int kt, uint32_t (&pk)[8], float& alpha,
                          const Exchange& xs, auto&& mid_hook) __attribute__((always_inline)) -> f32x16_t {
        uint32_t kxl[4] = {kx[0], kx[1], kx[2], kx[3]};
        asm volatile("" : "+v"(kxl[0]), "+v"(kxl[1]), "+v"(kxl[2]), "+v"(kxl[3]));
        constexpr int AHEAD = 6;  // K reads in flight ahead of their MFMA
        bf16x8_t kr[KSTEPS];
        f32x4_t po[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) po[q4] = xs[w ^ 2][q4][lane];
#pragma unroll
        for (int ks = 0; ks < AHEAD; ++ks)
            kr[ks] = __builtin_bit_cast(bf16x8_t, lds_read16(tile + kxl[ks & 3] + 128 * (ks >> 2)));
        f32x16_t sn = f32x16_t{};
        f32x16_t x = s_cur;
        // Optimistic max: P against the running max of the earlier tiles;
        // the tile's own max only when some lane's sum of P exceeds 2^8.
        const float nb = (m_run == -INFINITY) ? 0.0f : -m_run;
        float psum = 0.0f;
        float psb = 0.0f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks + AHEAD < KSTEPS)
                kr[ks + AHEAD] = __builtin_bit_cast(
                    bf16x8_t, lds_read16(tile + kxl[(ks + AHEAD) & 3] + 128 * ((ks + AHEAD) >> 2)));
            sn = mfma32x32x16(kr[ks], qreg[ks], sn);
            if (ks >= 2 && ks < 10) {  // logits and mask of elements 2(ks-2), 2(ks-2)+1
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * (ks - 2) + e;
                    float v = x[r] + po[r >> 2][r & 3];
                    v = kCap ? score_to_logit<true>(v, p.x_mul, p.cap_mul, p.cap_out) : v * p.x_mul;
                    const int key = kt + 8 * (r >> 2) + 4 * lh + (r & 3);
                    v = ((unsigned)(key - key_lo) <= (unsigned)key_span) ? v : -INFINITY;
                    x[r] = v;
                }
            }
            if (ks >= 10) {  // exp2 and packing of elements 2(ks-10), 2(ks-10)+1
                const int r = 2 * (ks - 10);
                const float p0 = fast_exp2(x[r] + nb);
                const float p1 = fast_exp2(x[r + 1] + nb);
                psum += p0 + p1;
                pk[r >> 1] = pack_bf16x2(p0, p1);
                psb = add_bf16x2(pk[r >> 1], psb);
            }
            if (ks == 6) mid_hook();
            __builtin_amdgcn_sched_barrier(0);
        }
        alpha = 1.0f;
        if (wave_any(m_run == -INFINITY || psum > 256.0f)) {
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, x[r]);
            mt = half_max(mt);
            const float m_new = fmaxf(m_run, mt);
            alpha = (m_new == m_run) ? 1.0f : fast_exp2(m_run - m_new);
            m_run = m_new;
            const float nb2 = (m_run == -INFINITY) ? 0.0f : -m_run;
            psum = 0.0f;
            psb = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(x[r] + nb2);
                const float p1 = fast_exp2(x[r + 1] + nb2);
                psum += p0 + p1;
                pk[r >> 1] = pack_bf16x2(p0, p1);
                psb = add_bf16x2(pk[r >> 1], psb);
            }
        }
        l_part = l_part * alpha + psum;
        lb_part = lb_part * alpha + psb;
        return sn;
    };
    // O^T += V^T P^T over the tile's two 16-key steps.
    auto pv_tile = [&](const char* tile, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
        uint32_t vxl[4] = {vx[0][0], vx[0][1], vx[1][0], vx[1][1]};
        asm volatile("" : "+v"(vxl[0]), "+v"(vxl[1]), "+v"(vxl[2]), "+v"(vxl[3]));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t pv = {pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) {
                const char* base = tile + 16 * ROWB * h + 128 * (cb >> 1);
                const u32x2_t r0 = lds_read_tr16(base + vxl[cb & 1]);
                const u32x2_t r1 = lds_read_tr16(base + vxl[2 + (cb & 1)]);
                const u32x4_t av = {r0[0], r0[1], r1[0], r1[1]};
                acc[cb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pb, acc[cb]);
            }
        }
        // Schedule: the transposing reads run PV_AHEAD MFMAs ahead.
        constexpr int PV_AHEAD = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_AHEAD, 0);
#pragma unroll
        for (int m = 0; m < 2 * CBLK - PV_AHEAD; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PV_AHEAD, 0);
    };

    // fp8: O^T += V^T P^T as pv_tile, with the conversion of a loaded tile
    // into its stage spread over the MFMAs: after MFMA m (2 <= m < 12) the
    // four conversions and the LDS write of half chunk m - 2 (chunk (m-2)/2,
    // its first or second 8 values), fenced so that the write issues while
    // the MFMA runs. A thread with no fifth chunk reloaded its first one,
    // so it rewrites the same values to the same place.
    auto pv_fill = [&](const char* tile, const uint32_t (&pk)[8], const Raw8& r, char* stage)
                       __attribute__((always_inline)) {
        uint32_t vxl[4] = {vx[0][0], vx[0][1], vx[1][0], vx[1][1]};
        asm volatile("" : "+v"(vxl[0]), "+v"(vxl[1]), "+v"(vxl[2]), "+v"(vxl[3]));
        constexpr int NM = 2 * CBLK;  // MFMAs: m = CBLK*h + cb
        constexpr int AHEAD = 4;
        u32x2_t ra[NM], rb2[NM];
        auto rd = [&](int m) __attribute__((always_inline)) {
            const int h = m / CBLK;
            const int cb = m % CBLK;
            const char* base = tile + 16 * ROWB * h + 128 * (cb >> 1);
            ra[m] = lds_read_tr16(base + vxl[cb & 1]);
            rb2[m] = lds_read_tr16(base + vxl[2 + (cb & 1)]);
        };
#pragma unroll
        for (int m = 0; m < AHEAD; ++m) rd(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + AHEAD < NM) rd(m + AHEAD);
            const int h = m / CBLK;
            const int cb = m % CBLK;
            const u32x4_t pv = {pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
            const u32x4_t av = {ra[m][0], ra[m][1], rb2[m][0], rb2[m][1]};
            acc[cb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, pv), acc[cb]);
            if (m >= 2 && m < 2 + 2 * LOADS8) {
                const int n = (m - 2) >> 1;
                const int half = (m - 2) & 1;
                uint32_t hv[4];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int wd = 2 * half + k;
                    hv[2 * k] = __builtin_bit_cast(uint32_t,
                                                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.v[n][wd], 1.0f, false));
                    hv[2 * k + 1] = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.v[n][wd], 1.0f, true));
                }
                typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
                *(lds_u32x4*)to_lds(stage + (lo8[n] ^ (16u * half))) = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (lo <= hi) {
        const int kt0 = lo & ~(BN - 1);
        const int ntiles = (hi - kt0) / BN + 1;
        // Contiguous cache: the loop's tiles read one tile's span, the last
        // tile of the split up to the segment's end, tiles past the split
        // nothing; the spans are set here so that a step's resource is a
        // compare, two selects and the tile's base address.
        const long long span64 = ((long long)(BN - 1) * kv_tok_stride + DQK) * ESZ;
        const uint32_t span = (uint32_t)(span64 > 0x7fffffffLL ? 0x7fffffffLL : span64);
        const int kt_last = kt0 + (ntiles - 1) * BN;
        long long last64 = ((long long)(sk - kt_last - 1) * kv_tok_stride + DQK) * ESZ;
        const uint32_t last_bytes = (uint32_t)(last64 < (long long)span ? last64 : (long long)span);
        auto loop_rsrc = [&](int kt, PageRef pr) __attribute__((always_inline)) -> __amdgpu_buffer_rsrc_t {
            if constexpr (kPaged) return tile_rsrc(kt, pr);
            const uint32_t bytes = kt > hi ? 0u : (kt == kt_last ? last_bytes : span);
            return make_rsrc(bytes ? KVseg + (long long)kt * kv_tok_stride * ESZ : KVseg, bytes);
        };
        // Tile j lives in stage j % 4. Past the end, tiles are issued as
        // zero-byte loads, so the count of loads behind each wait is fixed.
        f32x16_t s_mine = f32x16_t{};
        auto publish = [&](Exchange& xs) __attribute__((always_inline)) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                xs[w][q4][lane] = f32x4_t{s_mine[4 * q4], s_mine[4 * q4 + 1], s_mine[4 * q4 + 2], s_mine[4 * q4 + 3]};
        };
      if constexpr (!kFp8) {
        page_cursor_at(kt0);
        issue_tile(kt0, sT0);
        issue_tile(kt0 + BN, sT1);
        issue_tile(kt0 + 2 * BN, sT2);
        PageRef pg_fill = next_page(kt0 + 3 * BN);  // page of the tile the next step issues
        asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // this wave's loads of tile 0
        lds_barrier();
        s_mine = qk_tile(sT0);
        publish(sS);
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // this wave's loads of tile 1
        lds_barrier();
        // Step j: add the partner's partial scores of tile j; compute this
        // wave's partial scores of tile j+1 on the MFMAs while the vector ALU
        // runs the softmax of tile j; barrier (both partials of tile j read);
        // publish the partial of tile j+1; P V of tile j; wait for this wave's
        // loads of tile j+2 (tile j+3 may still run: 9 loads); barrier (tile
        // j+2 landed, partials of tile j+1 published, tile j consumed). The
        // loads of tile j+3 go into the stage of tile j-1 (consumed before
        // the previous step's closing barrier) in three parts spread over the
        // step, so that their issue overlaps the MFMAs.
        auto step = [&](auto stage_tag, int j) __attribute__((always_inline)) {
            constexpr int S = decltype(stage_tag)::value;
            char* const cur = S == 0 ? sT0 : S == 1 ? sT1 : S == 2 ? sT2 : sT3;
            char* const nxt = S == 0 ? sT1 : S == 1 ? sT2 : S == 2 ? sT3 : sT0;
            char* const prv = S == 0 ? sT3 : S == 1 ? sT0 : S == 2 ? sT1 : sT2;
            const int kt_fill = kt0 + (j + 3) * BN;  // tile j+3 -> the stage of tile j-1
            uint32_t pk[8];
            float alpha = 1.0f;
            const __amdgpu_buffer_rsrc_t rfill = loop_rsrc(kt_fill, pg_fill);
            pg_fill = next_page(kt_fill + BN);
            // Wait for the page-table read here, where no LDS read is in
            // flight: the scalar load shares the LDS wait counter and returns
            // out of order, so while it is pending every LDS wait of the step
            // would have to drain all reads.
            if constexpr (kPaged) asm volatile("" : "+s"(pg_fill.phys));
            issue_part(rfill, prv, 0, 3);
            // Every wave runs the same code (a row block past the group's rows
            // sees no key, so its results stay zero and are never read): the
            // compiler then keeps an exact count of the LDS reads in flight.
            // On the last step the scores are of a finished (zero-filled)
            // tile and are not used.
            s_mine = qk_softmax(nxt, s_mine, kt0 + j * BN, pk, alpha, sS,
                                [&]() __attribute__((always_inline)) { issue_part(rfill, prv, 3, 6); });
            lds_barrier();
            issue_part(rfill, prv, 6, LOADS);
            publish(sS);
            if (wave_any(alpha != 1.0f)) {
#pragma unroll
                for (int cb = 0; cb < CBLK; ++cb) acc[cb] *= alpha;
            }
            pv_tile(cur, pk);
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
            lds_barrier();
        };
        static_assert(LOADS == 9, "the vmcnt counts above assume 9 loads per tile");
        using st0 = std::integral_constant<int, 0>;
        using st1 = std::integral_constant<int, 1>;
        using st2 = std::integral_constant<int, 2>;
        using st3 = std::integral_constant<int, 3>;
        int j = 0;
        for (; j + STAGES <= ntiles; j += STAGES) {
            step(st0{}, j);
            step(st1{}, j + 1);
            step(st2{}, j + 2);
            step(st3{}, j + 3);
        }
        if (j < ntiles) step(st0{}, j);
        if (j + 1 < ntiles) step(st1{}, j + 1);
        if (j + 2 < ntiles) step(st2{}, j + 2);
        // Drain the look-ahead loads before the work group's LDS is released.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        // fp8 rows: tile j is loaded into registers in step j-3 (set j % 3)
        // and converted into its LDS stage j % 3 during the P V MFMAs of step
        // j-2: two steps of load latency covered with three register sets (a
        // fourth set left too few registers for the P V reads to run ahead).
        Raw8 R0, R1, R2;
        load8(kt0, R0);
        load8(kt0 + BN, R1);
        load8(kt0 + 2 * BN, R2);
        store8(R0, sT0);
        store8(R1, sT1);
        lds_barrier();
        s_mine = qk_tile(sT0);
        publish(sS);
        lds_barrier();
        // Step j: loads of tile j+3 into the registers of tile j (converted
        // in step j-2), in three parts; scores of tile j+1 with the softmax
        // of tile j; publish; P V of tile j with tile j+2 converted into the
        // stage of tile j-1 (last read in step j-1); barrier. The partial
        // scores of tile t go through exchange buffer t % 2: publishing tile
        // j+1's in step j overwrites tile j-1's, which the partner read in
        // step j-1, before the barrier that ended it; so one barrier per step
        // suffices.
        auto step8 = [&](auto stage_tag, int j, Raw8& rl, const Raw8& rc) __attribute__((always_inline)) {
            constexpr int S = decltype(stage_tag)::value;
            char* const cur = S == 0 ? sT0 : S == 1 ? sT1 : sT2;
            char* const nxt = S == 0 ? sT1 : S == 1 ? sT2 : sT0;
            char* const fill = S == 0 ? sT2 : S == 1 ? sT0 : sT1;
            uint32_t pk[8];
            float alpha = 1.0f;
            const __amdgpu_buffer_rsrc_t rs = loop_rsrc(kt0 + (j + 3) * BN, PageRef{0, 0});
            load8_part(rs, rl, 0, 2);
            s_mine = qk_softmax(nxt, s_mine, kt0 + j * BN, pk, alpha, (j & 1) ? sS1 : sS,
                                [&]() __attribute__((always_inline)) { load8_part(rs, rl, 2, 4); });
            load8_part(rs, rl, 4, LOADS8);
            publish((j & 1) ? sS : sS1);
            if (wave_any(alpha != 1.0f)) {
#pragma unroll
                for (int cb = 0; cb < CBLK; ++cb) acc[cb] *= alpha;
            }
            pv_fill(cur, pk, rc, fill);
            lds_barrier();
        };
        using st0 = std::integral_constant<int, 0>;
        using st1 = std::integral_constant<int, 1>;
        using st2 = std::integral_constant<int, 2>;
        int j = 0;
        for (; j + 3 <= ntiles; j += 3) {
            step8(st0{}, j, R0, R2);
            step8(st1{}, j + 1, R1, R0);
            step8(st2{}, j + 2, R2, R1);
        }
        if (j < ntiles) step8(st0{}, j, R0, R2);
        if (j + 1 < ntiles) step8(st1{}, j + 1, R1, R0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }

    // Partial (m, l, acc) of this split: row 32*rb + lr of the group, channels
    // 256*ch + 32*cb + 8*(r/4) + 4*lh + r%4.
    const long long pidx = (((long long)b * p.heads_kv + g) * p.m_groups + mg) * p.splits + sp;
    const float l_row = half_sum(l_part);
    const float lb_row = half_sum(lb_part);
    const int grow_idx = 32 * rb + lr;
    float* pacc = p.part_acc + (pidx * ROWS + grow_idx) * DV + 256 * ch + 4 * lh;
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4_t*>(pacc + 32 * cb + 8 * q4) =
                f32x4_t{acc[cb][4 * q4], acc[cb][4 * q4 + 1], acc[cb][4 * q4 + 2], acc[cb][4 * q4 + 3]};
    if (ch == 0 && lh == 0) {
        float* pml = p.part_ml + pidx * 3 * ROWS;
        pml[grow_idx] = m_run;
        pml[ROWS + grow_idx] = l_row;
        pml[2 * ROWS + grow_idx] = lb_row;
    }
}

// Merge the splits: M = max_s m_s, w_s = exp2(m_s - M),
// O = sum_s w_s acc_s / sum_s w_s lb_s (lb: sums of the bf16 weights the P V
// MFMAs used), LSE = ln2 * (M + log2 sum_s w_s l_s) (l: fp32 sums),
// with a running max over chunks of splits. One thread per (row, 16
// channels); 8 rows per work group.
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
    // One pass with a running max over chunks of CH splits; all loads of a
    // chunk are issued before any is used (one memory round trip per chunk).
    constexpr int CH = 2;
    float M = -INFINITY, L = 0.0f, Lb = 0.0f;
    float o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = 0.0f;
    for (int s0 = 0; s0 < p.splits; s0 += CH) {
        float ms[CH], ls[CH], lbs[CH];
        f32x4_t as[CH][4];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = s0 + c < p.splits;
            const long long pi = pidx0 + (in ? s0 + c : 0);
            ms[c] = in ? p.part_ml[pi * 3 * ROWS + row] : -INFINITY;
            ls[c] = p.part_ml[pi * 3 * ROWS + ROWS + row];
            lbs[c] = p.part_ml[pi * 3 * ROWS + 2 * ROWS + row];
            const f32x4_t* a = reinterpret_cast<const f32x4_t*>(p.part_acc + (pi * ROWS + row) * DV + d0);
#pragma unroll
            for (int j = 0; j < 4; ++j) as[c][j] = a[j];
        }
        float mc = M;
#pragma unroll
        for (int c = 0; c < CH; ++c) mc = fmaxf(mc, ms[c]);
        if (mc == -INFINITY) continue;  // nothing visible so far
        const float rs = fast_exp2(M - mc);  // 0 while M is -inf
        L *= rs;
        Lb *= rs;
#pragma unroll
        for (int j = 0; j < 16; ++j) o[j] *= rs;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float ws = fast_exp2(ms[c] - mc);  // 0 for splits past the end or with no keys
            L += ws * ls[c];
            Lb += ws * lbs[c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o[4 * j + 0] += ws * as[c][j][0];
                o[4 * j + 1] += ws * as[c][j][1];
                o[4 * j + 2] += ws * as[c][j][2];
                o[4 * j + 3] += ws * as[c][j][3];
            }
        }
        M = mc;
    }
    const float inv = (Lb > 0.0f) ? p.v_scale / Lb : 0.0f;  // v_scale: the fp8 cache's dequantisation scale
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

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream) {
    const long long units = (long long)p.batch * p.heads_kv * p.m_groups;
    if (units <= 0) return hipSuccess;
    const long long grid_split = units * p.splits;
    if (grid_split > 0x7fffffffLL || units * (ROWS / CROWS) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)grid_split);
    const bool cap = p.softcap > 0.0f;
    if (p.kv_fp8) {
        if (cap) hipLaunchKernelGGL((decode_split_kernel<true, false, true>), grid, dim3(NTHREADS), 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<false, false, true>), grid, dim3(NTHREADS), 0, stream, p);
    } else if (p.block_table) {
        if (cap) hipLaunchKernelGGL((decode_split_kernel<true, true, false>), grid, dim3(NTHREADS), 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<false, true, false>), grid, dim3(NTHREADS), 0, stream, p);
    } else {
        if (cap) hipLaunchKernelGGL((decode_split_kernel<true, false, false>), grid, dim3(NTHREADS), 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<false, false, false>), grid, dim3(NTHREADS), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(units * (ROWS / CROWS))), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mxfa
