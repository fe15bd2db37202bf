// mxfa_internal.h -- kernel parameter blocks and launcher declarations shared
// by the C-ABI layer (mxfa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfa {

// One forward problem (dense or packed). Dense problems leave cu_q/cu_k null
// and use seqlen_q/seqlen_k for every segment; packed problems read the
// segment bounds from cu_q/cu_k and use seqlen_q/seqlen_k as upper bounds.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;              // may be null
    const int32_t* cu_q;     // null for dense
    const int32_t* cu_k;
    int batch;
    int seqlen_q;            // dense: every segment; packed: max over segments
    int seqlen_k;
    int total_q;             // packed LSE row stride ([Hq, total_q])
    int heads_q;
    int heads_kv;
    int group;               // heads_q / heads_kv
    int causal;
    int window_left;         // -1 = unbounded
    int window_right;
    float softcap;           // 0 = off
    float scale;             // softmax scale
    float x_mul;             // score -> log2-domain logit multiplier (no cap: scale*log2e)
    float cap_mul;           // cap: 2*log2e*scale/cap
    float cap_out;           // cap: cap*log2e
    int n_qtiles;            // ceil(seqlen_q / BM), set by the launcher
    int xcd_cus;             // compute units per XCD (pairing of the first dispatch round), 0 = unknown
    // Packed problems: the work list the list kernel wrote (null for dense)
    // and an upper bound on its length (sizes the grid).
    const int* worklist;
    long long list_max;
};

// The work-list kernel of a packed forward: (segment, q tile) pairs of bm
// rows, ordered by the number of bn-key tiles they stream, most first.
struct WorkListParams {
    const int32_t* cu_q;
    const int32_t* cu_k;
    int* ws;                 // count, prefix sums, pairs (worklist_bytes())
    long long list_max;      // pairs the workspace holds; items past it are dropped
    int batch;
    int max_seqlen_k;
    int bm;
    int bn;
    int causal;
    int window_left;
    int window_right;
    int shift;               // set by the launcher
};

// One latent-KV split decode.
struct DecodeParams {
    const void* q;
    const void* kv;
    void* o;
    float* lse;              // may be null
    const int32_t* cu_q;
    const int32_t* cu_k;
    float* part_acc;         // [batch, m_groups, splits, 64, d_v] fp32
    float* part_ml;          // [batch, m_groups, splits, 3, 64] fp32 (max, sum of p, sum of bf16(p))
    int batch;
    int max_seqlen_q;
    int max_seqlen_k;
    int total_q;
    int heads_q;
    int heads_kv;
    int group;
    int m_groups;            // ceil(max_seqlen_q * group / 64)
    int splits;
    int causal;
    int window_left;
    int window_right;
    float softcap;
    float x_mul;
    float cap_mul;
    float cap_out;
    // Paged latent cache (null block_table: contiguous kv with cu_k).
    const int32_t* block_table;  // [batch, max_pages] physical page of each logical page
    const int32_t* seqlens_k;    // [batch] keys of each sequence
    int page_size;               // keys per page, a multiple of kDecodeTile
    int max_pages;               // row length of block_table
    int num_pages;               // pages in the cache (kv holds num_pages * page_size rows)
    // fp8 (OCP e4m3) latent cache: stored value x stands for v_scale * x; the
    // scale of the scores is folded into x_mul / cap_mul by the host.
    int kv_fp8;
    float v_scale;               // 1 for a bf16 cache
};

// Split-KV decode for standard heads (separate K and V).
struct GqaDecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;              // may be null
    const int32_t* cu_q;
    const int32_t* cu_k;
    float* part_acc;         // [batch, heads_kv, m_groups, splits, 32, head_dim] fp32 (splits > 1)
    float* part_ml;          // [batch, heads_kv, m_groups, splits, 3, 32] fp32 (max, sum of p, sum of bf16(p))
    int batch;
    int total_q;
    int heads_q;
    int heads_kv;
    int group;
    int m_groups;            // ceil(max_seqlen_q * group / 32)
    int splits;
    int causal;
    int window_left;
    int window_right;
    float softcap;
    float x_mul;
    float cap_mul;
    float cap_out;
};

// Page-table description of a paged latent cache, as the host receives it.
struct PagedKV {
    const int32_t* block_table;
    const int32_t* seqlens;
    int page_size;
    int max_pages;
    int num_pages;
};

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, hipStream_t stream);
// Shader-clock probe (clock_probe.hip): out[0] = shader-clock cycles,
// out[1] = 100 MHz real-time ticks over an interval of `ticks` ticks.
hipError_t launch_clock_probe(unsigned long long* out, unsigned ticks, hipStream_t stream);

hipError_t launch_varlen_worklist(const WorkListParams& p, hipStream_t stream);
size_t worklist_bytes(int batch, long long max_items);
hipError_t launch_fwd_f32(const FwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_gqa(const GqaDecodeParams& p, int head_dim, hipStream_t stream);

// Accelerator dies (XCDs) of the device, each with its own L2.
constexpr int kXcdCount = 8;

// Forward tiles: query rows per work group and keys per tile, bf16 and fp32.
constexpr int kFwdBf16Rows = 128;
constexpr int kFwdBf16Keys = 64;
constexpr int kFwdF32Rows = 32;
constexpr int kFwdF32Keys = 32;

// Rows of one decode work group: (query token, head-in-group) pairs.
constexpr int kDecodeRows = 64;
// Standard-head decode: rows per work group, keys per tile.
constexpr int kGqaRows = 32;
constexpr int kGqaTile = 64;
// Keys per decode tile; split boundaries are multiples of it.
constexpr int kDecodeTile = 32;

}  // namespace mxfa
