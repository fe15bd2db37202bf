/*
 * mxfa.h -- fused scaled-dot-product attention forward for MI355X (gfx950).
 *
 * C ABI of libmxfa.so. Every call computes, on the caller's HIP stream,
 *
 *     O = softmax(scale * Q K^T + mask) V        and      LSE = log sum exp(row scores)
 *
 * tile by tile with a running row max and sum, so the score matrix is never
 * stored. The operation is the one stated by the mxflashattn 1.4.0 page
 * (api.py: flash_attn_func / flash_attn_varlen_func; prefill.py:
 * prefill_chunked_reference) and computed, tile by tile, as in the
 * oxillama-runtime 0.1.0 page (src/flash_attention.rs, flash_attention).
 *
 * Semantics shared by every entry point
 * -------------------------------------
 *  - Row i of a segment with Sq queries and Sk keys sits at key position
 *    pos = i + (Sk - Sq) (bottom-right alignment, as in prefill_chunked_reference).
 *    Key j is visible iff 0 <= j < Sk, and j <= pos when causal, and
 *    j >= pos - window_left when window_left >= 0, and j <= pos + window_right
 *    when window_right >= 0 (window bounds inclusive; -1 = unbounded).
 *  - Score of a visible key: t = scale * <q_i, k_j>; when softcap > 0 it is
 *    replaced by softcap * tanh(t / softcap) before the softmax.
 *  - Query head h reads key/value head h / (heads_q / heads_kv) (grouped-query
 *    attention; flash_attention_gqa on the oxillama-runtime page).
 *  - A row that sees no key gets O = 0 and LSE = -inf.
 *  - LSE is float32, natural log.
 *  - bf16 inputs: products accumulate in fp32; the softmax weights p enter
 *    the P V product rounded to bf16, and O is divided by the sum of those
 *    rounded weights (so a row's weights sum to one), the LSE taken from the
 *    fp32 sum of p; O is rounded to bf16 with round-to-nearest-even. f32
 *    inputs: fp32 throughout.
 *
 * Ownership and execution
 * -----------------------
 *  - All tensor pointers are device pointers owned by the caller; the library
 *    keeps none of them after the call returns and allocates no device memory.
 *  - Work is enqueued on `stream` (NULL = the default stream) and is complete
 *    when the stream reaches that point. No call synchronises the device.
 *  - Tensors are contiguous in the layouts stated per call. q, k, v, kv and o
 *    must be 16-byte aligned; lse and cu_seqlens 4-byte aligned.
 *  - The contents of cu_seqlens (non-decreasing, starting at 0, last entry =
 *    total) are the caller's contract and are not checked on the device.
 *  - heads_q and heads_kv are at most MXFA_MAX_HEADS; beyond it a call
 *    returns MXFA_ERR_UNSUPPORTED (the kernels address one tile of keys, all
 *    kv heads of each key row, through a buffer range of under 2 GiB).
 *
 * Errors
 * ------
 *  Every call returns an mxfa_status. Arguments are checked on the host
 *  before anything is enqueued; on a non-OK status nothing was enqueued.
 *  mxfa_last_error() returns a message for the calling thread's last non-OK
 *  status. The library never aborts and never prints.
 */
#ifndef MXFA_H
#define MXFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mxfa_stream_t; /* the same handle as hipStream_t */

#define MXFA_MAX_HEADS 16384 /* largest heads_q and heads_kv any call accepts */

typedef enum {
    MXFA_OK = 0,
    MXFA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, inconsistent heads, ... */
    MXFA_ERR_UNSUPPORTED = 2, /* head dim, dtype or head count the library has no kernel for */
    MXFA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query says */
    MXFA_ERR_HIP = 4          /* the HIP runtime reported an error (launch, device query) */
} mxfa_status;

typedef enum { MXFA_F32 = 0, MXFA_BF16 = 1 } mxfa_dtype;

/*
 * Dense forward (flash_attn_func on the mxflashattn page).
 *   q   [batch, seqlen_q, heads_q,  head_dim]
 *   k,v [batch, seqlen_k, heads_kv, head_dim]
 *   o   [batch, seqlen_q, heads_q,  head_dim]     (written)
 *   lse [batch, heads_q, seqlen_q] float32       (written; may be NULL)
 * dtype: MXFA_F32 or MXFA_BF16 for q, k, v and o alike. head_dim: 64 or 128.
 * batch, seqlen_q, seqlen_k >= 0 (zero-sized calls return MXFA_OK).
 * heads_kv >= 1 divides heads_q. window_left/right >= -1. softcap >= 0 and
 * finite (0 = off). scale finite.
 */
mxfa_status mxfa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int batch, int seqlen_q, int seqlen_k, int heads_q, int heads_kv,
                     int head_dim, mxfa_dtype dtype, int causal, int window_left,
                     int window_right, float softcap, float scale, mxfa_stream_t stream);

/*
 * Packed variable-length forward (flash_attn_varlen_func on the mxflashattn
 * page; packed batches as in the lattice-inference page's
 * src/attention/standard.rs). Segment b owns query tokens
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key tokens
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); segments never attend to each other.
 *   q   [total_q, heads_q,  head_dim]      k, v [total_k, heads_kv, head_dim]
 *   o   [total_q, heads_q,  head_dim]      lse  [heads_q, total_q] float32 (may be NULL)
 *   cu_seqlens_q, cu_seqlens_k: int32 device arrays of batch + 1 entries.
 * max_seqlen_q / max_seqlen_k must bound every segment's length (they size the
 * work list; rows of a segment longer than max_seqlen_q may be left unwritten).
 * workspace: device memory of at least mxfa_fwd_varlen_workspace_bytes()
 * bytes for the same batch and max_seqlen_q, 16-byte aligned; owned by the
 * caller, overwritten (nothing in it needs clearing), not needed after the
 * stream passes the call. A first small kernel walks cu_seqlens on the device
 * and writes the list of (segment, query tile) pairs there, longest causal
 * work first; the forward kernel then runs exactly those tiles. Too small a
 * workspace: MXFA_ERR_WORKSPACE, nothing enqueued.
 * Other arguments as for mxfa_fwd.
 */
mxfa_status mxfa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                            int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                            int heads_q, int heads_kv, int head_dim, mxfa_dtype dtype, int causal,
                            int window_left, int window_right, float softcap, float scale,
                            void* workspace, size_t workspace_bytes, mxfa_stream_t stream);

/*
 * Workspace bytes mxfa_fwd_varlen needs (0 when batch or max_seqlen_q is 0):
 * a count, batch + 1 prefix sums and one (segment, q tile) pair per query
 * tile of batch segments of max_seqlen_q tokens, for either dtype. heads_q
 * and head_dim do not change it (every query head reads the same list); they
 * are part of the signature so that a future kernel may depend on them.
 * Host-only arithmetic, no device query.
 */
size_t mxfa_fwd_varlen_workspace_bytes(int batch, int max_seqlen_q, int heads_q, int head_dim);

/* Bytes of the static device array mxfa_fwd_varlen_noalloc keeps its work list in. */
#define MXFA_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * Allocation-free packed forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, computation and result as
 * mxfa_fwd_varlen (bit for bit), minus the workspace: the work list goes into
 * a static device array of the library, MXFA_NOALLOC_SCRATCH_BYTES bytes, one
 * copy per GPU, held from the library's load until the process ends (its
 * address is looked up once per device, on the first call made with that
 * device current). The list holds one entry per query tile, about 130,000
 * of them (16.7 million query tokens at the bf16 kernel's 128-row tiles,
 * 4.2 million at the fp32 kernel's 32); a problem whose list would not fit
 * returns MXFA_ERR_WORKSPACE with nothing enqueued. The call allocates nothing and calls no allocating
 * routine. Every call on a GPU shares that GPU's array, which keeps the last
 * call's contents (nothing in it needs clearing): calls that overlap on one
 * GPU -- on streams that do not order them -- race and must not be made.
 */
mxfa_status mxfa_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                                    int total_k, int heads_q, int heads_kv, int head_dim,
                                    mxfa_dtype dtype, int causal, int window_left, int window_right,
                                    float softcap, float scale, mxfa_stream_t stream);

/*
 * Split-KV decode over a shared latent KV (the kernelbot amd-mixed-mla
 * submission 588924 page: _flash_splitk then _reduce_splitk; the split /
 * combine scheme of the AstrAI v1.3.9 page's attn_decode_split_kv_mma.cuh).
 * The keys are the full kv rows; the values are their first head_dim_v
 * channels. Each split of the key range writes an un-normalised partial
 * (acc, row max, row sum) into the workspace; a combine kernel merges them.
 *   q   [total_q, heads_q,  head_dim_qk] bf16    kv [total_k, heads_kv, head_dim_qk] bf16
 *   o   [total_q, heads_q,  head_dim_v]  bf16    lse [heads_q, total_q] float32 (may be NULL)
 *   cu_seqlens_q, cu_seqlens_k as for mxfa_fwd_varlen.
 * Supported: head_dim_qk = 576, head_dim_v = 512, bf16.
 * num_splits: 0 picks a split count from the device's compute-unit count;
 * otherwise 1..64 (the result does not depend on it beyond fp32 rounding).
 * workspace: device memory of at least mxfa_decode_splitkv_workspace_bytes()
 * bytes with the same batch/max_seqlen_q/heads/num_splits arguments; owned by
 * the caller, overwritten, not needed after the stream passes the call.
 * Other arguments as for mxfa_fwd.
 */
mxfa_status mxfa_decode_splitkv(const void* q, const void* kv, void* o, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                                int total_k, int heads_q, int heads_kv, int head_dim_qk,
                                int head_dim_v, int causal, int window_left, int window_right,
                                float softcap, float scale, int num_splits, void* workspace,
                                size_t workspace_bytes, mxfa_stream_t stream);

/*
 * Split-KV decode over a latent cache stored as fp8 (the kernelbot
 * amd-mixed-mla submission 588924 page names an fp8 KV; the encoding is the
 * OCP 8-bit floating point E4M3 format) with one per-tensor scale: key row j
 * is kv_scale * e4m3(kv8[j]) and its value the first head_dim_v channels.
 * Same computation as mxfa_decode_splitkv on those rows; the kernel converts
 * the codes to bf16 exactly and folds kv_scale into the score scale and the
 * output.
 *   kv8 [total_k, heads_kv, head_dim_qk] uint8 E4M3 codes (16-byte aligned)
 * kv_scale: finite (scale * kv_scale too). NaN codes give NaN rows.
 * Other arguments, the workspace and its size query as for
 * mxfa_decode_splitkv.
 */
mxfa_status mxfa_decode_splitkv_fp8(const void* q, const void* kv8, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                                    int total_k, int heads_q, int heads_kv, int head_dim_qk,
                                    int head_dim_v, int causal, int window_left, int window_right,
                                    float softcap, float scale, float kv_scale, int num_splits,
                                    void* workspace, size_t workspace_bytes, mxfa_stream_t stream);

/*
 * Split-KV decode over a paged latent cache (the mxflashattn page's
 * flash_attn_with_kvcache interface: k/v cache of fixed-size pages, per-batch
 * cache_seqlens, block_table of page indices; the AstrAI v1.3.9 page's paged
 * decode reads one page-table entry per key tile). Same computation and
 * result as mxfa_decode_splitkv on the gathered keys.
 *   kv_cache [num_pages, page_size, heads_kv, head_dim_qk] bf16
 *   cache_seqlens int32 [batch]: keys of sequence b (bottom-right causal
 *     alignment against its queries, as in mxfa_decode_splitkv)
 *   block_table int32 [batch, max_pages], row-major, never NULL: key j of
 *     sequence b is row j % page_size of page block_table[b * max_pages +
 *     j / page_size]
 * page_size: a positive multiple of 32 (one key tile never straddles a page).
 * max_seqlen_k must bound cache_seqlens and be <= max_pages * page_size; it
 * sizes the split plan (a longer sequence is cut to max_pages * page_size
 * keys). Table entries of pages that hold keys must lie in [0, num_pages);
 * a tile whose entry lies outside is read as zeros (no memory outside the
 * cache is touched) and the affected rows' results are then unspecified.
 * Entries past a sequence's last page are never read.
 * Other arguments, the workspace and its size query as for
 * mxfa_decode_splitkv.
 */
mxfa_status mxfa_decode_splitkv_paged(const void* q, const void* kv_cache, void* o, float* lse,
                                      const int32_t* cu_seqlens_q, const int32_t* cache_seqlens,
                                      const int32_t* block_table, int batch, int max_seqlen_q,
                                      int max_seqlen_k, int total_q, int num_pages, int page_size,
                                      int max_pages, int heads_q, int heads_kv, int head_dim_qk,
                                      int head_dim_v, int causal, int window_left, int window_right,
                                      float softcap, float scale, int num_splits, void* workspace,
                                      size_t workspace_bytes, mxfa_stream_t stream);

/*
 * Split-KV decode for standard heads with separate K and V (grouped-query
 * attention at decode time: few query tokens per sequence). The split /
 * combine scheme of mxfa_decode_splitkv; the query heads that share a kv head
 * are packed into the rows of one MFMA tile (the AstrAI v1.3.9 page's
 * split-KV MMA decode, head packing), so each kv head's keys are read once
 * per key split for all of its query heads and tokens (up to 32 (token, head)
 * pairs per pass).
 *   q   [total_q, heads_q,  head_dim] bf16   k, v [total_k, heads_kv, head_dim] bf16
 *   o   [total_q, heads_q,  head_dim] bf16   lse  [heads_q, total_q] float32 (may be NULL)
 *   cu_seqlens_q, cu_seqlens_k as for mxfa_fwd_varlen (bottom-right causal
 *   alignment when a sequence has fewer queries than keys).
 * Supported: head_dim 64 or 128, bf16. Any query length is computed
 * correctly; the kernel is meant for short ones (it re-reads the keys once
 * per 32 (token, head) rows).
 * num_splits: 0 picks a split count from the device's compute-unit count;
 * otherwise 1..64. workspace: at least
 * mxfa_decode_splitkv_gqa_workspace_bytes() bytes (0 when the plan has one
 * split: then workspace may be NULL); owned by the caller, overwritten.
 * Other arguments as for mxfa_fwd.
 */
mxfa_status mxfa_decode_splitkv_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                                    int total_k, int heads_q, int heads_kv, int head_dim, int causal,
                                    int window_left, int window_right, float softcap, float scale,
                                    int num_splits, void* workspace, size_t workspace_bytes,
                                    mxfa_stream_t stream);

/* Workspace bytes mxfa_decode_splitkv_gqa needs (0 on error or for one split). */
size_t mxfa_decode_splitkv_gqa_workspace_bytes(int batch, int max_seqlen_q, int max_seqlen_k,
                                               int heads_q, int heads_kv, int head_dim,
                                               int num_splits);

/* Split count mxfa_decode_splitkv_gqa uses for these arguments (0 on error). */
int mxfa_decode_splitkv_gqa_num_splits(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q,
                                       int heads_kv, int num_splits);

/*
 * Workspace bytes mxfa_decode_splitkv needs for these arguments (0 when
 * nothing is needed). With num_splits = 0 it queries the current device's
 * compute-unit count (a host-side HIP query, no device work); if that fails
 * it returns 0 and sets mxfa_last_error().
 */
size_t mxfa_decode_splitkv_workspace_bytes(int batch, int max_seqlen_q, int max_seqlen_k,
                                           int heads_q, int heads_kv, int head_dim_v,
                                           int num_splits);

/* Split count mxfa_decode_splitkv uses for these arguments (0 on error). */
int mxfa_decode_splitkv_num_splits(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q,
                                   int heads_kv, int num_splits);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* mxfa_last_error(void);

/* Library version string, e.g. "mxfa 0.1.0 gfx950". */
const char* mxfa_version(void);

/*
 * Measurement aid, not part of attention: the shader clock the chip runs at.
 * One wave counts shader-clock cycles (s_memtime) against the fixed 100 MHz
 * real-time counter (s_memrealtime) for interval_us microseconds (1..1000)
 * and writes two uint64 values to out_device (device memory, 8-byte
 * aligned, caller-owned): [0] the cycles, [1] the real-time ticks (10 ns
 * each); cycles / ticks * 100 is the clock in MHz over the interval.
 * Enqueued on `stream` like the other calls: between a workload's calls it
 * reads the clock the chip holds under that load. Returns
 * MXFA_ERR_INVALID_ARG for a null or misaligned pointer or an interval out
 * of range, MXFA_ERR_HIP if the launch fails.
 */
mxfa_status mxfa_clock_probe(void* out_device, int interval_us, mxfa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFA_H */
