// mxfa_api.hip -- the C ABI of libmxfa.so: argument checks, launch planning
// and kernel launches on the caller's stream. Declared in include/mxfa.h.
//
// Every check runs on the host before anything is enqueued; no call
// synchronises the device (the mxflashattn 1.4.0 page's api.py keeps its
// device-syncing checks behind an opt-in switch for the same reason).
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "mxfa.h"
#include "mxfa_internal.h"

namespace {

thread_local char g_err[512] = "";

mxfa_status fail(mxfa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

mxfa_status hip_fail(hipError_t e, const char* what) {
    return fail(MXFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr float kLog2e = 1.4426950408889634f;

// Shared scalar checks of every entry point.
mxfa_status check_common(int heads_q, int heads_kv, int window_left, int window_right, float softcap,
                         float scale) {
    if (heads_q < 1 || heads_kv < 1) return fail(MXFA_ERR_INVALID_ARG, "heads_q and heads_kv must be >= 1");
    if (heads_q % heads_kv) return fail(MXFA_ERR_INVALID_ARG, "heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
    if (heads_q > MXFA_MAX_HEADS || heads_kv > MXFA_MAX_HEADS)
        return fail(MXFA_ERR_UNSUPPORTED, "heads_q (%d) and heads_kv (%d) must be at most %d", heads_q, heads_kv,
                    MXFA_MAX_HEADS);
    if (window_left < -1 || window_right < -1) return fail(MXFA_ERR_INVALID_ARG, "window bounds must be >= -1");
    if (!isfinite(softcap) || softcap < 0.0f) return fail(MXFA_ERR_INVALID_ARG, "softcap must be finite and >= 0");
    if (!isfinite(scale)) return fail(MXFA_ERR_INVALID_ARG, "scale must be finite");
    return MXFA_OK;
}

mxfa_status check_tensor(const void* p, const char* name, uintptr_t align) {
    if (!p) return fail(MXFA_ERR_INVALID_ARG, "%s is null", name);
    if (!aligned(p, align)) return fail(MXFA_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, (int)align);
    return MXFA_OK;
}

void fill_scaling(float scale, float softcap, float* x_mul, float* cap_mul, float* cap_out) {
    *x_mul = scale * kLog2e;
    if (softcap > 0.0f) {
        *cap_mul = 2.0f * kLog2e * scale / softcap;
        *cap_out = softcap * kLog2e;
    } else {
        *cap_mul = 0.0f;
        *cap_out = 0.0f;
    }
}

int device_cus(int* out);

// Work-list length bound of a packed forward with bm-row q tiles: no more
// than batch * ceil(max_seqlen_q / bm), nor ceil(total_q / bm) + batch.
long long varlen_list_max(int batch, int max_seqlen_q, int total_q, int bm) {
    const long long a = (long long)batch * ((max_seqlen_q + bm - 1) / bm);
    const long long b = ((long long)total_q + bm - 1) / bm + batch;
    return a < b ? a : b;
}

// Workspace bytes the size query promises: the list for the smallest q tile
// of any dtype, without total_q (every segment at max_seqlen_q).
size_t varlen_ws_bytes(int batch, int max_seqlen_q) {
    if (batch <= 0 || max_seqlen_q <= 0) return 0;
    const int bm = mxfa::kFwdF32Rows < mxfa::kFwdBf16Rows ? mxfa::kFwdF32Rows : mxfa::kFwdBf16Rows;
    return mxfa::worklist_bytes(batch, (long long)batch * ((max_seqlen_q + bm - 1) / bm));
}

mxfa_status launch_fwd(const mxfa::FwdParams& args, int head_dim, mxfa_dtype dtype, hipStream_t stream) {
    mxfa::FwdParams p = args;
    int cus = 0;
    if (device_cus(&cus) == 0 && cus % mxfa::kXcdCount == 0) p.xcd_cus = cus / mxfa::kXcdCount;
    hipError_t e = (dtype == MXFA_BF16) ? mxfa::launch_fwd_bf16(p, head_dim, stream)
                                        : mxfa::launch_fwd_f32(p, head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
    return MXFA_OK;
}

// Compute units of the current device, cached per device.
int device_cus(int* out) {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return (int)e;
        cache[dev] = cus > 0 ? cus : 1;
    }
    *out = cache[dev];
    return 0;
}

constexpr int kMaxSplits = 64;

// Split plan: aim for about one work group per compute unit (the split kernel
// keeps four 36 KB latent tiles in LDS, one group per CU).
int plan_splits(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q, int heads_kv, int requested,
                int* err) {
    *err = 0;
    const int group = heads_q / heads_kv;
    const long long m_groups = ((long long)max_seqlen_q * group + mxfa::kDecodeRows - 1) / mxfa::kDecodeRows;
    const long long units = (long long)batch * heads_kv * m_groups;
    const int tiles = (max_seqlen_k + mxfa::kDecodeTile - 1) / mxfa::kDecodeTile;
    if (requested > 0) return requested;
    int cus = 0;
    int e = device_cus(&cus);
    if (e) {
        *err = e;
        return 0;
    }
    if (units <= 0) return 1;
    long long s = (cus + units - 1) / units;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    return (int)s;
}

size_t decode_ws_bytes(int batch, int max_seqlen_q, int heads_q, int heads_kv, int head_dim_v, int splits) {
    const int group = heads_q / heads_kv;
    const long long m_groups = ((long long)max_seqlen_q * group + mxfa::kDecodeRows - 1) / mxfa::kDecodeRows;
    const long long parts = (long long)batch * heads_kv * m_groups * splits;
    return (size_t)parts * (size_t)mxfa::kDecodeRows * ((size_t)head_dim_v + 3) * sizeof(float);
}

// Split plan for the standard-head decode: about one work group per compute
// unit (two fit one CU at head dim 128, so the groups of a second round start
// while the first finish; fewer splits also keep the combine short), and at
// least two 64-key tiles per split.
int plan_gqa_splits(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q, int heads_kv, int requested,
                    int* err) {
    *err = 0;
    if (requested > 0) return requested;
    const int group = heads_q / heads_kv;
    const long long m_groups = ((long long)max_seqlen_q * group + mxfa::kGqaRows - 1) / mxfa::kGqaRows;
    const long long units = (long long)batch * heads_kv * m_groups;
    const long long tiles = ((long long)max_seqlen_k + mxfa::kGqaTile - 1) / mxfa::kGqaTile;
    int cus = 0;
    int e = device_cus(&cus);
    if (e) {
        *err = e;
        return 0;
    }
    if (units <= 0) return 1;
    long long s = ((long long)cus + units - 1) / units;
    if (s > tiles / 2) s = tiles / 2;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < 1) s = 1;
    return (int)s;
}

size_t gqa_ws_bytes(int batch, int max_seqlen_q, int heads_q, int heads_kv, int head_dim, int splits) {
    if (splits <= 1) return 0;
    const int group = heads_q / heads_kv;
    const long long m_groups = ((long long)max_seqlen_q * group + mxfa::kGqaRows - 1) / mxfa::kGqaRows;
    const long long parts = (long long)batch * heads_kv * m_groups * splits;
    return (size_t)parts * (size_t)mxfa::kGqaRows * ((size_t)head_dim + 3) * sizeof(float);
}

// Checks and launch shared by the contiguous (cu_k) and paged (pg) decode
// entry points; exactly one of cu_k and pg is non-null. total_k: key rows in kv.
// kv_fp8: kv holds OCP e4m3 values standing for kv_scale times themselves.
mxfa_status decode_common(const void* q, const void* kv, void* o, float* lse, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, const mxfa::PagedKV* pg, int batch, int max_seqlen_q,
                          int max_seqlen_k, int total_q, int total_k, int heads_q, int heads_kv, int head_dim_qk,
                          int head_dim_v, int causal, int window_left, int window_right, float softcap, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, mxfa_stream_t stream,
                          int kv_fp8 = 0, float kv_scale = 1.0f) {
    if (head_dim_qk != 576 || head_dim_v != 512)
        return fail(MXFA_ERR_UNSUPPORTED, "decode head dims (%d, %d): supported (576, 512)", head_dim_qk, head_dim_v);
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
        return fail(MXFA_ERR_INVALID_ARG, "batch, max lengths and totals must be >= 0");
    if (max_seqlen_q > total_q) return fail(MXFA_ERR_INVALID_ARG, "max_seqlen exceeds the total token count");
    if (num_splits < 0 || num_splits > kMaxSplits)
        return fail(MXFA_ERR_INVALID_ARG, "num_splits must be in [0, %d]", kMaxSplits);
    mxfa_status st = check_common(heads_q, heads_kv, window_left, window_right, softcap, scale);
    if (st != MXFA_OK) return st;
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return MXFA_OK;
    if ((st = check_tensor(cu_seqlens_q, "cu_seqlens_q", 4)) != MXFA_OK) return st;
    if (pg) {
        if ((st = check_tensor(pg->seqlens, "cache_seqlens", 4)) != MXFA_OK) return st;
        if ((st = check_tensor(pg->block_table, "block_table", 4)) != MXFA_OK) return st;
    } else if ((st = check_tensor(cu_seqlens_k, "cu_seqlens_k", 4)) != MXFA_OK) {
        return st;
    }
    if ((st = check_tensor(q, "q", 16)) != MXFA_OK) return st;
    if ((st = check_tensor(o, "o", 16)) != MXFA_OK) return st;
    if (total_k > 0 && (st = check_tensor(kv, "kv", 16)) != MXFA_OK) return st;
    if (kv_fp8 && (heads_kv * (long long)head_dim_qk) % 16)
        return fail(MXFA_ERR_INVALID_ARG, "fp8 kv rows must be a multiple of 16 bytes");
    if (lse && !aligned(lse, 4)) return fail(MXFA_ERR_INVALID_ARG, "lse is not 4-byte aligned");

    int err = 0;
    const int splits = plan_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits, &err);
    if (err) return hip_fail((hipError_t)err, "device query for the split count");
    const size_t need = decode_ws_bytes(batch, max_seqlen_q, heads_q, heads_kv, head_dim_v, splits);
    if (!workspace || workspace_bytes < need)
        return fail(MXFA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 16)) return fail(MXFA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");

    mxfa::DecodeParams p = {};
    p.q = q;
    p.kv = kv;
    p.o = o;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.batch = batch;
    p.max_seqlen_q = max_seqlen_q;
    p.max_seqlen_k = max_seqlen_k;
    p.total_q = total_q;
    p.heads_q = heads_q;
    p.heads_kv = heads_kv;
    p.group = heads_q / heads_kv;
    p.m_groups = (int)(((long long)max_seqlen_q * p.group + mxfa::kDecodeRows - 1) / mxfa::kDecodeRows);
    p.splits = splits;
    const long long parts = (long long)batch * heads_kv * p.m_groups * splits;
    p.part_acc = static_cast<float*>(workspace);
    p.part_ml = p.part_acc + parts * mxfa::kDecodeRows * head_dim_v;
    p.causal = causal ? 1 : 0;
    p.window_left = window_left;
    p.window_right = window_right;
    p.softcap = softcap;
    // The scores of an fp8 cache carry its scale: fold it into the score scale.
    fill_scaling(scale * kv_scale, softcap, &p.x_mul, &p.cap_mul, &p.cap_out);
    p.kv_fp8 = kv_fp8;
    p.v_scale = kv_scale;
    if (pg) {
        p.block_table = pg->block_table;
        p.seqlens_k = pg->seqlens;
        p.page_size = pg->page_size;
        p.max_pages = pg->max_pages;
        p.num_pages = pg->num_pages;
    }
    hipError_t e = mxfa::launch_decode_mla(p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    return MXFA_OK;
}

// Static scratch of the allocation-free entry point: one copy per GPU, in
// device memory from the library's load until the process ends. Host code
// uses only the address hipGetSymbolAddress gives for the current device.
__device__ __attribute__((aligned(256))) char scratch[MXFA_NOALLOC_SCRATCH_BYTES];

// Device address of this GPU's copy of scratch, looked up once per device
// with that device current. Null (and *err set) if the lookup fails.
void* scratch_device_ptr(hipError_t* err) {
    static std::mutex mu;
    static void* ptrs[64] = {nullptr};
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !ptr) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        ptrs[dev] = ptr;
    }
    return ptrs[dev];
}

// Checks and launches of the packed forward. static_scratch: the work list
// goes into this library's static device array (the allocation-free entry
// point) instead of the caller's workspace.
mxfa_status varlen_common(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int max_seqlen_q,
                          int max_seqlen_k, int total_q, int total_k, int heads_q, int heads_kv, int head_dim,
                          mxfa_dtype dtype, int causal, int window_left, int window_right, float softcap,
                          float scale, void* workspace, size_t workspace_bytes, bool static_scratch,
                          mxfa_stream_t stream) {
    if (dtype != MXFA_F32 && dtype != MXFA_BF16) return fail(MXFA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (head_dim != 64 && head_dim != 128) return fail(MXFA_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", head_dim);
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
        return fail(MXFA_ERR_INVALID_ARG, "batch, max lengths and totals must be >= 0");
    if (max_seqlen_q > total_q || max_seqlen_k > total_k)
        return fail(MXFA_ERR_INVALID_ARG, "max_seqlen exceeds the total token count");
    mxfa_status st = check_common(heads_q, heads_kv, window_left, window_right, softcap, scale);
    if (st != MXFA_OK) return st;
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return MXFA_OK;
    if ((st = check_tensor(cu_seqlens_q, "cu_seqlens_q", 4)) != MXFA_OK) return st;
    if ((st = check_tensor(cu_seqlens_k, "cu_seqlens_k", 4)) != MXFA_OK) return st;
    if ((st = check_tensor(q, "q", 16)) != MXFA_OK) return st;
    if ((st = check_tensor(o, "o", 16)) != MXFA_OK) return st;
    if (total_k > 0) {
        if ((st = check_tensor(k, "k", 16)) != MXFA_OK) return st;
        if ((st = check_tensor(v, "v", 16)) != MXFA_OK) return st;
    }
    if (lse && !aligned(lse, 4)) return fail(MXFA_ERR_INVALID_ARG, "lse is not 4-byte aligned");

    // The work list of the live q tiles goes into the workspace.
    const int bm = dtype == MXFA_BF16 ? mxfa::kFwdBf16Rows : mxfa::kFwdF32Rows;
    const int bn = dtype == MXFA_BF16 ? mxfa::kFwdBf16Keys : mxfa::kFwdF32Keys;
    const long long list_max = varlen_list_max(batch, max_seqlen_q, total_q, bm);
    const size_t need = mxfa::worklist_bytes(batch, list_max);
    if (static_scratch) {
        if (need > (size_t)MXFA_NOALLOC_SCRATCH_BYTES)
            return fail(MXFA_ERR_WORKSPACE,
                        "the work list needs %zu bytes; the allocation-free call holds at most %u "
                        "(use mxfa_fwd_varlen with a workspace)",
                        need, (unsigned)MXFA_NOALLOC_SCRATCH_BYTES);
        hipError_t e = hipSuccess;
        workspace = scratch_device_ptr(&e);
        if (!workspace) return hip_fail(e, "address of the static scratch array");
        workspace_bytes = MXFA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need)
        return fail(MXFA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 16)) return fail(MXFA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");

    mxfa::FwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.worklist = static_cast<const int*>(workspace);
    p.list_max = list_max;
    p.batch = batch;
    p.seqlen_q = max_seqlen_q;
    p.seqlen_k = max_seqlen_k;
    p.total_q = total_q;
    p.heads_q = heads_q;
    p.heads_kv = heads_kv;
    p.group = heads_q / heads_kv;
    p.causal = causal ? 1 : 0;
    p.window_left = window_left;
    p.window_right = window_right;
    p.softcap = softcap;
    p.scale = scale;
    fill_scaling(scale, softcap, &p.x_mul, &p.cap_mul, &p.cap_out);
    mxfa::WorkListParams wp = {};
    wp.cu_q = cu_seqlens_q;
    wp.cu_k = cu_seqlens_k;
    wp.ws = static_cast<int*>(workspace);
    wp.list_max = list_max;
    wp.batch = batch;
    wp.max_seqlen_k = max_seqlen_k;
    wp.bm = bm;
    wp.bn = bn;
    wp.causal = p.causal;
    wp.window_left = window_left;
    wp.window_right = window_right;
    hipError_t e = mxfa::launch_varlen_worklist(wp, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "work-list kernel launch");
    return launch_fwd(p, head_dim, dtype, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

const char* mxfa_last_error(void) { return g_err; }

const char* mxfa_version(void) { return "mxfa 0.1.0 gfx950"; }

mxfa_status mxfa_clock_probe(void* out_device, int interval_us, mxfa_stream_t stream) {
    g_err[0] = 0;
    if (interval_us < 1 || interval_us > 1000) return fail(MXFA_ERR_INVALID_ARG, "interval_us must be in [1, 1000]");
    mxfa_status st = check_tensor(out_device, "out_device", 8);
    if (st != MXFA_OK) return st;
    hipError_t e = mxfa::launch_clock_probe(static_cast<unsigned long long*>(out_device), (unsigned)interval_us * 100u,
                                            reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "clock probe launch");
    return MXFA_OK;
}

mxfa_status mxfa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int seqlen_q,
                     int seqlen_k, int heads_q, int heads_kv, int head_dim, mxfa_dtype dtype, int causal,
                     int window_left, int window_right, float softcap, float scale, mxfa_stream_t stream) {
    g_err[0] = 0;
    if (dtype != MXFA_F32 && dtype != MXFA_BF16) return fail(MXFA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (head_dim != 64 && head_dim != 128) return fail(MXFA_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", head_dim);
    if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return fail(MXFA_ERR_INVALID_ARG, "batch and sequence lengths must be >= 0");
    mxfa_status st = check_common(heads_q, heads_kv, window_left, window_right, softcap, scale);
    if (st != MXFA_OK) return st;
    if ((long long)batch * seqlen_q > 0x7fffffffLL || (long long)batch * seqlen_k > 0x7fffffffLL)
        return fail(MXFA_ERR_INVALID_ARG, "batch * seqlen exceeds 2^31 - 1 tokens");
    if ((long long)batch * seqlen_q == 0) return MXFA_OK;
    if ((st = check_tensor(q, "q", 16)) != MXFA_OK) return st;
    if ((st = check_tensor(o, "o", 16)) != MXFA_OK) return st;
    if (seqlen_k > 0) {
        if ((st = check_tensor(k, "k", 16)) != MXFA_OK) return st;
        if ((st = check_tensor(v, "v", 16)) != MXFA_OK) return st;
    }
    if (lse && !aligned(lse, 4)) return fail(MXFA_ERR_INVALID_ARG, "lse is not 4-byte aligned");

    mxfa::FwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.cu_q = nullptr;
    p.cu_k = nullptr;
    p.batch = batch;
    p.seqlen_q = seqlen_q;
    p.seqlen_k = seqlen_k;
    p.total_q = batch * seqlen_q;
    p.heads_q = heads_q;
    p.heads_kv = heads_kv;
    p.group = heads_q / heads_kv;
    p.causal = causal ? 1 : 0;
    p.window_left = window_left;
    p.window_right = window_right;
    p.softcap = softcap;
    p.scale = scale;
    fill_scaling(scale, softcap, &p.x_mul, &p.cap_mul, &p.cap_out);
    return launch_fwd(p, head_dim, dtype, reinterpret_cast<hipStream_t>(stream));
}

mxfa_status mxfa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch, int max_seqlen_q,
                            int max_seqlen_k, int total_q, int total_k, int heads_q, int heads_kv, int head_dim,
                            mxfa_dtype dtype, int causal, int window_left, int window_right, float softcap,
                            float scale, void* workspace, size_t workspace_bytes, mxfa_stream_t stream) {
    g_err[0] = 0;
    return varlen_common(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, total_q,
                         total_k, heads_q, heads_kv, head_dim, dtype, causal, window_left, window_right, softcap,
                         scale, workspace, workspace_bytes, false, stream);
}

mxfa_status mxfa_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int heads_q,
                                    int heads_kv, int head_dim, mxfa_dtype dtype, int causal, int window_left,
                                    int window_right, float softcap, float scale, mxfa_stream_t stream) {
    g_err[0] = 0;
    return varlen_common(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, total_q,
                         total_k, heads_q, heads_kv, head_dim, dtype, causal, window_left, window_right, softcap,
                         scale, nullptr, 0, true, stream);
}

size_t mxfa_fwd_varlen_workspace_bytes(int batch, int max_seqlen_q, int heads_q, int head_dim) {
    (void)heads_q;  // the list holds (segment, q tile) pairs; every query head reads the same list
    (void)head_dim;
    return varlen_ws_bytes(batch, max_seqlen_q);
}

int mxfa_decode_splitkv_num_splits(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q, int heads_kv,
                                   int num_splits) {
    g_err[0] = 0;
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv ||
        num_splits < 0 || num_splits > kMaxSplits) {
        fail(MXFA_ERR_INVALID_ARG, "invalid decode plan arguments");
        return 0;
    }
    int err = 0;
    const int s = plan_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits, &err);
    if (err) {
        hip_fail((hipError_t)err, "device query for the split count");
        return 0;
    }
    return s;
}

size_t mxfa_decode_splitkv_workspace_bytes(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q,
                                           int heads_kv, int head_dim_v, int num_splits) {
    const int s = mxfa_decode_splitkv_num_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits);
    if (s <= 0 || head_dim_v <= 0) return 0;
    return decode_ws_bytes(batch, max_seqlen_q, heads_q, heads_kv, head_dim_v, s);
}

mxfa_status mxfa_decode_splitkv(const void* q, const void* kv, void* o, float* lse, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k,
                                int total_q, int total_k, int heads_q, int heads_kv, int head_dim_qk,
                                int head_dim_v, int causal, int window_left, int window_right, float softcap,
                                float scale, int num_splits, void* workspace, size_t workspace_bytes,
                                mxfa_stream_t stream) {
    g_err[0] = 0;
    if (total_k < 0) return fail(MXFA_ERR_INVALID_ARG, "batch, max lengths and totals must be >= 0");
    if (max_seqlen_k > total_k) return fail(MXFA_ERR_INVALID_ARG, "max_seqlen exceeds the total token count");
    return decode_common(q, kv, o, lse, cu_seqlens_q, cu_seqlens_k, nullptr, batch, max_seqlen_q, max_seqlen_k,
                         total_q, total_k, heads_q, heads_kv, head_dim_qk, head_dim_v, causal, window_left,
                         window_right, softcap, scale, num_splits, workspace, workspace_bytes, stream);
}

mxfa_status mxfa_decode_splitkv_fp8(const void* q, const void* kv8, void* o, float* lse, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k,
                                    int total_q, int total_k, int heads_q, int heads_kv, int head_dim_qk,
                                    int head_dim_v, int causal, int window_left, int window_right, float softcap,
                                    float scale, float kv_scale, int num_splits, void* workspace,
                                    size_t workspace_bytes, mxfa_stream_t stream) {
    g_err[0] = 0;
    if (total_k < 0) return fail(MXFA_ERR_INVALID_ARG, "batch, max lengths and totals must be >= 0");
    if (max_seqlen_k > total_k) return fail(MXFA_ERR_INVALID_ARG, "max_seqlen exceeds the total token count");
    if (!isfinite(kv_scale) || !isfinite(scale * kv_scale))
        return fail(MXFA_ERR_INVALID_ARG, "kv_scale (and scale * kv_scale) must be finite");
    return decode_common(q, kv8, o, lse, cu_seqlens_q, cu_seqlens_k, nullptr, batch, max_seqlen_q, max_seqlen_k,
                         total_q, total_k, heads_q, heads_kv, head_dim_qk, head_dim_v, causal, window_left,
                         window_right, softcap, scale, num_splits, workspace, workspace_bytes, stream, 1, kv_scale);
}

mxfa_status mxfa_decode_splitkv_paged(const void* q, const void* kv_cache, void* o, float* lse,
                                      const int32_t* cu_seqlens_q, const int32_t* cache_seqlens,
                                      const int32_t* block_table, int batch, int max_seqlen_q, int max_seqlen_k,
                                      int total_q, int num_pages, int page_size, int max_pages, int heads_q,
                                      int heads_kv, int head_dim_qk, int head_dim_v, int causal, int window_left,
                                      int window_right, float softcap, float scale, int num_splits,
                                      void* workspace, size_t workspace_bytes, mxfa_stream_t stream) {
    g_err[0] = 0;
    if (num_pages < 0 || max_pages < 0)
        return fail(MXFA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 0");
    if (page_size <= 0 || page_size % mxfa::kDecodeTile)
        return fail(MXFA_ERR_INVALID_ARG, "page_size %d: must be a positive multiple of %d", page_size,
                    mxfa::kDecodeTile);
    if ((long long)max_seqlen_k > (long long)max_pages * page_size)
        return fail(MXFA_ERR_INVALID_ARG, "max_seqlen_k %d exceeds the block table's %lld keys", max_seqlen_k,
                    (long long)max_pages * page_size);
    if ((long long)num_pages * page_size > 0x7fffffffLL)
        return fail(MXFA_ERR_INVALID_ARG, "the cache holds more than 2^31 - 1 rows");
    mxfa::PagedKV pg = {block_table, cache_seqlens, page_size, max_pages, num_pages};
    return decode_common(q, kv_cache, o, lse, cu_seqlens_q, nullptr, &pg, batch, max_seqlen_q, max_seqlen_k,
                         total_q, num_pages * page_size, heads_q, heads_kv, head_dim_qk, head_dim_v, causal,
                         window_left, window_right, softcap, scale, num_splits, workspace, workspace_bytes, stream);
}

int mxfa_decode_splitkv_gqa_num_splits(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q, int heads_kv,
                                       int num_splits) {
    g_err[0] = 0;
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv ||
        num_splits < 0 || num_splits > kMaxSplits) {
        fail(MXFA_ERR_INVALID_ARG, "invalid decode plan arguments");
        return 0;
    }
    int err = 0;
    const int s = plan_gqa_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits, &err);
    if (err) {
        hip_fail((hipError_t)err, "device query for the split count");
        return 0;
    }
    return s;
}

size_t mxfa_decode_splitkv_gqa_workspace_bytes(int batch, int max_seqlen_q, int max_seqlen_k, int heads_q,
                                               int heads_kv, int head_dim, int num_splits) {
    const int s =
        mxfa_decode_splitkv_gqa_num_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits);
    if (s <= 0 || head_dim <= 0) return 0;
    return gqa_ws_bytes(batch, max_seqlen_q, heads_q, heads_kv, head_dim, s);
}

mxfa_status mxfa_decode_splitkv_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int heads_q,
                                    int heads_kv, int head_dim, int causal, int window_left, int window_right,
                                    float softcap, float scale, int num_splits, void* workspace,
                                    size_t workspace_bytes, mxfa_stream_t stream) {
    g_err[0] = 0;
    if (head_dim != 64 && head_dim != 128)
        return fail(MXFA_ERR_UNSUPPORTED, "decode head dim %d: supported 64, 128", head_dim);
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
        return fail(MXFA_ERR_INVALID_ARG, "batch, max lengths and totals must be >= 0");
    if (heads_kv > 0 && (long long)max_seqlen_q * (heads_q / heads_kv) > 0x7fffffffLL)
        return fail(MXFA_ERR_INVALID_ARG, "max_seqlen_q * heads_q / heads_kv exceeds 2^31 - 1");
    if (max_seqlen_q > total_q || max_seqlen_k > total_k)
        return fail(MXFA_ERR_INVALID_ARG, "max_seqlen exceeds the total token count");
    if (num_splits < 0 || num_splits > kMaxSplits)
        return fail(MXFA_ERR_INVALID_ARG, "num_splits must be in [0, %d]", kMaxSplits);
    mxfa_status st = check_common(heads_q, heads_kv, window_left, window_right, softcap, scale);
    if (st != MXFA_OK) return st;
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return MXFA_OK;
    if ((st = check_tensor(cu_seqlens_q, "cu_seqlens_q", 4)) != MXFA_OK) return st;
    if ((st = check_tensor(cu_seqlens_k, "cu_seqlens_k", 4)) != MXFA_OK) return st;
    if ((st = check_tensor(q, "q", 16)) != MXFA_OK) return st;
    if ((st = check_tensor(o, "o", 16)) != MXFA_OK) return st;
    if (total_k > 0) {
        if ((st = check_tensor(k, "k", 16)) != MXFA_OK) return st;
        if ((st = check_tensor(v, "v", 16)) != MXFA_OK) return st;
    }
    if (lse && !aligned(lse, 4)) return fail(MXFA_ERR_INVALID_ARG, "lse is not 4-byte aligned");

    int err = 0;
    const int splits = plan_gqa_splits(batch, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, num_splits, &err);
    if (err) return hip_fail((hipError_t)err, "device query for the split count");
    const size_t need = gqa_ws_bytes(batch, max_seqlen_q, heads_q, heads_kv, head_dim, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(MXFA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : 0);
        if (!aligned(workspace, 16)) return fail(MXFA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }

    mxfa::GqaDecodeParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.batch = batch;
    p.total_q = total_q;
    p.heads_q = heads_q;
    p.heads_kv = heads_kv;
    p.group = heads_q / heads_kv;
    p.m_groups = (int)(((long long)max_seqlen_q * p.group + mxfa::kGqaRows - 1) / mxfa::kGqaRows);
    p.splits = splits;
    if (need > 0) {
        const long long parts = (long long)batch * heads_kv * p.m_groups * splits;
        p.part_acc = static_cast<float*>(workspace);
        p.part_ml = p.part_acc + parts * mxfa::kGqaRows * head_dim;
    }
    p.causal = causal ? 1 : 0;
    p.window_left = window_left;
    p.window_right = window_right;
    p.softcap = softcap;
    fill_scaling(scale, softcap, &p.x_mul, &p.cap_mul, &p.cap_out);
    hipError_t e = mxfa::launch_decode_gqa(p, head_dim, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    return MXFA_OK;
}

}  // extern "C"
