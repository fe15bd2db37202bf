/*
 * A C11 caller of libmxfa.so that uses only include/mxfa.h and the HIP
 * runtime's C API (no Python, no C++). Test infrastructure: it shows the
 * boundary is a plain C ABI.
 *
 *   caller checks          host-side argument checks and the version string
 *                          (no device work; runs without a GPU)
 *   caller fwd <dir>       dense forward (bf16) on the inputs in <dir>
 *   caller varlen <dir>    packed forward (bf16), work list in a workspace
 *   caller decode <dir>    latent split-KV decode (bf16)
 *   caller fp8 <dir>       latent split-KV decode over an e4m3 cache
 *   caller paged <dir>     latent split-KV decode over a paged cache
 *   caller gqa <dir>       standard-head split-KV decode (bf16)
 *
 * <dir>/args.txt holds the call's integer and float arguments (see below);
 * the tensors are raw little-endian files (q.bin, k.bin, v.bin, kv.bin,
 * cu_q.bin, cu_k.bin, seqlens.bin, table.bin as the call needs). o.bin and
 * lse.bin are written back. Work runs on a stream the program creates; every
 * workspace size comes from the library's own size query. Exit status 0 on
 * success.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mxfa.h"

static void* read_file(const char* dir, const char* name, size_t* n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    fseek(f, 0, SEEK_END);
    long len = ftell(f);
    fseek(f, 0, SEEK_SET);
    void* buf = malloc(len > 0 ? (size_t)len : 1);
    if (buf && len > 0 && fread(buf, 1, (size_t)len, f) != (size_t)len) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    *n = len > 0 ? (size_t)len : 0;
    return buf;
}

static int write_file(const char* dir, const char* name, const void* data, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    int bad = fwrite(data, 1, n, f) != n;
    fclose(f);
    return bad;
}

/* Device copy of a host file (16 bytes at least, so the pointer is never null). */
static void* upload(const char* dir, const char* name, size_t* n) {
    void* h = read_file(dir, name, n);
    void* d = NULL;
    if (!h) return NULL;
    if (hipMalloc(&d, *n ? *n : 16) != hipSuccess) d = NULL;
    else if (*n && hipMemcpy(d, h, *n, hipMemcpyHostToDevice) != hipSuccess) d = NULL;
    free(h);
    return d;
}

static int download(const char* dir, const char* name, const void* d, size_t n) {
    void* h = malloc(n ? n : 1);
    int bad = !h || (n && hipMemcpy(h, d, n, hipMemcpyDeviceToHost) != hipSuccess) || write_file(dir, name, h, n);
    free(h);
    return bad;
}

static int checks(void) {
    void* a = (void*)(uintptr_t)0x100000; /* aligned, never dereferenced: every case fails on the host */
    if (mxfa_fwd(NULL, a, a, a, NULL, 1, 4, 4, 2, 1, 128, MXFA_BF16, 1, -1, -1, 0.0f, 0.1f, NULL) !=
            MXFA_ERR_INVALID_ARG || !mxfa_last_error()[0])
        return 1;
    if (mxfa_fwd(a, a, a, a, NULL, 1, 4, 4, 2, 1, 96, MXFA_BF16, 1, -1, -1, 0.0f, 0.1f, NULL) != MXFA_ERR_UNSUPPORTED)
        return 2;
    if (mxfa_fwd(a, a, a, a, NULL, 1, 4, 4, 3, 2, 128, MXFA_BF16, 1, -1, -1, 0.0f, 0.1f, NULL) != MXFA_ERR_INVALID_ARG)
        return 3;
    if (mxfa_decode_splitkv(a, a, a, NULL, (const int32_t*)a, (const int32_t*)a, 1, 1, 64, 1, 64, 16, 1, 576, 512,
                            0, -1, -1, 0.0f, 0.05f, 1, NULL, 0, NULL) != MXFA_ERR_WORKSPACE)
        return 4;
    if (mxfa_fwd(a, a, a, a, NULL, 0, 4, 4, 2, 1, 128, MXFA_BF16, 1, -1, -1, 0.0f, 0.1f, NULL) != MXFA_OK)
        return 5;
    if (mxfa_fwd_varlen(a, a, a, a, NULL, (const int32_t*)a, (const int32_t*)a, 2, 16, 16, 20, 20, 4, 2, 128,
                        MXFA_BF16, 1, -1, -1, 0.0f, 0.1f, a, mxfa_fwd_varlen_workspace_bytes(2, 16, 4, 128) - 1,
                        NULL) != MXFA_ERR_WORKSPACE)
        return 6;
    printf("%s\n", mxfa_version());
    return 0;
}

static int run(const char* mode, const char* dir) {
    size_t n = 0;
    char* args = read_file(dir, "args.txt", &n);
    if (!args) return 10;
    char* text = realloc(args, n + 1);
    if (!text) return 10;
    text[n] = 0;
    hipStream_t stream;
    if (hipStreamCreate(&stream) != hipSuccess) return 11;
    int rc = 0;
    mxfa_status st = MXFA_OK;
    if (strcmp(mode, "fwd") == 0) {
        /* batch sq sk hq hkv d causal wl wr softcap scale */
        int b, sq, sk, hq, hkv, d, causal, wl, wr;
        float cap, scale;
        if (sscanf(text, "%d %d %d %d %d %d %d %d %d %f %f", &b, &sq, &sk, &hq, &hkv, &d, &causal, &wl, &wr, &cap,
                   &scale) != 11)
            return 12;
        size_t nq, nk, nv;
        void* q = upload(dir, "q.bin", &nq);
        void* k = upload(dir, "k.bin", &nk);
        void* v = upload(dir, "v.bin", &nv);
        void* o = NULL;
        float* lse = NULL;
        const size_t no = nq, nl = (size_t)b * hq * sq * sizeof(float);
        if (!q || !k || !v || hipMalloc(&o, no ? no : 16) != hipSuccess ||
            hipMalloc((void**)&lse, nl ? nl : 16) != hipSuccess)
            return 13;
        st = mxfa_fwd(q, k, v, o, lse, b, sq, sk, hq, hkv, d, MXFA_BF16, causal, wl, wr, cap, scale,
                      (mxfa_stream_t)stream);
        if (st == MXFA_OK && hipStreamSynchronize(stream) == hipSuccess)
            rc = download(dir, "o.bin", o, no) || download(dir, "lse.bin", lse, nl);
        hipFree(q);
        hipFree(k);
        hipFree(v);
        hipFree(o);
        hipFree(lse);
    } else if (strcmp(mode, "varlen") == 0 || strcmp(mode, "gqa") == 0) {
        /* batch mq mk tq tk hq hkv d causal wl wr softcap scale splits */
        int b, mq, mk, tq, tk, hq, hkv, d, causal, wl, wr, splits;
        float cap, scale;
        if (sscanf(text, "%d %d %d %d %d %d %d %d %d %d %d %f %f %d", &b, &mq, &mk, &tq, &tk, &hq, &hkv, &d, &causal,
                   &wl, &wr, &cap, &scale, &splits) != 14)
            return 12;
        const int is_gqa = strcmp(mode, "gqa") == 0;
        size_t nq, nk, nv, ncq, nck;
        void* q = upload(dir, "q.bin", &nq);
        void* k = upload(dir, "k.bin", &nk);
        void* v = upload(dir, "v.bin", &nv);
        int32_t* cq = upload(dir, "cu_q.bin", &ncq);
        int32_t* ck = upload(dir, "cu_k.bin", &nck);
        const size_t ws_bytes = is_gqa ? mxfa_decode_splitkv_gqa_workspace_bytes(b, mq, mk, hq, hkv, d, splits)
                                       : mxfa_fwd_varlen_workspace_bytes(b, mq, hq, d);
        const size_t no = nq, nl = (size_t)hq * tq * sizeof(float);
        void *o = NULL, *ws = NULL;
        float* lse = NULL;
        if (!q || !k || !v || !cq || !ck || hipMalloc(&o, no ? no : 16) != hipSuccess ||
            hipMalloc((void**)&lse, nl ? nl : 16) != hipSuccess || hipMalloc(&ws, ws_bytes ? ws_bytes : 16) != hipSuccess)
            return 13;
        if (is_gqa)
            st = mxfa_decode_splitkv_gqa(q, k, v, o, lse, cq, ck, b, mq, mk, tq, tk, hq, hkv, d, causal, wl, wr, cap,
                                         scale, splits, ws, ws_bytes, (mxfa_stream_t)stream);
        else
            st = mxfa_fwd_varlen(q, k, v, o, lse, cq, ck, b, mq, mk, tq, tk, hq, hkv, d, MXFA_BF16, causal, wl, wr,
                                 cap, scale, ws, ws_bytes, (mxfa_stream_t)stream);
        if (st == MXFA_OK && hipStreamSynchronize(stream) == hipSuccess)
            rc = download(dir, "o.bin", o, no) || download(dir, "lse.bin", lse, nl);
        hipFree(q);
        hipFree(k);
        hipFree(v);
        hipFree(cq);
        hipFree(ck);
        hipFree(o);
        hipFree(lse);
        hipFree(ws);
    } else {
        /* decode, fp8: batch mq mk tq tk hq hkv causal wl wr softcap scale splits kv_scale
         * paged:       batch mq mk tq num_pages page_size max_pages hq hkv causal wl wr softcap scale splits */
        const int paged = strcmp(mode, "paged") == 0, fp8 = strcmp(mode, "fp8") == 0;
        int b, mq, mk, tq, tk = 0, hq, hkv, causal, wl, wr, splits, num_pages = 0, page_size = 0, max_pages = 0;
        float cap, scale, kv_scale = 1.0f;
        if (paged) {
            if (sscanf(text, "%d %d %d %d %d %d %d %d %d %d %d %d %f %f %d", &b, &mq, &mk, &tq, &num_pages, &page_size,
                       &max_pages, &hq, &hkv, &causal, &wl, &wr, &cap, &scale, &splits) != 15)
                return 12;
        } else {
            /* kv_scale is optional for the bf16 decode */
            const int got = sscanf(text, "%d %d %d %d %d %d %d %d %d %d %f %f %d %f", &b, &mq, &mk, &tq, &tk, &hq,
                                   &hkv, &causal, &wl, &wr, &cap, &scale, &splits, &kv_scale);
            if (got != 14 && !(got == 13 && !fp8)) return 12;
        }
        size_t nq, nkv, ncq, nck = 0, nsl = 0, ntb = 0;
        void* q = upload(dir, "q.bin", &nq);
        void* kv = upload(dir, "kv.bin", &nkv);
        int32_t* cq = upload(dir, "cu_q.bin", &ncq);
        int32_t* ck = paged ? NULL : upload(dir, "cu_k.bin", &nck);
        int32_t* seqlens = paged ? upload(dir, "seqlens.bin", &nsl) : NULL;
        int32_t* table = paged ? upload(dir, "table.bin", &ntb) : NULL;
        const size_t ws_bytes = mxfa_decode_splitkv_workspace_bytes(b, mq, mk, hq, hkv, 512, splits);
        const size_t no = (size_t)tq * hq * 512 * 2, nl = (size_t)hq * tq * sizeof(float);
        void *o = NULL, *ws = NULL;
        float* lse = NULL;
        if (!q || !kv || !cq || (paged ? (!seqlens || !table) : !ck) || hipMalloc(&o, no ? no : 16) != hipSuccess ||
            hipMalloc((void**)&lse, nl ? nl : 16) != hipSuccess || hipMalloc(&ws, ws_bytes ? ws_bytes : 16) != hipSuccess)
            return 13;
        if (paged)
            st = mxfa_decode_splitkv_paged(q, kv, o, lse, cq, seqlens, table, b, mq, mk, tq, num_pages, page_size,
                                           max_pages, hq, hkv, 576, 512, causal, wl, wr, cap, scale, splits, ws,
                                           ws_bytes, (mxfa_stream_t)stream);
        else if (fp8)
            st = mxfa_decode_splitkv_fp8(q, kv, o, lse, cq, ck, b, mq, mk, tq, tk, hq, hkv, 576, 512, causal, wl, wr,
                                         cap, scale, kv_scale, splits, ws, ws_bytes, (mxfa_stream_t)stream);
        else
            st = mxfa_decode_splitkv(q, kv, o, lse, cq, ck, b, mq, mk, tq, tk, hq, hkv, 576, 512, causal, wl, wr, cap,
                                     scale, splits, ws, ws_bytes, (mxfa_stream_t)stream);
        if (st == MXFA_OK && hipStreamSynchronize(stream) == hipSuccess)
            rc = download(dir, "o.bin", o, no) || download(dir, "lse.bin", lse, nl);
        hipFree(q);
        hipFree(kv);
        hipFree(cq);
        if (ck) hipFree(ck);
        if (seqlens) hipFree(seqlens);
        if (table) hipFree(table);
        hipFree(o);
        hipFree(lse);
        hipFree(ws);
    }
    hipStreamDestroy(stream);
    free(text);
    if (st != MXFA_OK) {
        fprintf(stderr, "mxfa status %d: %s\n", (int)st, mxfa_last_error());
        return 14;
    }
    return rc ? 15 : 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "checks") == 0) return checks();
    static const char* const modes[] = {"fwd", "varlen", "decode", "fp8", "paged", "gqa"};
    for (size_t i = 0; argc >= 3 && i < sizeof modes / sizeof modes[0]; ++i)
        if (strcmp(argv[1], modes[i]) == 0) return run(argv[1], argv[2]);
    fprintf(stderr, "usage: caller checks | caller {fwd|varlen|decode|fp8|paged|gqa} <dir>\n");
    return 2;
}
