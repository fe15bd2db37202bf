/*
 * attention_oracle.c -- plain fp64 CPU oracle for softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this library. The product path (the HIP
 * library) never links, loads or calls it, and it shares no code with it.
 *
 * What it computes is the plain, materialised definition of scaled
 * dot-product attention, one query row at a time, in double precision:
 *
 *   t_j   = scale * <q_i, k_j>                      for every visible key j
 *   s_j   = softcap > 0 ? softcap * tanh(t_j / softcap) : t_j
 *   P_ij  = exp(s_j - max s) / sum_j exp(s_j - max s)
 *   O_i   = sum_j P_ij v_j,      LSE_i = max s + ln sum_j exp(s_j - max s)
 *
 * Sources: the materialised "naive_attention" test helper of the
 * oxillama-runtime 0.1.0 page (src/flash_attention.rs, test module) gives the
 * S = scale*QK^T -> row softmax -> P*V sequence; the mxflashattn 1.4.0 page
 * (prefill.py, prefill_chunked_reference) gives bottom-right causal alignment
 * (query i sits at key position i + Sk - Sq), the grouped-query head mapping
 * (query head h reads kv head h / (Hq/Hkv)) and the zero output of a row that
 * sees no key; the lattice-inference 0.7.1 page (src/attention/standard.rs)
 * gives packed batches addressed by cumulative sequence lengths, with no
 * attention across segments; the kernelbot amd-mixed-mla submission 588924
 * page gives the shared latent KV where V is the leading channels of the kv
 * row. Window and softcap semantics are only named by a signature on the
 * mxflashattn page (flash_attn_func: window_size, softcap); the reading used
 * here is: key j is visible to row i iff i+off-left <= j <= i+off+right
 * (inclusive, -1 = unbounded, intersected with causal), and the cap applies
 * to the scaled score before masking. Masked keys take no part (their score
 * is -inf), so they are never computed.
 *
 * No blocking, no online softmax, no reordering: each row's full visible
 * score vector is materialised, then normalised, then multiplied by V.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC attention_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

typedef struct {
    const void* q;
    const void* k;
    const void* v;
    int dtype;               /* ORACLE_F32, ORACLE_BF16 (bit patterns, upcast exactly) or ORACLE_F64 */
    int64_t q_tok_stride;    /* element strides */
    int64_t q_head_stride;
    int64_t k_tok_stride;
    int64_t k_head_stride;
    int64_t v_tok_stride;
    int64_t v_head_stride;
    const int32_t* cu_q;     /* [batch+1] cumulative query lengths */
    const int32_t* cu_k;     /* [batch+1] cumulative key lengths */
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t d_qk;
    int32_t d_v;
    int32_t causal;
    int32_t window_left;     /* -1: unbounded */
    int32_t window_right;    /* -1: unbounded */
    double softcap;          /* 0: off */
    double scale;
} oracle_problem;

/* Exact upcast of one stored element to double. */
static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == ORACLE_F64) return ((const double*)base)[idx];
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Segment index b with cu_q[b] <= tok < cu_q[b+1] (linear scan). */
static int find_segment(const int32_t* cu, int32_t batch, int64_t tok) {
    for (int b = 0; b < batch; ++b)
        if (tok >= cu[b] && tok < cu[b + 1]) return b;
    return -1;
}

/*
 * Computes rows (tok[r], head[r]) for r in [0, n). Writes o[r*d_v + c],
 * lse[r] (natural log; -inf for a row that sees no key) and, when
 * max_psum_dev is non-null, the largest |sum_j P_ij - 1| over the rows.
 * Returns 0, or a negative code for bad arguments (-1) / allocation (-2).
 */
int oracle_rows(const oracle_problem* p, const int64_t* tok, const int32_t* head, int64_t n,
                double* o, double* lse, double* max_psum_dev, int threads) {
    if (!p || !tok || !head || !o || !lse) return -1;
    if (p->heads_kv <= 0 || p->heads_q <= 0 || p->heads_q % p->heads_kv) return -1;
    const int group = p->heads_q / p->heads_kv;
    int32_t max_sk = 0;
    for (int b = 0; b < p->batch; ++b) {
        int32_t sk = p->cu_k[b + 1] - p->cu_k[b];
        if (sk > max_sk) max_sk = sk;
    }
    int err = 0;
    double worst = 0.0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#endif
#pragma omp parallel reduction(max : worst)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_sk > 0 ? max_sk : 1));
        if (!s) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n; ++r) {
            if (!s) continue;
            double* out = o + r * p->d_v;
            const int b = find_segment(p->cu_q, p->batch, tok[r]);
            const int h = head[r];
            if (b < 0 || h < 0 || h >= p->heads_q) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            const int64_t sq = p->cu_q[b + 1] - p->cu_q[b];
            const int64_t sk = p->cu_k[b + 1] - p->cu_k[b];
            const int64_t i = tok[r] - p->cu_q[b];
            const int64_t off = sk - sq; /* bottom-right alignment */
            int64_t lo = 0, hi = sk - 1;
            if (p->causal && i + off < hi) hi = i + off;
            if (p->window_right >= 0 && i + off + p->window_right < hi) hi = i + off + p->window_right;
            if (p->window_left >= 0 && i + off - p->window_left > lo) lo = i + off - p->window_left;
            if (lo > hi) {
                for (int c = 0; c < p->d_v; ++c) out[c] = 0.0;
                lse[r] = -INFINITY;
                continue;
            }
            const int g = h / group;
            const int64_t qbase = tok[r] * p->q_tok_stride + (int64_t)h * p->q_head_stride;
            /* scores of the visible keys */
            for (int64_t j = lo; j <= hi; ++j) {
                const int64_t kbase = (p->cu_k[b] + j) * p->k_tok_stride + (int64_t)g * p->k_head_stride;
                double dot = 0.0;
                for (int c = 0; c < p->d_qk; ++c)
                    dot += load_elem(p->q, p->dtype, qbase + c) * load_elem(p->k, p->dtype, kbase + c);
                double t = p->scale * dot;
                if (p->softcap > 0.0) t = p->softcap * tanh(t / p->softcap);
                s[j - lo] = t;
            }
            /* row softmax */
            const int64_t cnt = hi - lo + 1;
            double m = s[0];
            for (int64_t j = 1; j < cnt; ++j)
                if (s[j] > m) m = s[j];
            double z = 0.0;
            for (int64_t j = 0; j < cnt; ++j) {
                s[j] = exp(s[j] - m);
                z += s[j];
            }
            double psum = 0.0;
            for (int64_t j = 0; j < cnt; ++j) {
                s[j] /= z;
                psum += s[j];
            }
            const double dev = fabs(psum - 1.0);
            if (dev > worst) worst = dev;
            /* O = P V */
            for (int c = 0; c < p->d_v; ++c) out[c] = 0.0;
            for (int64_t j = 0; j < cnt; ++j) {
                const int64_t vbase = (p->cu_k[b] + lo + j) * p->v_tok_stride + (int64_t)g * p->v_head_stride;
                for (int c = 0; c < p->d_v; ++c) out[c] += s[j] * load_elem(p->v, p->dtype, vbase + c);
            }
            lse[r] = m + log(z);
        }
        free(s);
    }
    if (max_psum_dev) *max_psum_dev = worst;
    return err;
}

/* Number of OpenMP threads a parallel region would use with `threads`. */
int oracle_threads(int threads) {
#ifdef _OPENMP
    if (threads > 0) return threads;
    return omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}
