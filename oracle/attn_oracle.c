/*
 * Exact attention oracle, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may call this code. The GPU library neither links nor calls
 * it, and it shares no code, header or table with the GPU library.
 *
 * What it computes is the plain definition of scaled-dot-product attention,
 * written out row by row, materialising each query row's full vector of scores
 * (the structure of the small exact kernel on the rustytorch
 * "flash_attention_forward.cu" page, function flash_attention_forward_small_kernel:
 * scores, then max, then sum of exponentials, then LSE = max + log(sum), then the
 * probability-weighted sum of V; and the materialising path of the llm.c
 * "attention.cuh" page, function attention_forward: QK^T, then row softmax, then
 * times V). It is never online or tiled.
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes):
 *   - scores are s_ij = scale * sum_t q_it k_jt with the scale applied before the
 *     mask, and the LSE is the natural log of sum_j exp(s_ij) over allowed keys
 *     (rustytorch page, OnlineSoftmaxState::get_log_sum_exp and the small kernel);
 *   - the causal mask is bottom-right aligned: key j is allowed for query row i
 *     iff j <= i + (Nk - Nq); with Nq == Nk this is the pages' j <= i;
 *   - masked keys are excluded from the row (no finite stand-in constant);
 *   - a row with no allowed key has O = 0 and LSE = -inf;
 *   - grouped-query attention maps query head h to key/value head
 *     floor(h * Hkv / Hq) (abaddon "attention.rs" page, flash_attention_f16);
 *   - decode: the single new query attends to every cached key 0..L_b-1 with no
 *     mask (abaddon page, flash_attention_cached_f16);
 *   - split-KV partials: chunk c covers keys [c*chunk, min((c+1)*chunk, L_b)); the
 *     partial is that chunk's own normalised output and LSE, and chunks past the
 *     end have O = 0 and LSE = -inf;
 *   - combine: global max M over the chunk LSEs, weights exp(LSE_c - M), output is
 *     the weighted mean of the chunk outputs, LSE = M + log(sum of weights); -inf
 *     chunks carry zero weight (aprender-gpu "flash_decoding/reduce_kernel.rs"
 *     page, FlashDecodingReduceKernel::build_ptx, its two passes over the chunks).
 *
 * Inputs are the raw 16-bit patterns of bf16 (dtype 0) or IEEE fp16 (dtype 1)
 * values, decoded here to fp64 without rounding. The fp32 `scale` is widened
 * exactly. Every sum is a sequential fp64 sum.
 *
 * Return value of every entry point: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- 16-bit float decoding (no rounding: both formats embed in fp64) ---- */

static double decode_bf16(uint16_t bits) {
    /* bf16 is the upper half of an IEEE binary32 pattern. */
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double decode_fp16(uint16_t bits) {
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

static double decode(uint16_t bits, int dtype) {
    return dtype == 0 ? decode_bf16(bits) : decode_fp16(bits);
}

/* Decodes n consecutive 16-bit values into out. */
static void decode_vec(const uint16_t* src, int64_t n, int dtype, double* out) {
    for (int64_t t = 0; t < n; ++t) out[t] = decode(src[t], dtype);
}

/*
 * One query row attending to keys [lo, hi) of one key/value head.
 *   qrow: the decoded query (d values)
 *   kh, vh: the raw key/value rows of this head, row-major [*, d]
 *   s: scratch of at least hi-lo doubles (the materialised score vector)
 *   vrow: scratch of d doubles
 * Writes o[0..d) and *lse.
 */
static void attend_row(const double* qrow, const uint16_t* kh, const uint16_t* vh,
                       int dtype, int64_t lo, int64_t hi, int d, double scale,
                       double* s, double* vrow, double* o, double* lse) {
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    if (hi <= lo) {
        *lse = -INFINITY;
        return;
    }
    /* 1. scores of every allowed key */
    for (int64_t j = lo; j < hi; ++j) {
        const uint16_t* krow = kh + j * (int64_t)d;
        double acc = 0.0;
        for (int t = 0; t < d; ++t) acc += qrow[t] * decode(krow[t], dtype);
        s[j - lo] = scale * acc;
    }
    /* 2. row maximum */
    double m = s[0];
    for (int64_t j = 1; j < hi - lo; ++j)
        if (s[j] > m) m = s[j];
    /* 3. exponentials relative to the maximum, and their sum */
    double l = 0.0;
    for (int64_t j = 0; j < hi - lo; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* 4. probability-weighted sum of the value rows */
    for (int64_t j = lo; j < hi; ++j) {
        decode_vec(vh + j * (int64_t)d, d, dtype, vrow);
        double p = s[j - lo] / l;
        for (int t = 0; t < d; ++t) o[t] += p * vrow[t];
    }
    /* 5. log-sum-exp, natural log */
    *lse = m + log(l);
}

/* Exclusive end of the allowed key range of query row i (keys 0..end-1). */
static int64_t causal_end(int64_t i, int Nq, int Nk, int causal) {
    if (!causal) return Nk;
    int64_t e = i + ((int64_t)Nk - (int64_t)Nq) + 1;
    if (e < 0) e = 0;
    if (e > Nk) e = Nk;
    return e;
}

static int check_fwd(int B, int Hq, int Hkv, int Nq, int Nk, int d, int dtype) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (dtype != 0 && dtype != 1) return -1;
    return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Attention forward over every row.
 *   q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d] (16-bit patterns, row-major)
 *   o [B,Hq,Nq,d] fp64, lse [B,Hq,Nq] fp64
 */
int oracle_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                    double* o, double* lse, int nthreads) {
    if (check_fwd(B, Hq, Hkv, Nq, Nk, d, dtype)) return -1;
    set_threads(nthreads);
    const int64_t nrows = (int64_t)B * Hq * Nq;
    const double sc = (double)scale;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = r % Nq;
            int64_t h = (r / Nq) % Hq;
            int64_t b = r / ((int64_t)Nq * Hq);
            int64_t g = h * Hkv / Hq;
            const uint16_t* kh = k + ((b * Hkv + g) * (int64_t)Nk) * d;
            const uint16_t* vh = v + ((b * Hkv + g) * (int64_t)Nk) * d;
            decode_vec(q + r * (int64_t)d, d, dtype, qrow);
            attend_row(qrow, kh, vh, dtype, 0, causal_end(i, Nq, Nk, causal), d, sc, s, vrow,
                       o + r * (int64_t)d, lse + r);
        }
        free(s);
        free(qrow);
        free(vrow);
    }
    return 0;
}

/*
 * Local (sliding-window) attention forward, the "local" mode flagged in the
 * flash-attention page's kernel traits: key j is allowed for query row i iff
 * i + off - window_left <= j <= i + off + window_right with off = Nk - Nq; a
 * negative bound is no bound on that side. Shapes and outputs as
 * oracle_attn_fwd. The allowed keys of a row are one contiguous range.
 */
int oracle_attn_fwd_local(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                          int window_left, int window_right, double* o, double* lse,
                          int nthreads) {
    if (check_fwd(B, Hq, Hkv, Nq, Nk, d, dtype)) return -1;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t nrows = (int64_t)B * Hq * Nq;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t i = r % Nq, h = (r / Nq) % Hq, b = r / ((int64_t)Nq * Hq);
            const int64_t g = h * Hkv / Hq;
            const int64_t centre = i + ((int64_t)Nk - Nq);
            int64_t lo = window_left < 0 ? 0 : centre - window_left;
            int64_t hi = window_right < 0 ? Nk : centre + window_right + 1;
            if (lo < 0) lo = 0;
            if (hi > Nk) hi = Nk;
            const uint16_t* kh = k + ((b * Hkv + g) * (int64_t)Nk) * d;
            const uint16_t* vh = v + ((b * Hkv + g) * (int64_t)Nk) * d;
            decode_vec(q + r * (int64_t)d, d, dtype, qrow);
            attend_row(qrow, kh, vh, dtype, lo, hi, d, sc, s, vrow, o + r * (int64_t)d, lse + r);
        }
        free(s);
        free(qrow);
        free(vrow);
    }
    return 0;
}

/*
 * Attention forward from a packed projection output qkv [B, N, 3, H, d] (the
 * layout the llm.c page's attention_forward permutes apart before its matrix
 * products): q, k and v of head h and token n are qkv[b][n][0|1|2][h]. Output
 * o [B, N, H, d] (token-major) and lse [B, H, N]. Each (b, h) gathers its
 * three row sets into contiguous scratch and attends as oracle_attn_fwd.
 */
int oracle_attn_fwd_qkvpacked(const uint16_t* qkv, int dtype, int B, int N, int H, int d,
                              float scale, int causal, double* o, double* lse, int nthreads) {
    if (check_fwd(B, H, H, N, N, d, dtype)) return -1;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t units = (int64_t)B * H;
    const int64_t tok = (int64_t)3 * H * d;  /* elements per token */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
        uint16_t* kg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * (size_t)d);
        uint16_t* vg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            const int64_t b = u / H, h = u % H;
            const uint16_t* base = qkv + b * (int64_t)N * tok;
            for (int64_t j = 0; j < N; ++j) {
                memcpy(kg + j * d, base + j * tok + (H + h) * (int64_t)d, sizeof(uint16_t) * (size_t)d);
                memcpy(vg + j * d, base + j * tok + (2 * H + h) * (int64_t)d,
                       sizeof(uint16_t) * (size_t)d);
            }
            for (int64_t i = 0; i < N; ++i) {
                decode_vec(base + i * tok + h * (int64_t)d, d, dtype, qrow);
                attend_row(qrow, kg, vg, dtype, 0, causal_end(i, N, N, causal), d, sc, s, vrow,
                           o + ((b * N + i) * H + h) * (int64_t)d, lse + (b * H + h) * (int64_t)N + i);
            }
        }
        free(s);
        free(qrow);
        free(vrow);
        free(kg);
        free(vg);
    }
    return 0;
}

/*
 * Attention forward for a chosen set of rows only (for spot checks of large
 * problems). rows holds n triples (b, h, i). o is [n, d], lse is [n].
 */
int oracle_attn_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         const int64_t* rows, int64_t n, double* o, double* lse, int nthreads) {
    if (check_fwd(B, Hq, Hkv, Nq, Nk, d, dtype)) return -1;
    for (int64_t r = 0; r < n; ++r) {
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= Hq || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= Nq)
            return -1;
    }
    set_threads(nthreads);
    const double sc = (double)scale;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n; ++r) {
            int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            int64_t g = h * Hkv / Hq;
            const uint16_t* kh = k + ((b * Hkv + g) * (int64_t)Nk) * d;
            const uint16_t* vh = v + ((b * Hkv + g) * (int64_t)Nk) * d;
            decode_vec(q + ((b * Hq + h) * (int64_t)Nq + i) * d, d, dtype, qrow);
            attend_row(qrow, kh, vh, dtype, 0, causal_end(i, Nq, Nk, causal), d, sc, s, vrow,
                       o + r * (int64_t)d, lse + r);
        }
        free(s);
        free(qrow);
        free(vrow);
    }
    return 0;
}

/*
 * Attention forward over a packed batch of sequences of different lengths (the
 * variable-length mode flagged in the flash-attention page's kernel traits).
 *   q [total_q, Hq, d], k and v [total_k, Hkv, d] (16-bit patterns, row-major)
 *   cu_q, cu_k [B+1]: sequence b owns query rows [cu_q[b], cu_q[b+1]) and key
 *   rows [cu_k[b], cu_k[b+1]); both start at 0, never decrease and end at
 *   total_q / total_k.
 *   o [total_q, Hq, d] fp64, lse [Hq, total_q] fp64
 * Each sequence is an independent attention problem with Nq_b = cu_q[b+1] -
 * cu_q[b] queries and Nk_b keys; the causal mask is bottom-right aligned within
 * it. Each (b, h) gathers its kv-head's key and value rows into contiguous
 * scratch, then every query row attends to them as in oracle_attn_fwd.
 */
int oracle_attn_fwd_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* cu_q, const int32_t* cu_k, int dtype, int B, int Hq,
                           int Hkv, int total_q, int total_k, int d, float scale, int causal,
                           double* o, double* lse, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || total_q <= 0 || total_k < 0 || d <= 0) return -1;
    if (Hq % Hkv != 0 || (dtype != 0 && dtype != 1)) return -1;
    if (cu_q[0] != 0 || cu_k[0] != 0 || cu_q[B] != total_q || cu_k[B] != total_k) return -1;
    int64_t max_nk = 0;
    for (int b = 0; b < B; ++b) {
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return -1;
        if (cu_k[b + 1] - cu_k[b] > max_nk) max_nk = cu_k[b + 1] - cu_k[b];
    }
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t units = (int64_t)B * Hq;
    const size_t nk_alloc = (size_t)(max_nk > 0 ? max_nk : 1);
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * nk_alloc);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
        uint16_t* kg = (uint16_t*)malloc(sizeof(uint16_t) * nk_alloc * (size_t)d);
        uint16_t* vg = (uint16_t*)malloc(sizeof(uint16_t) * nk_alloc * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            const int64_t b = u / Hq, h = u % Hq;
            const int64_t g = h * Hkv / Hq;
            const int64_t q0 = cu_q[b], k0 = cu_k[b];
            const int Nq = cu_q[b + 1] - cu_q[b], Nk = cu_k[b + 1] - cu_k[b];
            /* 1. this sequence's rows of kv-head g, contiguous */
            for (int64_t j = 0; j < Nk; ++j) {
                const int64_t src = ((k0 + j) * Hkv + g) * (int64_t)d;
                memcpy(kg + j * d, k + src, sizeof(uint16_t) * (size_t)d);
                memcpy(vg + j * d, v + src, sizeof(uint16_t) * (size_t)d);
            }
            /* 2. every query row of the sequence */
            for (int64_t i = 0; i < Nq; ++i) {
                const int64_t row = q0 + i;
                decode_vec(q + (row * Hq + h) * (int64_t)d, d, dtype, qrow);
                attend_row(qrow, kg, vg, dtype, 0, causal_end(i, Nq, Nk, causal), d, sc, s, vrow,
                           o + (row * Hq + h) * (int64_t)d, lse + h * (int64_t)total_q + row);
            }
        }
        free(s);
        free(qrow);
        free(vrow);
        free(kg);
        free(vg);
    }
    return 0;
}

/*
 * Attention backward: the gradients of L = sum_i dO_i . O_i with respect to q, k
 * and v, written out from the plain definition (the derivation that the
 * llm.c page's attention_backward and the flash-attention page's backward
 * kernel implement): for each query row i with allowed keys J_i,
 *   P_ij  = exp(s_ij) / sum_{j' in J_i} exp(s_ij')     s_ij = scale * q_i . k_j
 *   dv_j += P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dq_i  = scale * sum_j dS_ij k_j,     dk_j += scale * dS_ij q_i
 * dk and dv of kv-head g sum over every query head that reads it (GQA).
 *   q, do [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d] (16-bit patterns)
 *   dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d] fp64
 * Parallel over (b, kv-head), so each thread owns its dk / dv rows.
 */
int oracle_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dout, int dtype, int B, int Hq, int Hkv, int Nq, int Nk,
                    int d, float scale, int causal, double* dq, double* dk, double* dv,
                    int nthreads) {
    if (check_fwd(B, Hq, Hkv, Nq, Nk, d, dtype)) return -1;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t units = (int64_t)B * Hkv;
    const int group = Hq / Hkv;
#pragma omp parallel
    {
        double* sp = (double*)malloc(sizeof(double) * (size_t)Nk);   /* scores, then P */
        double* dp = (double*)malloc(sizeof(double) * (size_t)Nk);   /* dP, then dS */
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* dorow = (double*)malloc(sizeof(double) * (size_t)d);
        double* kd = (double*)malloc(sizeof(double) * (size_t)Nk * (size_t)d);
        double* vd = (double*)malloc(sizeof(double) * (size_t)Nk * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            const int64_t b = u / Hkv, g = u % Hkv;
            const int64_t kvbase = ((b * Hkv + g) * (int64_t)Nk) * d;
            decode_vec(k + kvbase, (int64_t)Nk * d, dtype, kd);
            decode_vec(v + kvbase, (int64_t)Nk * d, dtype, vd);
            double* dkh = dk + kvbase;
            double* dvh = dv + kvbase;
            for (int64_t x = 0; x < (int64_t)Nk * d; ++x) dkh[x] = dvh[x] = 0.0;
            for (int hh = 0; hh < group; ++hh) {
                const int64_t h = g * group + hh;  /* the heads with floor(h*Hkv/Hq) == g */
                for (int64_t i = 0; i < Nq; ++i) {
                    const int64_t qoff = ((b * Hq + h) * (int64_t)Nq + i) * d;
                    double* dqi = dq + qoff;
                    for (int t = 0; t < d; ++t) dqi[t] = 0.0;
                    const int64_t hi = causal_end(i, Nq, Nk, causal);
                    if (hi <= 0) continue;  /* no allowed key: no gradient */
                    decode_vec(q + qoff, d, dtype, qrow);
                    decode_vec(dout + qoff, d, dtype, dorow);
                    /* P_i: scores, max, exponentials, normalisation */
                    double m = -INFINITY;
                    for (int64_t j = 0; j < hi; ++j) {
                        double acc = 0.0;
                        for (int t = 0; t < d; ++t) acc += qrow[t] * kd[j * d + t];
                        sp[j] = sc * acc;
                        if (sp[j] > m) m = sp[j];
                    }
                    double l = 0.0;
                    for (int64_t j = 0; j < hi; ++j) {
                        sp[j] = exp(sp[j] - m);
                        l += sp[j];
                    }
                    for (int64_t j = 0; j < hi; ++j) sp[j] /= l;
                    /* dP_ij and D_i */
                    double Di = 0.0;
                    for (int64_t j = 0; j < hi; ++j) {
                        double acc = 0.0;
                        for (int t = 0; t < d; ++t) acc += dorow[t] * vd[j * d + t];
                        dp[j] = acc;
                        Di += sp[j] * acc;
                    }
                    /* dS, then the three gradients */
                    for (int64_t j = 0; j < hi; ++j) {
                        const double ds = sp[j] * (dp[j] - Di);
                        for (int t = 0; t < d; ++t) {
                            dqi[t] += sc * ds * kd[j * d + t];
                            dkh[j * d + t] += sc * ds * qrow[t];
                            dvh[j * d + t] += sp[j] * dorow[t];
                        }
                    }
                }
            }
        }
        free(sp);
        free(dp);
        free(qrow);
        free(dorow);
        free(kd);
        free(vd);
    }
    return 0;
}

static int check_decode(int B, int Hq, int Hkv, int max_len, int d, int dtype,
                        const int32_t* seq_lens) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_len <= 0 || d <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (dtype != 0 && dtype != 1) return -1;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > max_len) return -1;
    return 0;
}

/*
 * Single-token decode against a padded KV cache.
 *   q [B,Hq,d]; k_cache, v_cache [B,Hkv,max_len,d]; seq_lens [B]
 *   o [B,Hq,d] fp64; lse [B,Hq] fp64
 * The query of sequence b attends to keys 0..seq_lens[b]-1, unmasked.
 */
int oracle_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                  const int32_t* seq_lens, int dtype, int B, int Hq, int Hkv, int max_len,
                  int d, float scale, double* o, double* lse, int nthreads) {
    if (check_decode(B, Hq, Hkv, max_len, d, dtype, seq_lens)) return -1;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t nrows = (int64_t)B * Hq;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)max_len);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t b = r / Hq, h = r % Hq;
            int64_t g = h * Hkv / Hq;
            const uint16_t* kh = k_cache + ((b * Hkv + g) * (int64_t)max_len) * d;
            const uint16_t* vh = v_cache + ((b * Hkv + g) * (int64_t)max_len) * d;
            decode_vec(q + r * (int64_t)d, d, dtype, qrow);
            attend_row(qrow, kh, vh, dtype, 0, seq_lens[b], d, sc, s, vrow,
                       o + r * (int64_t)d, lse + r);
        }
        free(s);
        free(qrow);
        free(vrow);
    }
    return 0;
}

/*
 * Single-token decode against a paged KV cache (the layout of the aprender-gpu
 * page's "attention/paged/flash_decoding" module: fixed-size pages in a shared
 * pool, and a per-sequence table listing them in order).
 *   q [B,Hq,d]; k_pages, v_pages [num_pages, page_size, Hkv, d];
 *   block_table [B, max_pages]; seq_lens [B]
 *   o [B,Hq,d] fp64; lse [B,Hq] fp64
 * Key j of sequence b is row j % page_size of page block_table[b][j / page_size]
 * (kv-head g within that row). Each (b, h) first gathers its L_b key and value
 * rows through the table into contiguous scratch, then attends to them exactly
 * as oracle_decode does. A table entry that a sequence uses outside
 * [0, num_pages) is a bad argument.
 */
int oracle_decode_paged(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages,
                        const int32_t* block_table, const int32_t* seq_lens, int dtype, int B,
                        int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                        float scale, double* o, double* lse, int nthreads) {
    if (num_pages <= 0 || page_size <= 0 || max_pages <= 0) return -1;
    const int64_t max_len = (int64_t)max_pages * page_size;
    if (max_len > 0x7fffffff) return -1;
    if (check_decode(B, Hq, Hkv, (int)max_len, d, dtype, seq_lens)) return -1;
    for (int b = 0; b < B; ++b)
        for (int64_t j = 0; j < seq_lens[b]; j += page_size) {
            const int32_t pg = block_table[(int64_t)b * max_pages + j / page_size];
            if (pg < 0 || pg >= num_pages) return -1;
        }
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t nrows = (int64_t)B * Hq;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)max_len);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
        uint16_t* kg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)max_len * (size_t)d);
        uint16_t* vg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)max_len * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t b = r / Hq, h = r % Hq;
            int64_t g = h * Hkv / Hq;
            const int64_t L = seq_lens[b];
            /* 1. gather the sequence's rows of kv-head g through the block table */
            for (int64_t j = 0; j < L; ++j) {
                const int64_t pg = block_table[b * max_pages + j / page_size];
                const int64_t src = ((pg * page_size + j % page_size) * Hkv + g) * (int64_t)d;
                memcpy(kg + j * d, k_pages + src, sizeof(uint16_t) * (size_t)d);
                memcpy(vg + j * d, v_pages + src, sizeof(uint16_t) * (size_t)d);
            }
            /* 2. the plain decode row over the gathered keys */
            decode_vec(q + r * (int64_t)d, d, dtype, qrow);
            attend_row(qrow, kg, vg, dtype, 0, L, d, sc, s, vrow, o + r * (int64_t)d, lse + r);
        }
        free(s);
        free(qrow);
        free(vrow);
        free(kg);
        free(vg);
    }
    return 0;
}

/*
 * Split-KV partials: for every (b, h, c) with C = ceil(max_len / chunk) chunk
 * slots, the exact attention of the query over keys
 * [c*chunk, min((c+1)*chunk, seq_lens[b])), normalised within the chunk.
 *   part_o [B,Hq,C,d] fp64; part_lse [B,Hq,C] fp64.
 * Chunk slots at or past the end of the sequence get O = 0 and LSE = -inf.
 */
int oracle_decode_chunks(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* seq_lens, int dtype, int B, int Hq, int Hkv,
                         int max_len, int d, int chunk, float scale, double* part_o,
                         double* part_lse, int nthreads) {
    if (check_decode(B, Hq, Hkv, max_len, d, dtype, seq_lens)) return -1;
    if (chunk <= 0) return -1;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t C = ((int64_t)max_len + chunk - 1) / chunk;
    const int64_t nitems = (int64_t)B * Hq * C;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)chunk);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)d);
        double* vrow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < nitems; ++r) {
            int64_t c = r % C;
            int64_t h = (r / C) % Hq;
            int64_t b = r / (C * Hq);
            int64_t g = h * Hkv / Hq;
            int64_t lo = c * chunk;
            int64_t hi = lo + chunk;
            if (hi > seq_lens[b]) hi = seq_lens[b];
            const uint16_t* kh = k_cache + ((b * Hkv + g) * (int64_t)max_len) * d;
            const uint16_t* vh = v_cache + ((b * Hkv + g) * (int64_t)max_len) * d;
            decode_vec(q + (b * Hq + h) * (int64_t)d, d, dtype, qrow);
            attend_row(qrow, kh, vh, dtype, lo, hi, d, sc, s, vrow, part_o + r * (int64_t)d,
                       part_lse + r);
        }
        free(s);
        free(qrow);
        free(vrow);
    }
    return 0;
}

/*
 * Combine of split-KV partials (fp64 inputs, so it can also merge widened GPU
 * partials). For each (b, h) it merges the first n_c = ceil(seq_lens[b]/chunk)
 * chunk slots (capped at C):
 *   M = max_c LSE_c;  w_c = exp(LSE_c - M);  O = sum_c w_c O_c / sum_c w_c;
 *   LSE = M + log(sum_c w_c).
 * Chunks with LSE = -inf get weight 0. If every chunk is -inf (or n_c = 0) the
 * output is O = 0, LSE = -inf.
 *   part_o [B,Hq,C,d], part_lse [B,Hq,C]; o [B,Hq,d], lse [B,Hq].
 */
int oracle_combine(const double* part_o, const double* part_lse, const int32_t* seq_lens,
                   int B, int Hq, int C, int d, int chunk, double* o, double* lse) {
    if (B <= 0 || Hq <= 0 || C <= 0 || d <= 0 || chunk <= 0) return -1;
    for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
        int64_t b = r / Hq;
        if (seq_lens[b] < 0) return -1;
        int64_t nc = ((int64_t)seq_lens[b] + chunk - 1) / chunk;
        if (nc > C) nc = C;
        const double* po = part_o + r * (int64_t)C * d;
        const double* pl = part_lse + r * (int64_t)C;
        double* out = o + r * (int64_t)d;
        for (int t = 0; t < d; ++t) out[t] = 0.0;
        /* pass 1: global maximum over the chunk LSEs */
        double M = -INFINITY;
        for (int64_t c = 0; c < nc; ++c)
            if (pl[c] > M) M = pl[c];
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        /* pass 2: weights, weighted sum, normalisation */
        double wsum = 0.0;
        for (int64_t c = 0; c < nc; ++c) {
            if (pl[c] == -INFINITY) continue;
            double w = exp(pl[c] - M);
            wsum += w;
            for (int t = 0; t < d; ++t) out[t] += w * po[c * d + t];
        }
        for (int t = 0; t < d; ++t) out[t] /= wsum;
        lse[r] = M + log(wsum);
    }
    return 0;
}

/* Decodes n 16-bit patterns to fp64 (exposed so tests can pin the decoders). */
int oracle_decode_values(const uint16_t* src, int64_t n, int dtype, double* out) {
    if (dtype != 0 && dtype != 1) return -1;
    decode_vec(src, n, dtype, out);
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
