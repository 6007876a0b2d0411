/*
 * Plain CPU oracle for the sparse Flash-MLA Softmax-L1Norm.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code. The product
 * library never links it, and it shares no code with the HIP path.
 *
 * What it follows: the "SparseFlashMlaSoftmaxL1Norm" article (CANN
 * ops-transformer, pnsm.cn),
 *   - section 三阶段计算公式 (three-stage formula):
 *       stage 1  selectedKv = Gather(K, sparseIndices[i]), i < selectBlockCount
 *                in the sparse case, else selectedKv = K (the dense case,
 *                no sparse_indices: every key of the row's batch/sequence)
 *       stage 2  P = SimpleSoftmax(Mask(Q selectedKv^T * scale), softmaxLse)
 *       stage 3  softmaxL1Norm = ReduceSum(P, dimG) / G,   G = N1 / N2
 *   - section 参数说明 (parameters) for layouts, cu_seqlens, topk_length,
 *     cmp_residual_k and the output shape (B,S1,N2,S2) / (T1,N2,T2);
 *   - section 约束说明 (constraints) for mask_mode 3 = right-down causal.
 *
 * Readings taken where the page is silent (each one is listed with its
 * reason in the design notes of the repository):
 *   - indices of a TND sequence are local to that sequence: the k row is
 *     cu_seqlens_k[b] + idx and the output column is cu_seqlens_k[b] + idx;
 *   - an entry t of a row is used iff t < n, 0 <= idx < S2_b, and the key
 *     is visible; other entries contribute nothing. n (selectBlockCount) is
 *     topk_length clamped to [0, K]; without topk_length it is K for mask 0
 *     and min(K, number of keys visible to the row) for mask 3 (a row cannot
 *     select more blocks than it sees);
 *   - right-down causal with compression ratio r and residual res: query i of
 *     a sequence with S1_b queries and S2_b compressed keys is at original
 *     position i + S2_b*r + res - S1_b; compressed key j (original positions
 *     j*r .. (j+1)*r-1) is visible iff (j+1)*r <= i + 1 + S2_b*r + res - S1_b;
 *   - SimpleSoftmax with the forward lse is exp(s - lse) in the natural base,
 *     the scale applied to Q.K^T before the lse is subtracted;
 *   - every output element not hit by a used entry is 0 (rows with no used
 *     entry are all 0); repeated indices accumulate;
 *   - dense case (idx == NULL): the row's entries are its sequence's keys in
 *     order, entry t being key t (n = S2_b); topk_length does not apply;
 *     mask and output columns are those of the sparse case;
 *   - seqused_q / seqused_k (parameter table: the number of q / k tokens of
 *     each batch that actually take part), clamped to [0, S1_b] / [0, S2_b]:
 *     a query i >= seqused_q[b] uses no entry (its row is 0, its lse -inf),
 *     a key j >= seqused_k[b] is never used (as if not visible); the causal
 *     alignment keeps S1_b and S2_b. The pages give no example of either:
 *     parity of this reading is unpinned by the pages;
 *   - K-wide output (the shape-inference section: the last output dimension
 *     is K when sparse_indices is given, else S2 (BSND) or max_seqlen_k
 *     (TND)): entry t's value goes to column t of a row of that width,
 *     instead of to the key's column.
 *
 * The forward softmax_lse itself (oracle_lse) is not part of the operation:
 * it is the log-sum-exp over the same used entries that the forward pass
 * would produce, computed here so that test inputs are consistent. It is
 * returned rounded to fp32, the dtype the operation consumes.
 *
 * Everything is evaluated in double precision. q and k arrive as float32
 * arrays holding exactly the bf16/fp16 input values (the widening is exact).
 * The scale is the fp32-rounded softmax_scale, widened to double.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { LAYOUT_BSND = 0, LAYOUT_TND = 1 };

typedef struct {
    int64_t b;      /* batch (BSND) or sequence (TND) */
    int64_t i;      /* query position inside it */
    int64_t s1;     /* its number of queries */
    int64_t s2;     /* its number of (compressed) keys */
    int64_t kbase;  /* first k row belonging to it */
    int64_t col0;   /* first output column belonging to it */
    int64_t q_used; /* queries of it that take part (seqused_q, else s1) */
    int64_t k_used; /* keys of it that take part (seqused_k, else s2) */
} row_info;

typedef struct {
    const float* k;          /* (B*S2 | T2, D) */
    const int32_t* idx;      /* (R, K), or NULL: the dense case */
    const int32_t* topk_len; /* (R) or NULL */
    const int32_t* cu_q;     /* (B+1) for TND */
    const int32_t* cu_k;
    const int32_t* cmp_res;  /* (B) or NULL */
    const int32_t* su_q;     /* seqused_q (B) or NULL */
    const int32_t* su_k;     /* seqused_k (B) or NULL */
    int64_t layout, B, S1, S2, G, D, K, mask_mode, cmp_ratio;
    double scale;
} problem;

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

/* seqused limits of a decoded row */
static void set_used(const problem* p, row_info* ri) {
    ri->q_used = p->su_q ? clamp64(p->su_q[ri->b], 0, ri->s1) : ri->s1;
    ri->k_used = p->su_k ? clamp64(p->su_k[ri->b], 0, ri->s2) : ri->s2;
}

static int decode_row(const problem* p, int64_t r, row_info* ri) {
    if (p->layout == LAYOUT_BSND) {
        ri->b = r / p->S1;
        ri->i = r % p->S1;
        ri->s1 = p->S1;
        ri->s2 = p->S2;
        ri->kbase = ri->b * p->S2;
        ri->col0 = 0;
        set_used(p, ri);
        return 0;
    }
    for (int64_t b = 0; b < p->B; ++b) {
        if (r >= p->cu_q[b] && r < p->cu_q[b + 1]) {
            ri->b = b;
            ri->i = r - p->cu_q[b];
            ri->s1 = p->cu_q[b + 1] - p->cu_q[b];
            ri->s2 = p->cu_k[b + 1] - p->cu_k[b];
            ri->kbase = p->cu_k[b];
            ri->col0 = p->cu_k[b];
            set_used(p, ri);
            return 0;
        }
    }
    return -1;
}

static int visible(const problem* p, const row_info* ri, int64_t j) {
    if (p->mask_mode == 0) return 1;
    int64_t res = p->cmp_res ? p->cmp_res[ri->b] : 0;
    int64_t r = p->cmp_ratio;
    return (j + 1) * r <= ri->i + 1 + ri->s2 * r + res - ri->s1;
}

/* number of leading entries of row r that are looked at */
static int64_t selected_count(const problem* p, const row_info* ri, int64_t r) {
    if (ri->i >= ri->q_used) return 0; /* query not taking part */
    if (!p->idx) return ri->s2; /* dense: selectedKv = K */
    if (!p->topk_len) {
        if (p->mask_mode == 0) return p->K;
        int64_t nvis = 0;  /* keys of the row's sequence it can see */
        for (int64_t j = 0; j < ri->k_used; ++j) nvis += visible(p, ri, j);
        return nvis < p->K ? nvis : p->K;
    }
    int64_t n = p->topk_len[r];
    if (n < 0) n = 0;
    if (n > p->K) n = p->K;
    return n;
}

/* key index of entry t if the entry is used, else -1 */
static int64_t used_key(const problem* p, const row_info* ri, int64_t r, int64_t t) {
    int64_t j = p->idx ? p->idx[r * p->K + t] : t;
    if (j < 0 || j >= ri->k_used) return -1;
    if (!visible(p, ri, j)) return -1;
    return j;
}

/* s = scale * q[g] . k[kbase + j], all in double */
static double score(const problem* p, const float* qrow, int64_t g,
                    const row_info* ri, int64_t j) {
    const float* qg = qrow + g * p->D;
    const float* kj = p->k + (ri->kbase + j) * p->D;
    double acc = 0.0;
    for (int64_t d = 0; d < p->D; ++d) acc += (double)qg[d] * (double)kj[d];
    return p->scale * acc;
}

static void fill_problem(problem* p, const float* k, const int32_t* idx,
                         const int32_t* topk_len, const int32_t* cu_q,
                         const int32_t* cu_k, const int32_t* cmp_res,
                         const int32_t* su_q, const int32_t* su_k, int64_t layout, int64_t B, int64_t S1, int64_t S2,
                         int64_t G, int64_t D, int64_t K, int64_t mask_mode,
                         int64_t cmp_ratio, double scale) {
    p->k = k; p->idx = idx; p->topk_len = topk_len;
    p->cu_q = cu_q; p->cu_k = cu_k; p->cmp_res = cmp_res;
    p->su_q = su_q; p->su_k = su_k;
    p->layout = layout; p->B = B; p->S1 = S1; p->S2 = S2; p->G = G; p->D = D;
    p->K = K; p->mask_mode = mask_mode; p->cmp_ratio = cmp_ratio;
    p->scale = (double)(float)scale;
}

/*
 * Forward log-sum-exp over the used entries, per (row, head):
 *   lse[g] = log sum_{t used} exp(s[g, t]),  -inf when no entry is used.
 * Evaluated as m + log sum exp(s - m) with m the maximum (same value).
 *
 * q_rows:   (nrows, G, D) float32, the q rows listed in rows[]
 * rows:     row ids r in [0, R), R = B*S1 (BSND) or T1 (TND)
 * lse_rows: (nrows, G) float32 out
 * nused:    (nrows) int32 out, number of used entries per row
 * Returns 0, or -1 if a row id cannot be decoded.
 */
int oracle_lse(const float* q_rows, const float* k, const int32_t* idx,
               const int32_t* topk_len, const int32_t* cu_q, const int32_t* cu_k,
               const int32_t* cmp_res, const int32_t* su_q, const int32_t* su_k,
               int64_t layout, int64_t B, int64_t S1,
               int64_t S2, int64_t G, int64_t D, int64_t K, int64_t mask_mode,
               int64_t cmp_ratio, double scale, const int64_t* rows, int64_t nrows,
               float* lse_rows, int32_t* nused) {
    problem p;
    fill_problem(&p, k, idx, topk_len, cu_q, cu_k, cmp_res, su_q, su_k, layout, B, S1,
                 S2, G, D, K, mask_mode, cmp_ratio, scale);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t x = 0; x < nrows; ++x) {
        int64_t r = rows[x];
        row_info ri;
        if (decode_row(&p, r, &ri) != 0) { bad |= 1; continue; }
        const float* qrow = q_rows + x * G * D;
        int64_t n = selected_count(&p, &ri, r);
        double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int32_t used = 0;
        for (int64_t t = 0; t < n; ++t) used += used_key(&p, &ri, r, t) >= 0;
        nused[x] = used;
        for (int64_t g = 0; g < G; ++g) {
            double m = -INFINITY;
            int64_t cnt = 0;
            for (int64_t t = 0; t < n; ++t) {
                int64_t j = used_key(&p, &ri, r, t);
                if (j < 0) continue;
                s[cnt] = score(&p, qrow, g, &ri, j);
                if (s[cnt] > m) m = s[cnt];
                ++cnt;
            }
            double lse;
            if (cnt == 0) {
                lse = -INFINITY;
            } else {
                double sum = 0.0;
                for (int64_t c = 0; c < cnt; ++c) sum += exp(s[c] - m);
                lse = m + log(sum);
            }
            lse_rows[x * G + g] = (float)lse;
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * The operation itself, for the rows listed in rows[]:
 *   out[c] = 0 for every column c of the row, then for every used entry t
 *   with key j:  out[col0 + j] += (1/G) * sum_g exp(s[g, t] - lse[g])
 *   (K-wide output: out[t] instead of out[col0 + j]).
 *
 * lse_rows: (nrows, G) float32, the softmax_lse values of those rows
 * out_rows: (nrows, W) float32 out; W = S2 (BSND) or T2 (TND), or with
 *           kwide the K-wide width (K; dense: S2 or max_seqlen_k)
 */
int oracle_l1norm(const float* q_rows, const float* k, const float* lse_rows,
                  const int32_t* idx, const int32_t* topk_len, const int32_t* cu_q,
                  const int32_t* cu_k, const int32_t* cmp_res, const int32_t* su_q,
                  const int32_t* su_k, int64_t layout,
                  int64_t B, int64_t S1, int64_t S2, int64_t G, int64_t D, int64_t K,
                  int64_t mask_mode, int64_t cmp_ratio, double scale,
                  const int64_t* rows, int64_t nrows, int64_t kwide, int64_t W,
                  float* out_rows) {
    problem p;
    fill_problem(&p, k, idx, topk_len, cu_q, cu_k, cmp_res, su_q, su_k, layout, B, S1,
                 S2, G, D, K, mask_mode, cmp_ratio, scale);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t x = 0; x < nrows; ++x) {
        int64_t r = rows[x];
        row_info ri;
        if (decode_row(&p, r, &ri) != 0) { bad |= 1; continue; }
        const float* qrow = q_rows + x * G * D;
        const float* lse = lse_rows + x * G;
        double* acc = (double*)calloc((size_t)W, sizeof(double));
        int64_t n = selected_count(&p, &ri, r);
        for (int64_t t = 0; t < n; ++t) {
            int64_t j = used_key(&p, &ri, r, t);
            if (j < 0) continue;
            double psum = 0.0;
            for (int64_t g = 0; g < G; ++g)
                psum += exp(score(&p, qrow, g, &ri, j) - (double)lse[g]);
            const int64_t c = kwide ? t : ri.col0 + j;
            if (c >= W) { bad |= 2; continue; } /* no room: the caller's W is wrong */
            acc[c] += psum / (double)G;
        }
        float* o = out_rows + x * W;
        for (int64_t c = 0; c < W; ++c) o[c] = (float)acc[c];
        free(acc);
    }
    return bad ? -1 : 0;
}

/* Number of threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
