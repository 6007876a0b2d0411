/*
 * smla.h - C ABI of the sparse Flash-MLA Softmax-L1Norm library for MI355X
 * (gfx950).
 *
 * The operation is the one the "SparseFlashMlaSoftmaxL1Norm" article (CANN
 * ops-transformer, pnsm.cn) defines. For every query row it gathers the
 * row's top-k selected rows of the single shared latent K (N2 = 1, D = 512),
 * forms Q.K^T * scale for the G = N1/N2 query heads, masks the scores, turns
 * them into probabilities with the forward pass's log-sum-exp as
 * exp(s - lse), and averages the G probability rows into one fp32 row
 * (section 三阶段计算公式, three-stage formula; output shapes from section
 * 参数说明).
 *
 * As on the page, a call is split in two: a host metadata call that plans
 * the work split (section 算子定位与配套关系, metadata fields), then the
 * main call that runs on the GPU.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers unless the name ends in _host.
 *    Tensors are dense, row-major and contiguous in the stated layout.
 *  - The caller owns every buffer and the stream. The library allocates no
 *    device memory and needs no workspace.
 *  - All argument checks happen before anything is enqueued. On an error
 *    nothing is written and nothing is launched; smla_last_error() gives a
 *    message. A success of smla_softmax_l1norm means "enqueued on stream":
 *    results are ready once the stream has synchronised.
 *  - Calls are thread-safe and deterministic: the same inputs give the same
 *    bits on every run (the page's 约束说明 section states determinism).
 */
#ifndef SMLA_H
#define SMLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of int32 elements of a metadata buffer (64 on the page too). */
#define SMLA_METADATA_SIZE 64

/* Status codes. The first two reuse the numeric values of the page's aclnn
 * errors (section 调用方式一 aclnn API): 161001 = an illegal null pointer,
 * 161002 = an unsupported dtype / value or a missing required tensor. */
typedef int32_t smla_status_t;
enum {
    SMLA_SUCCESS = 0,
    SMLA_ERR_PARAM_NULLPTR = 161001,
    SMLA_ERR_PARAM_INVALID = 161002,
    SMLA_ERR_UNSUPPORTED = 161101, /* valid on the page, beyond this
                                      library's limits: a key sequence of
                                      more than 2^21 rows, topk above 2^24,
                                      or output rows wider than 0x1FFFFFFC
                                      columns (the kernels address key rows,
                                      index lists and output rows with
                                      32-bit byte offsets) */
    SMLA_ERR_RUNTIME = 561001      /* a HIP runtime call failed */
};

enum { SMLA_LAYOUT_BSND = 0, SMLA_LAYOUT_TND = 1 };
enum { SMLA_DTYPE_FP16 = 0, SMLA_DTYPE_BF16 = 1 };
enum { SMLA_MASK_NONE = 0, SMLA_MASK_RIGHT_DOWN_CAUSAL = 3 };

/* Metadata layout (int32[64]).
 * Fields 0..4 are the page's (section 算子定位与配套关系):
 *   [0] total      number of query rows to balance, R * N2
 *                  (R = B*S1 for BSND, T1 for TND)
 *   [1] former     rows per regular workgroup = ceil(total / cores)
 *   [2] remain     rows per tail workgroup    = floor(total / cores)
 *   [3] remainNum  number of tail workgroups: cores - (total mod cores)
 *                  when the division leaves a remainder, else 0
 *   [4] cores      workgroups launched = min(total, core budget); the page
 *                  caps this at 36 Ascend cores, here the budget is the
 *                  number of co-resident workgroups of the kernel on the
 *                  GPU (CU count x resident workgroups per CU)
 * Fields 5.. are this library's own, checked by smla_softmax_l1norm:
 *   [5] magic 0x534D4C41, [6] version, [7] layout, [8] N1, [9] N2, [10] D,
 *   [11] B, [12] max_seqlen_q, [13] max_seqlen_k, [14] topk,
 *   [15] mask_mode, [16] cmp_ratio, [17] R, [18] rows of k (B*S2 or T2),
 *   [19] row order (1 = snake: workgroup w takes rows w, 2C-1-w, 2C+w, ...),
 *   [20] head tiles per row (kernel variant), [21] device, [22] CU count,
 *   [23] resident workgroups per CU,
 *   [24] kernel: 0 = general (65..128 heads with topk > 2048: one wave
 *        per 32-head tile, two workgroups per CU), 1 = pipelined for
 *        65..128 heads (topk <= 2048 or the dense case: one 4-wave
 *        workgroup per CU, 64 heads per wave, 64-key tiles), 2 = pipelined
 *        for up to 64 heads (any topk or the dense case: one 4-wave
 *        workgroup per CU, every head and 16 keys per wave);
 *   [25] the longest key sequence (BSND: S2; TND: the longest
 *        cu_seqlens_k step);
 *        [26..63] zero.
 */
#define SMLA_META_MAGIC 0x534D4C41

/*
 * smla_l1norm_metadata - plan the work split (host only, no device work).
 *
 * Mirrors the page's sparse_flash_mla_softmax_l1_norm_metadata parameters
 * (section "metadata 前置算子"), with the sequence tensors in HOST memory.
 *
 *   num_heads_q, num_heads_k, head_dim  N1 in [1,128], N2 == 1, D == 512
 *   cu_seqlens_q_host, cu_seqlens_k_host  int32 (B+1), required for TND
 *                                         (prefix sums, first entry 0);
 *                                         ignored for BSND
 *   seqused_q_host, seqused_k_host      optional, not used (the split is
 *                                         by rows)
 *   cmp_residual_k_host, topk_length_host  optional, only range-checked
 *                                         lengths are not used for balance
 *   batch_size     B (> 0): batches for BSND, sequences for TND (the
 *                  length of cu_seqlens_q minus one)
 *   max_seqlen_q, max_seqlen_k  S1, S2: required > 0 for BSND (the padded
 *                  per-batch lengths); for TND 0 means "from cu_seqlens",
 *                  and a non-zero max_seqlen_k must cover the longest k
 *                  sequence
 *   topk           K, number of indices per row, >= 0; 0 = the dense case
 *                  (no sparse_indices: every key of the row's batch or
 *                  sequence is an entry; stage 1 of the page's formula
 *                  selects the whole K)
 *   layout_q, layout_k  SMLA_LAYOUT_*, must be equal
 *   mask_mode      0 or 3; cmp_ratio in [1,128]
 *   device         HIP device ordinal whose CU count sizes the grid
 *   core_budget    workgroups to split over; 0 = the device's co-resident
 *                  capacity for this problem's kernel variant
 *   metadata_host  out: int32[SMLA_METADATA_SIZE], caller-owned
 *
 * Errors: SMLA_ERR_PARAM_NULLPTR (metadata_host NULL, TND without
 * cu_seqlens), SMLA_ERR_PARAM_INVALID (out-of-range value, layout mismatch,
 * inconsistent cu_seqlens), SMLA_ERR_UNSUPPORTED (a key sequence longer than
 * 2^21 rows, topk above 2^24, more than 0x1FFFFFFC key rows),
 * SMLA_ERR_RUNTIME (device query failed; only when core_budget == 0).
 *
 * Core budget: not a page parameter. The page's metadata operator caps the
 * split at the device's core count; core_budget lets a caller (tests, or a
 * caller sharing the GPU) split over fewer workgroups instead.
 *
 * Environment: SMLA_LOG=1 prints one line per metadata call and per launch
 * (shapes, kernel, grid) on stderr.
 */
smla_status_t smla_l1norm_metadata(
    int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
    const int32_t* seqused_q_host, const int32_t* seqused_k_host,
    const int32_t* cmp_residual_k_host, const int32_t* topk_length_host,
    int64_t batch_size, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t topk,
    int32_t layout_q, int32_t layout_k, int64_t mask_mode, int64_t cmp_ratio,
    int32_t device, int32_t core_budget, int32_t* metadata_host);

/*
 * smla_softmax_l1norm - the main call; enqueues the kernel on `stream`.
 *
 * Mirrors the page's sparse_flash_mla_softmax_l1_norm / aclnn argument list
 * (sections 参数说明 and 调用方式一 aclnn API). Shapes, all row-major:
 *
 *   q              (B,S1,N1,D) | (T1,N1,D), dtype `dtype`
 *   k              (B,S2,N2,D) | (T2,N2,D), same dtype as q
 *   softmax_lse    fp32 (B,N2,S1,G) | (N2,T1,G), natural-log forward lse
 *   sparse_indices int32 (B,S1,N2,K) | (T1,N2,K), or NULL for the dense
 *                  case (then topk must be 0 and topk_length is ignored:
 *                  entry t of a row is key t of its batch/sequence, every
 *                  key in order). Entries index the keys of the row's own
 *                  batch/sequence
 *                  (0-based, local to a TND sequence); an entry is used iff
 *                  its position is < the row's entry count (topk_length
 *                  below), it lies in [0, S2_b) and
 *                  the mask lets the key through. Used entries of one row
 *                  must be distinct: the kernels write each entry's value
 *                  to its key's column, so with a repeated key one write
 *                  wins and the row loses both its sum of 1 and its
 *                  run-to-run determinism. Nothing checks this by default;
 *                  smla_check_indices checks host copies, and with
 *                  SMLA_CHECK_INDICES=1 in the environment every main call
 *                  copies its index lists to the host (synchronising the
 *                  stream) and fails with SMLA_ERR_PARAM_INVALID on a row
 *                  that repeats a key.
 *   cu_seqlens_q, cu_seqlens_k  int32 (B+1) device, required for TND
 *   seqused_q, seqused_k        int32 (B) device, optional (parameter
 *                  table: the q / k tokens of each batch that take part):
 *                  a query i >= seqused_q[b] uses no entry (its output row
 *                  is 0), a key j >= seqused_k[b] is never used (as if not
 *                  visible); the causal alignment keeps S1_b and S2_b. The
 *                  pages give no example of either: this reading is this
 *                  library's own
 *   cmp_residual_k int32 (B): original key length of batch b is
 *                  S2_b*cmp_ratio + cmp_residual_k[b]; required when
 *                  mask_mode == 3 and cmp_ratio != 1, else may be NULL (0)
 *   topk_length    int32 (B,S1,N2) | (T1,N2): entries per row to look at
 *                  (selectBlockCount), clamped to [0,K]; required when
 *                  mask_mode == 0 with sparse_indices; when NULL (mask_mode
 *                  3) a row looks at its first min(K, keys visible to it)
 *                  entries
 *   metadata_host  int32[64] from smla_l1norm_metadata for the same shapes
 *   dtype          SMLA_DTYPE_FP16 or SMLA_DTYPE_BF16
 *   batch_size, seqlen_q, seqlen_k  B,S1,S2 (BSND) | B,T1,T2 (TND)
 *   num_heads_q, num_heads_k, head_dim, topk  N1, N2 (== 1), D (== 512), K
 *   softmax_scale  the page's FLOAT32 attribute; rounded to fp32 once
 *   max_seqlen_k   accepted for the dense TND shape rule; must be >= 0
 *   cmp_ratio      [1,128]; mask_mode 0 (none) or 3 (right-down causal:
 *                  compressed key j of batch b is visible to query i iff
 *                  (j+1)*cmp_ratio <= i + 1 + S2_b*cmp_ratio + res_b - S1_b)
 *   layout_q, layout_k  SMLA_LAYOUT_*, must be equal
 *   softmax_l1_norm fp32 out (B,S1,N2,S2) | (T1,N2,T2); every element is
 *                  written (zeros outside the used entries). For TND a row's
 *                  non-zeros lie in its own sequence's columns
 *                  cu_seqlens_k[b] + j.
 *   stream         hipStream_t (NULL = the default stream)
 *
 * Errors: SMLA_ERR_PARAM_INVALID when q, k, softmax_lse or softmax_l1_norm
 * is NULL (as on the page) or a value/shape is out of range or does not
 * match the metadata; SMLA_ERR_PARAM_NULLPTR when a conditionally required
 * pointer is NULL (metadata, cu_seqlens for TND, cmp_residual_k,
 * topk_length);
 * SMLA_ERR_UNSUPPORTED beyond the limits listed with the status codes;
 * SMLA_ERR_RUNTIME if the launch fails. An empty q (R == 0) or an empty
 * output (S2/T2 == 0) returns SMLA_SUCCESS once the attributes are checked,
 * before any pointer or the metadata is looked at, and launches nothing.
 */
smla_status_t smla_softmax_l1norm(
    const void* q, const void* k, const float* softmax_lse,
    const int32_t* sparse_indices, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, const int32_t* seqused_q, const int32_t* seqused_k,
    const int32_t* cmp_residual_k, const int32_t* topk_length,
    const int32_t* metadata_host, int32_t dtype, int64_t batch_size, int64_t seqlen_q,
    int64_t seqlen_k, int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    int64_t topk, double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
    int64_t mask_mode, int32_t layout_q, int32_t layout_k, float* softmax_l1_norm,
    void* stream);

/*
 * smla_softmax_l1norm_kwide - the main call with the K-wide output of the
 * article's shape-inference section (源码实现解读, shape 推导): the last
 * output dimension is K when sparse_indices is given, and without it S2
 * (BSND) or max_seqlen_k (TND). Entry t of a row (index t of its
 * sparse_indices row, or key t without them) puts its value in column t;
 * columns of unused entries are 0.
 *
 * Arguments are smla_softmax_l1norm's, with
 *
 *   softmax_l1_norm fp32 out (B,S1,N2,K') | (T1,N2,K'), K' = topk, or
 *                  without sparse_indices S2 (BSND) or max_seqlen_k (TND);
 *                  every element written
 *   max_seqlen_k   without sparse_indices in TND: the output width; it
 *                  must equal the metadata's (field 13)
 *
 * Errors: as smla_softmax_l1norm, plus SMLA_ERR_PARAM_INVALID for a TND
 * max_seqlen_k that differs from the metadata's without sparse_indices.
 * A width of 0 returns SMLA_SUCCESS and launches nothing.
 */
smla_status_t smla_softmax_l1norm_kwide(
    const void* q, const void* k, const float* softmax_lse,
    const int32_t* sparse_indices, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, const int32_t* seqused_q, const int32_t* seqused_k,
    const int32_t* cmp_residual_k, const int32_t* topk_length,
    const int32_t* metadata_host, int32_t dtype, int64_t batch_size, int64_t seqlen_q,
    int64_t seqlen_k, int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    int64_t topk, double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
    int64_t mask_mode, int32_t layout_q, int32_t layout_k, float* softmax_l1_norm,
    void* stream);

/*
 * smla_softmax_lse - the forward softmax_lse that smla_softmax_l1norm
 * consumes, computed on the GPU over the same used entries; enqueues one
 * kernel on `stream`.
 *
 * The article's parameter table (section 参数说明, input softmax_lse)
 * defines this input as the forward attention pass's log-sum-exp and refers
 * to the sparse_flash_mla operator for its formula, which the pages do not
 * print; this call computes the plain definition over the entries that
 * stage 1 and the mask of section 三阶段计算公式 use:
 *
 *   softmax_lse[row, g] = log sum_{t used} exp(softmax_scale * q[row,g,:] . k[key(t),:])
 *
 * in the natural base, -inf for a row with no used entry. It then holds
 * that the main call's output rows sum to 1 for every row with a used
 * entry.
 *
 * Arguments are those of smla_softmax_l1norm (same meaning, same layouts,
 * same metadata from smla_l1norm_metadata), without the softmax_lse input
 * and with softmax_lse as the output:
 *
 *   softmax_lse    fp32 out (B,N2,S1,G) | (N2,T1,G), every element written
 *
 * The work is split over the metadata's rows with this kernel's own
 * co-residency on the device's CUs (metadata field 22), or over the
 * metadata's core count (field 4) when the metadata was made with a
 * core_budget.
 *
 * Errors: as smla_softmax_l1norm (SMLA_ERR_PARAM_INVALID when q, k or
 * softmax_lse is NULL; k may be NULL when there are no keys). An empty q
 * (R == 0) returns SMLA_SUCCESS and launches nothing; with no keys
 * (T2 == 0) every row is -inf.
 */
smla_status_t smla_softmax_lse(
    const void* q, const void* k, const int32_t* sparse_indices,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* seqused_q,
    const int32_t* seqused_k, const int32_t* cmp_residual_k, const int32_t* topk_length,
    const int32_t* metadata_host, int32_t dtype, int64_t batch_size, int64_t seqlen_q,
    int64_t seqlen_k, int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    int64_t topk, double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
    int64_t mask_mode, int32_t layout_q, int32_t layout_k, float* softmax_lse,
    void* stream);

/*
 * smla_check_indices - host check of the distinct-entries precondition of
 * the main calls (parameter table, sparse_indices: the selected key blocks
 * of a row; a selection names each key once).
 *
 *   sparse_indices_host  int32 (rows, topk) in host memory
 *   topk_length_host     int32 (rows) in host memory, or NULL (then every
 *                        one of the topk entries is looked at)
 *   rows, topk           the list's shape (>= 0)
 *   first_bad_row        out, may be NULL: the first row that repeats a key,
 *                        -1 when none does
 *
 * Looks at entries t < n (n = topk_length[row] clamped to [0, topk]) with a
 * non-negative index, and fails on the first row in which two of them name
 * the same key. This is stricter than the kernels need: a repeated key that
 * lies past S2_b or that the mask hides is never used, but is flagged too.
 *
 * Errors: SMLA_ERR_PARAM_INVALID (negative sizes, or a repeated key: the
 * message names the row, the key and both entries), SMLA_ERR_PARAM_NULLPTR
 * (sparse_indices_host NULL with rows and topk > 0). Host only.
 */
smla_status_t smla_check_indices(const int32_t* sparse_indices_host,
                                 const int32_t* topk_length_host, int64_t rows, int64_t topk,
                                 int64_t* first_bad_row);

/* Elements of the output for the given shapes: B*S1*N2*S2 (BSND) or
 * T1*N2*T2 (TND); -1 for an unknown layout or a negative size. Host only. */
int64_t smla_output_numel(int32_t layout, int64_t batch_size, int64_t seqlen_q,
                          int64_t num_heads_k, int64_t seqlen_k);

/* Message for the last non-success status returned on this thread ("" if
 * none). The pointer stays valid until the next call on this thread. */
const char* smla_last_error(void);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t smla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
