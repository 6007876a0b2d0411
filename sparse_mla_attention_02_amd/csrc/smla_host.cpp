// Host side of the C ABI declared in include/smla.h: argument checks, the
// metadata work split, and the kernel launch.
//
// Argument rules follow the "SparseFlashMlaSoftmaxL1Norm" article:
// parameter table and shape notes (section 参数说明), constraints (section
// 约束说明), metadata fields (section 算子定位与配套关系) and aclnn error
// codes (section 调用方式一 aclnn API).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "smla.h"
#include "smla_internal.h"

namespace {

thread_local std::string g_last_error;

smla_status_t fail(smla_status_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

smla_status_t ok() {
    g_last_error.clear();
    return SMLA_SUCCESS;
}

// Per (device, head tiles, layout, kernel variant): CU count and
// co-resident workgroups per CU, queried once.
std::mutex g_cap_mu;
std::map<std::tuple<int, int, bool, int>, std::pair<int, int>> g_cap;

hipError_t device_capacity(int device, int ht, bool tnd, int64_t G, int64_t topk, int* cus,
                           int* per_cu) {
    const int variant = smla::kernel_variant(G, topk);
    {
        std::lock_guard<std::mutex> lk(g_cap_mu);
        auto it = g_cap.find({device, ht, tnd, variant});
        if (it != g_cap.end()) {
            *cus = it->second.first;
            *per_cu = it->second.second;
            return hipSuccess;
        }
    }
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return e;
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    int occ = 0;
    e = smla::resident_per_cu(ht, true, tnd, G, topk, &occ);
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    if (occ <= 0) return hipErrorInvalidConfiguration;
    std::lock_guard<std::mutex> lk(g_cap_mu);
    g_cap[{device, ht, tnd, variant}] = {n, occ};
    *cus = n;
    *per_cu = occ;
    return hipSuccess;
}

constexpr int32_t kVersion = 2;
constexpr int64_t kHeadDim = 512;
// Limits of the kernels' 32-bit buffer offsets: a key row is addressed as
// key * 1024 bytes from its sequence's first row, an index list as entry * 4
// bytes, an output row as column * 4 bytes (signed 32-bit range).
constexpr int64_t kMaxKeysPerSeq = int64_t(1) << 21;
constexpr int64_t kMaxTopk = int64_t(1) << 24;
constexpr int64_t kMaxWidth = 0x1FFFFFFC;

const char* kernel_name(int variant) {
    return variant == smla::kKernelNarrow ? "smla_narrow_kernel"
           : variant == smla::kKernelWide ? "smla_wide_kernel"
                                           : "smla_l1norm_kernel";
}

// SMLA_LOG=1: one line on stderr per metadata call and per launch.
bool log_on() {
    static const bool on = [] {
        const char* v = std::getenv("SMLA_LOG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}
// SMLA_CHECK_INDICES=1: the main calls copy the index lists to the host and
// reject a row whose used entries repeat a key (see smla_check_indices).
bool check_indices_on() {
    static const bool on = [] {
        const char* v = std::getenv("SMLA_CHECK_INDICES");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// Shared checks of the scalar attributes of both calls.
smla_status_t check_common(int64_t n1, int64_t n2, int64_t d, int32_t layout_q,
                           int32_t layout_k, int64_t mask_mode, int64_t cmp_ratio) {
    if (layout_q != SMLA_LAYOUT_BSND && layout_q != SMLA_LAYOUT_TND)
        return fail(SMLA_ERR_PARAM_INVALID, "layout_q must be BSND or TND");
    if (layout_k != layout_q)
        return fail(SMLA_ERR_PARAM_INVALID, "layout_q and layout_k must be equal");
    if (n2 != 1)
        return fail(SMLA_ERR_PARAM_INVALID, "num_heads_k (N2) must be 1, got %lld",
                    (long long)n2);
    if (n1 < 1 || n1 > 128)
        return fail(SMLA_ERR_PARAM_INVALID, "num_heads_q (N1) must be in [1,128], got %lld",
                    (long long)n1);
    if (n1 % n2 != 0)
        return fail(SMLA_ERR_PARAM_INVALID, "N1 must be divisible by N2");
    if (d != kHeadDim)
        return fail(SMLA_ERR_PARAM_INVALID, "head_dim (D) must be 512, got %lld",
                    (long long)d);
    if (mask_mode != SMLA_MASK_NONE && mask_mode != SMLA_MASK_RIGHT_DOWN_CAUSAL)
        return fail(SMLA_ERR_PARAM_INVALID, "mask_mode must be 0 or 3, got %lld",
                    (long long)mask_mode);
    if (cmp_ratio < 1 || cmp_ratio > 128)
        return fail(SMLA_ERR_PARAM_INVALID, "cmp_ratio must be in [1,128], got %lld",
                    (long long)cmp_ratio);
    return SMLA_SUCCESS;
}

// Checks a host prefix-sum array of B+1 entries; returns its total and max step.
smla_status_t check_cu(const int32_t* cu, int64_t B, const char* name, int64_t* total,
                       int64_t* maxlen) {
    if (cu[0] != 0) return fail(SMLA_ERR_PARAM_INVALID, "%s[0] must be 0", name);
    int64_t mx = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t step = (int64_t)cu[b + 1] - cu[b];
        if (step < 0)
            return fail(SMLA_ERR_PARAM_INVALID, "%s must be non-decreasing", name);
        if (step > mx) mx = step;
    }
    *total = cu[B];
    *maxlen = mx;
    return SMLA_SUCCESS;
}

// Rows [0, rows) of a host index list: the first row whose entries t < n
// (n = topk_length[r] clamped to [0, K], or K) repeat a non-negative key.
// Returns -1 when every row is fine; *t0/*t1 get the two entry positions.
int64_t first_repeat(const int32_t* idx, const int32_t* tlen, int64_t rows, int64_t K,
                     int64_t* t0, int64_t* t1) {
    std::vector<std::pair<int32_t, int32_t>> v;
    v.reserve((size_t)K);
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = K;
        if (tlen) n = std::min<int64_t>(std::max<int64_t>(tlen[r], 0), K);
        v.clear();
        const int32_t* row = idx + r * K;
        for (int64_t t = 0; t < n; ++t)
            if (row[t] >= 0) v.emplace_back(row[t], (int32_t)t);
        std::sort(v.begin(), v.end());
        for (size_t i = 1; i < v.size(); ++i)
            if (v[i].first == v[i - 1].first) {
                *t0 = v[i - 1].second;
                *t1 = v[i].second;
                return r;
            }
    }
    return -1;
}

}  // namespace

extern "C" {

int32_t smla_version(void) { return 10000 * 0 + 100 * 2 + 0; }

smla_status_t smla_check_indices(const int32_t* sparse_indices_host,
                                 const int32_t* topk_length_host, int64_t rows, int64_t topk,
                                 int64_t* first_bad_row) {
    if (first_bad_row) *first_bad_row = -1;
    if (rows < 0 || topk < 0) return fail(SMLA_ERR_PARAM_INVALID, "rows and topk must be >= 0");
    if (rows == 0 || topk == 0) return ok();
    if (!sparse_indices_host) return fail(SMLA_ERR_PARAM_NULLPTR, "sparse_indices_host is NULL");
    int64_t t0 = 0, t1 = 0;
    const int64_t r = first_repeat(sparse_indices_host, topk_length_host, rows, topk, &t0, &t1);
    if (r >= 0) {
        if (first_bad_row) *first_bad_row = r;
        return fail(SMLA_ERR_PARAM_INVALID,
                    "row %lld repeats key %d at entries %lld and %lld (used entries of a row "
                    "must be distinct)", (long long)r, sparse_indices_host[r * topk + t0],
                    (long long)t0, (long long)t1);
    }
    return ok();
}

const char* smla_last_error(void) { return g_last_error.c_str(); }

int64_t smla_output_numel(int32_t layout, int64_t batch_size, int64_t seqlen_q,
                          int64_t num_heads_k, int64_t seqlen_k) {
    if (batch_size < 0 || seqlen_q < 0 || num_heads_k < 0 || seqlen_k < 0) return -1;
    if (layout == SMLA_LAYOUT_BSND) return batch_size * seqlen_q * num_heads_k * seqlen_k;
    if (layout == SMLA_LAYOUT_TND) return seqlen_q * num_heads_k * seqlen_k;
    return -1;
}

smla_status_t smla_l1norm_metadata(
    int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
    const int32_t* seqused_q_host, const int32_t* seqused_k_host,
    const int32_t* cmp_residual_k_host, const int32_t* topk_length_host,
    int64_t batch_size, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t topk,
    int32_t layout_q, int32_t layout_k, int64_t mask_mode, int64_t cmp_ratio,
    int32_t device, int32_t core_budget, int32_t* metadata_host) {
    // (the split is by rows; these refine nothing here)
    (void)cmp_residual_k_host;
    (void)topk_length_host;
    (void)seqused_q_host;
    (void)seqused_k_host;
    if (!metadata_host) return fail(SMLA_ERR_PARAM_NULLPTR, "metadata_host is NULL");
    smla_status_t st = check_common(num_heads_q, num_heads_k, head_dim, layout_q, layout_k,
                                    mask_mode, cmp_ratio);
    if (st != SMLA_SUCCESS) return st;
    // topk == 0: the dense case (no sparse_indices)
    if (topk < 0) return fail(SMLA_ERR_PARAM_INVALID, "topk must be >= 0");
    if (core_budget < 0) return fail(SMLA_ERR_PARAM_INVALID, "core_budget must be >= 0");

    int64_t B = batch_size, R = 0, rows_k = 0, mq = max_seqlen_q, mk = max_seqlen_k;
    if (layout_q == SMLA_LAYOUT_BSND) {
        if (batch_size <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0)
            return fail(SMLA_ERR_PARAM_INVALID,
                        "BSND needs batch_size, max_seqlen_q and max_seqlen_k > 0");
        R = batch_size * max_seqlen_q;
        rows_k = batch_size * max_seqlen_k;
    } else {
        if (!cu_seqlens_q_host || !cu_seqlens_k_host)
            return fail(SMLA_ERR_PARAM_NULLPTR, "TND needs cu_seqlens_q and cu_seqlens_k");
        if (batch_size <= 0)
            return fail(SMLA_ERR_PARAM_INVALID,
                        "TND needs batch_size = len(cu_seqlens_q) - 1 > 0");
        int64_t tq, tk, mxq, mxk;
        if ((st = check_cu(cu_seqlens_q_host, B, "cu_seqlens_q", &tq, &mxq)) != SMLA_SUCCESS)
            return st;
        if ((st = check_cu(cu_seqlens_k_host, B, "cu_seqlens_k", &tk, &mxk)) != SMLA_SUCCESS)
            return st;
        if (max_seqlen_q < 0 || max_seqlen_k < 0)
            return fail(SMLA_ERR_PARAM_INVALID, "max_seqlen_q/k must be >= 0");
        if (mq == 0) mq = mxq;
        if (mk == 0) mk = mxk;
        if (mk < mxk)
            return fail(SMLA_ERR_PARAM_INVALID,
                        "max_seqlen_k is smaller than the longest cu_seqlens_k sequence");
        R = tq;
        rows_k = tk;
    }
    if (R > INT32_MAX || rows_k > INT32_MAX || B > INT32_MAX)
        return fail(SMLA_ERR_PARAM_INVALID, "sizes exceed the int32 metadata fields");
    // the longest key sequence (BSND: S2; TND: the longest cu_seqlens_k step)
    int64_t longest_k = mk;
    if (layout_q == SMLA_LAYOUT_TND) {
        int64_t tk, mxk;
        (void)check_cu(cu_seqlens_k_host, B, "cu_seqlens_k", &tk, &mxk);
        longest_k = mxk;
    }
    if (longest_k > kMaxKeysPerSeq)
        return fail(SMLA_ERR_UNSUPPORTED,
                    "a key sequence of %lld rows exceeds the supported %lld (32-bit key "
                    "offsets)", (long long)longest_k, (long long)kMaxKeysPerSeq);
    if (topk > kMaxTopk)
        return fail(SMLA_ERR_UNSUPPORTED, "topk %lld exceeds the supported %lld",
                    (long long)topk, (long long)kMaxTopk);
    if (rows_k > kMaxWidth)
        return fail(SMLA_ERR_UNSUPPORTED,
                    "%lld key rows (the output row width) exceed the supported %lld "
                    "(32-bit output offsets)", (long long)rows_k, (long long)kMaxWidth);

    const int ht = smla::head_tiles_for(num_heads_q / num_heads_k);
    int cus = 0, per_cu = 0;
    int64_t budget = core_budget;
    if (core_budget == 0) {
        hipError_t e = device_capacity(device, ht, layout_q == SMLA_LAYOUT_TND,
                                       num_heads_q / num_heads_k, topk, &cus, &per_cu);
        if (e != hipSuccess)
            return fail(SMLA_ERR_RUNTIME, "device %d capacity query failed: %s", device,
                        hipGetErrorString(e));
        budget = (int64_t)cus * per_cu;
    }

    const int64_t total = R * num_heads_k;
    const int64_t cores = total < budget ? total : budget;
    int32_t* m = metadata_host;
    std::memset(m, 0, sizeof(int32_t) * SMLA_METADATA_SIZE);
    m[0] = (int32_t)total;
    if (cores > 0) {
        const int64_t q = total / cores, rem = total % cores;
        m[1] = (int32_t)(rem ? q + 1 : q);
        m[2] = (int32_t)q;
        m[3] = (int32_t)(rem ? cores - rem : 0);
    }
    m[4] = (int32_t)cores;
    m[5] = SMLA_META_MAGIC;
    m[6] = kVersion;
    m[7] = layout_q;
    m[8] = (int32_t)num_heads_q;
    m[9] = (int32_t)num_heads_k;
    m[10] = (int32_t)head_dim;
    m[11] = (int32_t)B;
    m[12] = (int32_t)mq;
    m[13] = (int32_t)mk;
    m[14] = (int32_t)topk;
    m[15] = (int32_t)mask_mode;
    m[16] = (int32_t)cmp_ratio;
    m[17] = (int32_t)R;
    m[18] = (int32_t)rows_k;
    m[19] = 1;  // snake row order
    m[20] = ht;
    m[21] = device;
    m[22] = cus;
    m[23] = per_cu;
    m[24] = smla::kernel_variant(num_heads_q / num_heads_k, topk);  // kernel variant
    m[25] = (int32_t)longest_k;
    if (log_on())
        std::fprintf(stderr,
                     "smla: metadata layout=%s R=%lld N1=%lld K=%lld mask=%lld cmp=%lld "
                     "rows_k=%lld longest_k=%lld cores=%d rows/core=%d/%d tail=%d "
                     "kernel=%s cus=%d per_cu=%d\n",
                     layout_q == SMLA_LAYOUT_TND ? "TND" : "BSND", (long long)R,
                     (long long)num_heads_q, (long long)topk, (long long)mask_mode,
                     (long long)cmp_ratio, (long long)rows_k, (long long)longest_k, m[4],
                     m[1], m[2], m[3], kernel_name(m[24]), cus, per_cu);
    return ok();
}

}  // extern "C"

namespace {

// Checks shared by the main call (softmax_lse in, softmax_l1_norm out; kwide:
// the K-wide output) and the lse call (lse_in NULL, out = softmax_lse), then
// the kernel arguments. *nothing_to_do is set when there are no rows (the
// page: an empty q returns directly) or, for the main call, an empty output
// row.
smla_status_t prepare(const void* q, const void* k, const int32_t* sparse_indices,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      const int32_t* seqused_q, const int32_t* seqused_k,
                      const int32_t* cmp_residual_k, const int32_t* topk_length,
                      const int32_t* metadata_host, int32_t dtype, int64_t batch_size,
                      int64_t seqlen_q, int64_t seqlen_k, int64_t num_heads_q,
                      int64_t num_heads_k, int64_t head_dim, int64_t topk,
                      double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
                      int64_t mask_mode, int32_t layout_q, int32_t layout_k, bool lse_call,
                      bool kwide, const float* lse_in, float* out,
                      smla::KernelArgs* out_args, bool* nothing_to_do) {
    *nothing_to_do = false;
    if (dtype != SMLA_DTYPE_FP16 && dtype != SMLA_DTYPE_BF16)
        return fail(SMLA_ERR_PARAM_INVALID, "dtype must be FLOAT16 or BFLOAT16");
    smla_status_t st = check_common(num_heads_q, num_heads_k, head_dim, layout_q, layout_k,
                                    mask_mode, cmp_ratio);
    if (st != SMLA_SUCCESS) return st;
    if (max_seqlen_k < 0) return fail(SMLA_ERR_PARAM_INVALID, "max_seqlen_k must be >= 0");
    if (batch_size < 0 || seqlen_q < 0 || seqlen_k < 0)
        return fail(SMLA_ERR_PARAM_INVALID, "sizes must be >= 0");
    const bool tnd = layout_q == SMLA_LAYOUT_TND;
    if (tnd && batch_size < 1)
        return fail(SMLA_ERR_PARAM_INVALID, "TND needs batch_size >= 1");

    const int64_t R = tnd ? seqlen_q : batch_size * seqlen_q;
    const int64_t rows_k = tnd ? seqlen_k : batch_size * seqlen_k;
    const bool dense = !sparse_indices;
    // output row width: S2 / T2, or K-wide (the shape-inference section) K,
    // without sparse_indices S2 (BSND) or max_seqlen_k (TND)
    const int64_t W = !kwide ? seqlen_k : (!dense ? topk : (tnd ? max_seqlen_k : seqlen_k));
    // empty q (both calls) or empty output row (main call): nothing is read
    // or written. Without keys every lse row is -inf, which the lse call
    // still writes.
    if (R == 0 || (!lse_call && W == 0)) {
        *nothing_to_do = true;
        return SMLA_SUCCESS;
    }

    if (lse_call && (!q || (!k && rows_k > 0) || !out))
        return fail(SMLA_ERR_PARAM_INVALID, "q, k and softmax_lse (output) are required");
    if (!lse_call && (!q || !k || !lse_in || !out))
        return fail(SMLA_ERR_PARAM_INVALID,
                    "q, k, softmax_lse and softmax_l1_norm are required");
    // no sparse_indices: the dense case, every key of the row's batch or
    // sequence (stage 1 of the page's formula selects the whole K); topk
    // is then 0 and topk_length does not apply
    if (dense && topk != 0)
        return fail(SMLA_ERR_PARAM_INVALID, "topk must be 0 without sparse_indices");
    if (!dense && topk < 1)
        return fail(SMLA_ERR_PARAM_INVALID, "topk must be >= 1 with sparse_indices");
    if (!metadata_host)
        return fail(SMLA_ERR_PARAM_NULLPTR,
                    "metadata is required (from smla_l1norm_metadata)");
    if (tnd && (!cu_seqlens_q || !cu_seqlens_k))
        return fail(SMLA_ERR_PARAM_NULLPTR, "TND needs cu_seqlens_q and cu_seqlens_k");
    if (mask_mode == SMLA_MASK_RIGHT_DOWN_CAUSAL && cmp_ratio != 1 && !cmp_residual_k)
        return fail(SMLA_ERR_PARAM_NULLPTR,
                    "cmp_residual_k is required when mask_mode == 3 and cmp_ratio != 1");
    if (!dense && mask_mode == SMLA_MASK_NONE && !topk_length)
        return fail(SMLA_ERR_PARAM_NULLPTR,
                    "topk_length is required when mask_mode == 0 with sparse_indices");
    if (R > INT32_MAX || rows_k > INT32_MAX || topk > INT32_MAX)
        return fail(SMLA_ERR_PARAM_INVALID, "sizes exceed the supported range");
    if (topk > kMaxTopk)
        return fail(SMLA_ERR_UNSUPPORTED, "topk %lld exceeds the supported %lld",
                    (long long)topk, (long long)kMaxTopk);
    if (W > kMaxWidth)
        return fail(SMLA_ERR_UNSUPPORTED,
                    "output rows of %lld columns exceed the supported %lld (32-bit output "
                    "offsets)", (long long)W, (long long)kMaxWidth);

    const int32_t* m = metadata_host;
    if (m[5] != SMLA_META_MAGIC || m[6] != kVersion)
        return fail(SMLA_ERR_PARAM_INVALID, "metadata was not made by smla_l1norm_metadata");
    if (m[7] != layout_q || m[8] != num_heads_q || m[9] != num_heads_k ||
        m[10] != head_dim || m[11] != batch_size || m[14] != topk ||
        m[15] != mask_mode || m[16] != cmp_ratio || m[17] != R || m[18] != rows_k ||
        m[0] != R * num_heads_k)
        return fail(SMLA_ERR_PARAM_INVALID, "metadata does not match the call's shapes");
    if (!tnd && (m[12] != seqlen_q || m[13] != seqlen_k))
        return fail(SMLA_ERR_PARAM_INVALID, "metadata does not match S1/S2");
    if (kwide && dense && tnd && m[13] != max_seqlen_k)
        return fail(SMLA_ERR_PARAM_INVALID,
                    "K-wide TND output without sparse_indices: max_seqlen_k must be the "
                    "metadata's max_seqlen_k");
    if (m[4] < 1 || m[4] > m[0])
        return fail(SMLA_ERR_PARAM_INVALID, "metadata core count is out of range");
    if (m[25] < 0 || m[25] > kMaxKeysPerSeq || (!tnd && m[25] != seqlen_k))
        return fail(SMLA_ERR_PARAM_INVALID, "metadata longest key sequence is out of range");

    smla::KernelArgs& a = *out_args;
    a = smla::KernelArgs{};
    a.q = q;
    a.k = k;
    a.lse = lse_in;
    a.out = out;
    a.idx = sparse_indices;
    a.topk_len = dense ? nullptr : topk_length;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.cmp_res = cmp_residual_k;
    a.su_q = seqused_q;
    a.su_k = seqused_k;
    a.kwide = kwide ? 1 : 0;
    a.R = R;
    a.W = W;
    a.rows_k = rows_k;
    a.B = (int32_t)batch_size;
    a.S1 = tnd ? 0 : (int32_t)seqlen_q;
    a.S2 = tnd ? 0 : (int32_t)seqlen_k;
    a.G = (int32_t)(num_heads_q / num_heads_k);
    // dense: entries per row at most the longest key sequence (S2, or the
    // maximum of cu_seqlens_k as the metadata call resolved it)
    a.K = dense ? (tnd ? m[13] : (int32_t)seqlen_k) : (int32_t)topk;
    a.dense = dense ? 1 : 0;
    a.mask_mode = (int32_t)mask_mode;
    a.cmp_ratio = (int32_t)cmp_ratio;
    const float scale32 = (float)softmax_scale;  // the attribute is FLOAT32
    a.c_scale = scale32 * 1.4426950408889634f;
    a.inv_g = 1.0f / (float)a.G;
    a.num_wg = m[4];
    a.snake = m[19];
    return SMLA_SUCCESS;
}

// SMLA_CHECK_INDICES: copies the index lists (and topk_length) of a main
// call to the host on its stream, waits, and checks them.
smla_status_t check_device_indices(const smla::KernelArgs& a, hipStream_t stream) {
    if (a.dense || !a.idx) return SMLA_SUCCESS;
    std::vector<int32_t> idx((size_t)(a.R * a.K)), tl;
    hipError_t e = hipMemcpyAsync(idx.data(), a.idx, idx.size() * 4, hipMemcpyDeviceToHost,
                                  stream);
    if (e == hipSuccess && a.topk_len) {
        tl.resize((size_t)a.R);
        e = hipMemcpyAsync(tl.data(), a.topk_len, tl.size() * 4, hipMemcpyDeviceToHost,
                           stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(SMLA_ERR_RUNTIME, "index check copy failed: %s", hipGetErrorString(e));
    int64_t t0 = 0, t1 = 0;
    const int64_t r = first_repeat(idx.data(), a.topk_len ? tl.data() : nullptr, a.R, a.K,
                                   &t0, &t1);
    if (r >= 0)
        return fail(SMLA_ERR_PARAM_INVALID,
                    "row %lld repeats key %d at entries %lld and %lld (used entries of a row "
                    "must be distinct)", (long long)r, idx[(size_t)(r * a.K + t0)],
                    (long long)t0, (long long)t1);
    return SMLA_SUCCESS;
}

void log_launch(const char* call, const smla::KernelArgs& a, int ht, int32_t dtype,
                const char* kernel, int32_t grid, int32_t block, void* stream) {
    if (!log_on()) return;
    std::fprintf(stderr,
                 "smla: %s kernel=%s grid=%d block=%d R=%lld W=%lld G=%d K=%d head_tiles=%d "
                 "dtype=%s dense=%d kwide=%d mask=%d cmp=%d stream=%p\n",
                 call, kernel, grid, block, (long long)a.R, (long long)a.W, a.G, a.K, ht,
                 dtype == SMLA_DTYPE_BF16 ? "bf16" : "fp16", a.dense, a.kwide, a.mask_mode,
                 a.cmp_ratio, stream);
}

// Enqueues the main kernel for prepared arguments (both main calls).
smla_status_t run_main(const char* call, const smla::KernelArgs& a, int32_t dtype,
                       int32_t layout_q, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (check_indices_on()) {
        smla_status_t st = check_device_indices(a, s);
        if (st != SMLA_SUCCESS) return st;
    }
    const int ht = smla::head_tiles_for(a.G);
    const int variant = smla::kernel_variant(a.G, a.dense ? 0 : a.K);
    log_launch(call, a, ht, dtype, kernel_name(variant), a.num_wg,
               variant == smla::kKernelGeneral ? 64 * ht : 256, stream);
    hipError_t e = smla::launch(a, ht, dtype == SMLA_DTYPE_BF16, layout_q == SMLA_LAYOUT_TND,
                                s);
    if (e != hipSuccess)
        return fail(SMLA_ERR_RUNTIME, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Co-resident workgroups per CU of the lse kernel, queried once per variant.
std::mutex g_lse_occ_mu;
std::map<std::tuple<int, bool, bool, int>, int> g_lse_occ;  // (ht, bf16, tnd, variant)

hipError_t lse_capacity(int ht, bool bf16, bool tnd, int64_t G, int64_t topk, int* per_cu) {
    std::lock_guard<std::mutex> lk(g_lse_occ_mu);
    const int var = smla::lse_variant(G, topk);
    auto it = g_lse_occ.find({ht, bf16, tnd, var});
    if (it != g_lse_occ.end()) {
        *per_cu = it->second;
        return hipSuccess;
    }
    int occ = 0;
    hipError_t e = smla::lse_resident_per_cu(ht, bf16, tnd, G, topk, &occ);
    if (e != hipSuccess) return e;
    if (occ <= 0) return hipErrorInvalidConfiguration;
    g_lse_occ[{ht, bf16, tnd, var}] = occ;
    *per_cu = occ;
    return hipSuccess;
}

}  // namespace

extern "C" {

smla_status_t smla_softmax_l1norm(
    const void* q, const void* k, const float* softmax_lse,
    const int32_t* sparse_indices, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, const int32_t* seqused_q, const int32_t* seqused_k,
    const int32_t* cmp_residual_k, const int32_t* topk_length,
    const int32_t* metadata_host, int32_t dtype, int64_t batch_size, int64_t seqlen_q,
    int64_t seqlen_k, int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    int64_t topk, double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
    int64_t mask_mode, int32_t layout_q, int32_t layout_k, float* softmax_l1_norm,
    void* stream) {
    smla::KernelArgs a;
    bool nothing = false;
    smla_status_t st = prepare(q, k, sparse_indices, cu_seqlens_q, cu_seqlens_k, seqused_q,
                               seqused_k, cmp_residual_k, topk_length, metadata_host, dtype,
                               batch_size, seqlen_q, seqlen_k, num_heads_q, num_heads_k,
                               head_dim, topk, softmax_scale, max_seqlen_k, cmp_ratio,
                               mask_mode, layout_q, layout_k, false, false, softmax_lse,
                               softmax_l1_norm, &a, &nothing);
    if (st != SMLA_SUCCESS) return st;
    if (nothing) return ok();
    return run_main("smla_softmax_l1norm", a, dtype, layout_q, stream);
}

smla_status_t smla_softmax_l1norm_kwide(
    const void* q, const void* k, const float* softmax_lse,
    const int32_t* sparse_indices, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, const int32_t* seqused_q, const int32_t* seqused_k,
    const int32_t* cmp_residual_k, const int32_t* topk_length,
    const int32_t* metadata_host, int32_t dtype, int64_t batch_size, int64_t seqlen_q,
    int64_t seqlen_k, int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    int64_t topk, double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
    int64_t mask_mode, int32_t layout_q, int32_t layout_k, float* softmax_l1_norm,
    void* stream) {
    smla::KernelArgs a;
    bool nothing = false;
    smla_status_t st = prepare(q, k, sparse_indices, cu_seqlens_q, cu_seqlens_k, seqused_q,
                               seqused_k, cmp_residual_k, topk_length, metadata_host, dtype,
                               batch_size, seqlen_q, seqlen_k, num_heads_q, num_heads_k,
                               head_dim, topk, softmax_scale, max_seqlen_k, cmp_ratio,
                               mask_mode, layout_q, layout_k, false, true, softmax_lse,
                               softmax_l1_norm, &a, &nothing);
    if (st != SMLA_SUCCESS) return st;
    if (nothing) return ok();
    return run_main("smla_softmax_l1norm_kwide", a, dtype, layout_q, stream);
}

smla_status_t smla_softmax_lse(
    const void* q, const void* k, const int32_t* sparse_indices,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* seqused_q,
    const int32_t* seqused_k, const int32_t* cmp_residual_k, const int32_t* topk_length,
    const int32_t* metadata_host, int32_t dtype, int64_t batch_size, int64_t seqlen_q,
    int64_t seqlen_k, int64_t num_heads_q, int64_t num_heads_k, int64_t head_dim,
    int64_t topk, double softmax_scale, int64_t max_seqlen_k, int64_t cmp_ratio,
    int64_t mask_mode, int32_t layout_q, int32_t layout_k, float* softmax_lse,
    void* stream) {
    smla::KernelArgs a;
    bool nothing = false;
    smla_status_t st = prepare(q, k, sparse_indices, cu_seqlens_q, cu_seqlens_k, seqused_q,
                               seqused_k, cmp_residual_k, topk_length, metadata_host, dtype,
                               batch_size, seqlen_q, seqlen_k, num_heads_q, num_heads_k,
                               head_dim, topk, softmax_scale, max_seqlen_k, cmp_ratio,
                               mask_mode, layout_q, layout_k, true, false, nullptr,
                               softmax_lse, &a, &nothing);
    if (st != SMLA_SUCCESS) return st;
    if (nothing) return ok();
    const int ht = smla::head_tiles_for(a.G);
    const bool bf16 = dtype == SMLA_DTYPE_BF16, tnd = layout_q == SMLA_LAYOUT_TND;
    // the metadata's split was sized for the main call's kernel; this kernel
    // has its own co-residency on the same CUs (field 22). With a caller's
    // core budget (field 22 is 0) the metadata's core count stands.
    const int32_t* m = metadata_host;
    if (m[22] > 0) {
        int per_cu = 0;
        hipError_t e = lse_capacity(ht, bf16, tnd, a.G, a.dense ? 0 : a.K, &per_cu);
        if (e != hipSuccess)
            return fail(SMLA_ERR_RUNTIME, "occupancy query failed: %s", hipGetErrorString(e));
        const int64_t cap = (int64_t)m[22] * per_cu;
        a.num_wg = (int32_t)(a.R < cap ? a.R : cap);
    }
    const int var = smla::lse_variant(a.G, a.dense ? 0 : a.K);
    log_launch("smla_softmax_lse", a, ht, dtype,
               var == smla::kLseNarrow ? "smla_lse_narrow_kernel"
               : var == smla::kLseWide ? "smla_lse_wide_kernel" : "smla_lse_kernel",
               a.num_wg, var != smla::kLseGeneral ? 256 : 64 * (ht == 4 ? 2 : ht), stream);
    hipError_t e = smla::launch_lse(a, ht, bf16, tnd, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SMLA_ERR_RUNTIME, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
