// A complete host program on the C ABI: the call sequence of the
// "SparseFlashMlaSoftmaxL1Norm" article's aclnn example (section 调用方式一
// aclnn API: set the device, create a stream, create the tensors, run the
// metadata pre-operator, run the operator, synchronise, copy the result
// back, release everything), written for HIP.
//
// The forward softmax_lse the operator consumes comes from the library's
// own smla_softmax_lse call, so every row with a used entry must sum to 1
// (section 三阶段计算公式: the output is the head mean of probability rows).
// The program checks that, checks that non-zeros sit only at selected
// columns, and exits with status 0 when both hold.
//
// Shapes: BSND, B = 1, S1 = 96, S2 = 320, N1 = 64 (G = 64), N2 = 1, D = 512,
// topk = 160, right-down causal mask; bf16 q and k.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "smla.h"

#define HIP_OK(x)                                                                    \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));      \
            return 2;                                                                \
        }                                                                            \
    } while (0)
#define SMLA_OK(x)                                                                   \
    do {                                                                             \
        smla_status_t s_ = (x);                                                      \
        if (s_ != SMLA_SUCCESS) {                                                    \
            std::fprintf(stderr, "%s failed: %d %s\n", #x, s_, smla_last_error());   \
            return 3;                                                                \
        }                                                                            \
    } while (0)

namespace {

// Deterministic values in [-1, 1) from a 64-bit linear congruential generator.
struct Lcg {
    uint64_t s;
    float next() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (float)((s >> 40) & 0xffffff) / 8388608.0f - 1.0f;
    }
};

// fp32 -> bf16 bits, round to nearest even (finite inputs).
uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fff + ((u >> 16) & 1);
    return (uint16_t)(u >> 16);
}

}  // namespace

int main() {
    const int64_t B = 1, S1 = 96, S2 = 320, N1 = 64, N2 = 1, D = 512, K = 160;
    const int64_t mask_mode = SMLA_MASK_RIGHT_DOWN_CAUSAL, cmp_ratio = 1;
    const double scale = 1.0 / std::sqrt((double)D);

    // 1. device and stream
    HIP_OK(hipSetDevice(0));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    // 2. host inputs: q, k and, per row, distinct visible keys (key j is
    // visible to query i iff j <= i + S2 - S1), -1 padded
    Lcg g{12345};
    std::vector<uint16_t> q((size_t)(B * S1 * N1 * D)), k((size_t)(B * S2 * N2 * D));
    for (auto& v : q) v = to_bf16(g.next());
    for (auto& v : k) v = to_bf16(g.next());
    std::vector<int32_t> idx((size_t)(B * S1 * N2 * K), -1), tlen((size_t)(B * S1 * N2));
    for (int64_t i = 0; i < S1; ++i) {
        const int64_t vis = std::min<int64_t>(S2, i + 1 + S2 - S1);
        const int64_t n = std::min<int64_t>(K, vis);
        // every second visible key from the newest one back, then the rest
        int64_t t = 0;
        for (int64_t j = vis - 1; j >= 0 && t < n; j -= 2) idx[(size_t)(i * K + t++)] = (int32_t)j;
        for (int64_t j = vis - 2; j >= 0 && t < n; j -= 2) idx[(size_t)(i * K + t++)] = (int32_t)j;
        tlen[(size_t)i] = (int32_t)n;
    }
    SMLA_OK(smla_check_indices(idx.data(), tlen.data(), B * S1 * N2, K, nullptr));

    // 3. device tensors
    void *dq, *dk;
    int32_t *didx, *dtlen;
    float *dlse, *dout;
    const int64_t out_numel = smla_output_numel(SMLA_LAYOUT_BSND, B, S1, N2, S2);
    HIP_OK(hipMalloc(&dq, q.size() * 2));
    HIP_OK(hipMalloc(&dk, k.size() * 2));
    HIP_OK(hipMalloc(&didx, idx.size() * 4));
    HIP_OK(hipMalloc(&dtlen, tlen.size() * 4));
    HIP_OK(hipMalloc(&dlse, (size_t)(B * N2 * S1 * N1) * 4));
    HIP_OK(hipMalloc(&dout, (size_t)out_numel * 4));
    HIP_OK(hipMemcpy(dq, q.data(), q.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, k.data(), k.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(didx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dtlen, tlen.data(), tlen.size() * 4, hipMemcpyHostToDevice));

    // 4. the metadata pre-operator (host), then the forward lse and the
    // operator on the stream
    int32_t meta[SMLA_METADATA_SIZE];
    SMLA_OK(smla_l1norm_metadata(N1, N2, D, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 tlen.data(), B, S1, S2, K, SMLA_LAYOUT_BSND, SMLA_LAYOUT_BSND,
                                 mask_mode, cmp_ratio, 0, 0, meta));
    SMLA_OK(smla_softmax_lse(dq, dk, didx, nullptr, nullptr, nullptr, nullptr, nullptr, dtlen,
                             meta, SMLA_DTYPE_BF16, B, S1, S2, N1, N2, D, K, scale, 0,
                             cmp_ratio, mask_mode, SMLA_LAYOUT_BSND, SMLA_LAYOUT_BSND, dlse,
                             stream));
    SMLA_OK(smla_softmax_l1norm(dq, dk, dlse, didx, nullptr, nullptr, nullptr, nullptr, nullptr,
                                dtlen, meta, SMLA_DTYPE_BF16, B, S1, S2, N1, N2, D, K, scale, 0,
                                cmp_ratio, mask_mode, SMLA_LAYOUT_BSND, SMLA_LAYOUT_BSND, dout,
                                stream));

    // 5. synchronise and copy back
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<float> out((size_t)out_numel);
    HIP_OK(hipMemcpy(out.data(), dout, out.size() * 4, hipMemcpyDeviceToHost));

    // 6. checks: row sums and support
    double worst = 0.0;
    int64_t off_support = 0;
    for (int64_t i = 0; i < S1; ++i) {
        std::vector<char> sel((size_t)S2, 0);
        for (int64_t t = 0; t < tlen[(size_t)i]; ++t) sel[(size_t)idx[(size_t)(i * K + t)]] = 1;
        double sum = 0.0;
        for (int64_t c = 0; c < S2; ++c) {
            const float v = out[(size_t)(i * S2 + c)];
            sum += v;
            if (v != 0.0f && !sel[(size_t)c]) ++off_support;
        }
        if (tlen[(size_t)i] > 0) worst = std::max(worst, std::fabs(sum - 1.0));
    }

    // 7. release
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(didx));
    HIP_OK(hipFree(dtlen));
    HIP_OK(hipFree(dlse));
    HIP_OK(hipFree(dout));
    HIP_OK(hipStreamDestroy(stream));

    std::printf("smla_example: %lld rows, workgroups %d, max |row sum - 1| = %.3e, "
                "values off the selected columns = %lld\n",
                (long long)S1, meta[4], worst, (long long)off_support);
    if (worst > 1e-4 || off_support != 0) {
        std::printf("smla_example: FAILED\n");
        return 1;
    }
    std::printf("smla_example: OK\n");
    return 0;
}
