// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

// Everything a kernel launch needs, passed by value as the kernel argument.
struct KernelArgs {
    const void* q;            // (R, G, 512) bf16/fp16, N2 == 1 so N1 == G
    const void* k;            // (rows_k, 512) bf16/fp16
    const float* lse;         // (R, G) fp32
    const int32_t* idx;       // (R, K) int32; NULL when dense
    const int32_t* topk_len;  // (R) or nullptr
    const int32_t* cu_q;      // (B+1) for TND
    const int32_t* cu_k;      // (B+1) for TND
    const int32_t* cmp_res;   // (B) or nullptr
    const int32_t* su_q;      // seqused_q (B) or nullptr
    const int32_t* su_k;      // seqused_k (B) or nullptr
    float* out;               // (R, W) fp32; the lse kernel: (R, G) fp32 softmax_lse
    int64_t R;                // query rows
    int64_t W;                // output row width (S2 or T2; K-wide: the entry count)
    int64_t rows_k;           // rows of k (B*S2 or T2)
    int32_t B;                // batches or sequences
    int32_t S1, S2;           // BSND per-batch lengths
    int32_t G;                // query heads per kv head
    int32_t K;                // indices per row
    int32_t mask_mode;        // 0 or 3
    int32_t cmp_ratio;        // [1, 128]
    float c_scale;            // softmax_scale * log2(e)
    float inv_g;              // 1 / G
    int32_t num_wg;           // workgroups launched (metadata field 4)
    int32_t snake;            // row order: 1 = snake, 0 = plain strided
    int32_t dense;            // 1: no sparse_indices, entry t of a row is key t (idx NULL)
    int32_t kwide;            // 1: entry t's value goes to column t of a W = K wide row
};

// Head tiles of 32 heads each that one row needs: 1, 2 or 4.
inline int head_tiles_for(int64_t G) { return G <= 32 ? 1 : (G <= 64 ? 2 : 4); }

// Enqueue the kernel variant for (head_tiles, bf16, tnd).
hipError_t launch(const KernelArgs& a, int head_tiles, bool bf16, bool tnd,
                  hipStream_t stream);

// The main call's kernels (metadata field 24): the general kernel (one wave
// per 32-head tile), the pipelined kernel for 65..128 heads (64 heads per
// wave, 64-key tiles, index list in LDS), the pipelined kernel for up to 64
// heads (every head per wave, 16 keys per wave).
enum { kKernelGeneral = 0, kKernelWide = 1, kKernelNarrow = 2 };

// The kernel that runs rows of G heads with `topk` indices (0: dense).
int kernel_variant(int64_t G, int64_t topk);

// Co-resident workgroups per CU of the kernel used for (G, topk).
hipError_t resident_per_cu(int head_tiles, bool bf16, bool tnd, int64_t G, int64_t topk,
                           int* out);

// Most indices per row that the pipelined kernel for 65..128 heads takes (its
// index list sits in LDS); longer rows take the general kernel.
constexpr int kWideIndexCap = 2048;

// The three kernels of the main call, one source file each.
hipError_t launch_general(const KernelArgs& a, int head_tiles, bool bf16, bool tnd,
                          hipStream_t stream);
hipError_t general_resident_per_cu(int head_tiles, bool bf16, bool tnd, int* out);
hipError_t launch_wide(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream);
hipError_t wide_resident_per_cu(bool bf16, bool tnd, int* out);
hipError_t launch_narrow(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream);
hipError_t narrow_resident_per_cu(bool bf16, bool tnd, int* out);

// The forward softmax_lse call: a.out receives (R, G) fp32. Rows of up to 64
// heads take the pipelined small-head kernel (any K), rows of 65..128 heads
// with at most kWideIndexCap indices (or dense rows) the pipelined kernel for
// 65..128 heads, other shapes the general one.
enum { kLseGeneral = 0, kLseWide = 1, kLseNarrow = 2 };
inline int lse_variant(int64_t G, int64_t topk) {
    return G <= 64 ? kLseNarrow : (topk <= kWideIndexCap ? kLseWide : kLseGeneral);
}
hipError_t launch_lse(const KernelArgs& a, int head_tiles, bool bf16, bool tnd,
                      hipStream_t stream);
hipError_t launch_lse_wide(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream);
hipError_t launch_lse_narrow(const KernelArgs& a, bool bf16, bool tnd, hipStream_t stream);

// Co-resident workgroups per CU of the lse kernel used for (G, topk).
hipError_t lse_resident_per_cu(int head_tiles, bool bf16, bool tnd, int64_t G, int64_t topk,
                               int* out);
hipError_t lse_wide_resident_per_cu(bool bf16, bool tnd, int* out);
hipError_t lse_narrow_resident_per_cu(bool bf16, bool tnd, int* out);

}  // namespace smla
