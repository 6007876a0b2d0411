// Choice of the main call's kernel for a shape, and its launch.
#include "smla_internal.h"

namespace smla {

int kernel_variant(int64_t G, int64_t topk) {
    // (the dense case, topk 0, has no index list: no limit on its entries)
    if (G <= 64) return kKernelNarrow;
    return topk <= kWideIndexCap ? kKernelWide : kKernelGeneral;
}

hipError_t launch(const KernelArgs& a, int ht, bool bf16, bool tnd, hipStream_t stream) {
    switch (kernel_variant(a.G, a.dense ? 0 : a.K)) {
        case kKernelNarrow: return launch_narrow(a, bf16, tnd, stream);
        case kKernelWide: return launch_wide(a, bf16, tnd, stream);
        default: return launch_general(a, ht, bf16, tnd, stream);
    }
}

hipError_t resident_per_cu(int ht, bool bf16, bool tnd, int64_t G, int64_t topk, int* out) {
    switch (kernel_variant(G, topk)) {
        case kKernelNarrow: return narrow_resident_per_cu(bf16, tnd, out);
        case kKernelWide: return wide_resident_per_cu(bf16, tnd, out);
        default: return general_resident_per_cu(ht, bf16, tnd, out);
    }
}

}  // namespace smla
