// Split-KV matrix-core kernel instances for 8-bit (E4M3) caches with F16 or BF16
// queries (split from the 16-bit instances so the two compile in parallel).
#include "decode_mfma.hpp"

namespace kvattn {

const void* select_mfma_fp8(int dtype, int head_dim, int rows, int cache_mode) {
    if (dtype == F16)
        return head_dim == 128 ? mfma_kernel_r<F16, FP8, 128>(rows, cache_mode)
                               : mfma_kernel_r<F16, FP8, 64>(rows, cache_mode);
    return head_dim == 128 ? mfma_kernel_r<BF16, FP8, 128>(rows, cache_mode)
                           : mfma_kernel_r<BF16, FP8, 64>(rows, cache_mode);
}

}  // namespace kvattn
