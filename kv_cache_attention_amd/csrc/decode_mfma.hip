// Instance selection and launch of the split-KV matrix-core kernel (the kernel is in
// decode_mfma.hpp; instances with 8-bit caches are compiled in decode_mfma_fp8.hip).
#include "decode_mfma.hpp"

namespace kvattn {

const void* select_mfma_fp8(int dtype, int head_dim, int rows, int cache_mode);

// 16 rows or more per KV head; above 64 the rows run in blocks of 64 (4 row tiles).
bool mfma_supported(int dtype, int head_dim, int rows) {
    return (dtype == F16 || dtype == BF16) && (head_dim == 64 || head_dim == 128) && rows >= 16;
}
int mfma_rows_per_block(int rows) {
    constexpr int MAXR = KVATTN_MFMA_MAX_R * 16;
    return rows <= MAXR ? (rows + 15) / 16 * 16 : MAXR;
}

const void* select_mfma_kernel(int dtype, int kv_dtype, int head_dim, int rows, int cache_mode) {
    if (!mfma_supported(dtype, head_dim, rows)) return nullptr;
    if (kv_dtype == FP8) return select_mfma_fp8(dtype, head_dim, rows, cache_mode);
    if (kv_dtype != dtype) return nullptr;
    if (dtype == F16)
        return head_dim == 128 ? mfma_kernel_r<F16, F16, 128>(rows, cache_mode)
                               : mfma_kernel_r<F16, F16, 64>(rows, cache_mode);
    return head_dim == 128 ? mfma_kernel_r<BF16, BF16, 128>(rows, cache_mode)
                           : mfma_kernel_r<BF16, BF16, 64>(rows, cache_mode);
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int kv_dtype, int head_dim,
                              int grid, hipStream_t st) {
    const void* k = select_mfma_kernel(dtype, kv_dtype, head_dim, p.rows, p.cache_mode);
    if (!k) return hipErrorInvalidValue;
    DecodeParams pp = p;
    void* args[] = {&pp};
    return hipLaunchKernel(k, dim3(grid), dim3(MFMA_THREADS), args, 0, st);
}

}  // namespace kvattn
