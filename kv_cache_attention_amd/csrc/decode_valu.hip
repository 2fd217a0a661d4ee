// Vector-ALU split-KV kernel: instance dispatch and launch (the kernel itself is in
// decode_valu.hpp; its instances are compiled per element type in valu_*.hip).
#include "decode_valu.hpp"

namespace kvattn {

const void* select_valu_f16(int head_dim, int rows_per_block, int cache_mode, bool masked);
const void* select_valu_bf16(int head_dim, int rows_per_block, int cache_mode, bool masked);
const void* select_valu_f32(int head_dim, int rows_per_block, int cache_mode, bool masked);
const void* select_valu_f16_fp8(int head_dim, int rows_per_block, int cache_mode, bool masked);
const void* select_valu_bf16_fp8(int head_dim, int rows_per_block, int cache_mode, bool masked);

int valu_threads(int rows) { return 64 * valu_waves(valu_rows_per_block(rows)); }

int valu_rows_per_block(int rows) {
    if (rows <= 1) return 1;
    if (rows <= 2) return 2;
    if (rows <= 4) return 4;
    if (rows <= 8) return 8;
    return 16;
}

const void* select_valu_kernel(int dtype, int kv_dtype, int head_dim, int rows, int cache_mode,
                               bool masked) {
    const int rpb = valu_rows_per_block(rows);
    if (kv_dtype == FP8) {
        if (dtype == F16) return select_valu_f16_fp8(head_dim, rpb, cache_mode, masked);
        if (dtype == BF16) return select_valu_bf16_fp8(head_dim, rpb, cache_mode, masked);
        return nullptr;
    }
    switch (dtype) {
    case F16: return select_valu_f16(head_dim, rpb, cache_mode, masked);
    case BF16: return select_valu_bf16(head_dim, rpb, cache_mode, masked);
    default: return select_valu_f32(head_dim, rpb, cache_mode, masked);
    }
}

hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int kv_dtype, int head_dim,
                              int grid, hipStream_t st) {
    const void* k = select_valu_kernel(dtype, kv_dtype, head_dim, p.rows, p.cache_mode,
                                       valu_masked(p.q_len, p.mask_mode));
    if (!k) return hipErrorInvalidValue;
    DecodeParams pp = p;
    void* args[] = {&pp};
    return hipLaunchKernel(k, dim3(grid), dim3(valu_threads(p.rows)), args, 0, st);
}

}  // namespace kvattn
