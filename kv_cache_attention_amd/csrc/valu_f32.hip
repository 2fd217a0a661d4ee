// Vector-ALU decode kernel instances for F32 queries and F32 caches (split
// from the other element types so the instances compile in parallel).
#include "decode_valu.hpp"

namespace kvattn {

const void* select_valu_f32(int head_dim, int rows_per_block, int cache_mode, bool masked) {
    return head_dim == 128 ? valu_kernel_r<F32, F32, 128>(rows_per_block, cache_mode, masked)
                           : valu_kernel_r<F32, F32, 64>(rows_per_block, cache_mode, masked);
}

}  // namespace kvattn
