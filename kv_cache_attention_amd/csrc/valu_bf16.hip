// Vector-ALU decode kernel instances for BF16 queries and BF16 caches (split
// from the other element types so the instances compile in parallel).
#include "decode_valu.hpp"

namespace kvattn {

const void* select_valu_bf16(int head_dim, int rows_per_block, int cache_mode, bool masked) {
    return head_dim == 128 ? valu_kernel_r<BF16, BF16, 128>(rows_per_block, cache_mode, masked)
                           : valu_kernel_r<BF16, BF16, 64>(rows_per_block, cache_mode, masked);
}

}  // namespace kvattn
