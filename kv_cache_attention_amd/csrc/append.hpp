// KV append: arguments of the scatter kernel (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace kvattn {

struct AppendParams {
    const char* k_new;  // [batch, q_len, Hkv, D] rows, the caches' element type
    const char* v_new;
    char* k_cache;
    char* v_cache;
    const int32_t* block_table;  // PAGED only
    const int32_t* seq_lens;
    int64_t stride_seq, stride_head, stride_tok;  // cache strides, elements
    int64_t n_chunks;  // 2 * batch * q_len * Hkv * row_bytes / 16
    int32_t batch, num_kv_heads, q_len, elem_bytes, row_bytes;
    int32_t cache_mode, capacity, log2_block, num_blocks, blocks_per_seq, n_sink;
};

hipError_t launch_append(const AppendParams& a, hipStream_t st);

}  // namespace kvattn
