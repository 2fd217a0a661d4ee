// KV append: the q_len new K and V rows of every sequence written to the cache
// slots of their positions, before the decode reads them.  A new token's key and
// value are written back to memory as part of each decode step (dothoosh.com
// speculative-decoding article, "bypassing the memory bottleneck"); the slot of a
// position follows the cache form: contiguous, paged (page table from logical
// 16-token pages to physical blocks, nextadmin.net lesson "PagedAttention"), or
// the StreamingLLM ring whose first n_sink positions keep their slots while later
// ones roll over the rest (dothoosh.com StreamingLLM article, "The StreamingLLM
// solution").
//
// The copy is HBM-bound and tiny next to the decode (q_len rows per sequence and
// KV head): one thread moves 16 bytes, consecutive threads the consecutive chunks
// of a row, so every row is written with full 16-byte stores.
#include "append.hpp"

namespace kvattn {

template <int CACHE>
__global__ __launch_bounds__(256) void append_kernel(const AppendParams a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = a.row_bytes / 16;  // 16-byte chunks per row
    if (idx >= a.n_chunks) return;
    int64_t r = idx / cpr;
    const int c = (int)(idx - r * cpr);
    const int kvh = (int)(r % a.num_kv_heads);
    r /= a.num_kv_heads;
    const int i = (int)(r % a.q_len);
    r /= a.q_len;
    const int b = (int)(r % a.batch);
    const bool is_v = r >= a.batch;

    int32_t T = a.seq_lens[b];
    if (T < 0) T = 0;
    const int32_t P = T - a.q_len + i;
    if (P < 0) return;  // no slot: fewer positions than new rows
    int64_t unit;
    int32_t slot;
    if constexpr (CACHE == CONTIGUOUS) {
        if (P >= a.capacity) return;
        unit = b;
        slot = P;
    } else if constexpr (CACHE == RING) {
        unit = b;
        slot = P < a.n_sink ? P : a.n_sink + (P - a.n_sink) % (a.capacity - a.n_sink);
    } else {
        if (P >= a.capacity) return;
        const int32_t blk = a.block_table[(int64_t)b * a.blocks_per_seq + (P >> a.log2_block)];
        if ((uint32_t)blk >= (uint32_t)a.num_blocks) return;  // entry outside the pool
        unit = blk;
        slot = P & ((1 << a.log2_block) - 1);
    }
    const int64_t dst = (unit * a.stride_seq + (int64_t)kvh * a.stride_head +
                         (int64_t)slot * a.stride_tok) * a.elem_bytes + (int64_t)c * 16;
    const int64_t src = (((int64_t)b * a.q_len + i) * a.num_kv_heads + kvh) * a.row_bytes +
                        (int64_t)c * 16;
    const uint4 v = *reinterpret_cast<const uint4*>((is_v ? a.v_new : a.k_new) + src);
    *reinterpret_cast<uint4*>((is_v ? a.v_cache : a.k_cache) + dst) = v;
}

hipError_t launch_append(const AppendParams& a, hipStream_t st) {
    if (a.n_chunks <= 0) return hipSuccess;
    const dim3 block(256), grid((unsigned)((a.n_chunks + 255) / 256));
    switch (a.cache_mode) {
    case CONTIGUOUS:
        hipLaunchKernelGGL(append_kernel<CONTIGUOUS>, grid, block, 0, st, a);
        break;
    case PAGED:
        hipLaunchKernelGGL(append_kernel<PAGED>, grid, block, 0, st, a);
        break;
    default:
        hipLaunchKernelGGL(append_kernel<RING>, grid, block, 0, st, a);
        break;
    }
    return hipGetLastError();
}

}  // namespace kvattn
