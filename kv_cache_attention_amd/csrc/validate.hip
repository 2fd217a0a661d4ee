// Debug validation of the device-resident arguments of a step (handles created with
// KVATTN_FLAG_DEBUG): the sequence lengths and the page-table entries a decode or an
// append will read.  The kernels never trust these values - they clamp lengths and
// skip page entries outside the pool, so a bad value cannot make them read outside
// the caller's buffers - but a clamped or skipped value still means the caller's
// bookkeeping is wrong (the page table is caller data that maps logical 16-token
// pages to physical blocks: nextadmin.net lesson "KV cache and Flash Attention",
// section "PagedAttention").  This kernel records such values as bits of one
// validation word in the handle's workspace; kvattn_check reads and clears it.
#include "launch.hpp"

namespace kvattn {

__global__ __launch_bounds__(256) void validate_kernel(const ValidateParams v) {
    const int b = blockIdx.x;  // one workgroup per sequence
    if (b >= v.batch) return;
    const int32_t T = v.seq_lens[b];
    uint32_t bad = 0;
    if (T < 0 || (v.cache_mode != RING && T > v.capacity)) bad |= VALIDATE_SEQ_LEN;
    if (v.cache_mode == PAGED && T > 0) {
        // every page a row of this sequence can reach: pages 0 .. ceil(T / block) - 1
        const int32_t Tc = T > v.capacity ? v.capacity : T;
        const int32_t pages = (Tc + (1 << v.log2_block) - 1) >> v.log2_block;
        for (int32_t pg = threadIdx.x; pg < pages; pg += blockDim.x) {
            const int32_t blk = v.block_table[(int64_t)b * v.blocks_per_seq + pg];
            if ((uint32_t)blk >= (uint32_t)v.num_blocks) bad |= VALIDATE_BLOCK_ID;
        }
    }
    if (v.tree_mask && threadIdx.x < v.q_len && v.q_len < 64) {
        // a row's word may name only new positions 0 .. q_len - 1
        const uint64_t w = v.tree_mask[(int64_t)b * v.q_len + threadIdx.x];
        if (w >> v.q_len) bad |= VALIDATE_TREE_BITS;
    }
    if (bad) __hip_atomic_fetch_or(v.word, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_validate(const ValidateParams& v, hipStream_t st) {
    if (v.batch <= 0) return hipSuccess;
    hipLaunchKernelGGL(validate_kernel, dim3(v.batch), dim3(256), 0, st, v);
    return hipGetLastError();
}

}  // namespace kvattn
