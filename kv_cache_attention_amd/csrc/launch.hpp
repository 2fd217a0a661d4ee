// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace kvattn {

// Vector-ALU split-KV kernel (any row count; rows above 16 run in blocks of 16).
// `grid` workgroups share the step's work in equal slices.
hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int kv_dtype, int head_dim,
                              int grid, hipStream_t st);
// The vector-ALU instance tests each score against its row's mask when the rows of a
// sequence attend different sets: q_len > 1, or any token-tree decode.  The launch and
// the occupancy query that sizes its grid both go through this predicate.
inline bool valu_masked(int q_len, int mask_mode) { return q_len > 1 || mask_mode == MASK_TREE; }
int valu_rows_per_block(int rows);
int valu_threads(int rows);  // workgroup size of the instance serving `rows`
// kv_dtype: element type of the caches (FP8 = 8-bit E4M3 codes, with F16/BF16 queries)
const void* select_valu_kernel(int dtype, int kv_dtype, int head_dim, int rows, int cache_mode,
                               bool masked);

// Matrix-core split-KV kernel for 16 to 64 rows per KV head (f16 / bf16 queries;
// caches of the same type or 8-bit E4M3 codes).
hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int kv_dtype, int head_dim,
                              int grid, hipStream_t st);
bool mfma_supported(int dtype, int head_dim, int rows);
int mfma_rows_per_block(int rows);  // rows of one segment (whole 16-row tiles, at most 64)
const void* select_mfma_kernel(int dtype, int kv_dtype, int head_dim, int rows, int cache_mode);
constexpr int kMfmaThreads = 256;

// Matrix-core kernel for chunked prefill: more than 64 rows per KV head (f16 / bf16,
// every cache form) in blocks of kPrefillRows rows, one segment each.
hipError_t launch_prefill_mfma(const DecodeParams& p, int dtype, int head_dim, int grid,
                               hipStream_t st);
bool prefill_supported(int dtype, int head_dim, int rows, int cache_mode);
const void* select_prefill_kernel(int dtype, int head_dim, int rows, int cache_mode);
#ifndef KVATTN_PF_WAVES
#define KVATTN_PF_WAVES 8  // waves per workgroup
#endif
#ifndef KVATTN_PF_RW
#define KVATTN_PF_RW 2     // 16-row tiles per wave
#endif
#ifndef KVATTN_PF_AHEAD
#define KVATTN_PF_AHEAD 2  // K/V tiles in flight in registers (1 or 2)
#endif
#ifndef KVATTN_MFMA_MAX_R
#define KVATTN_MFMA_MAX_R 4  // 16-row tiles of a split-KV matrix-core row block (1 .. 4)
#endif
#ifndef KVATTN_PF_MIN_ROWS
#define KVATTN_PF_MIN_ROWS 64  // segments with more rows than this take the prefill kernel
#endif
constexpr int kPrefillThreads = KVATTN_PF_WAVES * 64;
constexpr int kPrefillRows = KVATTN_PF_WAVES * KVATTN_PF_RW * 16;

// Debug validation of seq_lens, the page table and token-tree words (handles created
// with KVATTN_FLAG_DEBUG): bits of *word are set for each kind of bad value found.
enum : uint32_t { VALIDATE_SEQ_LEN = 1u, VALIDATE_BLOCK_ID = 2u, VALIDATE_TREE_BITS = 4u };
struct ValidateParams {
    const int32_t* seq_lens;
    const int32_t* block_table;  // PAGED only
    const uint64_t* tree_mask;   // token-tree decodes only
    uint32_t* word;              // the handle's validation word (device)
    int32_t batch, q_len, cache_mode, capacity, log2_block, num_blocks, blocks_per_seq;
};
hipError_t launch_validate(const ValidateParams& v, hipStream_t st);

// Measurement: a plain streaming read of `bytes` (a multiple of 16) at `buf`.
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int num_cus,
                              hipStream_t st);

// Test entry: the slots each new row attends, through the kernels' own gather code.
hipError_t launch_debug_gather(const DecodeParams& p, int max_slots, int32_t* slots_out,
                               int32_t* counts_out, hipStream_t st);

}  // namespace kvattn
