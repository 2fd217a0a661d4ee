/*
 * kvattn - one decode step of attention over a KV cache, on AMD MI355X (gfx950).
 *
 * The operation (dothoosh.com StreamingLLM article, "The softmax problem"):
 *
 *     out = softmax(Q K^T / sqrt(d)) V
 *
 * for a block of q_len new query rows of each sequence against that sequence's
 * cached keys and values ("KV cache" item of the nextadmin.net lesson "KV cache
 * and Flash Attention": each new token is one query against the cached keys).
 * q_len = 1 is plain autoregressive decode; q_len = 1 + k is the verification
 * pass of speculative decoding, where every new row sees all earlier positions
 * (dothoosh.com speculative-decoding article, "verify phase"); q_len in the
 * hundreds is a chunk of a prefill against the cached prefix (the lesson's
 * FlashAttention section: query tiles against key/value tiles, softmax kept
 * running), the rows then run in blocks of up to 256 on the matrix cores.
 *
 * Cache forms:
 *   CONTIGUOUS  each sequence owns `capacity` consecutive slots; position p is slot p.
 *   PAGED       16-token (block_size) blocks from a shared pool; a page table maps
 *               logical page p / block_size to a physical block (lesson, "PagedAttention").
 *   RING        StreamingLLM cache: the first n_sink positions keep slots 0..n_sink-1
 *               for ever, later positions roll over the remaining capacity - n_sink
 *               slots: slot = n_sink + (p - n_sink) mod (capacity - n_sink)
 *               (StreamingLLM article, "The StreamingLLM solution").
 *
 * Masks:
 *   KVATTN_MASK_CAUSAL       new row i of a sequence of T positions sits at
 *                            P = T - q_len + i and sees every position p <= P.
 *   KVATTN_MASK_SINK_WINDOW  row at P sees p <= P with p < n_sink (attention sinks)
 *                            or p >= P - window + 1 (the `window` most recent
 *                            positions, its own included).
 *   KVATTN_MASK_TREE         token-tree verification (kvattn_decode_tree): the q_len
 *                            new positions P0 = T - q_len .. T - 1 are a tree of draft
 *                            tokens; row i sees every p < P0 and P0 + j iff bit j
 *                            of its mask word is set (its ancestors and itself).
 *
 * Layouts (row-major, head_dim innermost and contiguous; element type = dtype, or
 * kv_dtype for the caches):
 *   q, out       [batch, q_len, num_q_heads, head_dim]
 *   CONTIGUOUS and RING caches
 *                token-major (default): [batch, capacity, num_kv_heads, head_dim]
 *                head-major:            [batch, num_kv_heads, capacity, head_dim]
 *   PAGED cache  token-major (default): [num_blocks, block_size, num_kv_heads, head_dim]
 *                head-major:            [num_blocks, num_kv_heads, block_size, head_dim]
 *   block_table  int32 [batch, capacity / block_size]  (PAGED only)
 *   seq_lens     int32 [batch]: T_b, every cached position of sequence b including
 *                the q_len new ones, whose K and V are already in the cache.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped-query attention).
 *
 * Memory: every pointer passed to kvattn_decode is a device pointer owned by the
 * caller and must stay valid until the work enqueued on the handle's stream has
 * finished.  The handle owns one device workspace, allocated by kvattn_create;
 * kvattn_decode never allocates, never synchronises and never copies to the host,
 * so a call can be captured into a HIP graph and replayed: the decode step of the
 * dothoosh.com Moondream article ("Mechanism one: the ping-pong slot system") avoids
 * runtime device allocation because it synchronises the device, and keeps its
 * buffers at fixed addresses so the step can be recorded once as a graph and
 * replayed.
 *
 * Errors: every entry point returns KVATTN_OK (0) or a negative code and never
 * aborts; kvattn_last_error() gives the text of the calling thread's last error.
 * Values that live on the device (seq_lens, block_table) are not checked on the
 * host: the kernels clamp T to what the cache can hold (CONTIGUOUS/PAGED: T <=
 * capacity) and skip page-table entries outside [0, num_blocks), so they never
 * read outside the caller's buffers; a row with no attended position (T < q_len)
 * gets zeros.  Handles created with KVATTN_FLAG_DEBUG also record such values
 * on the device, for kvattn_check to report.
 *
 * Threads: one handle serves one stream; concurrent decode calls on one handle
 * race on its workspace.  Use one handle per in-flight step.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KVATTN_API __attribute__((visibility("default")))
#else
#define KVATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum kvattn_status {
    KVATTN_OK = 0,
    KVATTN_ERR_INVALID_ARG = -1,   /* null pointer, bad enum, inconsistent sizes */
    KVATTN_ERR_UNSUPPORTED = -2,   /* dtype / head_dim / mode combination not built */
    KVATTN_ERR_CAPACITY = -3,      /* batch or q_len beyond what the handle was created for */
    KVATTN_ERR_HIP = -4,           /* a HIP runtime call failed (text in kvattn_last_error) */
    KVATTN_ERR_DEVICE_DATA = -5    /* kvattn_check: device-resident arguments were out of range */
};

enum kvattn_dtype { KVATTN_F32 = 0, KVATTN_F16 = 1, KVATTN_BF16 = 2, KVATTN_FP8_E4M3 = 3 };
enum kvattn_cache_mode { KVATTN_CONTIGUOUS = 0, KVATTN_PAGED = 1, KVATTN_RING = 2 };
enum kvattn_mask_mode { KVATTN_MASK_CAUSAL = 0, KVATTN_MASK_SINK_WINDOW = 1, KVATTN_MASK_TREE = 2 };
enum kvattn_layout { KVATTN_LAYOUT_TOKEN_MAJOR = 0, KVATTN_LAYOUT_HEAD_MAJOR = 1 };

typedef struct kvattn_config {
    int32_t dtype;          /* kvattn_dtype: q, both caches and out share it */
    int32_t num_q_heads;    /* Hq >= 1 */
    int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;       /* 64 or 128 */
    int32_t max_batch;      /* >= 1 */
    int32_t max_q_len;      /* 1 .. 1024 (token-tree masks: q_len <= 64) */
    int32_t cache_mode;     /* kvattn_cache_mode */
    int32_t capacity;       /* CONTIGUOUS / RING: slots per sequence; PAGED: positions per
                               sequence = block_size * (row length of block_table) */
    int32_t block_size;     /* PAGED: power of two (16 in the lesson); otherwise ignored */
    int32_t num_blocks;     /* PAGED: blocks in the pool; otherwise ignored */
    int32_t layout;         /* kvattn_layout */
    float scale;            /* 0 => 1 / sqrt(head_dim) */
    uint32_t flags;         /* KVATTN_FLAG_* bits, 0 for the defaults */
    int32_t kv_dtype;       /* element type of both caches: 0 or dtype = the same as q;
                               KVATTN_FP8_E4M3 (q F16 or BF16) = 8-bit OCP E4M3 codes, the
                               real value being code * the KV head's scale
                               (kvattn_set_kv_scales) */
} kvattn_config;

/* Flags.
 * KVATTN_FLAG_DETERMINISTIC: every decode with the same inputs returns the same
 *   bits.  By default the waves of a workgroup take tiles of positions from a
 *   shared queue, so the order in which partial sums are added (and with it the
 *   last bits of the result) depends on timing; with this flag each wave takes a
 *   fixed set of tiles, at some cost in speed when memory bandwidth is shared
 *   unevenly.  The result then depends only on the logical positions, not on
 *   where a paged cache keeps them. */
#define KVATTN_FLAG_DETERMINISTIC 1u

/* KVATTN_FLAG_DEBUG: every decode and append first enqueues a check of its
 *   device-resident arguments - seq_lens (T < 0, or T > capacity for CONTIGUOUS and
 *   PAGED caches), the page-table entries of pages 0 .. ceil(T / block_size) - 1
 *   (a block id outside [0, num_blocks)) and token-tree words (bits at or beyond
 *   q_len) - and records what it finds in a word of the workspace, which
 *   kvattn_check reads.  Without the flag the same values are clamped or skipped by
 *   the kernels silently.  Costs one small extra launch per call. */
#define KVATTN_FLAG_DEBUG 2u

typedef struct kvattn_handle kvattn_handle;

/* Validate `cfg`, plan the work decomposition and allocate the handle's device
 * workspace (split partials, merge counters) on the current HIP device.  This is the
 * only call that allocates device memory: later calls reuse the workspace at its
 * fixed address (the no-runtime-allocation, fixed-buffer rule of the Moondream
 * article's ping-pong slot system, dothoosh.com).  *out is NULL on error. */
KVATTN_API int kvattn_create(const kvattn_config* cfg, kvattn_handle** out);

/*
 * Enqueue one decode step on the handle's stream and return.
 *   q            [batch, q_len, Hq, D]           device, read
 *   k_cache      cache of keys (layout above)     device, read
 *   v_cache      cache of values (same layout)    device, read
 *   block_table  [batch, capacity / block_size]   device, read; PAGED only, else NULL
 *   seq_lens     [batch] int32                    device, read
 *   q_len        1 .. max_q_len
 *   mask_mode    kvattn_mask_mode; RING requires KVATTN_MASK_SINK_WINDOW
 *   n_sink       >= 0, window >= 1               (SINK_WINDOW only; ignored for CAUSAL)
 *                RING: n_sink + window + q_len - 1 <= capacity and n_sink < capacity
 *   out          [batch, q_len, Hq, D]           device, written
 * batch is the handle's current batch (kvattn_set_batch; initially max_batch).
 * One kernel launch; several, one per batch range and in order on the stream, when
 * batch x KV heads x query-row blocks x the longest attended set the arguments allow
 * (capacity, or n_sink + window + q_len - 1 for SINK_WINDOW) exceeds 2^30 position
 * units (the kernels index that range in 32 bits); KVATTN_ERR_CAPACITY if a single
 * sequence exceeds it.  The environment variable KVATTN_MAX_FLAT, read when a handle
 * is created, lowers the limit (tests of the batch-range launches).
 */
KVATTN_API int kvattn_decode(kvattn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens, int32_t q_len,
                  int32_t mask_mode, int32_t n_sink, int32_t window, void* out);

/*
 * Enqueue the write of each sequence's q_len new K and V rows into the caches:
 * row i of sequence b goes to the slot of logical position P = T_b - q_len + i
 * (T_b = seq_lens[b]) - the step of a decode that writes the new token's key and
 * value back to memory before attending (dothoosh.com speculative-decoding
 * article, "bypassing the memory bottleneck"), through the same position-to-slot
 * mapping the decode reads with: CONTIGUOUS slot P; PAGED block
 * block_table[b][P / block_size], offset P % block_size (lesson, "PagedAttention");
 * RING the first n_sink positions keep their slots, later ones roll over the other
 * capacity - n_sink slots, overwriting the position capacity - n_sink earlier
 * (StreamingLLM article, "The StreamingLLM solution").
 *   k_new, v_new [batch, q_len, Hkv, D], the caches' element type   device, read
 *   k_cache, v_cache  caches (layout above)                          device, written
 *   block_table, seq_lens                                            as for kvattn_decode
 *   q_len        1 .. max_q_len
 *   n_sink       RING: the sink count the decodes use (0 .. capacity - 1); else ignored
 * Rows without a slot are not written: P < 0 (T < q_len), P >= capacity (CONTIGUOUS,
 * PAGED), or a page-table entry outside [0, num_blocks).  Only the new rows' slots
 * are written.  Pointers 16-byte aligned.  No allocation, no synchronisation.
 */
KVATTN_API int kvattn_append(kvattn_handle* h, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                             int32_t q_len, int32_t n_sink);

/* kvattn_append and kvattn_decode in one launch: the step writes the new tokens'
 * keys and values back to the cache and attends over them (dothoosh.com
 * speculative-decoding article, "The memory-bandwidth wall").  The result and the
 * caches afterwards are those of kvattn_append followed by kvattn_decode: each
 * workgroup writes the new rows that its share of the step reads before loading it
 * (the new positions are the last of every attended list, and no attended position
 * shares a slot with a new one), so no step-wide ordering is needed.  Arguments as
 * for the two calls; a RING cache uses n_sink for both (with
 * KVATTN_MASK_SINK_WINDOW).  k_new / v_new must not overlap the caches.  Launches
 * over batch ranges as kvattn_decode does, each range writing its own sequences'
 * rows. */
KVATTN_API int kvattn_append_decode(kvattn_handle* h, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int32_t q_len, int32_t mask_mode, int32_t n_sink,
                                    int32_t window, void* out);

/*
 * Enqueue one decode step whose new rows form a token tree (SpecInfer verifies a
 * tree of draft tokens in one pass with a tree-shaped attention mask - dothoosh.com
 * speculative-decoding article; EAGLE-2 builds such trees dynamically - aioapex.com
 * article): row i of sequence b sees every cached position before the new block
 * (p < T - q_len) and new position T - q_len + j iff bit j of tree_mask[b * q_len + i]
 * is set.  A row that sees nothing returns zeros.
 *   tree_mask    [batch, q_len] uint64             device, read
 *   q_len        1 .. min(max_q_len, 64); CONTIGUOUS or PAGED caches
 * Other arguments and behaviour as kvattn_decode.
 */
KVATTN_API int kvattn_decode_tree(kvattn_handle* h, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t q_len,
                                  const uint64_t* tree_mask, void* out);

/*
 * kvattn_decode without a handle and without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same operation, arguments, layouts and kernels as
 * kvattn_decode (the configuration in `cfg`, the batch and the stream given per call);
 * the step's partials, arrival counters and unit queue live in a static 32 MiB device
 * array that each GPU holds from the library's load until the process ends.
 *   cfg          as for kvattn_create; 16-bit or fp32 caches (kv_dtype 0 or dtype),
 *                no KVATTN_FLAG_DEBUG
 *   batch        0 .. cfg->max_batch
 *   stream       hipStream_t (NULL = the null stream)
 * KVATTN_ERR_CAPACITY, with nothing enqueued, when the step needs more than the array
 * holds: more than 65,536 segments (batch x KV heads x row blocks) or partials beyond
 * 32 MiB (the decode and verify shapes fit; large prefill chunks need a handle).
 * All calls on one GPU share its array, so calls that overlap on one GPU race: order
 * them on one stream.  Never allocates, never synchronises.
 */
KVATTN_API int kvattn_decode_noalloc(const kvattn_config* cfg, int32_t batch, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     int32_t q_len, int32_t mask_mode, int32_t n_sink,
                                     int32_t window, void* out, void* stream);

/* Free the workspace and the handle.  NULL is a no-op.  No enqueued decode may
 * still be using the handle (as a ping-pong slot of the Moondream article is released
 * only once the step that used it has completed). */
KVATTN_API void kvattn_destroy(kvattn_handle* h);

/* Stream for later decode calls (a hipStream_t; NULL = the null stream).  A handle's
 * workspace serves one step at a time: calls on one handle are ordered by its one
 * stream.  Two steps in flight at once (the two alternating slots of the Moondream
 * article's ping-pong system) take two handles, each with its own workspace, on one
 * stream or on two.  Switch a handle's stream only once its earlier work is done. */
KVATTN_API int kvattn_set_stream(kvattn_handle* h, void* stream);

/* Batch for later decode calls, 0 .. max_batch (0 enqueues nothing).  Host-side
 * state only: no device work, no allocation (sizes stay within what kvattn_create
 * allocated for max_batch). */
KVATTN_API int kvattn_set_batch(kvattn_handle* h, int32_t batch);

/* Dequantisation scales of an 8-bit cache (kv_dtype KVATTN_FP8_E4M3): float32
 * [num_kv_heads] device arrays for K and V, read by later decode calls (borrowed:
 * they must stay valid while those calls are in flight).  Scales must be positive
 * and finite.  Required before decoding an 8-bit cache; ignored otherwise. */
KVATTN_API int kvattn_set_kv_scales(kvattn_handle* h, const float* k_scale, const float* v_scale);

/* Force the length of the work units the step is cut into (attended positions of
 * a (sequence, KV head) segment; a multiple of 64, or 0 to let the library choose).
 * Every unit then has exactly this length (the last one of the step may be shorter),
 * so segments are cut into many pieces.  For tests of split-count invariance. */
KVATTN_API int kvattn_set_split_len(kvattn_handle* h, int32_t split_len);

/* The decomposition a decode with these host arguments would use: n_split = the
 * workgroups launched (one per compute unit for the automatic plan), split_len =
 * the minimum unit length in positions (the exact unit length is placed on the
 * device from seq_lens), and the kernel family (0 = vector-ALU rows, 1 =
 * matrix-core rows, 2 = chunked-prefill blocks of 256 rows on the matrix cores). */
KVATTN_API int kvattn_plan(kvattn_handle* h, int32_t q_len, int32_t mask_mode, int32_t n_sink,
                int32_t window, int32_t* n_split, int32_t* split_len, int32_t* kernel);

/* Device bytes kvattn_create would allocate for `cfg`. */
KVATTN_API int kvattn_workspace_bytes(const kvattn_config* cfg, size_t* bytes);

/*
 * Debug handles (KVATTN_FLAG_DEBUG): wait for the handle's stream, then report and
 * clear the validation word the step's checks wrote since the last kvattn_check.
 * KVATTN_OK if every checked value was in range; KVATTN_ERR_DEVICE_DATA otherwise
 * (kvattn_last_error names the kinds of bad values: lengths, block ids, tree bits -
 * the page table maps logical pages to physical blocks and is the caller's data,
 * nextadmin.net lesson "KV cache and Flash Attention", section "PagedAttention").
 * KVATTN_ERR_INVALID_ARG for a handle without the flag.  Synchronises: not for use
 * under graph capture.
 */
KVATTN_API int kvattn_check(kvattn_handle* h);

/*
 * Measurement yardstick (no handle): enqueue on `stream` (a hipStream_t, NULL = the
 * null stream) one plain streaming read of `bytes` bytes at the device pointer `buf`
 * (16-byte aligned, bytes a multiple of 16), every byte loaded once.  A decode step
 * is bounded below by its bytes / the device's bandwidth (dothoosh.com
 * speculative-decoding article, "The memory-bandwidth wall"); timing this read gives
 * the bandwidth a read-only stream reaches in practice.  `sink`: one device uint32,
 * written only when the fold of the data hits one particular value.  No allocation.
 */
KVATTN_API int kvattn_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Text of the calling thread's last error ("" if none). */
KVATTN_API const char* kvattn_last_error(void);

/*
 * Test entry: for each (b, i) with b < batch, i < q_len, write the flat slot
 * indices (rows of the [slots, Hkv, D] view of the cache; PAGED: block * block_size
 * + offset) of every position row i of sequence b attends, in increasing
 * position order, to slots_out[(b * q_len + i) * max_slots + j], and the count to
 * counts_out[b * q_len + i] (counts beyond max_slots are still counted; only the
 * first max_slots slots are written).  Uses the same device gather code as the
 * decode kernels.  Device pointers; enqueued on the handle's stream.
 */
KVATTN_API int kvattn_debug_gather(kvattn_handle* h, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t q_len, int32_t mask_mode, int32_t n_sink, int32_t window,
                        int32_t max_slots, int32_t* slots_out, int32_t* counts_out);

/* Test entry: kvattn_debug_gather for a tree mask (tree_mask as for
 * kvattn_decode_tree). */
KVATTN_API int kvattn_debug_gather_tree(kvattn_handle* h, const int32_t* block_table,
                                        const int32_t* seq_lens, int32_t q_len,
                                        const uint64_t* tree_mask, int32_t max_slots,
                                        int32_t* slots_out, int32_t* counts_out);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
