// C-ABI host side of kvattn: argument validation, work decomposition, the
// handle's workspace, and the launches on the caller's stream.  kvattn_create
// allocates and clears the workspace (and waits for the clear); kvattn_decode
// allocates nothing and never synchronises: one kernel launch per call (one per batch
// range when the call's flat range exceeds 2^30 position units).
#include "../../include/kvattn.h"

#include <hip/hip_runtime.h>

#include "append.hpp"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

// Work decomposition: the flat list of (sequence, KV head, row block) segments is
// cut into kUnitsPerWg large units per workgroup, with as many workgroups as the
// GPU holds resident at once for the kernel instance (occupancy x compute units),
// and a tail of kTailPct percent of the work in about kTailUnits smaller units per
// workgroup that a device-wide queue hands to whichever workgroup is free.  A unit
// is at least kMinChunk positions (kMinChunkMfma for the matrix-core kernel, whose
// per-piece epilogue is heavier).  The split points are placed on the device from
// seq_lens.
#ifndef KVATTN_UNITS_PER_WG
#define KVATTN_UNITS_PER_WG 1
#endif
#ifndef KVATTN_TAIL_PCT
#define KVATTN_TAIL_PCT 0
#endif
#ifndef KVATTN_TAIL_UNITS
#define KVATTN_TAIL_UNITS 2
#endif
constexpr int kMaxResidentWorkgroups = 1024;
constexpr int kMinForcedUnits = 512;
constexpr int kUnitsPerWg = KVATTN_UNITS_PER_WG;  // large units per workgroup
constexpr int kTailPct = KVATTN_TAIL_PCT;         // share of the work in the tail
constexpr int kTailUnits = KVATTN_TAIL_UNITS;     // tail units per workgroup
static_assert(kTailPct >= 0 && kTailPct < 100 && kTailUnits >= 1, "tail shape");
constexpr int kMinChunk = 256;
constexpr int kMinChunkMfma = 512;
constexpr int kChunkQuantum = 64;
constexpr int kMaxQLen = 1024;  // chunked prefill: hundreds of new rows per sequence

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

}  // namespace

struct kvattn_handle {
    kvattn_config cfg;
    int device;
    int num_cus;
    int resident[kMaxQLen + 1][2];  // per (q_len, masked instance): workgroups resident at once
    hipStream_t stream;
    int32_t batch;
    int32_t forced_chunk;
    int64_t flat_max;       // largest flat range of one launch (kvattn::kFlatMax)
    const float* k_scale;   // 8-bit caches: per-KV-head dequantisation scales (device)
    const float* v_scale;
    float* ws;              // partials: acc [ws_part_rows, D] (the handle's allocation starts here)
    float* ws_ml;           // partials: (m, l) [ws_part_rows, 2]
    int32_t* counters;      // arrival counters, one per segment, zero between calls
    int32_t* queue;         // unit queue: two words, zero between calls
    int64_t ws_part_rows;   // partial rows (slot x segment row) the workspace holds
    int64_t n_units;        // arrival counters available (batch x segments per sequence)
    uint32_t* vword;        // debug validation word (NULL without a workspace for it)
    int64_t stride_seq, stride_head, stride_tok;
};

namespace {

int rows_of(const kvattn_config& c, int q_len) {
    return q_len * (c.num_q_heads / c.num_kv_heads);
}

// Longest attended union per sequence that a decode with these arguments can see.
int64_t max_attended(const kvattn_config& c, int q_len, int mask_mode, int n_sink, int window) {
    int64_t cap = c.capacity;
    if (mask_mode == KVATTN_MASK_SINK_WINDOW) {
        const int64_t u = (int64_t)n_sink + window + q_len - 1;
        return u < cap ? u : cap;
    }
    return cap;
}

// Element type of the caches (the config's kv_dtype, 0 meaning the same as dtype).
int kv_dtype_of(const kvattn_config& c) { return c.kv_dtype == 0 ? c.dtype : c.kv_dtype; }

// 16 to 64 rows per KV head (and more, in 64-row blocks, where the prefill kernel does
// not apply): 16-bit caches of the query's type, or 8-bit E4M3 caches.
bool use_mfma(const kvattn_config& c, int q_len) {
    const int kv = kv_dtype_of(c);
    return (kv == c.dtype || kv == KVATTN_FP8_E4M3) &&
           kvattn::mfma_supported(c.dtype, c.head_dim, rows_of(c, q_len));
}

// Chunked prefill (more than 64 rows per KV head, 16-bit caches of every form): the
// prefill kernel's 256-row blocks.
bool use_prefill(const kvattn_config& c, int q_len) {
    return kv_dtype_of(c) == c.dtype &&
           kvattn::prefill_supported(c.dtype, c.head_dim, rows_of(c, q_len), c.cache_mode);
}

// Rows of one segment as laid out in the workspace (the kernel instance's row block;
// the matrix-core kernel pads to whole 16-row tiles, at most 64 rows a block).
int seg_rows_of(const kvattn_config& c, int q_len) {
    const int rows = rows_of(c, q_len);
    if (use_prefill(c, q_len)) return kvattn::kPrefillRows;
    if (use_mfma(c, q_len)) return kvattn::mfma_rows_per_block(rows);
    return kvattn::valu_rows_per_block(rows);
}

int row_blocks_of(const kvattn_config& c, int q_len) {
    const int rows = rows_of(c, q_len);
    const int rpb = seg_rows_of(c, q_len);
    return (rows + rpb - 1) / rpb;
}

int64_t segs_per_seq_of(const kvattn_config& c, int q_len) {
    return (int64_t)c.num_kv_heads * row_blocks_of(c, q_len);
}

// Arrival counters: one per segment.
int64_t counter_units(const kvattn_config& c) {
    int64_t best = 0;
    for (int ql = 1; ql <= c.max_q_len; ++ql)
        best = std::max(best, (int64_t)c.max_batch * segs_per_seq_of(c, ql));
    return best;
}

int validate_config(const kvattn_config* c) {
    if (!c) return fail(KVATTN_ERR_INVALID_ARG, "config is NULL");
    if (c->dtype < KVATTN_F32 || c->dtype > KVATTN_BF16)
        return fail(KVATTN_ERR_UNSUPPORTED, "dtype must be F32, F16 or BF16");
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(KVATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c->num_q_heads < 1 || c->num_kv_heads < 1 || c->num_q_heads % c->num_kv_heads)
        return fail(KVATTN_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    if (c->max_batch < 1) return fail(KVATTN_ERR_INVALID_ARG, "max_batch must be >= 1");
    // the kernels address a position's row in 32 bits (bytes)
    if ((int64_t)c->num_kv_heads * c->head_dim * 4 >= (int64_t)1 << 32)
        return fail(KVATTN_ERR_UNSUPPORTED, "num_kv_heads too large");
    if (c->max_q_len < 1 || c->max_q_len > kMaxQLen)
        return fail(KVATTN_ERR_UNSUPPORTED, "max_q_len must be in 1..1024");
    if (c->capacity < 1) return fail(KVATTN_ERR_INVALID_ARG, "capacity must be >= 1");
    if (c->layout != KVATTN_LAYOUT_TOKEN_MAJOR && c->layout != KVATTN_LAYOUT_HEAD_MAJOR)
        return fail(KVATTN_ERR_INVALID_ARG, "unknown layout");
    if (c->kv_dtype != 0 && c->kv_dtype != c->dtype && c->kv_dtype != KVATTN_FP8_E4M3)
        return fail(KVATTN_ERR_UNSUPPORTED, "kv_dtype must be 0, dtype or FP8_E4M3");
    if (c->kv_dtype == KVATTN_FP8_E4M3 && c->dtype != KVATTN_F16 && c->dtype != KVATTN_BF16)
        return fail(KVATTN_ERR_UNSUPPORTED, "8-bit caches need F16 or BF16 queries");
    if (c->flags & ~(KVATTN_FLAG_DETERMINISTIC | KVATTN_FLAG_DEBUG))
        return fail(KVATTN_ERR_INVALID_ARG, "unknown flag bits");
    if (!(c->scale >= 0.0f) || std::isinf(c->scale))
        return fail(KVATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
    switch (c->cache_mode) {
    case KVATTN_CONTIGUOUS:
    case KVATTN_RING:
        break;
    case KVATTN_PAGED:
        if (!is_pow2(c->block_size))
            return fail(KVATTN_ERR_INVALID_ARG, "block_size must be a power of two");
        if (c->capacity % c->block_size)
            return fail(KVATTN_ERR_INVALID_ARG, "capacity must be a multiple of block_size");
        if (c->num_blocks < 1) return fail(KVATTN_ERR_INVALID_ARG, "num_blocks must be >= 1");
        // the kernels address within a block in 32 bits (bytes)
        if ((int64_t)c->block_size * c->num_kv_heads * c->head_dim * 4 >= (int64_t)1 << 32)
            return fail(KVATTN_ERR_UNSUPPORTED, "block_size x num_kv_heads x head_dim too large");
        break;
    default:
        return fail(KVATTN_ERR_INVALID_ARG, "unknown cache_mode");
    }
    return KVATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int validate_decode_args(const kvattn_handle* h, int32_t q_len, int32_t mask_mode,
                         int32_t n_sink, int32_t window) {
    const kvattn_config& c = h->cfg;
    if (q_len < 1) return fail(KVATTN_ERR_INVALID_ARG, "q_len must be >= 1");
    if (q_len > c.max_q_len) return fail(KVATTN_ERR_CAPACITY, "q_len exceeds max_q_len");
    if (mask_mode != KVATTN_MASK_CAUSAL && mask_mode != KVATTN_MASK_SINK_WINDOW &&
        mask_mode != KVATTN_MASK_TREE)
        return fail(KVATTN_ERR_INVALID_ARG, "unknown mask_mode");
    if (mask_mode == KVATTN_MASK_TREE) {
        if (q_len > 64) return fail(KVATTN_ERR_INVALID_ARG, "tree mask: q_len must be <= 64");
        if (c.cache_mode == KVATTN_RING)
            return fail(KVATTN_ERR_UNSUPPORTED, "tree mask: contiguous or paged caches only");
    }
    if (mask_mode == KVATTN_MASK_SINK_WINDOW) {
        if (n_sink < 0) return fail(KVATTN_ERR_INVALID_ARG, "n_sink must be >= 0");
        if (window < 1) return fail(KVATTN_ERR_INVALID_ARG, "window must be >= 1");
    }
    if (c.cache_mode == KVATTN_RING) {
        if (mask_mode != KVATTN_MASK_SINK_WINDOW)
            return fail(KVATTN_ERR_INVALID_ARG, "a ring cache needs the sink/window mask");
        if (n_sink >= c.capacity)
            return fail(KVATTN_ERR_INVALID_ARG, "ring: n_sink must be below capacity");
        if ((int64_t)n_sink + window + q_len - 1 > c.capacity)
            return fail(KVATTN_ERR_INVALID_ARG,
                        "ring: n_sink + window + q_len - 1 exceeds capacity (attended slots would be overwritten)");
    }
    return KVATTN_OK;
}

// Workgroups of the kernel instance a decode with q_len would launch that fit on
// the device at once (occupancy query).
int resident_for(const kvattn_config& c, int q_len, bool masked, int num_cus) {
    const int rows = rows_of(c, q_len);
    const bool prefill = use_prefill(c, q_len);
    const bool mfma = use_mfma(c, q_len);
    const void* k = prefill ? kvattn::select_prefill_kernel(c.dtype, c.head_dim, rows, c.cache_mode)
                    : mfma  ? kvattn::select_mfma_kernel(c.dtype, kv_dtype_of(c), c.head_dim, rows, c.cache_mode)
                            : kvattn::select_valu_kernel(c.dtype, kv_dtype_of(c), c.head_dim, rows,
                                                         c.cache_mode, masked);
    const int threads = prefill ? kvattn::kPrefillThreads
                        : mfma  ? kvattn::kMfmaThreads
                                : kvattn::valu_threads(rows);
    int per_cu = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return std::min(per_cu * num_cus, kMaxResidentWorkgroups);
}

int resident_workgroups(kvattn_handle* h, int q_len, int mask_mode) {
    const bool masked = kvattn::valu_masked(q_len, mask_mode);
    int& r = h->resident[q_len][masked ? 1 : 0];
    if (r <= 0) r = resident_for(h->cfg, q_len, masked, h->num_cus);
    return r;
}

// Partial rows the workspace needs for decodes with q_len: one slot per unit plus
// one per segment (the pieces of a step fill at most that many), each holding a
// segment's rows.  Units: at most kUnitsPerWg + kTailUnits per launched workgroup
// (at most kMaxResidentWorkgroups), and no more than one plus what the longest
// possible flat range holds at the default minimum unit (every unit is at least
// that long; the head/tail boundary adds one); forced unit lengths (tests) may use
// up to kMinForcedUnits.  Host-only: the bound does not depend on the device.
int64_t part_rows_for(const kvattn_config& c, int q_len) {
    const int64_t segs = (int64_t)c.max_batch * segs_per_seq_of(c, q_len);
    const int64_t w_max = segs * max_attended(c, q_len, KVATTN_MASK_CAUSAL, 0, 0);
    const int64_t by_len = ceil_div(w_max, use_mfma(c, q_len) ? kMinChunkMfma : kMinChunk);
    const int64_t units = std::min<int64_t>((int64_t)kMaxResidentWorkgroups * (kUnitsPerWg + kTailUnits),
                                            std::max<int64_t>(by_len + 1, kMinForcedUnits));
    return (units + segs) * seg_rows_of(c, q_len);
}

int64_t workspace_part_rows(const kvattn_config& c) {
    int64_t best = 0;
    for (int ql = 1; ql <= c.max_q_len; ++ql) best = std::max(best, part_rows_for(c, ql));
    return best;
}

// acc and (m, l) of the partials, one arrival counter per segment, the unit queue
// (two words), the debug validation word.
size_t workspace_size(const kvattn_config& c, int64_t part_rows) {
    return (size_t)part_rows * (size_t)(c.head_dim + 2) * sizeof(float) +
           (size_t)(counter_units(c) + 3) * sizeof(int32_t);
}

// Grid and minimum unit length of a decode with these host arguments.  The work
// itself is only known on the device (seq_lens); the grid is sized for the most
// the arguments allow: batch x segments x the longest attended set.
int plan_for(kvattn_handle* h, int32_t q_len, int32_t mask_mode, int32_t n_sink,
             int32_t window, int* grid, int* min_chunk) {
    const kvattn_config& c = h->cfg;
    const int64_t n_att = std::max<int64_t>(1, max_attended(c, q_len, mask_mode, n_sink, window));
    const int64_t w_max = std::max<int64_t>(1, (int64_t)h->batch * segs_per_seq_of(c, q_len) * n_att);
    *min_chunk = h->forced_chunk > 0 ? h->forced_chunk
                                     : (use_mfma(c, q_len) ? kMinChunkMfma : kMinChunk);
    const int64_t units_max = ceil_div(w_max, *min_chunk);  // units are >= min_chunk
    const int64_t g = std::min<int64_t>(resident_workgroups(h, q_len, mask_mode), units_max);
    // units of the step: exactly min_chunk long when forced; otherwise at most
    // kUnitsPerWg per workgroup (plus the tail's, when there is one) and one more for
    // the rounding of the unit length
    const int64_t units = h->forced_chunk > 0
                              ? units_max
                              : std::min<int64_t>(units_max + 1,
                                                  g * (kUnitsPerWg + (kTailPct > 0 ? kTailUnits : 0)) + 1);
    const int64_t need =
        (units + (int64_t)h->batch * segs_per_seq_of(c, q_len)) * seg_rows_of(c, q_len);
    if (need > h->ws_part_rows)
        return fail(KVATTN_ERR_CAPACITY, "unit count exceeds the workspace");
    if ((int64_t)h->batch * segs_per_seq_of(c, q_len) > h->n_units)
        return fail(KVATTN_ERR_CAPACITY, "segment count exceeds the workspace's arrival counters");
    *grid = (int)std::max<int64_t>(1, g);
    return KVATTN_OK;
}

}  // namespace

extern "C" {

const char* kvattn_last_error(void) { return g_last_error.c_str(); }

int kvattn_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(KVATTN_ERR_INVALID_ARG, "buf and sink must be non-NULL");
    if (!aligned16(buf) || bytes % 16)
        return fail(KVATTN_ERR_INVALID_ARG, "buf must be 16-byte aligned and bytes a multiple of 16");
    if (bytes == 0) return KVATTN_OK;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = kvattn::launch_stream_read(buf, (int64_t)bytes, sink, cus,
                                       reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVATTN_ERR_HIP, std::string("stream read: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

int kvattn_check(kvattn_handle* h) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    if (!(h->cfg.flags & KVATTN_FLAG_DEBUG))
        return fail(KVATTN_ERR_INVALID_ARG, "kvattn_check needs a handle created with KVATTN_FLAG_DEBUG");
    uint32_t w = 0;
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e == hipSuccess) e = hipMemcpy(&w, h->vword, sizeof(w), hipMemcpyDeviceToHost);
    if (e == hipSuccess && w) {
        e = hipMemsetAsync(h->vword, 0, sizeof(w), h->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    }
    if (e != hipSuccess) return fail(KVATTN_ERR_HIP, std::string("kvattn_check: ") + hipGetErrorString(e));
    if (!w) return KVATTN_OK;
    std::string msg = "device-resident arguments out of range since the last check:";
    if (w & kvattn::VALIDATE_SEQ_LEN) msg += " seq_lens (negative, or above capacity)";
    if (w & kvattn::VALIDATE_BLOCK_ID) msg += " block_table (block ids outside [0, num_blocks))";
    if (w & kvattn::VALIDATE_TREE_BITS) msg += " tree_mask (bits at or beyond q_len)";
    return fail(KVATTN_ERR_DEVICE_DATA, msg);
}

int kvattn_workspace_bytes(const kvattn_config* cfg, size_t* bytes) {
    int rc = validate_config(cfg);
    if (rc) return rc;
    if (!bytes) return fail(KVATTN_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = workspace_size(*cfg, workspace_part_rows(*cfg));
    return KVATTN_OK;
}

}  // extern "C"

namespace {

// Host-side state of a handle that does not depend on where its workspace lives:
// configuration, cache strides, the current device and its compute-unit count.
int init_handle(kvattn_handle* h, const kvattn_config* cfg) {
    h->cfg = *cfg;
    h->stream = nullptr;
    h->batch = cfg->max_batch;
    h->forced_chunk = 0;
    // KVATTN_MAX_FLAT lowers the per-launch flat range (tests of the batch-range split
    // on small shapes); it cannot raise it
    h->flat_max = kvattn::kFlatMax;
    if (const char* e = std::getenv("KVATTN_MAX_FLAT")) {
        const long long v = std::atoll(e);
        if (v >= 1 && v < h->flat_max) h->flat_max = v;
    }
    h->k_scale = nullptr;
    h->v_scale = nullptr;
    const int64_t D = cfg->head_dim, H = cfg->num_kv_heads;
    const int64_t unit = cfg->cache_mode == KVATTN_PAGED ? cfg->block_size : cfg->capacity;
    if (cfg->layout == KVATTN_LAYOUT_TOKEN_MAJOR) {
        h->stride_tok = H * D;
        h->stride_head = D;
    } else {
        h->stride_tok = D;
        h->stride_head = unit * D;
    }
    h->stride_seq = unit * H * D;
    hipError_t e = hipGetDevice(&h->device);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&h->num_cus, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) return fail(KVATTN_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    for (auto& r : h->resident) r[0] = r[1] = 0;
    h->ws = nullptr;
    h->ws_ml = nullptr;
    h->counters = nullptr;
    h->queue = nullptr;
    h->vword = nullptr;
    h->ws_part_rows = 0;
    h->n_units = 0;
    return KVATTN_OK;
}

}  // namespace

extern "C" {

int kvattn_create(const kvattn_config* cfg, kvattn_handle** out) {
    if (!out) return fail(KVATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int rc = validate_config(cfg);
    if (rc) return rc;
    kvattn_handle* h = new (std::nothrow) kvattn_handle();
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "host allocation failed");
    rc = init_handle(h, cfg);
    if (rc) {
        delete h;
        return rc;
    }
    hipError_t e;
    h->ws_part_rows = workspace_part_rows(*cfg);
    h->n_units = counter_units(*cfg);
    // the merge addresses partials with 32-bit byte offsets
    if ((double)h->ws_part_rows * cfg->head_dim * sizeof(float) >= 2147483648.0) {
        delete h;
        return fail(KVATTN_ERR_CAPACITY, "workspace would exceed 2 GiB; lower max_batch or max_q_len");
    }
    const size_t bytes = workspace_size(*cfg, h->ws_part_rows);
    e = hipMalloc(reinterpret_cast<void**>(&h->ws), bytes);
    if (e != hipSuccess) {
        delete h;
        return fail(KVATTN_ERR_HIP, std::string("hipMalloc(workspace): ") + hipGetErrorString(e));
    }
    // the arrival counters start at zero; every decode leaves them at zero
    e = hipMemset(h->ws, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(h->ws);
        delete h;
        return fail(KVATTN_ERR_HIP, std::string("hipMemset(workspace): ") + hipGetErrorString(e));
    }
    h->ws_ml = h->ws + h->ws_part_rows * cfg->head_dim;
    h->counters = reinterpret_cast<int32_t*>(h->ws + h->ws_part_rows * (cfg->head_dim + 2));
    h->queue = h->counters + h->n_units;
    h->vword = reinterpret_cast<uint32_t*>(h->queue + 2);
    *out = h;
    return KVATTN_OK;
}

void kvattn_destroy(kvattn_handle* h) {
    if (!h) return;
    if (h->ws) (void)hipFree(h->ws);
    delete h;
}

int kvattn_set_stream(kvattn_handle* h, void* stream) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    h->stream = reinterpret_cast<hipStream_t>(stream);
    return KVATTN_OK;
}

int kvattn_set_batch(kvattn_handle* h, int32_t batch) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    if (batch < 0) return fail(KVATTN_ERR_INVALID_ARG, "batch must be >= 0");
    if (batch > h->cfg.max_batch) return fail(KVATTN_ERR_CAPACITY, "batch exceeds max_batch");
    h->batch = batch;
    return KVATTN_OK;
}

int kvattn_set_kv_scales(kvattn_handle* h, const float* k_scale, const float* v_scale) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    if (!k_scale || !v_scale) return fail(KVATTN_ERR_INVALID_ARG, "scales must be non-NULL");
    h->k_scale = k_scale;
    h->v_scale = v_scale;
    return KVATTN_OK;
}

int kvattn_set_split_len(kvattn_handle* h, int32_t split_len) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    if (split_len < 0 || split_len % kChunkQuantum || split_len > (1 << 24))
        return fail(KVATTN_ERR_INVALID_ARG,
                    "split_len must be 0 or a positive multiple of 64 up to 2^24");
    h->forced_chunk = split_len;
    return KVATTN_OK;
}

int kvattn_plan(kvattn_handle* h, int32_t q_len, int32_t mask_mode, int32_t n_sink,
                int32_t window, int32_t* n_split, int32_t* split_len, int32_t* kernel) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    int rc = validate_decode_args(h, q_len, mask_mode, n_sink, window);
    if (rc) return rc;
    int grid, chunk;
    rc = plan_for(h, q_len, mask_mode, n_sink, window, &grid, &chunk);
    if (rc) return rc;
    if (n_split) *n_split = grid;
    if (split_len) *split_len = chunk;
    if (kernel) *kernel = use_prefill(h->cfg, q_len) ? 2 : (use_mfma(h->cfg, q_len) ? 1 : 0);
    return KVATTN_OK;
}

static void fill_params(const kvattn_handle* h, kvattn::DecodeParams& p, const void* q,
                        const void* k, const void* v, const int32_t* bt, const int32_t* sl,
                        int32_t q_len, int32_t mask_mode, int32_t n_sink, int32_t window,
                        void* out, int min_chunk, const uint64_t* tree = nullptr) {
    const kvattn_config& c = h->cfg;
    p.q = q;
    p.k = k;
    p.v = v;
    p.block_table = bt;
    p.seq_lens = sl;
    p.out = out;
    p.ws_acc = h->ws;
    p.ws_ml = h->ws_ml;
    p.counters = h->counters;
    p.queue = h->queue;
    p.stride_seq = h->stride_seq;
    p.stride_head = h->stride_head;
    p.stride_tok = h->stride_tok;
    p.batch = h->batch;
    p.num_q_heads = c.num_q_heads;
    p.num_kv_heads = c.num_kv_heads;
    p.group = c.num_q_heads / c.num_kv_heads;
    p.q_len = q_len;
    p.rows = rows_of(c, q_len);
    p.cache_mode = c.cache_mode;
    p.mask_mode = mask_mode;
    p.n_sink = mask_mode == KVATTN_MASK_SINK_WINDOW ? n_sink : 0;
    p.window = mask_mode == KVATTN_MASK_SINK_WINDOW ? window : 0;
    p.capacity = c.capacity;
    p.log2_block = c.cache_mode == KVATTN_PAGED ? ilog2(c.block_size) : 0;
    p.num_blocks = c.cache_mode == KVATTN_PAGED ? c.num_blocks : 0;
    p.blocks_per_seq = c.cache_mode == KVATTN_PAGED ? c.capacity / c.block_size : 0;
    p.row_blocks = row_blocks_of(c, q_len);
    p.segs_per_seq = (int32_t)segs_per_seq_of(c, q_len);
    p.seg_rows = seg_rows_of(c, q_len);
    p.min_chunk = min_chunk;
    p.units_per_wg = h->forced_chunk > 0 ? 0 : kUnitsPerWg;  // 0: units of exactly min_chunk
    p.tail_pct = h->forced_chunk > 0 ? 0 : kTailPct;
    p.tail_units = kTailUnits;
    p.deterministic = (c.flags & KVATTN_FLAG_DETERMINISTIC) ? 1 : 0;
    p.k_scale = kv_dtype_of(c) == KVATTN_FP8_E4M3 ? h->k_scale : nullptr;
    p.v_scale = kv_dtype_of(c) == KVATTN_FP8_E4M3 ? h->v_scale : nullptr;
    p.tree_mask = mask_mode == KVATTN_MASK_TREE ? tree : nullptr;
    p.k_new = nullptr;
    p.v_new = nullptr;
    const float scale = c.scale > 0.0f ? c.scale : 1.0f / std::sqrt((float)c.head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;
}

}  // extern "C"

namespace {

// Checks and parameters of a decode; *grid = 0 when there is nothing to launch.
int prepare_decode(kvattn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens, int32_t q_len,
                   int32_t mask_mode, int32_t n_sink, int32_t window, void* out,
                   kvattn::DecodeParams& p, int* grid, const uint64_t* tree = nullptr) {
    *grid = 0;
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    int rc = validate_decode_args(h, q_len, mask_mode, n_sink, window);
    if (rc) return rc;
    if ((mask_mode == KVATTN_MASK_TREE) != (tree != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "a tree mask goes with kvattn_decode_tree (tree_mask non-NULL)");
    if (h->batch == 0) return KVATTN_OK;
    if (!q || !k_cache || !v_cache || !seq_lens || !out)
        return fail(KVATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, seq_lens and out must be non-NULL");
    if ((h->cfg.cache_mode == KVATTN_PAGED) != (block_table != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "block_table must be given exactly for a paged cache");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(KVATTN_ERR_INVALID_ARG, "q, caches and out must be 16-byte aligned");
    if (kv_dtype_of(h->cfg) == KVATTN_FP8_E4M3 && (!h->k_scale || !h->v_scale))
        return fail(KVATTN_ERR_INVALID_ARG, "an 8-bit cache needs kvattn_set_kv_scales first");
    int chunk;
    rc = plan_for(h, q_len, mask_mode, n_sink, window, grid, &chunk);
    if (rc) return rc;
    fill_params(h, p, q, k_cache, v_cache, block_table, seq_lens, q_len, mask_mode, n_sink,
                window, out, chunk, tree);
    return KVATTN_OK;
}

int dtype_bytes(int dtype) {
    return dtype == KVATTN_F32 ? 4 : (dtype == KVATTN_FP8_E4M3 ? 1 : 2);
}

// Parameters of sequences b0 .. b0 + nb - 1 of a decode: the batch-indexed arguments
// start at sequence b0 (caches of the contiguous and ring forms hold a region per
// sequence; a paged pool is shared and its page table starts at row b0).
void batch_range(const kvattn_handle* h, kvattn::DecodeParams& p, int32_t b0, int32_t nb) {
    const kvattn_config& c = h->cfg;
    const int64_t qrow = (int64_t)p.q_len * c.num_q_heads * c.head_dim * dtype_bytes(c.dtype);
    const int64_t eb = dtype_bytes(kv_dtype_of(c));
    p.q = static_cast<const char*>(p.q) + b0 * qrow;
    p.out = static_cast<char*>(p.out) + b0 * qrow;
    p.seq_lens += b0;
    if (c.cache_mode == KVATTN_PAGED) {
        p.block_table += (int64_t)b0 * p.blocks_per_seq;
    } else {
        p.k = static_cast<const char*>(p.k) + b0 * p.stride_seq * eb;
        p.v = static_cast<const char*>(p.v) + b0 * p.stride_seq * eb;
    }
    if (p.tree_mask) p.tree_mask += (int64_t)b0 * p.q_len;
    const int64_t nrow = (int64_t)p.q_len * c.num_kv_heads * c.head_dim * eb;
    if (p.k_new) p.k_new += b0 * nrow;
    if (p.v_new) p.v_new += b0 * nrow;
    p.batch = nb;
}

int launch_range(kvattn_handle* h, const kvattn::DecodeParams& p, int grid, int32_t q_len) {
    hipError_t e =
        use_prefill(h->cfg, q_len)
            ? kvattn::launch_prefill_mfma(p, h->cfg.dtype, h->cfg.head_dim, grid, h->stream)
        : use_mfma(h->cfg, q_len)
            ? kvattn::launch_decode_mfma(p, h->cfg.dtype, kv_dtype_of(h->cfg), h->cfg.head_dim,
                                         grid, h->stream)
            : kvattn::launch_decode_valu(p, h->cfg.dtype, kv_dtype_of(h->cfg), h->cfg.head_dim,
                                         grid, h->stream);
    if (e != hipSuccess)
        return fail(KVATTN_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

// One launch, or one per batch range when the flat range the arguments allow (batch x
// segments per sequence x the longest attended set, whatever seq_lens holds) exceeds
// the per-launch limit: the kernels index it in 32 bits.  The ranges are enqueued in
// order on the handle's stream and share its workspace (each leaves the arrival
// counters and the unit queue at zero); the grid sized for the whole batch serves each.
int launch_decode(kvattn_handle* h, const kvattn::DecodeParams& p, int grid, int32_t q_len) {
    if (grid == 0) return KVATTN_OK;
    const int64_t per_seq =
        (int64_t)p.segs_per_seq *
        std::max<int64_t>(1, max_attended(h->cfg, q_len, p.mask_mode, p.n_sink, p.window));
    if ((int64_t)p.batch * per_seq <= h->flat_max) return launch_range(h, p, grid, q_len);
    const int64_t per_launch = h->flat_max / per_seq;
    if (per_launch < 1)
        return fail(KVATTN_ERR_CAPACITY,
                    "one sequence's work (segments x attended positions) exceeds 2^30");
    for (int64_t b0 = 0; b0 < p.batch; b0 += per_launch) {
        kvattn::DecodeParams pr = p;
        batch_range(h, pr, (int32_t)b0, (int32_t)std::min<int64_t>(per_launch, p.batch - b0));
        const int rc = launch_range(h, pr, grid, q_len);
        if (rc) return rc;
    }
    return KVATTN_OK;
}

// Checks and parameters of an append; a->n_chunks = 0 when there is nothing to write.
int prepare_append(kvattn_handle* h, const void* k_new, const void* v_new, void* k_cache,
                   void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                   int32_t q_len, int32_t n_sink, kvattn::AppendParams* a) {
    a->n_chunks = 0;
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    const kvattn_config& c = h->cfg;
    if (q_len < 1) return fail(KVATTN_ERR_INVALID_ARG, "q_len must be >= 1");
    if (q_len > c.max_q_len) return fail(KVATTN_ERR_CAPACITY, "q_len exceeds max_q_len");
    if (c.cache_mode == KVATTN_RING && (n_sink < 0 || (int64_t)n_sink + q_len > c.capacity))
        return fail(KVATTN_ERR_INVALID_ARG, "ring append: need 0 <= n_sink and n_sink + q_len <= capacity");
    if (h->batch == 0) return KVATTN_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens)
        return fail(KVATTN_ERR_INVALID_ARG, "k_new, v_new, caches and seq_lens must be non-NULL");
    if ((c.cache_mode == KVATTN_PAGED) != (block_table != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "block_table must be given exactly for a paged cache");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(KVATTN_ERR_INVALID_ARG, "k_new, v_new and caches must be 16-byte aligned");
    const int kv = kv_dtype_of(c);
    const int eb = kv == KVATTN_F32 ? 4 : (kv == KVATTN_FP8_E4M3 ? 1 : 2);
    a->k_new = static_cast<const char*>(k_new);
    a->v_new = static_cast<const char*>(v_new);
    a->k_cache = static_cast<char*>(k_cache);
    a->v_cache = static_cast<char*>(v_cache);
    a->block_table = block_table;
    a->seq_lens = seq_lens;
    a->stride_seq = h->stride_seq;
    a->stride_head = h->stride_head;
    a->stride_tok = h->stride_tok;
    a->batch = h->batch;
    a->num_kv_heads = c.num_kv_heads;
    a->q_len = q_len;
    a->elem_bytes = eb;
    a->row_bytes = c.head_dim * eb;  // a multiple of 16 (head_dim 64 or 128)
    a->cache_mode = c.cache_mode;
    a->capacity = c.capacity;
    a->log2_block = c.cache_mode == KVATTN_PAGED ? ilog2(c.block_size) : 0;
    a->num_blocks = c.cache_mode == KVATTN_PAGED ? c.num_blocks : 0;
    a->blocks_per_seq = c.cache_mode == KVATTN_PAGED ? c.capacity / c.block_size : 0;
    a->n_sink = c.cache_mode == KVATTN_RING ? n_sink : 0;
    a->n_chunks = 2 * (int64_t)h->batch * q_len * c.num_kv_heads * (a->row_bytes / 16);
    return KVATTN_OK;
}

// Handles created with KVATTN_FLAG_DEBUG: enqueue the check of the step's
// device-resident arguments (lengths, page-table entries, tree words) ahead of its
// kernels; kvattn_check reports what it found.
int maybe_validate(kvattn_handle* h, const int32_t* block_table, const int32_t* seq_lens,
                   int32_t q_len, const uint64_t* tree) {
    const kvattn_config& c = h->cfg;
    if (!(c.flags & KVATTN_FLAG_DEBUG) || h->batch == 0 || !h->vword) return KVATTN_OK;
    kvattn::ValidateParams v;
    v.seq_lens = seq_lens;
    v.block_table = c.cache_mode == KVATTN_PAGED ? block_table : nullptr;
    v.tree_mask = tree;
    v.word = h->vword;
    v.batch = h->batch;
    v.q_len = q_len;
    v.cache_mode = c.cache_mode;
    v.capacity = c.capacity;
    v.log2_block = c.cache_mode == KVATTN_PAGED ? ilog2(c.block_size) : 0;
    v.num_blocks = c.cache_mode == KVATTN_PAGED ? c.num_blocks : 0;
    v.blocks_per_seq = c.cache_mode == KVATTN_PAGED ? c.capacity / c.block_size : 0;
    const hipError_t e = kvattn::launch_validate(v, h->stream);
    if (e != hipSuccess)
        return fail(KVATTN_ERR_HIP, std::string("validation launch: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

int launch_append(kvattn_handle* h, const kvattn::AppendParams& a) {
    hipError_t e = kvattn::launch_append(a, h->stream);
    if (e != hipSuccess)
        return fail(KVATTN_ERR_HIP, std::string("append launch: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

}  // namespace

extern "C" {

int kvattn_decode(kvattn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens, int32_t q_len,
                  int32_t mask_mode, int32_t n_sink, int32_t window, void* out) {
    kvattn::DecodeParams p;
    int grid;
    int rc = prepare_decode(h, q, k_cache, v_cache, block_table, seq_lens, q_len, mask_mode,
                            n_sink, window, out, p, &grid);
    if (rc) return rc;
    if (grid > 0 && (rc = maybe_validate(h, block_table, seq_lens, q_len, nullptr))) return rc;
    return launch_decode(h, p, grid, q_len);
}

int kvattn_decode_tree(kvattn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens, int32_t q_len,
                       const uint64_t* tree_mask, void* out) {
    kvattn::DecodeParams p;
    int grid;
    if (!tree_mask) return fail(KVATTN_ERR_INVALID_ARG, "tree_mask is NULL");
    int rc = prepare_decode(h, q, k_cache, v_cache, block_table, seq_lens, q_len,
                            KVATTN_MASK_TREE, 0, 0, out, p, &grid, tree_mask);
    if (rc) return rc;
    if (grid > 0 && (rc = maybe_validate(h, block_table, seq_lens, q_len, tree_mask))) return rc;
    return launch_decode(h, p, grid, q_len);
}

int kvattn_append(kvattn_handle* h, const void* k_new, const void* v_new, void* k_cache,
                  void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                  int32_t q_len, int32_t n_sink) {
    kvattn::AppendParams a;
    int rc = prepare_append(h, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len,
                            n_sink, &a);
    if (rc) return rc;
    if (a.n_chunks == 0) return KVATTN_OK;
    if ((rc = maybe_validate(h, block_table, seq_lens, q_len, nullptr))) return rc;
    return launch_append(h, a);
}

int kvattn_append_decode(kvattn_handle* h, const void* q, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t q_len, int32_t mask_mode,
                         int32_t n_sink, int32_t window, void* out) {
    // every check of both calls first, so an error launches nothing
    kvattn::DecodeParams p;
    int grid;
    int rc = prepare_decode(h, q, k_cache, v_cache, block_table, seq_lens, q_len, mask_mode,
                            n_sink, window, out, p, &grid);
    if (rc) return rc;
    kvattn::AppendParams a;
    rc = prepare_append(h, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len,
                        mask_mode == KVATTN_MASK_SINK_WINDOW ? n_sink : 0, &a);
    if (rc) return rc;
    if (grid == 0) return KVATTN_OK;  // no sequence holds a position: nothing to write
    if ((rc = maybe_validate(h, block_table, seq_lens, q_len, nullptr))) return rc;
    // one launch: the decode's workgroups write the new rows they read
    p.k_new = static_cast<const char*>(k_new);
    p.v_new = static_cast<const char*>(v_new);
    return launch_decode(h, p, grid, q_len);
}

}  // extern "C"

namespace {

int debug_gather(kvattn_handle* h, const int32_t* block_table, const int32_t* seq_lens,
                 int32_t q_len, int32_t mask_mode, int32_t n_sink, int32_t window,
                 const uint64_t* tree, int32_t max_slots, int32_t* slots_out,
                 int32_t* counts_out) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    int rc = validate_decode_args(h, q_len, mask_mode, n_sink, window);
    if (rc) return rc;
    if ((mask_mode == KVATTN_MASK_TREE) != (tree != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "a tree mask needs its words (and only it)");
    if (h->batch == 0) return KVATTN_OK;
    if (!seq_lens || !slots_out || !counts_out || max_slots < 0)
        return fail(KVATTN_ERR_INVALID_ARG, "seq_lens, slots_out and counts_out must be non-NULL");
    if ((h->cfg.cache_mode == KVATTN_PAGED) != (block_table != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "block_table must be given exactly for a paged cache");
    kvattn::DecodeParams p;
    fill_params(h, p, nullptr, nullptr, nullptr, block_table, seq_lens, q_len, mask_mode, n_sink,
                window, nullptr, 1 << 30, tree);
    hipError_t e = kvattn::launch_debug_gather(p, max_slots, slots_out, counts_out, h->stream);
    if (e != hipSuccess)
        return fail(KVATTN_ERR_HIP, std::string("gather launch: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

}  // namespace

extern "C" {

int kvattn_debug_gather(kvattn_handle* h, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t q_len, int32_t mask_mode, int32_t n_sink, int32_t window,
                        int32_t max_slots, int32_t* slots_out, int32_t* counts_out) {
    return debug_gather(h, block_table, seq_lens, q_len, mask_mode, n_sink, window, nullptr,
                        max_slots, slots_out, counts_out);
}

int kvattn_debug_gather_tree(kvattn_handle* h, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t q_len, const uint64_t* tree_mask,
                             int32_t max_slots, int32_t* slots_out, int32_t* counts_out) {
    if (!tree_mask) return fail(KVATTN_ERR_INVALID_ARG, "tree_mask is NULL");
    return debug_gather(h, block_table, seq_lens, q_len, KVATTN_MASK_TREE, 0, 0, tree_mask,
                        max_slots, slots_out, counts_out);
}

}  // extern "C"

// ---------------------------------------------------------------- decode without allocation
//
// For callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc): kvattn_decode_noalloc takes no
// handle.  Its partials, arrival counters and unit queue live in `scratch`, a
// file-scope device array of kScratchBytes that each GPU holds from the library's load
// until the process ends.  In host code the array's name is only a stand-in: its
// device address comes from hipGetSymbolAddress, once per device (with that device
// current), and that pointer is what the kernels receive.  Layout: the unit queue
// (two words) at offset 0, kScratchCounters arrival counters at offset 256, the
// partials after them; every call leaves the queue and the counters at zero, and the
// array starts zeroed (and is zeroed once more, by a fill kernel, at a device's first
// call).  Every call on a GPU shares its array: calls that overlap on one GPU race.

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int64_t kScratchCounters = 1 << 16;
constexpr size_t kScratchHead = 256 + (size_t)kScratchCounters * sizeof(int32_t);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

// The device address of this device's scratch array (looked up and cleared at the
// device's first call, on the caller's stream).
int scratch_of(int device, hipStream_t st, unsigned char** out) {
    if (device < 0 || device >= kMaxDevices) return fail(KVATTN_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(KVATTN_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        const int64_t words = (int64_t)(kScratchHead / sizeof(uint32_t));
        hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, st, static_cast<uint32_t*>(ptr),
                           words);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(KVATTN_ERR_HIP, std::string("scratch clear: ") + hipGetErrorString(e));
        g_scratch_ptr[device] = static_cast<unsigned char*>(ptr);
    }
    *out = g_scratch_ptr[device];
    return KVATTN_OK;
}

}  // namespace

extern "C" {

int kvattn_decode_noalloc(const kvattn_config* cfg, int32_t batch, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t q_len, int32_t mask_mode,
                          int32_t n_sink, int32_t window, void* out, void* stream) {
    int rc = validate_config(cfg);
    if (rc) return rc;
    if (kv_dtype_of(*cfg) == KVATTN_FP8_E4M3)
        return fail(KVATTN_ERR_UNSUPPORTED, "kvattn_decode_noalloc: 8-bit caches need a handle (scales)");
    if (cfg->flags & KVATTN_FLAG_DEBUG)
        return fail(KVATTN_ERR_UNSUPPORTED, "kvattn_decode_noalloc: no debug validation without a handle");
    if (batch < 0) return fail(KVATTN_ERR_INVALID_ARG, "batch must be >= 0");
    if (batch > cfg->max_batch) return fail(KVATTN_ERR_CAPACITY, "batch exceeds max_batch");
    if (q_len < 1) return fail(KVATTN_ERR_INVALID_ARG, "q_len must be >= 1");
    if (q_len > cfg->max_q_len) return fail(KVATTN_ERR_CAPACITY, "q_len exceeds max_q_len");
    kvattn_handle h;
    rc = init_handle(&h, cfg);
    if (rc) return rc;
    h.batch = batch;
    h.stream = reinterpret_cast<hipStream_t>(stream);
    // what the scratch holds after its head: partial rows of head_dim + 2 floats, and
    // the arrival counters; the plan is checked against these before anything is enqueued
    h.ws_part_rows = (int64_t)((kScratchBytes - kScratchHead) /
                               ((size_t)(cfg->head_dim + 2) * sizeof(float)));
    h.n_units = kScratchCounters;
    kvattn::DecodeParams p;
    int grid;
    rc = prepare_decode(&h, q, k_cache, v_cache, block_table, seq_lens, q_len, mask_mode, n_sink,
                        window, out, p, &grid);
    if (rc == KVATTN_ERR_CAPACITY)
        return fail(rc, "kvattn_decode_noalloc: the step needs more than the 32 MiB scratch holds (" +
                            g_last_error + "); use a handle (kvattn_create)");
    if (rc) return rc;
    if (grid == 0) return KVATTN_OK;
    unsigned char* base = nullptr;
    rc = scratch_of(h.device, h.stream, &base);
    if (rc) return rc;
    p.queue = reinterpret_cast<int32_t*>(base);
    p.counters = reinterpret_cast<int32_t*>(base + 256);
    p.ws_acc = reinterpret_cast<float*>(base + kScratchHead);
    p.ws_ml = p.ws_acc + h.ws_part_rows * cfg->head_dim;
    return launch_decode(&h, p, grid, q_len);
}

}  // extern "C"
