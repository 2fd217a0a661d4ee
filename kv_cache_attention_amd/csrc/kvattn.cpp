// C-ABI host side of kvattn: argument validation, work decomposition, the
// handle's workspace, and the launches on the caller's stream.  kvattn_create
// allocates and clears the workspace (and waits for the clear); kvattn_decode
// allocates nothing and never synchronises: one kernel launch per call.
#include "../../include/kvattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

// Split-KV decomposition: as many work items as the GPU holds resident at once
// (the kernel instance's occupancy x compute units), so the whole step runs in one
// round with no tail, each split at least kMinSplitLen positions.  The workspace
// is sized for the largest target any kernel instance could ask for (8 per CU on
// 256 CUs).
constexpr int kMaxResidentWorkgroups = 2048;
constexpr int kMinSplitLen = 256;
constexpr int kMinSplitLenMfma = 512;
constexpr int kSplitQuantum = 64;
constexpr int kMaxSplits = 1024;
constexpr int kMaxQLen = 64;

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
    int resident[65];       // per q_len: workgroups of its kernel instance resident at once
    hipStream_t stream;
    int32_t batch;
    int32_t forced_split_len;
    float* ws;              // split partials: acc [ws_rows, D], (m, l) [ws_rows, 2], counters
    int64_t ws_rows;        // partial rows the workspace holds
    int64_t n_units;        // arrival counters (batch x KV heads x row blocks)
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

bool use_mfma(const kvattn_config& c, int q_len) {
    return kvattn::mfma_supported(c.dtype, c.head_dim, rows_of(c, q_len));
}

int row_blocks_of(const kvattn_config& c, int q_len) {
    if (use_mfma(c, q_len)) return 1;
    const int rows = rows_of(c, q_len);
    const int rpb = kvattn::valu_rows_per_block(rows);
    return (rows + rpb - 1) / rpb;
}

// Automatic split count for `batch` sequences of up to n_att attended positions,
// aiming at `target` resident workgroups.
void auto_plan(const kvattn_config& c, int batch, int q_len, int64_t n_att, int target,
               int* n_split, int* split_len) {
    const bool mfma = use_mfma(c, q_len);
    const int64_t units = (int64_t)(batch > 0 ? batch : 1) * c.num_kv_heads * row_blocks_of(c, q_len);
    int ns = ceil_div(target, units);
    const int ns_cap = ceil_div(n_att > 0 ? n_att : 1, mfma ? kMinSplitLenMfma : kMinSplitLen);
    if (ns > ns_cap) ns = ns_cap;
    if (ns < 1) ns = 1;
    if (ns > kMaxSplits) ns = kMaxSplits;
    int len = ceil_div(n_att > 0 ? n_att : 1, ns);
    len = ceil_div(len, kSplitQuantum) * kSplitQuantum;
    *split_len = len;
    *n_split = ceil_div(n_att > 0 ? n_att : 1, len);
}

int64_t workspace_rows(const kvattn_config& c) {
    // largest batch x splits product the automatic plan can ask for, over every batch
    // size and q_len the handle accepts; plus room for up to 64 forced splits
    int64_t best = 0;
    for (int ql = 1; ql <= c.max_q_len; ++ql) {
        for (int b = 1; b <= c.max_batch; ++b) {
            int ns, len;
            auto_plan(c, b, ql, c.capacity, kMaxResidentWorkgroups, &ns, &len);
            const int64_t rows = (int64_t)b * ql * c.num_q_heads * ns;
            if (rows > best) best = rows;
        }
    }
    const int64_t floor_splits = std::min<int64_t>(64, ceil_div(c.capacity, kSplitQuantum));
    const int64_t fl = (int64_t)c.max_batch * c.max_q_len * c.num_q_heads * floor_splits;
    return best > fl ? best : fl;
}

// Arrival counters: one per (sequence, KV head, block of 16 rows).
int64_t counter_units(const kvattn_config& c) {
    const int64_t rows = (int64_t)c.max_q_len * (c.num_q_heads / c.num_kv_heads);
    return (int64_t)c.max_batch * c.num_kv_heads * ((rows + 15) / 16);
}

size_t workspace_size(const kvattn_config& c, int64_t ws_rows) {
    return (size_t)ws_rows * (size_t)(c.head_dim + 2) * sizeof(float) +
           (size_t)counter_units(c) * sizeof(int32_t);
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
    if (c->max_q_len < 1 || c->max_q_len > kMaxQLen)
        return fail(KVATTN_ERR_UNSUPPORTED, "max_q_len must be in 1..64");
    if (c->capacity < 1) return fail(KVATTN_ERR_INVALID_ARG, "capacity must be >= 1");
    if (c->layout != KVATTN_LAYOUT_TOKEN_MAJOR && c->layout != KVATTN_LAYOUT_HEAD_MAJOR)
        return fail(KVATTN_ERR_INVALID_ARG, "unknown layout");
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
    if (mask_mode != KVATTN_MASK_CAUSAL && mask_mode != KVATTN_MASK_SINK_WINDOW)
        return fail(KVATTN_ERR_INVALID_ARG, "unknown mask_mode");
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
// the device at once (occupancy query, cached per q_len).
int resident_workgroups(kvattn_handle* h, int q_len) {
    int& r = h->resident[q_len];
    if (r > 0) return r;
    const kvattn_config& c = h->cfg;
    const int rows = rows_of(c, q_len);
    const bool mfma = use_mfma(c, q_len);
    const void* k = mfma ? kvattn::select_mfma_kernel(c.dtype, c.head_dim, rows, c.cache_mode)
                         : kvattn::select_valu_kernel(c.dtype, c.head_dim, rows, c.cache_mode,
                                                      q_len > 1);
    int per_cu = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(
                  &per_cu, k, mfma ? kvattn::kMfmaThreads : kvattn::kValuThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    r = std::min(per_cu * h->num_cus, kMaxResidentWorkgroups);
    return r;
}

int plan_for(kvattn_handle* h, int32_t q_len, int32_t mask_mode, int32_t n_sink,
             int32_t window, int* n_split, int* split_len) {
    const kvattn_config& c = h->cfg;
    const int64_t n_att = max_attended(c, q_len, mask_mode, n_sink, window);
    if (h->forced_split_len > 0) {
        *split_len = h->forced_split_len;
        *n_split = ceil_div(n_att > 0 ? n_att : 1, h->forced_split_len);
    } else {
        auto_plan(c, h->batch, q_len, n_att, resident_workgroups(h, q_len), n_split, split_len);
    }
    if (*n_split > 1) {
        const int64_t need = (int64_t)h->batch * q_len * c.num_q_heads * *n_split;
        if (need > h->ws_rows)
            return fail(KVATTN_ERR_CAPACITY, "split count exceeds the handle's workspace");
    }
    return KVATTN_OK;
}

}  // namespace

extern "C" {

const char* kvattn_last_error(void) { return g_last_error.c_str(); }

int kvattn_workspace_bytes(const kvattn_config* cfg, size_t* bytes) {
    int rc = validate_config(cfg);
    if (rc) return rc;
    if (!bytes) return fail(KVATTN_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = workspace_size(*cfg, workspace_rows(*cfg));
    return KVATTN_OK;
}

int kvattn_create(const kvattn_config* cfg, kvattn_handle** out) {
    if (!out) return fail(KVATTN_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int rc = validate_config(cfg);
    if (rc) return rc;
    kvattn_handle* h = new (std::nothrow) kvattn_handle();
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "host allocation failed");
    h->cfg = *cfg;
    h->stream = nullptr;
    h->batch = cfg->max_batch;
    h->forced_split_len = 0;
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
    if (e != hipSuccess) {
        delete h;
        return fail(KVATTN_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    }
    for (int& r : h->resident) r = 0;
    h->ws_rows = workspace_rows(*cfg);
    h->n_units = counter_units(*cfg);
    // the merge addresses partials with 32-bit byte offsets
    if ((double)h->ws_rows * cfg->head_dim * sizeof(float) >= 2147483648.0) {
        delete h;
        return fail(KVATTN_ERR_CAPACITY, "workspace would exceed 2 GiB; lower max_batch or max_q_len");
    }
    const size_t bytes = workspace_size(*cfg, h->ws_rows);
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

int kvattn_set_split_len(kvattn_handle* h, int32_t split_len) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    if (split_len < 0 || split_len % kSplitQuantum)
        return fail(KVATTN_ERR_INVALID_ARG, "split_len must be 0 or a positive multiple of 64");
    h->forced_split_len = split_len;
    return KVATTN_OK;
}

int kvattn_plan(kvattn_handle* h, int32_t q_len, int32_t mask_mode, int32_t n_sink,
                int32_t window, int32_t* n_split, int32_t* split_len, int32_t* kernel) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    int rc = validate_decode_args(h, q_len, mask_mode, n_sink, window);
    if (rc) return rc;
    int ns, len;
    rc = plan_for(h, q_len, mask_mode, n_sink, window, &ns, &len);
    if (rc) return rc;
    if (n_split) *n_split = ns;
    if (split_len) *split_len = len;
    if (kernel) *kernel = use_mfma(h->cfg, q_len) ? 1 : 0;
    return KVATTN_OK;
}

static void fill_params(const kvattn_handle* h, kvattn::DecodeParams& p, const void* q,
                        const void* k, const void* v, const int32_t* bt, const int32_t* sl,
                        int32_t q_len, int32_t mask_mode, int32_t n_sink, int32_t window,
                        void* out, int n_split, int split_len) {
    const kvattn_config& c = h->cfg;
    p.q = q;
    p.k = k;
    p.v = v;
    p.block_table = bt;
    p.seq_lens = sl;
    p.out = out;
    p.ws_acc = h->ws;
    p.ws_ml = h->ws + h->ws_rows * c.head_dim;
    p.counters = reinterpret_cast<int32_t*>(h->ws + h->ws_rows * (c.head_dim + 2));
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
    p.n_split = n_split;
    p.split_len = split_len;
    const float scale = c.scale > 0.0f ? c.scale : 1.0f / std::sqrt((float)c.head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;
}

int kvattn_decode(kvattn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens, int32_t q_len,
                  int32_t mask_mode, int32_t n_sink, int32_t window, void* out) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    int rc = validate_decode_args(h, q_len, mask_mode, n_sink, window);
    if (rc) return rc;
    if (h->batch == 0) return KVATTN_OK;
    if (!q || !k_cache || !v_cache || !seq_lens || !out)
        return fail(KVATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, seq_lens and out must be non-NULL");
    if ((h->cfg.cache_mode == KVATTN_PAGED) != (block_table != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "block_table must be given exactly for a paged cache");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(KVATTN_ERR_INVALID_ARG, "q, caches and out must be 16-byte aligned");
    int ns, len;
    rc = plan_for(h, q_len, mask_mode, n_sink, window, &ns, &len);
    if (rc) return rc;
    kvattn::DecodeParams p;
    fill_params(h, p, q, k_cache, v_cache, block_table, seq_lens, q_len, mask_mode, n_sink,
                window, out, ns, len);
    hipError_t e = use_mfma(h->cfg, q_len)
                       ? kvattn::launch_decode_mfma(p, h->cfg.dtype, h->cfg.head_dim, h->stream)
                       : kvattn::launch_decode_valu(p, h->cfg.dtype, h->cfg.head_dim, h->stream);
    if (e != hipSuccess)
        return fail(KVATTN_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

int kvattn_debug_gather(kvattn_handle* h, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t q_len, int32_t mask_mode, int32_t n_sink, int32_t window,
                        int32_t max_slots, int32_t* slots_out, int32_t* counts_out) {
    if (!h) return fail(KVATTN_ERR_INVALID_ARG, "handle is NULL");
    int rc = validate_decode_args(h, q_len, mask_mode, n_sink, window);
    if (rc) return rc;
    if (h->batch == 0) return KVATTN_OK;
    if (!seq_lens || !slots_out || !counts_out || max_slots < 0)
        return fail(KVATTN_ERR_INVALID_ARG, "seq_lens, slots_out and counts_out must be non-NULL");
    if ((h->cfg.cache_mode == KVATTN_PAGED) != (block_table != nullptr))
        return fail(KVATTN_ERR_INVALID_ARG, "block_table must be given exactly for a paged cache");
    kvattn::DecodeParams p;
    fill_params(h, p, nullptr, nullptr, nullptr, block_table, seq_lens, q_len, mask_mode, n_sink,
                window, nullptr, 1, 1 << 30);
    hipError_t e = kvattn::launch_debug_gather(p, max_slots, slots_out, counts_out, h->stream);
    if (e != hipSuccess)
        return fail(KVATTN_ERR_HIP, std::string("gather launch: ") + hipGetErrorString(e));
    return KVATTN_OK;
}

}  // extern "C"
