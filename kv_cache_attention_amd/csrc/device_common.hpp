// Device-side building blocks shared by every kernel of the library: the
// per-launch parameter block, the attended-set and gather arithmetic (the one
// definition of which cache slot holds which position), element conversions
// and wavefront reductions.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvattn {

enum : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };  // FP8: OCP E4M3 codes
enum : int { CONTIGUOUS = 0, PAGED = 1, RING = 2 };
enum : int { MASK_CAUSAL = 0, MASK_SINK_WINDOW = 1, MASK_TREE = 2 };

// Everything a decode launch needs, passed by value as the kernel argument.
// Largest flat range (position-units: attended positions x segments, summed over the
// batch) of one launch; the host cuts a launch over batch ranges to stay within it, so
// the plan's indices are 32-bit with room for a unit past the end.
constexpr int32_t kFlatMax = 1 << 30;

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* out;
    float* ws_acc;        // [slots, seg_rows, D]  partial rows of split segments, normalised:
                          // the query type for 16-bit queries, fp32 for fp32 queries
    float* ws_ml;         // [slots, seg_rows, 2]  (running max m, sum l), log2 domain
    int32_t* counters;    // [batch, Hkv, row blocks] arrivals per segment, 0 between calls
    int32_t* queue;       // [2]: units taken beyond the first per workgroup, workgroups done
    int64_t stride_seq;   // elements: sequence (contiguous/ring) or block (paged)
    int64_t stride_head;  // elements: KV head
    int64_t stride_tok;   // elements: slot within a sequence / block
    int32_t batch, num_q_heads, num_kv_heads, group, q_len, rows;
    int32_t cache_mode, mask_mode, n_sink, window;
    int32_t capacity, log2_block, num_blocks, blocks_per_seq;
    int32_t row_blocks;   // segments per (sequence, KV head): blocks of query rows
    int32_t segs_per_seq; // num_kv_heads * row_blocks
    int32_t seg_rows;     // rows per segment as laid out in the workspace
    int32_t min_chunk;    // smallest unit (positions)
    int32_t units_per_wg; // units per workgroup the flat range is cut into (0: units of
                          // exactly min_chunk positions)
    int32_t tail_pct;     // share (percent) of the flat range left to a dynamic tail (0: none)
    int32_t tail_units;   // tail units per workgroup
    int32_t deterministic;  // waves take fixed tiles instead of a shared queue
    const float* k_scale; // 8-bit caches: [Hkv] dequantisation scales (else NULL)
    const float* v_scale;
    const uint64_t* tree_mask;  // MASK_TREE: [batch, q_len] words, bit j = attends new position j
    // Append fused into the decode: [batch, q_len, Hkv, D] rows of the cache's element
    // type for positions T - q_len .. T - 1, written to their slots by the workgroups
    // that read them (NULL: the caches already hold them)
    const char* k_new;
    const char* v_new;
    float scale_log2;     // softmax scale * log2(e): scores are kept in the exp2 domain
};

// Lazy rescaling of the running softmax: a row's reference maximum moves only when a
// score exceeds it by more than 2^RESCALE_SLACK (log2 units).  Until then the weights
// exp2(s - m) stay below 2^RESCALE_SLACK, well inside the range of the 16-bit types
// they may be packed to, and O and the row sum keep one common reference, so the
// normalised result is the same quantity; the accumulators are rescaled far less often.
constexpr float RESCALE_SLACK = 8.0f;

// The attended positions of one sequence, over all q_len new rows, are the union
// [0, sink) + [tail, T): sink positions (attention sinks) and one trailing run.
// Work is indexed by j in [0, count): j < sink -> position j, else tail + (j - sink).
struct SeqSpan {
    int32_t T;      // clamped length
    int32_t sink;   // attended sink positions
    int32_t tail;   // first position of the trailing run
    int32_t count;  // attended positions in the union
    int32_t ring_pos0;  // RING: first attended position at or past n_sink ...
    int32_t ring0;      // ... and its offset within the rolling slots
};

// The span of a sequence whose length (as seq_lens holds it) is T.
__device__ __forceinline__ SeqSpan seq_span_of(const DecodeParams& p, int32_t T) {
    SeqSpan s;
    if (T < 0) T = 0;
    // Contiguous and paged caches cannot hold more than `capacity` positions.
    if (p.cache_mode != RING && T > p.capacity) T = p.capacity;
    s.T = T;
    s.sink = 0;
    s.tail = 0;
    if (p.mask_mode == MASK_SINK_WINDOW) {
        const int32_t sk = min(p.n_sink, T);
        // first position any row's window reaches: row 0 sits at T - q_len
        const int64_t w0 = max<int64_t>((int64_t)T - p.q_len - p.window + 1, 0);
        if (w0 > sk) {
            s.sink = sk;
            s.tail = (int32_t)w0;
        }
    }
    s.count = s.sink + (T - s.tail);
    // Ring slots: positions past the sinks roll over R = capacity - n_sink slots.  The
    // attended ones past the sinks are consecutive and span at most R positions, so
    // their slots follow from one modulo at the first of them.
    s.ring_pos0 = max(s.tail, p.n_sink);
    s.ring0 = 0;
    if (p.cache_mode == RING && p.n_sink < p.capacity)
        s.ring0 = (s.ring_pos0 - p.n_sink) % (p.capacity - p.n_sink);
    return s;
}

__device__ __forceinline__ SeqSpan seq_span(const DecodeParams& p, int b) {
    return seq_span_of(p, p.seq_lens[b]);
}

// Logical position of work index j.
__device__ __forceinline__ int32_t span_pos(const SeqSpan& s, int32_t j) {
    return j < s.sink ? j : s.tail + (j - s.sink);
}

// Where position `pos` of sequence b lives: `unit` is the sequence (contiguous,
// ring) or the pool block (paged) and `idx` the slot inside it.  unit < 0 when the
// page table names a block outside the pool (the position is then skipped).
struct Loc {
    int64_t unit;
    int32_t idx;
};

template <int CACHE>
__device__ __forceinline__ Loc locate(const DecodeParams& p, const SeqSpan& s, int b,
                                      int32_t pos) {
    Loc l;
    if constexpr (CACHE == CONTIGUOUS) {
        (void)s;
        l.unit = b;
        l.idx = pos;
    } else if constexpr (CACHE == RING) {
        l.unit = b;
        if (pos < p.n_sink) {
            l.idx = pos;  // sinks are never evicted
        } else {
            const int32_t R = p.capacity - p.n_sink;
            int32_t r = s.ring0 + (pos - s.ring_pos0);
            if (r >= R) r -= R;
            l.idx = p.n_sink + r;
        }
    } else {
        (void)s;
        const int32_t blk = p.block_table[(int64_t)b * p.blocks_per_seq + (pos >> p.log2_block)];
        l.unit = (uint32_t)blk < (uint32_t)p.num_blocks ? (int64_t)blk : -1;
        l.idx = pos & ((1 << p.log2_block) - 1);
    }
    return l;
}

// Paged caches in two steps, so the page-table read can be issued ahead of use:
// the table entry of position pos, then the location it gives.
__device__ __forceinline__ int32_t page_entry(const DecodeParams& p, int b, int32_t pos) {
    return p.block_table[(int64_t)b * p.blocks_per_seq + (pos >> p.log2_block)];
}
__device__ __forceinline__ Loc paged_loc(const DecodeParams& p, int32_t blk, int32_t pos) {
    Loc l;
    l.unit = (uint32_t)blk < (uint32_t)p.num_blocks ? (int64_t)blk : -1;
    l.idx = pos & ((1 << p.log2_block) - 1);
    return l;
}

// Element offset of the (location, KV head) row of a cache.  Slot indices are
// non-negative and the strides of a position and of a page block are below 2^32 (the
// host checks the block's at create), so a lane's share is one 32 x 32 -> 64-bit
// product; the sequence's and the head's shares are the same across the workgroup.
template <int CACHE>
__device__ __forceinline__ int64_t row_offset(const DecodeParams& p, const Loc& l, int kvh) {
    const uint64_t slot = (uint64_t)(uint32_t)l.idx * (uint32_t)p.stride_tok;
    if constexpr (CACHE == PAGED)
        return (int64_t)((uint64_t)(uint32_t)l.unit * (uint32_t)p.stride_seq + slot) +
               (int64_t)kvh * p.stride_head;
    else
        return l.unit * p.stride_seq + (int64_t)kvh * p.stride_head + (int64_t)slot;
}

// Flat slot index, independent of the layout: b * capacity + slot, or
// block * block_size + offset.
template <int CACHE>
__device__ __forceinline__ int64_t flat_slot(const DecodeParams& p, const Loc& l) {
    if (l.unit < 0) return -1;
    if constexpr (CACHE == PAGED)
        return (l.unit << p.log2_block) + l.idx;
    else
        return l.unit * p.capacity + l.idx;
}

// Does new row i (query position T - q_len + i) of sequence b attend position pos?
__device__ __forceinline__ bool row_attends(const DecodeParams& p, const SeqSpan& s, int b,
                                            int i, int32_t pos) {
    const int32_t P0 = s.T - p.q_len;
    if (p.mask_mode == MASK_TREE) {
        if (pos < P0) return true;
        return pos < s.T && ((p.tree_mask[(int64_t)b * p.q_len + i] >> (pos - P0)) & 1);
    }
    const int32_t P = P0 + i;
    if (pos > P) return false;
    if (p.mask_mode == MASK_CAUSAL) return true;
    return pos < p.n_sink || pos >= P - p.window + 1;
}

// ---------------------------------------------------------------- element types

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));

template <int DT> struct Elem;
template <> struct Elem<F32> { static constexpr int bytes = 4; };
template <> struct Elem<F16> { static constexpr int bytes = 2; };
template <> struct Elem<BF16> { static constexpr int bytes = 2; };
template <> struct Elem<FP8> { static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Round-to-nearest-even stores.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---------------------------------------------------------------- cross-lane sums

// Sum over aligned groups of N lanes (N = 4, 8, 16 or 32); every lane of the group
// receives the same value.  Steps pair lanes with commutative adds, so all lanes
// hold bit-identical results.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
    // quad_perm [1,0,3,2]: swap neighbours
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, false);
    // quad_perm [2,3,0,1]: swap pairs
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, false);
    if constexpr (N == 4) return x;
    // row_half_mirror: lane i <-> 7 - i within each 8
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, false);
    if constexpr (N >= 16) {
        // row_mirror: lane i <-> 15 - i within each 16
        x += __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, false);
    }
    if constexpr (N == 32) {
        x += __shfl_xor(x, 16, 64);
    }
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x, unknown to the optimiser from here on (an empty asm statement that claims to
// change it): arithmetic on the result stays where the source puts it.  Per-thread
// offsets used only after a piece's first loads (LDS slots, Q rows, the epilogue's
// chunks) would otherwise be computed once ahead of the whole unit loop - before any
// K/V load goes out, at one wave per SIMD - and held in registers (or spilled) across it.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// K/V stream loads: each cached byte is read once per step, so the loads carry the
// nontemporal hint (global_load ... nt), which keeps the stream from displacing
// cache lines other data still needs; measured on MI355X, plain reads of a 512 MiB
// buffer ran about 10 % faster with it.
template <typename T>
__device__ __forceinline__ T load_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

}  // namespace kvattn
