// Log-sum-exp merge of split-KV partials, run by the last workgroup of a
// segment (sequence, KV head, row block) to finish its piece.
//
// Each piece k of a segment leaves, per row r, its normalised rows o_k[d] = acc_k[d] /
// l_k and its running max m_k and sum l_k (exp2 domain) in workspace slot slot0 + k,
// row r (slot-major: index (slot * seg_rows + r)).  The row's result is
//     M = max_k m_k,  L = sum_k l_k 2^(m_k - M),  out = sum_k l_k 2^(m_k - M) o_k / L
// - the same rescaling identity the online softmax applies across tiles (Flash
// Attention section of the nextadmin.net lesson "KV cache and Flash Attention"),
// applied once more across pieces.  Empty pieces (m = -inf, l = 0) weigh 0.
//
// The rows o_k are kept in the query's type for 16-bit queries (rounded to nearest
// even, half the bytes of fp32: a bounded value, |o_k| <= max |v|, rounded once more
// than the output is) and in fp32 for fp32 queries; (m_k, l_k) are fp32.
//
// Arrival protocol: every workgroup of a segment writes its partial with
// device-scope stores (they write through the per-XCD L2 to the device-coherent
// level), waits until they are acknowledged, and takes a ticket from the
// segment's counter with a device-scope atomic.  The workgroup that draws the
// last ticket reads the partials with device-scope loads (which do not hit a
// possibly stale L2 line), merges, and puts the counter back to zero for the next
// call.  No L2-wide write-back or invalidate is needed - a per-workgroup full-L2
// fence would cost more than the whole piece - and nothing waits on another
// workgroup, so no schedule can hang.
#pragma once

#include "device_common.hpp"

namespace kvattn {

template <int DT>
__device__ __forceinline__ void store_elem(void* out, int64_t idx, float x) {
    if constexpr (DT == F32)
        reinterpret_cast<float*>(out)[idx] = x;
    else if constexpr (DT == F16)
        reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(x);
    else
        reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(x);
}

// Row id (in out's [batch, q_len, Hq] order) of row rg of KV head kvh.
__device__ __forceinline__ int64_t row_id_of(const DecodeParams& p, int b, int kvh, int rg) {
    const int i = rg / p.group;
    const int h = kvh * p.group + (rg - i * p.group);
    return ((int64_t)b * p.q_len + i) * p.num_q_heads + h;
}

// Device-scope (cross-XCD coherent) partial stores and loads.
__device__ __forceinline__ void store_partial(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Vector loads of partials with the device-scope cache policy (SC1: the load is
// served from the device-coherent level, never from a stale per-XCD L2 line),
// through a buffer resource over the partial arrays (byte offsets < 2^31, which
// the host guarantees by bounding the workspace).
constexpr int kCachePolicyDevice = 16;  // SC1
constexpr int kBufferDword3 = 0x00020000;

// Bits of x in the partial rows' type (16-bit queries).
template <int DT>
__device__ __forceinline__ uint32_t part_bits(float x) {
    return DT == F16 ? f32_to_f16_bits(x) : f32_to_bf16_bits(x);
}
template <int DT>
__device__ __forceinline__ float part_value(uint32_t w16) {
    if constexpr (DT == F16) return f16_lo(w16);
    else return bf16_lo(w16);
}

// Two floats as a pair of 16-bit values (lo in the low half), rounded to nearest even
// by the conversion instructions.
template <int DT>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {lo, hi};
    if constexpr (DT == F16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Vector device-scope stores of four normalised partial elements starting at element
// `elem` (same buffer resources as the reader).
template <int DT>
__device__ __forceinline__ void store_partial4(const DecodeParams& p, int64_t elem, float4 o) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(p.ws_acc, 0, 0x7fffffff, kBufferDword3);
    if constexpr (DT == F32) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u4 w = {__float_as_uint(o.x), __float_as_uint(o.y), __float_as_uint(o.z),
                      __float_as_uint(o.w)};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)(elem * 4), 0, kCachePolicyDevice);
    } else {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 w = {pack_pair<DT>(o.x, o.y), pack_pair<DT>(o.z, o.w)};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)(elem * 2), 0, kCachePolicyDevice);
    }
}
// One normalised partial element.
template <int DT>
__device__ __forceinline__ void store_partial1(const DecodeParams& p, int64_t elem, float o) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(p.ws_acc, 0, 0x7fffffff, kBufferDword3);
    if constexpr (DT == F32)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), r, (int)(elem * 4), 0,
                                              kCachePolicyDevice);
    else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)part_bits<DT>(o), r, (int)(elem * 2), 0,
                                              kCachePolicyDevice);
}
__device__ __forceinline__ void store_partial_ml(const DecodeParams& p, int64_t part, float m,
                                                 float l) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(p.ws_ml, 0, 0x7fffffff, 0x00020000);
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 w = {__float_as_uint(m), __float_as_uint(l)};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)(part * 8), 0, kCachePolicyDevice);
}

struct PartialReader {
    __amdgpu_buffer_rsrc_t acc, ml;
    __device__ PartialReader(const DecodeParams& p)
        : acc(__builtin_amdgcn_make_buffer_rsrc(p.ws_acc, 0, 0x7fffffff, kBufferDword3)),
          ml(__builtin_amdgcn_make_buffer_rsrc(p.ws_ml, 0, 0x7fffffff, kBufferDword3)) {}
    // four normalised partial elements starting at element `elem`
    template <int DT>
    __device__ float4 acc4(int64_t elem) const {
        if constexpr (DT == F32) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(acc, (int)(elem * 4), 0,
                                                                 kCachePolicyDevice);
            return float4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                          __uint_as_float(v[3])};
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(acc, (int)(elem * 2), 0,
                                                                kCachePolicyDevice);
            return float4{part_value<DT>(v[0] & 0xffffu), part_value<DT>(v[0] >> 16),
                          part_value<DT>(v[1] & 0xffffu), part_value<DT>(v[1] >> 16)};
        }
    }
    // (m, l) of partial `part`
    __device__ float2 ml2(int64_t part) const {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(ml, (int)(part * 8), 0,
                                                            kCachePolicyDevice);
        return float2{__uint_as_float(v[0]), __uint_as_float(v[1])};
    }
};

// Partials per segment up to which the merge computes each row's weights once (and
// keeps them in LDS); beyond it, it folds the partials in with the running rescaling.
constexpr int kWeightParts = 16;

// Shared memory the merge needs (floats); W: with room for the two-pass form's weights.
template <int NROWS, int THREADS, bool W = false>
struct MergeSmem {
    float4 red[THREADS];                 // split groups' accumulators ...
    float2 red_ml[THREADS];              // ... and their running (max, sum)
    float w[W ? NROWS : 1][kWeightParts];  // row r's weight of partial k
};

// Four consecutive output elements, rounded to nearest even, in one store (the output
// and every row of it are 16-byte aligned).
template <int DT>
__device__ __forceinline__ void store_out4(void* out, int64_t idx, float4 v) {
    if constexpr (DT == F32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = v;
    } else {
        const uint2 w = {pack_pair<DT>(v.x, v.y), pack_pair<DT>(v.z, v.w)};
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = w;
    }
}

// The merge of more than kWeightParts partials (merge_partials below).
//
// One pass over the partials: each thread owns float4 chunks of (row, d) - split
// groups share the threads left over - and folds the partials in as it reads them,
// with the same rescaling identity:
//     M' = max(M, m_k),  L' = L 2^(M - M') + l_k 2^(m_k - M'),  A' = A 2^(M - M') + l_k o_k 2^(m_k - M').
// Every load of a step (US partials x the thread's chunks, accumulators and (max,
// sum) words together) is issued before any is used, so a merge of up to US x split
// groups partials costs one memory latency.
template <int DT, int D, int NROWS, int THREADS, bool W>
__device__ __forceinline__ void merge_online(const DecodeParams& p, int b, int kvh, int row0,
                                             int64_t slot0, int nvalid,
                                             MergeSmem<NROWS, THREADS, W>& sm, int roff) {
    static_assert(THREADS % 64 == 0, "whole waves");
    const int tid = threadIdx.x;
    constexpr float NEG_INF = -__builtin_inff();
    const int NR = p.seg_rows;  // partial k of row r: index (slot0 + k) * NR + r
    const PartialReader rd(p);

    constexpr int E4 = NROWS * D / 4;
    constexpr int SG = E4 >= THREADS ? 1 : THREADS / E4;
    constexpr int EPT = E4 >= THREADS ? (E4 + THREADS - 1) / THREADS : 1;
    constexpr int US = 4;  // partials per step
    static_assert(E4 >= THREADS || THREADS % E4 == 0, "shape");
    static_assert(SG == 1 || EPT == 1, "split groups hold one chunk each");
    const int sg = E4 >= THREADS ? 0 : tid / E4;
    int e4[EPT], r[EPT];
    bool live[EPT];
    int64_t part0[EPT];
    float mx[EPT], ls[EPT];
    float4 a[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = E4 >= THREADS ? tid + k * THREADS : tid % E4;
        const bool in = e < E4;  // chunks past the last one (E4 not a multiple of THREADS)
        e4[k] = in ? e : 0;
        r[k] = e4[k] / (D / 4);
        live[k] = in && row0 + r[k] < p.rows;
        part0[k] = live[k] ? slot0 * NR + roff + r[k] : 0;
        mx[k] = NEG_INF;
        ls[k] = 0.0f;
        a[k] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // folds (m, l, acc) into the thread's running (mx, ls, a)
    auto fold = [&](int k, float m, float l, float4 v) __attribute__((always_inline)) {
        const float mn = fmaxf(mx[k], m);
        const float mu = mn == NEG_INF ? 0.0f : mn;
        const float fa = fast_exp2(mx[k] - mu);  // 0 while nothing was folded in
        const float fb = fast_exp2(m - mu);      // 0 for an empty piece
        ls[k] = ls[k] * fa + l * fb;
        a[k].x = a[k].x * fa + v.x * fb;
        a[k].y = a[k].y * fa + v.y * fb;
        a[k].z = a[k].z * fa + v.z * fb;
        a[k].w = a[k].w * fa + v.w * fb;
        mx[k] = mn;
    };
    for (int sp0 = sg; sp0 < nvalid; sp0 += US * SG) {
        float4 v[US][EPT];
        float2 w[US][EPT];
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int sp = sp0 + u * SG;
            const int spc = sp < nvalid ? sp : sg;  // clamped: a valid partial, weight 0
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int64_t part = part0[k] + (int64_t)spc * NR;
                v[u][k] = rd.template acc4<DT>(part * D + (e4[k] % (D / 4)) * 4);
                w[u][k] = rd.ml2(part);
            }
        }
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const bool in = sp0 + u * SG < nvalid;
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const float l = in ? w[u][k].y : 0.0f;  // acc = l * o
                const float4 o = v[u][k];
                fold(k, in ? w[u][k].x : NEG_INF, l, float4{o.x * l, o.y * l, o.z * l, o.w * l});
            }
        }
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        if constexpr (SG > 1) {
            sm.red[tid] = a[k];
            sm.red_ml[tid] = float2{mx[k], ls[k]};
            __syncthreads();
            if (sg == 0) {
                // groups g >= nvalid were given no partial: their state is empty and
                // folding it in changes nothing (factor 1 on the sum, 0 on it), so with
                // many groups (one or two rows) the fold stops at nvalid
                const int ng = SG > 4 ? (nvalid < SG ? nvalid : SG) : SG;
                for (int g2 = 1; g2 < ng; ++g2) {
                    const float2 o = sm.red_ml[g2 * E4 + e4[k]];
                    fold(k, o.x, o.y, sm.red[g2 * E4 + e4[k]]);
                }
            }
        }
        if (sg == 0 && live[k]) {
            const float inv = ls[k] > 0.0f ? 1.0f / ls[k] : 0.0f;
            const int64_t o = row_id_of(p, b, kvh, row0 + r[k]) * D + (e4[k] % (D / 4)) * 4;
            store_elem<DT>(p.out, o, a[k].x * inv);
            store_elem<DT>(p.out, o + 1, a[k].y * inv);
            store_elem<DT>(p.out, o + 2, a[k].z * inv);
            store_elem<DT>(p.out, o + 3, a[k].w * inv);
        }
    }
}

// The same merge in two passes, for up to kWeightParts partials: one thread per row
// reads the row's (max, sum) words and computes its weights
//     w_k = l_k 2^(m_k - M) / L,   M = max_k m_k,  L = sum_k l_k 2^(m_k - M)
// once, into LDS; then every output element is sum_k w_k o_k - four fused multiply-adds
// per partial for four elements, where the running rescaling costs two exponentials, a
// maximum and a dozen multiplies per partial and element group.  The rows of the
// first partials are requested before the weights are worked out, so their latency and
// that of the (max, sum) words overlap.
template <int DT, int D, int NROWS, int THREADS>
__device__ __forceinline__ void merge_weighted(const DecodeParams& p, int b, int kvh, int row0,
                                               int64_t slot0, int nvalid,
                                               MergeSmem<NROWS, THREADS, true>& sm, int roff) {
    static_assert(THREADS % 64 == 0 && NROWS <= THREADS, "whole waves, a thread per row");
    const int tid = threadIdx.x;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr int KW = kWeightParts;
    const int NR = p.seg_rows;  // partial k of row r: index (slot0 + k) * NR + r
    const PartialReader rd(p);

    constexpr int E4 = NROWS * D / 4;
    constexpr int SG = E4 >= THREADS ? 1 : THREADS / E4;
    constexpr int EPT = E4 >= THREADS ? (E4 + THREADS - 1) / THREADS : 1;
    constexpr int US = 4;  // partials per step
    static_assert(E4 >= THREADS || THREADS % E4 == 0, "shape");
    static_assert(SG == 1 || EPT == 1, "split groups hold one chunk each");
    const int sg = E4 >= THREADS ? 0 : tid / E4;
    int e4[EPT], r[EPT];
    bool live[EPT];
    int64_t part0[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e = E4 >= THREADS ? tid + k * THREADS : tid % E4;
        const bool in = e < E4;
        e4[k] = in ? e : 0;
        r[k] = e4[k] / (D / 4);
        live[k] = in && row0 + r[k] < p.rows;
        part0[k] = live[k] ? slot0 * NR + roff + r[k] : 0;
    }
    // partials sg, sg + SG, ... of this thread's chunks, US at a time (past nvalid:
    // partial 0 again, weighted 0)
    float4 v[US][EPT];
    auto load_step = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int kk = k0 + u * SG;
            const int kc = kk < nvalid ? kk : 0;
#pragma unroll
            for (int k = 0; k < EPT; ++k)
                v[u][k] = rd.template acc4<DT>((part0[k] + (int64_t)kc * NR) * D +
                                               (e4[k] % (D / 4)) * 4);
        }
    };
    load_step(sg);

    if (tid < NROWS && row0 + tid < p.rows) {
        float2 ml[KW];
#pragma unroll
        for (int k = 0; k < KW; ++k)
            ml[k] = k < nvalid ? rd.ml2((slot0 + k) * NR + roff + tid) : float2{NEG_INF, 0.0f};
        float M = NEG_INF;
#pragma unroll
        for (int k = 0; k < KW; ++k) M = fmaxf(M, ml[k].x);
        const float Mu = M == NEG_INF ? 0.0f : M;
        float e[KW], L = 0.0f;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            e[k] = ml[k].y * fast_exp2(ml[k].x - Mu);  // 0 for an empty piece or k >= nvalid
            L += e[k];
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
        for (int k = 0; k < KW; ++k) sm.w[tid][k] = e[k] * inv;
    }
    __syncthreads();  // the weights are in LDS

    float4 a[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) a[k] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    auto accumulate = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int kk = k0 + u * SG;
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const float w = kk < nvalid ? sm.w[r[k]][kk] : 0.0f;
                a[k].x = fmaf(w, v[u][k].x, a[k].x);
                a[k].y = fmaf(w, v[u][k].y, a[k].y);
                a[k].z = fmaf(w, v[u][k].z, a[k].z);
                a[k].w = fmaf(w, v[u][k].w, a[k].w);
            }
        }
    };
    accumulate(sg);
    for (int k0 = sg + US * SG; k0 < nvalid; k0 += US * SG) {
        load_step(k0);
        accumulate(k0);
    }
    if constexpr (SG > 1) {  // the split groups' sums, in group order
        sm.red[tid] = a[0];
        __syncthreads();
        if (sg == 0) {
            for (int g2 = 1; g2 < SG && g2 < nvalid; ++g2) {  // later groups hold zeros
                const float4 o = sm.red[g2 * E4 + e4[0]];
                a[0].x += o.x;
                a[0].y += o.y;
                a[0].z += o.z;
                a[0].w += o.w;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k)
        if (sg == 0 && live[k])
            store_out4<DT>(p.out, row_id_of(p, b, kvh, row0 + r[k]) * D + (e4[k] % (D / 4)) * 4,
                           a[k]);
}

// Merges the nvalid partials of rows row0 .. row0 + NROWS - 1 of KV head kvh (rows
// roff .. of slots slot0 ..) into the output and puts the segment's counter back to
// zero.  Called by every thread of the workgroup that drew the segment's last ticket.
// With a scratch that has room for weights (W), the two-pass form where it applies: the
// matrix-core decode kernel, whose registers hold both forms (in the vector-ALU
// kernels the second form pushed scalar values out of registers inside the tile loop).
template <int DT, int D, int NROWS, int THREADS, bool W>
__device__ __forceinline__ void merge_partials(const DecodeParams& p, int b, int kvh, int row0,
                                               int64_t unit, int64_t slot0, int nvalid,
                                               MergeSmem<NROWS, THREADS, W>& sm, int roff = 0) {
    bool done = false;
    if constexpr (W) {
        if (nvalid <= kWeightParts) {
            merge_weighted<DT, D, NROWS, THREADS>(p, b, kvh, row0, slot0, nvalid, sm, roff);
            done = true;
        }
    }
    if (!done) merge_online<DT, D, NROWS, THREADS>(p, b, kvh, row0, slot0, nvalid, sm, roff);
    if (threadIdx.x == 0) atomicExch(p.counters + unit, 0);  // ready for the next call
}

// Called by every thread of the workgroup after it wrote its partial into slot
// slot0 + (its piece) of segment `unit`: takes the segment's ticket once every
// thread's stores are acknowledged; true for the workgroup that drew the last one.
__device__ __forceinline__ bool arrive(const DecodeParams& p, int64_t unit, int nvalid) {
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
    __syncthreads();                 // ... and every other thread's
    if (threadIdx.x == 0) s_last = atomicAdd(p.counters + unit, 1) == nvalid - 1;
    __syncthreads();
    return s_last;
}

// arrive, then (last workgroup of the segment) merge rows row0 .. row0 + NROWS - 1.
template <int DT, int D, int NROWS, int THREADS, bool W>
__device__ __forceinline__ void arrive_and_merge(const DecodeParams& p, int b, int kvh, int row0, int64_t unit,
                                 int64_t slot0, int nvalid, MergeSmem<NROWS, THREADS, W>& sm) {
    if (arrive(p, unit, nvalid))
        merge_partials<DT, D, NROWS, THREADS>(p, b, kvh, row0, unit, slot0, nvalid, sm);
}

}  // namespace kvattn
