// Log-sum-exp merge of split-KV partials, run by the last workgroup of a
// (sequence, KV head, row block) to finish.
//
// Each split s leaves, per row, its unnormalised accumulator acc_s[d] and its
// running max m_s and sum l_s (exp2 domain).  The row's result is
//     M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  out = sum_s acc_s 2^(m_s - M) / L
// - the same rescaling identity the online softmax applies across tiles (Flash
// Attention section of the nextadmin.net lesson "KV cache and Flash Attention"),
// applied once more across splits.  Empty splits (m = -inf, l = 0) weigh 0.
//
// Arrival protocol: every workgroup of a unit writes its partial with
// device-scope stores (they write through the per-XCD L2 to the device-coherent
// level), waits until they are acknowledged, and takes a ticket from the unit's
// counter with a device-scope atomic.  The workgroup that draws the last ticket
// reads the partials with device-scope loads (which do not hit a possibly stale
// L2 line), merges, and puts the counter back to zero for the next call.  No
// L2-wide write-back or invalidate is needed - a per-workgroup full-L2 fence
// would cost more than the whole split - and nothing waits on another
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
__device__ __forceinline__ float load_partial(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Shared memory the merge needs (floats).
template <int NROWS, int THREADS>
struct MergeSmem {
    float M[NROWS];
    float L[NROWS];
    float4 red[THREADS];
};

// Called by every thread of the workgroup after it wrote its partial.  Returns
// after the merge (last workgroup) or right away (the others).
template <int DT, int D, int NROWS, int THREADS>
__device__ void arrive_and_merge(const DecodeParams& p, int b, int kvh, int row0, int unit,
                                 int nvalid, MergeSmem<NROWS, THREADS>& sm) {
    static_assert(THREADS % 64 == 0, "whole waves");
    __shared__ int s_last;
    const int tid = threadIdx.x;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
    __syncthreads();                 // ... and every other thread's
    if (tid == 0) s_last = atomicAdd(p.counters + unit, 1) == nvalid - 1;
    __syncthreads();
    if (!s_last) return;

    constexpr float NEG_INF = -__builtin_inff();
    constexpr int NW = THREADS / 64;
    const int wave = tid / 64, lane = tid % 64;
    const int n_split = p.n_split;

    // per row: M and L over the splits (one wave per row, lanes across splits)
    for (int r = wave; r < NROWS; r += NW) {
        const int rg = row0 + r;
        if (rg >= p.rows) continue;
        const float* ml = p.ws_ml + row_id_of(p, b, kvh, rg) * n_split * 2;
        float mx = NEG_INF;
        for (int sp = lane; sp < nvalid; sp += 64) mx = fmaxf(mx, load_partial(ml + sp * 2));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float mu = mx == NEG_INF ? 0.0f : mx;
        float ls = 0.0f;
        for (int sp = lane; sp < nvalid; sp += 64)
            ls += load_partial(ml + sp * 2 + 1) * fast_exp2(load_partial(ml + sp * 2) - mu);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
        if (lane == 0) {
            sm.M[r] = mu;
            sm.L[r] = ls;
        }
    }
    __syncthreads();

    // accumulators: float4 chunks of (row, d); split groups share the remaining threads
    constexpr int E4 = NROWS * D / 4;
    constexpr int SG = E4 >= THREADS ? 1 : THREADS / E4;
    constexpr int EPT = E4 >= THREADS ? E4 / THREADS : 1;
    static_assert(E4 >= THREADS ? E4 % THREADS == 0 : THREADS % E4 == 0, "shape");
    const int sg = E4 >= THREADS ? 0 : tid / E4;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
        const int e4 = E4 >= THREADS ? tid + k * THREADS : tid % E4;
        const int r = e4 / (D / 4);
        const int d4 = e4 - r * (D / 4);
        const int rg = row0 + r;
        float4 a = {0.0f, 0.0f, 0.0f, 0.0f};
        int64_t rid = 0;
        if (rg < p.rows) {
            rid = row_id_of(p, b, kvh, rg);
            const float* ml = p.ws_ml + rid * n_split * 2;
            const float* acc = p.ws_acc + rid * n_split * D + d4 * 4;
            const float mu = sm.M[r];
            auto ld4 = [&](int sp_) {
                const float* q = acc + (int64_t)sp_ * D;
                return float4{load_partial(q), load_partial(q + 1), load_partial(q + 2),
                              load_partial(q + 3)};
            };
            int sp = sg;
            // four independent loads in flight per step
            for (; sp + 3 * SG < nvalid; sp += 4 * SG) {
                float4 v[4];
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    v[u] = ld4(sp + u * SG);
                    w[u] = fast_exp2(load_partial(ml + (sp + u * SG) * 2) - mu);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a.x += w[u] * v[u].x;
                    a.y += w[u] * v[u].y;
                    a.z += w[u] * v[u].z;
                    a.w += w[u] * v[u].w;
                }
            }
            for (; sp < nvalid; sp += SG) {
                const float4 v = ld4(sp);
                const float w = fast_exp2(load_partial(ml + sp * 2) - mu);
                a.x += w * v.x;
                a.y += w * v.y;
                a.z += w * v.z;
                a.w += w * v.w;
            }
        }
        if constexpr (SG > 1) {
            sm.red[tid] = a;
            __syncthreads();
            if (sg == 0 && rg < p.rows) {
                for (int g2 = 1; g2 < SG; ++g2) {
                    const float4 o = sm.red[g2 * E4 + e4];
                    a.x += o.x;
                    a.y += o.y;
                    a.z += o.z;
                    a.w += o.w;
                }
            }
        }
        if (sg == 0 && rg < p.rows) {
            const float L = sm.L[r];
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            const int64_t o = rid * D + d4 * 4;
            store_elem<DT>(p.out, o, a.x * inv);
            store_elem<DT>(p.out, o + 1, a.y * inv);
            store_elem<DT>(p.out, o + 2, a.z * inv);
            store_elem<DT>(p.out, o + 3, a.w * inv);
        }
    }
    if (tid == 0) atomicExch(p.counters + unit, 0);  // ready for the next call
}

}  // namespace kvattn
