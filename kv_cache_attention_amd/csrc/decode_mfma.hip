// Split-KV decode on the matrix cores, for 16 to 64 query rows per KV head
// (speculative verification with grouped-query attention: q_len new tokens x
// the query heads that share one KV head).
//
// Rows this wide make the step a dense contraction: per cached position every
// row does d multiply-adds for Q K^T and d for P V, ~10 flops per byte of K/V at
// 40 rows, beyond what the vector ALUs sustain at HBM speed, so both products
// run as v_mfma_f32_16x16x32_{bf16,f16} tiles with fp32 accumulation.
//
// One workgroup (4 wave64) owns a (sequence, KV head, split); each wave takes
// every 4th tile of 32 positions.  Per tile and wave:
//   S^T[32 x rows] = K[32 x d] . Q^T[d x rows]   K straight from HBM into the
//                     A operand (each lane's 16 bytes are 8 consecutive d of one
//                     position: the operand layout), Q^T held in registers;
//   online softmax per row over the tile (running max / sum, as in the Flash
//                     Attention section of the nextadmin.net lesson "KV cache
//                     and Flash Attention"), P rounded to the input type;
//   O^T[d x rows]  += V^T[d x 32] . P^T[32 x rows]   V needs positions along each
//                     lane's 8 operand elements while HBM holds it d-contiguous,
//                     so V goes HBM -> registers -> LDS and is read back
//                     transposed (2-byte reads from a padded, bank-conflict-free
//                     layout).
// The S^T accumulator already holds, per lane, 4 consecutive positions of one
// row for each 16-position half; two halves give the 8 positions of the P^T
// operand, and V^T is read back with the same position permutation.
// The next tile's K and V are loaded before the current tile's math: K into a
// second register buffer, V into the one V buffer just emptied into LDS.  The
// four waves then merge through LDS and the workgroup writes the final rows (its
// sequence needs one split) or its partial (acc, m, l); the last workgroup of the
// (sequence, KV head) merges the partials (split_merge.hpp).
#include "device_common.hpp"
#include "launch.hpp"
#include "split_merge.hpp"

namespace kvattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int MFMA_THREADS = 256;
constexpr int MFMA_WAVES = MFMA_THREADS / 64;
constexpr int TILE = 32;  // positions per wave step

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two fp32 -> one dword of two 16-bit values (round to nearest even)
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (DT == F16)
        return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
    else
        return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

template <int D>
struct MfmaGeo {
    static constexpr int KS = D / 32;                // k-steps of 32 along d
    static constexpr int DT16 = D / 16;              // 16-wide d tiles of the output
    static constexpr int VROW = D * 2 + 8;           // LDS bytes per staged V row (padded)
    static constexpr int VBUF = TILE * VROW;         // LDS bytes per wave
};

template <int DT, int D, int R, int CACHE>
__global__ __launch_bounds__(MFMA_THREADS) void decode_mfma_kernel(const DecodeParams p) {
    using G = MfmaGeo<D>;
    constexpr int KS = G::KS, DT16 = G::DT16, VROW = G::VROW;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr int NQ = R * 16;  // padded rows

    // V staging (per wave) during the loop; reused for the cross-wave merge after it.
    constexpr int SMEM_V = MFMA_WAVES * G::VBUF;
    constexpr int SMEM_O = NQ * D * 4;
    static_assert(SMEM_O <= SMEM_V, "merge buffer must fit in the staging area");
    __shared__ __attribute__((aligned(16))) char smem[SMEM_V];
    __shared__ float sm_m[MFMA_WAVES][NQ];
    __shared__ float sm_l[MFMA_WAVES][NQ];

    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const SeqSpan s = seq_span(p, b);
    const int nvalid = valid_splits(p, s);
    if (split >= nvalid) return;
    const int32_t j0 = split * p.split_len;
    const int32_t j1 = min(j0 + p.split_len, s.count);

    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int l = tid % 64;
    const int lr = l % 16;  // operand row / output column
    const int lq = l / 16;  // operand k-group / output row group

    // Q^T operand fragments: row n = qt*16 + lr, d chunk (ks*4 + lq)*8.
    u32x4 qf[R][KS];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        const int n = qt * 16 + lr;
        const bool ok = n < p.rows;
        const int i = ok ? n / p.group : 0;
        const int h = kvh * p.group + (ok ? n - i * p.group : 0);
        const int64_t base = (((int64_t)b * p.q_len + i) * p.num_q_heads + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int64_t off = base + (ks * 4 + lq) * 8;
            qf[qt][ks] = ok ? *reinterpret_cast<const u32x4*>(
                                  reinterpret_cast<const uint16_t*>(p.q) + off)
                            : u32x4{0, 0, 0, 0};
        }
    }
    // rows' new-token index (for the causal / window mask), -1 for padding rows
    int row_i[R];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        const int n = qt * 16 + lr;
        row_i[qt] = n < p.rows ? n / p.group : p.q_len - 1;
    }

    f32x4 o[DT16][R];
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
        for (int qt = 0; qt < R; ++qt) o[dt][qt] = f32x4{0, 0, 0, 0};
    float m[R], lsum[R];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        m[qt] = NEG_INF;
        lsum[qt] = 0.0f;
    }

    char* vbuf = smem + wave * G::VBUF;
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k);
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v);

    // K and V of one tile, in the A-operand lane mapping:
    // position tile + tt*16 + lr, d chunk (ks*4 + lq)*8.
    auto load_tile = [&](int32_t tb, u32x4 (&kf)[2][KS], u32x4 (&vf)[2][KS]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int32_t j = tb + tt * 16 + lr;
            bool val = j < j1;
            int64_t off = 0;
            if (val) {
                const Loc L = locate<CACHE>(p, s, b, span_pos(s, j));
                val = L.unit >= 0;
                off = row_offset(p, L, kvh);
            }
            // positions past the split or behind an invalid page entry are not
            // loaded (they may hold NaN) and enter as zeros
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int64_t e = off + (ks * 4 + lq) * 8;
                kf[tt][ks] = val ? *reinterpret_cast<const u32x4*>(kp + e) : u32x4{0, 0, 0, 0};
                vf[tt][ks] = val ? *reinterpret_cast<const u32x4*>(vp + e) : u32x4{0, 0, 0, 0};
            }
        }
    };

    const int32_t step = MFMA_WAVES * TILE;
    int32_t tb = j0 + wave * TILE;
    // K is double-buffered in registers; V has one register buffer, emptied into
    // LDS before the next tile's V is loaded into it.
    u32x4 kc[2][KS], kn[2][KS], vr[2][KS];
    if (tb < j1) load_tile(tb, kc, vr);

    // new row i sits at T - q_len + i; rows see positions <= their own
    const int32_t P0 = s.T - p.q_len;
    const bool sink_window = p.mask_mode == MASK_SINK_WINDOW;

    for (; tb < j1; tb += step) {
        // stage this tile's V rows in LDS: [position][d], padded rows
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                char* dst = vbuf + (tt * 16 + lr) * VROW + (ks * 4 + lq) * 16;
                *reinterpret_cast<uint2*>(dst) = uint2{vr[tt][ks][0], vr[tt][ks][1]};
                *reinterpret_cast<uint2*>(dst + 8) = uint2{vr[tt][ks][2], vr[tt][ks][3]};
            }
        // prefetch the next tile
        const bool more = tb + step < j1;
        if (more) load_tile(tb + step, kn, vr);

        // S^T = K . Q^T
        f32x4 st[2][R];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int qt = 0; qt < R; ++qt) {
                f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32<DT>(kc[tt][ks], qf[qt][ks], acc);
                st[tt][qt] = acc;
            }

        // scale, mask, online softmax (per row: lane column lr of each row tile)
        const bool edge = tb + TILE > j1 || (p.q_len > 1 && (sink_window ||
                                                             span_pos(s, min(tb + TILE, j1) - 1) > P0));
        uint32_t pf[R][4];
        bool rescale = false;
        float alpha[R];
#pragma unroll
        for (int qt = 0; qt < R; ++qt) {
            float x[2][4];
            float mt = NEG_INF;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = st[tt][qt][e] * p.scale_log2;
                    if (edge) {
                        const int32_t j = tb + tt * 16 + lq * 4 + e;
                        bool ok = j < j1;
                        if (ok) ok = row_attends(p, s, row_i[qt], span_pos(s, j));
                        v = ok ? v : NEG_INF;
                    }
                    x[tt][e] = v;
                    mt = fmaxf(mt, v);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m[qt], mt);
            const float m_use = m_new == NEG_INF ? 0.0f : m_new;
            alpha[qt] = fast_exp2(m[qt] - m_use);
            rescale |= m_new != m[qt];
            m[qt] = m_new;
            float ps = 0.0f;
            float pw[2][4];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pw[tt][e] = fast_exp2(x[tt][e] - m_use);
                    ps += pw[tt][e];
                }
            lsum[qt] = lsum[qt] * alpha[qt] + ps;
            // P^T operand: k = 8*lq + e -> positions 4*lq+e (first half), 16+4*lq+e (second)
            pf[qt][0] = pack2<DT>(pw[0][0], pw[0][1]);
            pf[qt][1] = pack2<DT>(pw[0][2], pw[0][3]);
            pf[qt][2] = pack2<DT>(pw[1][0], pw[1][1]);
            pf[qt][3] = pack2<DT>(pw[1][2], pw[1][3]);
        }
        if (__any(rescale)) {
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
                for (int qt = 0; qt < R; ++qt) o[dt][qt] *= alpha[qt];
        }

        // O^T += V^T . P^T, V^T read back transposed from LDS
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) {
            const char* col = vbuf + (dt * 16 + lr) * 2;
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const char* r0 = col + (h * 16 + lq * 4) * VROW;
                const uint32_t a0 = *reinterpret_cast<const uint16_t*>(r0);
                const uint32_t a1 = *reinterpret_cast<const uint16_t*>(r0 + VROW);
                const uint32_t a2 = *reinterpret_cast<const uint16_t*>(r0 + 2 * VROW);
                const uint32_t a3 = *reinterpret_cast<const uint16_t*>(r0 + 3 * VROW);
                w[2 * h] = a0 | (a1 << 16);
                w[2 * h + 1] = a2 | (a3 << 16);
            }
            const u32x4 va = {w[0], w[1], w[2], w[3]};
#pragma unroll
            for (int qt = 0; qt < R; ++qt) {
                const u32x4 pb = {pf[qt][0], pf[qt][1], pf[qt][2], pf[qt][3]};
                o[dt][qt] = mfma16x16x32<DT>(va, pb, o[dt][qt]);
            }
        }
        __builtin_amdgcn_wave_barrier();

        if (more) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kc[tt][ks] = kn[tt][ks];
        }
    }

    // ---- merge the four waves: per row (m, l), then sum of rescaled O in LDS
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        float lt = lsum[qt];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        lsum[qt] = lt;
        if (lq == 0) {
            sm_m[wave][qt * 16 + lr] = m[qt];
            sm_l[wave][qt * 16 + lr] = lt;
        }
    }
    __syncthreads();  // also: every wave is done with its V staging area
    float f[R];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        const int n = qt * 16 + lr;
        float M = NEG_INF;
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w) M = fmaxf(M, sm_m[w][n]);
        const float Mu = M == NEG_INF ? 0.0f : M;
        f[qt] = fast_exp2(m[qt] - Mu);
    }
    float* osum = reinterpret_cast<float*>(smem);  // [NQ][D]
    for (int w = 0; w < MFMA_WAVES; ++w) {
        if (wave == w) {
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
                for (int qt = 0; qt < R; ++qt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float* dst = osum + (qt * 16 + lr) * D + dt * 16 + lq * 4 + e;
                        const float v = o[dt][qt][e] * f[qt];
                        *dst = w == 0 ? v : *dst + v;
                    }
        }
        __syncthreads();
    }
    // rows out: thread -> (row, d)
    for (int idx = tid; idx < NQ * D; idx += MFMA_THREADS) {
        const int n = idx / D;
        const int d = idx - n * D;
        if (n >= p.rows) continue;
        float M = NEG_INF;
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w) M = fmaxf(M, sm_m[w][n]);
        const float Mu = M == NEG_INF ? 0.0f : M;
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w) L += sm_l[w][n] * fast_exp2(sm_m[w][n] - Mu);
        const float A = osum[idx];
        const int64_t rid = row_id_of(p, b, kvh, n);
        if (nvalid == 1) {
            store_elem<DT>(p.out, rid * D + d, L > 0.0f ? A / L : 0.0f);
        } else {
            const int64_t part = rid * p.n_split + split;
            store_partial(p.ws_acc + part * D + d, A);
            if (d == 0) {
                store_partial(p.ws_ml + part * 2, M);
                store_partial(p.ws_ml + part * 2 + 1, L);
            }
        }
    }
    if (nvalid > 1) {
        // the staging area is free again: the merge's scratch lives there
        static_assert(sizeof(MergeSmem<NQ, MFMA_THREADS>) <= SMEM_V, "merge scratch");
        __syncthreads();
        auto& msm = *reinterpret_cast<MergeSmem<NQ, MFMA_THREADS>*>(smem);
        arrive_and_merge<DT, D, NQ, MFMA_THREADS>(p, b, kvh, 0, b * p.num_kv_heads + kvh, nvalid,
                                                  msm);
    }
}

bool mfma_supported(int dtype, int head_dim, int rows) {
    return (dtype == F16 || dtype == BF16) && (head_dim == 64 || head_dim == 128) &&
           rows >= 16 && rows <= 64;
}

template <int DT, int D, int R>
static hipError_t launch_mfma_c(const DecodeParams& p, hipStream_t st) {
    dim3 grid(p.n_split, p.num_kv_heads, p.batch);
    switch (p.cache_mode) {
    case CONTIGUOUS:
        hipLaunchKernelGGL((decode_mfma_kernel<DT, D, R, CONTIGUOUS>), grid, dim3(MFMA_THREADS), 0, st, p);
        break;
    case PAGED:
        hipLaunchKernelGGL((decode_mfma_kernel<DT, D, R, PAGED>), grid, dim3(MFMA_THREADS), 0, st, p);
        break;
    default:
        hipLaunchKernelGGL((decode_mfma_kernel<DT, D, R, RING>), grid, dim3(MFMA_THREADS), 0, st, p);
        break;
    }
    return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_mfma_r(const DecodeParams& p, hipStream_t st) {
    switch ((p.rows + 15) / 16) {
    case 1: return launch_mfma_c<DT, D, 1>(p, st);
    case 2: return launch_mfma_c<DT, D, 2>(p, st);
    case 3: return launch_mfma_c<DT, D, 3>(p, st);
    default: return launch_mfma_c<DT, D, 4>(p, st);
    }
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int head_dim, hipStream_t st) {
    if (!mfma_supported(dtype, head_dim, p.rows)) return hipErrorInvalidValue;
    if (dtype == F16)
        return head_dim == 128 ? launch_mfma_r<F16, 128>(p, st) : launch_mfma_r<F16, 64>(p, st);
    return head_dim == 128 ? launch_mfma_r<BF16, 128>(p, st) : launch_mfma_r<BF16, 64>(p, st);
}

}  // namespace kvattn
