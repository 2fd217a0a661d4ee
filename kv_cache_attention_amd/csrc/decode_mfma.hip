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
// every 4th tile of 64 positions (32 for 49-64 rows).  Per tile and wave:
//   S^T[64 x rows] = K[64 x d] . Q^T[d x rows]   K straight from HBM into the
//                     A operand (each lane's 16 bytes are 8 consecutive d of one
//                     position: the operand layout), Q^T held in registers;
//   online softmax per row over the tile (running max / sum, as in the Flash
//                     Attention section of the nextadmin.net lesson "KV cache
//                     and Flash Attention"), P rounded to the input type;
//   O^T[d x rows]  += V^T[d x 64] . P^T[64 x rows]   V needs positions along each
//                     lane's 8 operand elements while HBM holds it d-contiguous,
//                     so V goes HBM -> registers -> LDS and is read back
//                     transposed (2-byte reads from a padded, bank-conflict-free
//                     layout).
// The S^T accumulator already holds, per lane, 4 consecutive positions of one
// row for each 16-position half; two halves give the 8 positions of the P^T
// operand, and V^T is read back with the same position permutation.
// The next tile's V is loaded as soon as this tile's V sits in LDS, its K as soon
// as S^T has consumed this tile's K, so both are in flight during the rest.  The
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
// Positions per wave step: 64 (32 when four row tiles leave too few registers).
template <int R>
struct MfmaTile {
    static constexpr int TILE = R <= 3 ? 64 : 32;
    static constexpr int TT = TILE / 16;  // 16-position sub-tiles (S^T accumulators)
    static constexpr int KK = TILE / 32;  // 32-position k-steps of P V
};

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> one dword of two 16-bit values (v_cvt_pk_*: round to nearest even)
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    if constexpr (DT == F16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// max / sum with the lanes 16 and 32 away (gfx950 permlane swaps, no LDS round trip)
__device__ __forceinline__ float xmax_16_32(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float xsum_16_32(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

template <int D, int TILE>
struct MfmaGeo {
    static constexpr int KS = D / 32;                // k-steps of 32 along d
    static constexpr int DT16 = D / 16;              // 16-wide d tiles of the output
    static constexpr int VROW = D * 2 + 8;           // LDS bytes per staged V row (padded)
    static constexpr int VBUF = TILE * VROW;         // LDS bytes per wave
};

template <int DT, int D, int R, int CACHE>
__global__ __launch_bounds__(MFMA_THREADS) void decode_mfma_kernel(const DecodeParams p) {
    constexpr int TILE = MfmaTile<R>::TILE, TT = MfmaTile<R>::TT, KK = MfmaTile<R>::KK;
    using G = MfmaGeo<D, TILE>;
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

    // K and V of one tile, in the A-operand lane mapping: position tile + tt*16 + lr,
    // d chunk (ks*4 + lq)*8.  Loads are branch-free: a position past the split is
    // clamped to the split's last one (an attended, finite row) and its scores are
    // masked; a paged position behind an out-of-pool entry reads block 0 and both
    // its score and its V are discarded by selects.
    bool pvalid[TT];
    int64_t offs[TT];
    auto locate_tile = [&](int32_t tb) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int32_t j = min(tb + tt * 16 + lr, j1 - 1);
            Loc L = locate<CACHE>(p, s, b, span_pos(s, j));
            pvalid[tt] = L.unit >= 0;
            L.unit = L.unit >= 0 ? L.unit : 0;
            offs[tt] = row_offset(p, L, kvh);
        }
    };
    auto load_k = [&](u32x4 (&kf)[TT][KS]) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[tt][ks] = *reinterpret_cast<const u32x4*>(kp + offs[tt] + (ks * 4 + lq) * 8);
    };
    auto load_v = [&](u32x4 (&vf)[TT][KS]) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                vf[tt][ks] = *reinterpret_cast<const u32x4*>(vp + offs[tt] + (ks * 4 + lq) * 8);
    };

    const int32_t step = MFMA_WAVES * TILE;
    int32_t tb = j0 + wave * TILE;
    // One register buffer each for K and V.  The next tile's V is loaded as soon as
    // this tile's V is in LDS, the next tile's K as soon as S^T has consumed this
    // tile's K; both are in flight during the softmax and P V of this tile.
    u32x4 kc[TT][KS], vr[TT][KS];
    bool cur_valid[TT];
    if (tb < j1) {
        locate_tile(tb);
        load_k(kc);
        load_v(vr);
    }

    // new row i sits at T - q_len + i; rows see positions <= their own
    const int32_t P0 = s.T - p.q_len;
    const bool sink_window = p.mask_mode == MASK_SINK_WINDOW;
    // per row tile: the row's last visible position and window start
    int32_t hi[R], lo[R];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        hi[qt] = P0 + row_i[qt];
        lo[qt] = sink_window ? hi[qt] - p.window + 1 : 0;
    }
    const float c = p.scale_log2;

    for (; tb < j1; tb += step) {
        // stage this tile's V rows in LDS: [position][d], padded rows
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            cur_valid[tt] = pvalid[tt];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 v = vr[tt][ks];
                if constexpr (CACHE == PAGED) {
                    if (!pvalid[tt]) v = u32x4{0, 0, 0, 0};
                }
                char* dst = vbuf + (tt * 16 + lr) * VROW + (ks * 4 + lq) * 16;
                *reinterpret_cast<uint2*>(dst) = uint2{v[0], v[1]};
                *reinterpret_cast<uint2*>(dst + 8) = uint2{v[2], v[3]};
            }
        }
        const bool more = tb + step < j1;
        if (more) {
            locate_tile(tb + step);
            load_v(vr);
        }

        // S^T = K . Q^T
        f32x4 st[TT][R];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int qt = 0; qt < R; ++qt) {
                f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32<DT>(kc[tt][ks], qf[qt][ks], acc);
                st[tt][qt] = acc;
            }
        if (more) load_k(kc);

        // Mask only where it can bite: a partial tile, rows that do not all see the
        // tile's last position (q_len > 1), the window mask, or a bad page entry.
        bool all_pages = true;
        if constexpr (CACHE == PAGED) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) all_pages = all_pages && __all(cur_valid[tt]);
        }
        const bool edge = (tb + TILE > j1) || !all_pages ||
                          (p.q_len > 1 && (sink_window ||
                                           span_pos(s, min(tb + TILE, j1) - 1) > P0));
        if (edge) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t j = tb + tt * 16 + lq * 4 + e;
                    const int32_t pos = span_pos(s, min(j, j1 - 1));
                    bool pv = true;
                    if constexpr (CACHE == PAGED) {
                        const int32_t blk = page_entry(p, b, pos);
                        pv = (uint32_t)blk < (uint32_t)p.num_blocks;
                    }
#pragma unroll
                    for (int qt = 0; qt < R; ++qt) {
                        const bool ok = (j < j1) & pv & (pos <= hi[qt]) &
                                        ((pos < p.n_sink) | (pos >= lo[qt]));
                        st[tt][qt][e] = ok ? st[tt][qt][e] : NEG_INF;
                    }
                }
            }
        }

        // online softmax per row (row = lane column lr of each row tile); scores
        // stay raw, the scale enters through the exp2 argument
        uint32_t pf[KK][R][4];
        bool rescale = false;
        float alpha[R];
#pragma unroll
        for (int qt = 0; qt < R; ++qt) {
            float mt = st[0][qt][0];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) mt = fmaxf(mt, st[tt][qt][e]);
            mt = xmax_16_32(mt);
            const float m_new = fmaxf(m[qt], mt * c);
            const float m_use = m_new == NEG_INF ? 0.0f : m_new;
            alpha[qt] = fast_exp2(m[qt] - m_use);
            rescale |= m_new != m[qt];
            m[qt] = m_new;
            float ps = 0.0f;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                float pw[2][4];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pw[h][e] = fast_exp2(fmaf(st[2 * kk + h][qt][e], c, -m_use));
                        ps += pw[h][e];
                    }
                // P^T operand of k-step kk: k = 8*lq + e -> positions kk*32 + 4*lq + e
                // (first half) and kk*32 + 16 + 4*lq + e (second half)
                pf[kk][qt][0] = pack2<DT>(pw[0][0], pw[0][1]);
                pf[kk][qt][1] = pack2<DT>(pw[0][2], pw[0][3]);
                pf[kk][qt][2] = pack2<DT>(pw[1][0], pw[1][1]);
                pf[kk][qt][3] = pack2<DT>(pw[1][2], pw[1][3]);
            }
            lsum[qt] = lsum[qt] * alpha[qt] + ps;
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
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt) {
                const char* col = vbuf + (dt * 16 + lr) * 2;
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const char* r0 = col + (kk * 32 + h * 16 + lq * 4) * VROW;
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
                    const u32x4 pb = {pf[kk][qt][0], pf[kk][qt][1], pf[kk][qt][2], pf[kk][qt][3]};
                    o[dt][qt] = mfma16x16x32<DT>(va, pb, o[dt][qt]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- merge the four waves: per row (m, l), then sum of rescaled O in LDS
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        const float lt = xsum_16_32(lsum[qt]);
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
