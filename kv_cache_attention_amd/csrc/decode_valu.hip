// Split-KV flash-decoding on the vector ALUs, for up to 16 query rows per KV head.
//
// One workgroup (256 lanes = 4 wave64) owns one (sequence, KV head, split): a
// run of split_len attended positions.  Each position's K row (and V row) of
// head_dim elements is read by one "lane group" of head_dim*bytes/16 lanes with
// one 16-byte load per lane, so a wave instruction covers whole 256-byte rows and
// every byte of K and V is loaded exactly once, straight into registers (each
// byte feeds exactly one lane, so staging it through LDS would add a write and a
// read with no reuse).  All query rows that share the KV head (the GQA group
// times the q_len new tokens) live in every lane, so one K/V fetch serves the
// whole group.
//
// Per tile of U positions a lane group forms the scores with packed dot
// products, sums them over its lanes with DPP, and folds them into its own
// running (max, sum, accumulator) - the online softmax of the Flash Attention
// section of the nextadmin.net lesson "KV cache and Flash Attention" (running
// max and sum across tiles, rescale the old terms by exp(m_old - m_new), which
// is 0 when nothing was seen yet).  Scores are kept in the exp2 domain
// (scale * log2 e folded into one multiply).  At the end the lane groups of a
// wave merge through cross-lane shuffles, the four waves through LDS, and the
// workgroup writes either the final rows (its sequence needs one split) or its
// unnormalised partial (acc, m, l); the last workgroup of the (sequence, KV
// head) to finish merges the partials (split_merge.hpp).
//
// Paged caches: the page-table entries of the next tile are read while the
// current tile is processed, so the K/V loads never wait on a table read.
#include "device_common.hpp"
#include "launch.hpp"
#include "split_merge.hpp"

namespace kvattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT, int D>
struct Geo {
    static constexpr int EB = Elem<DT>::bytes;
    static constexpr int EPL = 16 / EB;   // elements per lane (one 16-byte load)
    static constexpr int LPR = D / EPL;   // lanes per (position, head) row
};

constexpr int VALU_THREADS = 256;

__device__ __forceinline__ u32x4 load16(const void* base, int64_t elem_off, int eb) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + elem_off * eb);
}

// q . k over one lane's 16 bytes
template <int DT>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b) {
    float s = 0.0f;
    // (each vector element goes through a scalar first: bit-casting a vector
    // element expression directly is miscompiled to element 0 by this toolchain)
    if constexpr (DT == F16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = a[e], y = b[e];
            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, x),
                                       __builtin_bit_cast(half2_t, y), s, false);
        }
    } else if constexpr (DT == BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = a[e], y = b[e];
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short2_t, x),
                                                __builtin_bit_cast(short2_t, y), s, false);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(__uint_as_float(a[e]), __uint_as_float(b[e]), s);
    }
    return s;
}

// one lane's 16 bytes as EPL floats
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4& w, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (DT == F16) {
            f[2 * e] = f16_lo(w[e]);
            f[2 * e + 1] = f16_hi(w[e]);
        } else if constexpr (DT == BF16) {
            f[2 * e] = bf16_lo(w[e]);
            f[2 * e + 1] = bf16_hi(w[e]);
        } else {
            f[e] = __uint_as_float(w[e]);
        }
    }
}

// MASKED: q_len > 1, so rows of one sequence attend different position sets and
// every score gets its row's causal / window test (with one new row the attended
// union is exactly that row's set and no per-row test is needed).
template <int DT, int D, int ROWS, int CACHE, int U, bool MASKED>
__global__ __launch_bounds__(VALU_THREADS) void decode_valu_kernel(const DecodeParams p,
                                                                   int row_blocks) {
    using G = Geo<DT, D>;
    constexpr int EPL = G::EPL, LPR = G::LPR, EB = G::EB;
    constexpr int NLG = VALU_THREADS / LPR;  // lane groups per workgroup
    constexpr float NEG_INF = -__builtin_inff();

    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z / row_blocks;
    const int rb = blockIdx.z - b * row_blocks;

    const SeqSpan s = seq_span(p, b);
    const int nvalid = valid_splits(p, s);
    if (split >= nvalid) return;
    const int32_t j0 = split * p.split_len;
    const int32_t j1 = min(j0 + p.split_len, s.count);

    const int tid = threadIdx.x;
    const int lane = tid % LPR;
    const int lg = tid / LPR;
    const int d0 = lane * EPL;

    // Query rows of this KV head: row r = i * group + hg  (new token i, head kvh*group+hg)
    u32x4 qv[ROWS];
    int row_i[ROWS];
    int64_t row_id[ROWS];  // index of the row in out's [batch, q_len, Hq] order
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int rg = rb * ROWS + r;
        const bool ok = rg < p.rows;
        const int i = ok ? rg / p.group : 0;
        const int h = kvh * p.group + (ok ? rg - i * p.group : 0);
        row_i[r] = ok ? i : -1;
        row_id[r] = ((int64_t)b * p.q_len + i) * p.num_q_heads + h;
        qv[r] = ok ? load16(p.q, row_id[r] * D + d0, EB) : u32x4{0, 0, 0, 0};
    }

    float m[ROWS], l[ROWS], acc[ROWS][EPL];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        m[r] = NEG_INF;
        l[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = 0.0f;
    }
    // per-row bounds for MASKED: row r attends pos iff pos <= hi[r] and
    // (pos < n_sink or pos >= lo[r])  (lo = 0 for the causal mask)
    int32_t hi[ROWS], lo[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int32_t P = s.T - p.q_len + (row_i[r] >= 0 ? row_i[r] : p.q_len - 1);
        hi[r] = P;
        lo[r] = p.mask_mode == MASK_SINK_WINDOW ? P - p.window + 1 : 0;
    }

    // Loads are branch-free: a lane whose position lies past the split (or behind a
    // page-table entry outside the pool) loads a clamped, valid address and its
    // data is discarded by selects (score -> -inf, V -> 0), never multiplied in.
    // Paged caches read the page-table entries one tile ahead of use.
    constexpr int32_t TW = NLG * U;  // positions per workgroup tile
    int32_t blk[U];
    auto pages = [&](int32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j = min(base + u * NLG + lg, j1 - 1);
            blk[u] = page_entry(p, b, span_pos(s, j));
        }
    };
    if constexpr (CACHE == PAGED) pages(j0);

    for (int32_t base = j0; base < j1; base += TW) {
        u32x4 kw[U], vw[U];
        int32_t pos[U];
        bool val[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j = base + u * NLG + lg;
            val[u] = j < j1;
            pos[u] = span_pos(s, min(j, j1 - 1));
            Loc L;
            if constexpr (CACHE == PAGED) {
                L = paged_loc(p, blk[u], pos[u]);
                val[u] = val[u] && L.unit >= 0;
                L.unit = L.unit >= 0 ? L.unit : 0;
            } else {
                L = locate<CACHE>(p, s, b, pos[u]);
            }
            const int64_t off = row_offset(p, L, kvh) + d0;
            kw[u] = load16(p.k, off, EB);
            vw[u] = load16(p.v, off, EB);
        }
        if constexpr (CACHE == PAGED) pages(base + TW);
        // raw scores q.k; the softmax scale (times log2 e) is applied inside the
        // exp2 argument, so the running max m is kept in scaled units
        float sc[ROWS][U];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float x = group_sum<LPR>(dot16<DT>(qv[r], kw[u]));
                bool ok = val[u];
                if constexpr (MASKED)
                    ok = ok & (pos[u] <= hi[r]) & ((pos[u] < p.n_sink) | (pos[u] >= lo[r]));
                sc[r][u] = ok ? x : NEG_INF;
            }
        }
        float vf[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            unpack16<DT>(vw[u], vf[u]);
            // a paged position behind an out-of-pool entry was read from block 0 and
            // may hold anything; every other discarded lane read an attended position
            if constexpr (CACHE == PAGED) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) vf[u][e] = val[u] ? vf[u][e] : 0.0f;
            }
        }
        const float c = p.scale_log2;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            float mt = sc[r][0];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, sc[r][u]);
            const float m_new = fmaxf(m[r], mt * c);  // c > 0: max commutes with the scale
            const float m_use = m_new == NEG_INF ? 0.0f : m_new;
            if (__any(m_new != m[r])) {  // rescale only when some lane's max moved
                const float alpha = fast_exp2(m[r] - m_use);  // 0 while nothing was seen
                l[r] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[r][e] *= alpha;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float pw = fast_exp2(fmaf(sc[r][u], c, -m_use));
                l[r] += pw;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[r][e] = fmaf(pw, vf[u][e], acc[r][e]);
            }
            m[r] = m_new;
        }
    }

    // Merge the lane groups of each wave (butterfly over lane offsets LPR .. 32).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float mo = __shfl_xor(m[r], off, 64);
            const float lo = __shfl_xor(l[r], off, 64);
            const float M = fmaxf(m[r], mo);
            const float Mu = M == NEG_INF ? 0.0f : M;
            const float a = fast_exp2(m[r] - Mu);
            const float c = fast_exp2(mo - Mu);
            l[r] = l[r] * a + lo * c;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ao = __shfl_xor(acc[r][e], off, 64);
                acc[r][e] = acc[r][e] * a + ao * c;
            }
            m[r] = M;
        }
    }

    // Merge the four waves through LDS.
    constexpr int NW = VALU_THREADS / 64;
    __shared__ float sm_acc[NW][ROWS][D];
    __shared__ float sm_ml[NW][ROWS][2];
    const int wave = tid / 64;
    const int lw = tid % 64;
    if (lw < LPR) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_acc[wave][r][d0 + e] = acc[r][e];
            if (lw == 0) {
                sm_ml[wave][r][0] = m[r];
                sm_ml[wave][r][1] = l[r];
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < ROWS * D; idx += VALU_THREADS) {
        const int r = idx / D;
        const int d = idx - r * D;
        if (rb * ROWS + r >= p.rows) continue;
        float M = NEG_INF;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_ml[w][r][0]);
        const float Mu = M == NEG_INF ? 0.0f : M;
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(sm_ml[w][r][0] - Mu);
            L += sm_ml[w][r][1] * f;
            A += sm_acc[w][r][d] * f;
        }
        const int64_t rid = row_id_of(p, b, kvh, rb * ROWS + r);
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
        __shared__ MergeSmem<ROWS, VALU_THREADS> msm;
        const int unit = (b * p.num_kv_heads + kvh) * row_blocks + rb;
        arrive_and_merge<DT, D, ROWS, VALU_THREADS>(p, b, kvh, rb * ROWS, unit, nvalid, msm);
    }
}

// ---------------------------------------------------------------- host launchers

// Positions per lane group per tile.
#ifndef KVATTN_VALU_U_SMALL
#define KVATTN_VALU_U_SMALL 8   // 1 or 2 rows
#endif
#ifndef KVATTN_VALU_U_MID
#define KVATTN_VALU_U_MID 8     // 4 rows
#endif
#ifndef KVATTN_VALU_U_LARGE
#define KVATTN_VALU_U_LARGE 4   // 8 or 16 rows
#endif

// Kernel selection: one instance per (dtype, head_dim, row bucket, cache form,
// per-row mask); launches and occupancy queries go through the same choice.
template <int DT, int D, int ROWS, int CACHE>
static const void* valu_kernel_t(bool masked) {
    constexpr int U = ROWS <= 2 ? KVATTN_VALU_U_SMALL
                                : (ROWS <= 4 ? KVATTN_VALU_U_MID : KVATTN_VALU_U_LARGE);
    return masked ? reinterpret_cast<const void*>(&decode_valu_kernel<DT, D, ROWS, CACHE, U, true>)
                  : reinterpret_cast<const void*>(&decode_valu_kernel<DT, D, ROWS, CACHE, U, false>);
}

template <int DT, int D, int ROWS>
static const void* valu_kernel_c(int cache_mode, bool masked) {
    switch (cache_mode) {
    case CONTIGUOUS: return valu_kernel_t<DT, D, ROWS, CONTIGUOUS>(masked);
    case PAGED: return valu_kernel_t<DT, D, ROWS, PAGED>(masked);
    default: return valu_kernel_t<DT, D, ROWS, RING>(masked);
    }
}

template <int DT, int D>
static const void* valu_kernel_r(int rows_per_block, int cache_mode, bool masked) {
    switch (rows_per_block) {
    case 1: return valu_kernel_c<DT, D, 1>(cache_mode, masked);
    case 2: return valu_kernel_c<DT, D, 2>(cache_mode, masked);
    case 4: return valu_kernel_c<DT, D, 4>(cache_mode, masked);
    case 8: return valu_kernel_c<DT, D, 8>(cache_mode, masked);
    default: return valu_kernel_c<DT, D, 16>(cache_mode, masked);
    }
}

int valu_rows_per_block(int rows) {
    if (rows <= 1) return 1;
    if (rows <= 2) return 2;
    if (rows <= 4) return 4;
    if (rows <= 8) return 8;
    return 16;
}

const void* select_valu_kernel(int dtype, int head_dim, int rows, int cache_mode, bool masked) {
    const int rpb = valu_rows_per_block(rows);
    if (head_dim == 128) {
        switch (dtype) {
        case F16: return valu_kernel_r<F16, 128>(rpb, cache_mode, masked);
        case BF16: return valu_kernel_r<BF16, 128>(rpb, cache_mode, masked);
        default: return valu_kernel_r<F32, 128>(rpb, cache_mode, masked);
        }
    }
    switch (dtype) {
    case F16: return valu_kernel_r<F16, 64>(rpb, cache_mode, masked);
    case BF16: return valu_kernel_r<BF16, 64>(rpb, cache_mode, masked);
    default: return valu_kernel_r<F32, 64>(rpb, cache_mode, masked);
    }
}

hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int head_dim, hipStream_t st) {
    const int rpb = valu_rows_per_block(p.rows);
    int row_blocks = (p.rows + rpb - 1) / rpb;
    const void* k = select_valu_kernel(dtype, head_dim, p.rows, p.cache_mode, p.q_len > 1);
    DecodeParams pp = p;
    void* args[] = {&pp, &row_blocks};
    return hipLaunchKernel(k, dim3(p.n_split, p.num_kv_heads, p.batch * row_blocks),
                           dim3(VALU_THREADS), args, 0, st);
}

}  // namespace kvattn
