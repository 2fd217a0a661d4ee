// Matrix-core kernel for chunked prefill: hundreds of new query rows per KV head
// against the cached prefix.  The query tiles against key/value tiles with a
// running softmax of FlashAttention (nextadmin.net lesson "KV cache and Flash
// Attention", the tiling trick), shaped for gfx950:
//
//  * a workgroup of 8 waves owns a block of 256 rows of one KV head (one segment of
//    the flat decomposition, work_plan.hpp); each wave owns 32 rows (two 16-row
//    tiles) and keeps their Q^T operand fragments in registers;
//  * the workgroup streams the segment's positions in tiles of 32 through two LDS
//    buffers: while tile t is computed from one, every thread holds its share of the
//    next KVATTN_PF_AHEAD tiles in registers (loads in flight) and, after its matrix
//    work, stores tile t + 1 into the other buffer; one barrier per tile.  Each K/V
//    byte is fetched once per row block (the split-KV kernel fetches it once per 64
//    rows);
//  * S^T = K . Q^T with K read from LDS in the A-operand layout (rows padded by 16
//    bytes: the 16 positions one read touches fall on distinct banks), the running
//    (max, sum) per row, O^T += V^T . P^T with V^T read back with the gfx950
//    transposed LDS read, as in the split-KV kernel.
// Contiguous, ring and paged caches (a paged position behind a page-table entry
// outside the pool is staged as a zero V row and a masked score: skipped); causal,
// sink/window and token-tree masks.  A segment's pieces and their merge are the
// split-KV kernel's (split_merge.hpp).
#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"
#include "split_merge.hpp"
#include "work_plan.hpp"
#include "fused_append.hpp"

namespace kvattn {

constexpr int PF_WAVES = KVATTN_PF_WAVES;
constexpr int PF_THREADS = kPrefillThreads;
constexpr int PF_RW = KVATTN_PF_RW;             // 16-row tiles per wave
constexpr int PF_AHEAD = KVATTN_PF_AHEAD;       // tiles in flight in registers (1 or 2)
// Deeper rings are not offered: a four-tile ring (four waves of 16 rows) faulted once on
// a ring-cache case, and the cause was not established.
static_assert(PF_AHEAD == 1 || PF_AHEAD == 2, "prefetch depth");
constexpr int PF_ROWS = kPrefillRows;           // rows per workgroup (one segment)

template <int DT, int D, int CACHE>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_mfma_kernel(const DecodeParams p) {
    constexpr float NEG_INF = -__builtin_inff();
    constexpr int KS = D / 32;             // k-steps of 32 along d (S = K Q^T)
    constexpr int DT16 = D / 16;           // 16-wide d tiles of the output
    constexpr int CPR = D * 2 / 16;        // 16-byte chunks per K or V row
    constexpr int KROW = D * 2 + 16;       // LDS bytes per K row (A-operand reads: no conflict)
    constexpr int VROW = D * 2 + 32;       // LDS bytes per V row (transposed reads: no conflict)
    constexpr int TCH = TILE * CPR;        // chunks of one tile's K (and of its V)
    constexpr int NCH = 2 * TCH / PF_THREADS;  // chunks per thread per tile (K and V)
    static_assert(2 * TCH % PF_THREADS == 0 && NCH >= 1, "tile chunks per thread");

    constexpr int NB = 2;  // LDS tile buffers
    __shared__ __attribute__((aligned(16))) char kbuf[NB][TILE * KROW];
    __shared__ __attribute__((aligned(16))) char vbuf[NB][TILE * VROW];
    // paged caches: 1 where the tile's position has its page in the pool, else 0
    __shared__ __attribute__((aligned(16))) uint8_t in_pool[CACHE == PAGED ? NB : 1][TILE];
    constexpr int MROWS = 64;  // rows the merge takes at a time (bounds its registers)
    __shared__ MergeSmem<MROWS, PF_THREADS> msm;

    const int wg = blockIdx.x;
    const int n_wg = gridDim.x;
    const FlatPlan fp = plan_flat<PF_THREADS>(p, n_wg);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int l = tid % 64;
    const int lr = l % 16;  // operand row / output column
    const int lq = l / 16;  // operand k-group / output row group
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k);
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v);
    const float c = p.scale_log2;

    for_each_unit(p, fp, wg, n_wg, [&](int32_t ui) __attribute__((always_inline)) {
    if (p.k_new) append_unit_rows<CACHE, D, 2, PF_THREADS>(p, fp, ui);
    for_each_piece(p, fp, ui, [&](const Piece& pc, const SeqSpan& s) __attribute__((always_inline)) {
    const int b = pc.b;
    const int kvh = pc.seg / p.row_blocks;
    const int row0 = (pc.seg - kvh * p.row_blocks) * PF_ROWS;
    const int wrow0 = row0 + wave * PF_RW * 16;  // this wave's first row
    const int32_t j0 = pc.ja;
    const int32_t j1 = pc.jb;
    const int32_t n_tiles = (j1 - j0 + TILE - 1) / TILE;

    // rows' new-token index (padding rows act as the last) and their mask bounds; a
    // tree mask lets a row see every position before the new block and new position
    // P0 + j iff bit j of its word is set
    const int32_t P0 = s.T - p.q_len;
    const bool sink_window = p.mask_mode == MASK_SINK_WINDOW;
    const bool tree = p.mask_mode == MASK_TREE;
    int32_t hi[PF_RW];
    uint64_t tm[PF_RW];
#pragma unroll
    for (int qt = 0; qt < PF_RW; ++qt) {
        const int n = wrow0 + qt * 16 + lr;
        const int i = n < p.rows ? n / p.group : p.q_len - 1;
        hi[qt] = tree ? s.T - 1 : P0 + i;
        tm[qt] = tree ? p.tree_mask[(int64_t)b * p.q_len + i] : ~0ull;
    }
    // smallest position a row of this wave sits at (a tree's rows all see up to P0 - 1)
    const int32_t hi_first = tree ? P0 - 1 : P0 + min(wrow0, p.rows - 1) / p.group;

    // Q^T operand fragments of the wave's rows (B operand: lane l holds d chunk
    // ks * 4 + l / 16 of row l % 16)
    u32x4 qf[PF_RW][KS];
#pragma unroll
    for (int qt = 0; qt < PF_RW; ++qt) {
        const int n = wrow0 + qt * 16 + lr;
        const bool ok = n < p.rows;
        const int i = ok ? n / p.group : 0;
        const int h = kvh * p.group + (ok ? n - i * p.group : 0);
        const int64_t base = (((int64_t)b * p.q_len + i) * p.num_q_heads + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qt][ks] = ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                                             base + (ks * 4 + lq) * 8)
                            : u32x4{0, 0, 0, 0};
    }

    // A tile's K and V chunks: chunk cc of the tile (K first, then V) is position
    // cc / CPR (within the kind), 16 bytes cc % CPR of its row.  Positions past the
    // piece read its last position (in bounds; their scores are masked), so loads of
    // tiles past the last one are harmless and need no branch.
    // A paged position whose page-table entry lies outside the pool reads block 0 (in
    // bounds) and is flagged: its V chunks are staged as zeros, its in_pool byte as 0.
    struct Stage {
        u32x4 w[NCH];
        uint32_t ok;  // paged: bit k set when chunk k's page is in the pool
    };
    Stage stg[PF_AHEAD];  // staging registers: tile t sits in slot t % PF_AHEAD
    auto load_tile = [&](int32_t t, Stage& stage) __attribute__((always_inline)) {
        stage.ok = 0;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int cc = tid + k * PF_THREADS;
            const int kind = cc / TCH;
            const int rem = cc - kind * TCH;
            const int32_t j = min(j0 + t * TILE + rem / CPR, j1 - 1);
            Loc L = locate<CACHE>(p, s, b, span_pos(s, j));
            if constexpr (CACHE == PAGED) {
                stage.ok |= (L.unit >= 0 ? 1u : 0u) << k;
                L.unit = L.unit >= 0 ? L.unit : 0;
            }
            const int64_t off = row_offset<CACHE>(p, L, kvh) + (rem % CPR) * 8;
            stage.w[k] = *reinterpret_cast<const u32x4*>((kind ? vp : kp) + off);
        }
    };
    auto store_tile = [&](int buf, const Stage& stage) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int cc = tid + k * PF_THREADS;
            const int kind = cc / TCH;
            const int rem = cc - kind * TCH;
            char* dst = kind ? vbuf[buf] + (rem / CPR) * VROW : kbuf[buf] + (rem / CPR) * KROW;
            u32x4 w = stage.w[k];
            if constexpr (CACHE == PAGED) {
                const bool ok = (stage.ok >> k) & 1u;
                if (kind && !ok) w = u32x4{0, 0, 0, 0};
                if (!kind && rem % CPR == 0) in_pool[buf][rem / CPR] = ok ? 1 : 0;
            }
            *reinterpret_cast<u32x4*>(dst + (rem % CPR) * 16) = w;
        }
    };

    f32x4 o[DT16][PF_RW];
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
        for (int qt = 0; qt < PF_RW; ++qt) o[dt][qt] = f32x4{0, 0, 0, 0};
    float m[PF_RW], lsum[PF_RW];
#pragma unroll
    for (int qt = 0; qt < PF_RW; ++qt) {
        m[qt] = NEG_INF;
        lsum[qt] = 0.0f;
    }

    // Tiles 0 .. PF_AHEAD - 1 go in flight, tile 0 into LDS.  Step t then loads tile
    // t + PF_AHEAD into the slot tile t left (stored a step ago), computes tile t from
    // its buffer, stores tile t + 1 (loaded PF_AHEAD - 1 steps ago) into the other
    // buffer (last read in step t - 1) and meets the others at the barrier.
    if (n_tiles > 0) {
#pragma unroll
        for (int a = 0; a < PF_AHEAD; ++a) load_tile(a, stg[a]);
        store_tile(0, stg[0]);
    }
    __syncthreads();
    auto tile = [&](int32_t t, Stage& mine, const Stage& next) __attribute__((always_inline)) {
        const int cur = t % NB;
        load_tile(t + PF_AHEAD, mine);
        const int32_t tb = j0 + t * TILE;
        const char* kb = kbuf[cur];
        // S^T = K . Q^T: each K fragment serves both row tiles, each Q fragment both halves
        f32x4 st[2][PF_RW];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int qt = 0; qt < PF_RW; ++qt) st[tt][qt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(
                    kb + (tt * 16 + lr) * KROW + (ks * 32 + lq * 8) * 2);
#pragma unroll
                for (int qt = 0; qt < PF_RW; ++qt)
                    st[tt][qt] = mfma16x16x32<DT>(kf, qf[qt][ks], st[tt][qt]);
            }
        }

        // mask where it can bite: a partial tile, rows that do not all see the tile's
        // last position, the window mask, or (paged) a position whose page is not in
        // the pool; the lane's positions tt * 16 + lq * 4 + e have their in_pool
        // bytes in one word per tt
        uint32_t pool_w[2] = {0x01010101u, 0x01010101u};
        if constexpr (CACHE == PAGED) {
            pool_w[0] = *reinterpret_cast<const uint32_t*>(&in_pool[cur][lq * 4]);
            pool_w[1] = *reinterpret_cast<const uint32_t*>(&in_pool[cur][16 + lq * 4]);
        }
        const bool edge = (tb + TILE > j1) || sink_window ||
                          span_pos(s, min(tb + TILE, j1) - 1) > hi_first ||
                          (CACHE == PAGED && __any((pool_w[0] & pool_w[1]) != 0x01010101u));
        if (edge) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t j = tb + tt * 16 + lq * 4 + e;
                    const int32_t pos = span_pos(s, min(j, j1 - 1));
                    const int32_t rel = pos - P0;
                    const uint64_t bit = rel >= 0 ? 1ull << (rel & 63) : 0ull;
                    const bool pooled = (pool_w[tt] >> (8 * e)) & 1u;
#pragma unroll
                    for (int qt = 0; qt < PF_RW; ++qt) {
                        const bool ok = (j < j1) & pooled & (pos <= hi[qt]) &
                                        (!sink_window | (pos < p.n_sink) |
                                         (pos > hi[qt] - p.window)) &
                                        ((rel < 0) | ((tm[qt] & bit) != 0));
                        st[tt][qt][e] = ok ? st[tt][qt][e] : NEG_INF;
                    }
                }
            }
        }

        // online softmax per row (the lane's column lr of each row tile)
        uint32_t pf[PF_RW][4];
        // The weights are taken against the current reference at once, beside the
        // tile's maximum; only when some row's reference has to move (lazy rescaling:
        // rare after a piece's first tile) are they taken again against the new one.
        float pw[PF_RW][2][4], m_top[PF_RW];
        bool move = false;
#pragma unroll
        for (int qt = 0; qt < PF_RW; ++qt) {
            const float m_use = m[qt] == NEG_INF ? 0.0f : m[qt];
            float mt = st[0][qt][0];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pw[qt][tt][e] = fast_exp2(fmaf(st[tt][qt][e], c, -m_use));
                    mt = fmaxf(mt, st[tt][qt][e]);
                }
            mt = xmax_16_32(mt);
            m_top[qt] = fmaxf(m[qt], mt * c);
            move |= m_top[qt] > m[qt] + RESCALE_SLACK;
        }
        if (__any(move)) {
#pragma unroll
            for (int qt = 0; qt < PF_RW; ++qt) {
                const float m_new = m_top[qt] > m[qt] + RESCALE_SLACK ? m_top[qt] : m[qt];
                const float m_use = m_new == NEG_INF ? 0.0f : m_new;
                const float alpha = fast_exp2(m[qt] - m_use);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pw[qt][tt][e] = fast_exp2(fmaf(st[tt][qt][e], c, -m_use));
                lsum[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT16; ++dt) o[dt][qt] *= alpha;
                m[qt] = m_new;
            }
        }
#pragma unroll
        for (int qt = 0; qt < PF_RW; ++qt) {
            float ps = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) ps += pw[qt][tt][e];
            lsum[qt] += ps;
            pf[qt][0] = pack2<DT>(pw[qt][0][0], pw[qt][0][1]);
            pf[qt][1] = pack2<DT>(pw[qt][0][2], pw[qt][0][3]);
            pf[qt][2] = pack2<DT>(pw[qt][1][0], pw[qt][1][1]);
            pf[qt][3] = pack2<DT>(pw[qt][1][2], pw[qt][1][3]);
        }

        // O^T += V^T . P^T, V^T through the transposed read (lane layout as in the
        // split-KV kernel: lane j of a 16-lane group gets d = dt * 16 + j at 4 positions)
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef s16x4 __attribute__((address_space(3))) * lds_s16x4;
        const uint32_t vrow0 =
            (uint32_t)(size_t)vbuf[cur] + (lq * 4 + lr / 4) * VROW + (lr % 4) * 8;
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) {
            const uint32_t a0 = vrow0 + dt * 32;
            const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(size_t)a0);
            const s16x4 h1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(size_t)(a0 + 16 * VROW));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w0 = __builtin_bit_cast(u32x2, h0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, h1);
            const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
#pragma unroll
            for (int qt = 0; qt < PF_RW; ++qt) {
                const u32x4 pb = {pf[qt][0], pf[qt][1], pf[qt][2], pf[qt][3]};
                o[dt][qt] = mfma16x16x32<DT>(va, pb, o[dt][qt]);
            }
        }
        if (t + 1 < n_tiles) store_tile((t + 1) % NB, next);
        __syncthreads();
    };
    // unrolled by two so every slot index is a constant (PF_AHEAD 1: both steps use slot 0)
    for (int32_t t = 0; t < n_tiles;) {
        tile(t, stg[0], stg[1 % PF_AHEAD]);
        if (++t >= n_tiles) break;
        tile(t, stg[1 % PF_AHEAD], stg[0]);
        ++t;
    }

    // rows out: each wave writes its own rows (final rows, or this piece's partial)
#pragma unroll
    for (int qt = 0; qt < PF_RW; ++qt) {
        const float lt = xsum_16_32(lsum[qt]);
        const int nb = wave * PF_RW * 16 + qt * 16 + lr;  // row within the segment
        const bool live = row0 + nb < p.rows;
        const int64_t rid = live ? row_id_of(p, b, kvh, row0 + nb) : 0;
        const int64_t part = (int64_t)(pc.slot0 + pc.part) * PF_ROWS + nb;
        if (live && pc.nparts > 1 && lq == 0) store_partial_ml(p, part, m[qt], lt);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) {
            if (!live) continue;
            const int d = dt * 16 + lq * 4;
            const f32x4 v = o[dt][qt];
            if (pc.nparts == 1) {
                const uint2 w = {pack2<DT>(v[0] * inv, v[1] * inv), pack2<DT>(v[2] * inv, v[3] * inv)};
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + rid * D + d) = w;
            } else {  // normalised partial rows
                store_partial4<DT>(p, part * D + d,
                                   float4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv});
            }
        }
    }
    if (pc.nparts > 1 && arrive(p, pc.unit, pc.nparts)) {
#pragma unroll 1
        for (int r0 = 0; r0 < PF_ROWS && row0 + r0 < p.rows; r0 += MROWS) {
            merge_partials<DT, D, MROWS, PF_THREADS>(p, b, kvh, row0 + r0, pc.unit, pc.slot0,
                                                     pc.nparts, msm, r0);
            __syncthreads();  // msm is reused by the next rows
        }
    }
    __syncthreads();  // LDS is reused by the next piece
    });
    });
    zero_empty_sequences<DT, PF_THREADS, D>(p, wg, n_wg);
}

bool prefill_supported(int dtype, int head_dim, int rows, int cache_mode) {
    (void)cache_mode;  // every cache form
    return (dtype == F16 || dtype == BF16) && (head_dim == 64 || head_dim == 128) &&
           rows > KVATTN_PF_MIN_ROWS;
}

template <int DT, int D>
static const void* prefill_kernel_c(int cache_mode) {
    return cache_mode == RING    ? reinterpret_cast<const void*>(&prefill_mfma_kernel<DT, D, RING>)
           : cache_mode == PAGED ? reinterpret_cast<const void*>(&prefill_mfma_kernel<DT, D, PAGED>)
                                 : reinterpret_cast<const void*>(&prefill_mfma_kernel<DT, D, CONTIGUOUS>);
}

const void* select_prefill_kernel(int dtype, int head_dim, int rows, int cache_mode) {
    if (!prefill_supported(dtype, head_dim, rows, cache_mode)) return nullptr;
    if (dtype == F16)
        return head_dim == 128 ? prefill_kernel_c<F16, 128>(cache_mode)
                               : prefill_kernel_c<F16, 64>(cache_mode);
    return head_dim == 128 ? prefill_kernel_c<BF16, 128>(cache_mode)
                           : prefill_kernel_c<BF16, 64>(cache_mode);
}

hipError_t launch_prefill_mfma(const DecodeParams& p, int dtype, int head_dim, int grid,
                               hipStream_t st) {
    const void* k = select_prefill_kernel(dtype, head_dim, p.rows, p.cache_mode);
    if (!k) return hipErrorInvalidValue;
    DecodeParams pp = p;
    void* args[] = {&pp};
    return hipLaunchKernel(k, dim3(grid), dim3(PF_THREADS), args, 0, st);
}

}  // namespace kvattn
