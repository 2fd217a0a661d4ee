// Split-KV flash-decoding on the vector ALUs, for up to 16 query rows per KV head.
//
// One workgroup per compute unit streams one equal slice of the step's work (the
// balanced decomposition of work_plan.hpp): a run of attended positions of one
// or more (sequence, KV head, row block) segments.  Each position's K row (and
// V row) of head_dim elements is read by one "lane group" of head_dim*bytes/16
// lanes with one 16-byte load per lane, so a wave instruction covers whole
// 256-byte rows and every byte of K and V is loaded exactly once, straight into
// registers (each byte feeds exactly one lane, so staging it through LDS would
// add a write and a read with no reuse).  All query rows that share the KV head
// (the GQA group times the q_len new tokens) live in every lane, so one K/V
// fetch serves the whole group.
//
// Within a piece the waves take wave tiles (U positions per lane group) from a
// counter in LDS, so a wave that the memory system serves faster takes more
// tiles and the compute unit finishes at its average pace rather than at its
// slowest wave's.  Per tile a lane group forms the scores with packed dot
// products, sums them over its lanes with DPP, and folds them into its own
// running (max, sum, accumulator) - the online softmax of the Flash Attention
// section of the nextadmin.net lesson "KV cache and Flash Attention" (running
// max and sum across tiles, rescale the old terms by exp(m_old - m_new), which
// is 0 when nothing was seen yet).  Scores are kept in the exp2 domain
// (scale * log2 e folded into one multiply).  At the end of a piece the lane
// groups of a wave merge through cross-lane shuffles, the waves through LDS, and
// the workgroup writes either the final rows (the piece is a whole segment) or
// its partial (normalised rows, running max and sum); the last piece of a segment to finish
// merges the partials (split_merge.hpp).
//
// Loads are rolling: a wave issues the next tile's K as soon as the current
// tile's scores have consumed K, and its V as soon as the current V is
// accumulated, so every wave has loads in flight while it computes.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"
#include "split_merge.hpp"
#include "work_plan.hpp"
#include "fused_append.hpp"

namespace kvattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Per-lane load of a cache of element type KT: 16 bytes, or 8 for 8-bit codes (8
// elements a lane either way, which keeps the lane's accumulators and query
// fragment the size of the 16-bit case).
template <int KT> struct KVec { typedef u32x4 T; static constexpr int DW = 4; };
template <> struct KVec<FP8> { typedef u32x2 T; static constexpr int DW = 2; };

// Lane geometry for a cache of element type KT: one load per lane covers EPL
// consecutive elements of a (position, head) row.
template <int KT, int D>
struct Geo {
    static constexpr int EB = Elem<KT>::bytes;
    static constexpr int EPL = KVec<KT>::DW * 4 / EB;  // elements per lane (one load)
    static constexpr int LPR = D / EPL;                // lanes per (position, head) row
};

// A lane's query elements (EPL of them, type DT): one 16-byte load.
template <int DT, int KT>
struct QFrag {
    static constexpr int N = (KVec<KT>::DW * 4 / Elem<KT>::bytes) * Elem<DT>::bytes / 16;
    static_assert(N == 1, "one 16-byte query load per lane");
    u32x4 w[N];
};

__device__ __forceinline__ u32x4 load16(const void* base, int64_t elem_off, int eb) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + elem_off * eb);
}

// q . k over one lane's 16 bytes of K
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// q . k for a lane: K in its own type, or 8-bit codes converted exactly to the
// query's 16-bit type two at a time (every E4M3 value is a binary16 and a bfloat16
// value) and fed to the same packed dot products.  The K scale is applied to the
// score by the caller.
template <int DT, int KT>
__device__ __forceinline__ float dot_q(const QFrag<DT, KT>& q, const typename KVec<KT>::T& k) {
    if constexpr (KT != FP8) {
        return dot16<DT>(q.w[0], k);
    } else {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t w = k[e];  // codes of elements 4e .. 4e+3
            const uint32_t q0 = q.w[0][2 * e], q1 = q.w[0][2 * e + 1];
            if constexpr (DT == F16) {
                const half2_t k0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
                const half2_t k1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
                s = __builtin_amdgcn_fdot2(k0, __builtin_bit_cast(half2_t, q0), s, false);
                s = __builtin_amdgcn_fdot2(k1, __builtin_bit_cast(half2_t, q1), s, false);
            } else {
                const bf16x2_t k0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
                const bf16x2_t k1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
                s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short2_t, k0),
                                                    __builtin_bit_cast(short2_t, q0), s, false);
                s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short2_t, k1),
                                                    __builtin_bit_cast(short2_t, q1), s, false);
            }
        }
        return s;
    }
}

// one lane's load of V as EPL floats (8-bit codes unscaled)
template <int KT>
__device__ __forceinline__ void unpack16(const typename KVec<KT>::T& w, float* f) {
#pragma unroll
    for (int e = 0; e < KVec<KT>::DW; ++e) {
        if constexpr (KT == F16) {
            f[2 * e] = f16_lo(w[e]);
            f[2 * e + 1] = f16_hi(w[e]);
        } else if constexpr (KT == BF16) {
            f[2 * e] = bf16_lo(w[e]);
            f[2 * e + 1] = bf16_hi(w[e]);
        } else if constexpr (KT == FP8) {
            const uint32_t x = w[e];
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
            f[4 * e] = lo[0];
            f[4 * e + 1] = lo[1];
            f[4 * e + 2] = hi[0];
            f[4 * e + 3] = hi[1];
        } else {
            f[e] = __uint_as_float(w[e]);
        }
    }
}

// acc[r][e] += sum_u p[r][u] * v[u][e] for 8-bit V codes (unscaled), two positions
// per packed dot product: a byte permute interleaves the codes of positions u and
// u+1, one exact conversion gives the (v[u][e], v[u+1][e]) pair in the query's
// 16-bit type, and v_dot2 adds p[r][u] v[u][e] + p[r][u+1] v[u+1][e] with the
// weights rounded to that type (as the matrix-core path rounds P).  Paged caches:
// codes behind an out-of-pool page entry are replaced by 0 (= +0.0).
template <int DT, int ROWS, int U, bool ZERO_BAD>
__device__ __forceinline__ void accumulate_fp8_pairs(const u32x2 (&vw)[U], const bool (&vok)[U],
                                                     const float (&pw)[ROWS][U],
                                                     float (&acc)[ROWS][8]) {
    static_assert(U % 2 == 0, "positions are taken in pairs");
#pragma unroll
    for (int u = 0; u < U; u += 2) {
        uint32_t pp[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) pp[r] = pack_pair<DT>(pw[r][u], pw[r][u + 1]);
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
            uint32_t w0 = vw[u][e4], w1 = vw[u + 1][e4];  // codes of elements 4e4 .. 4e4+3
            if constexpr (ZERO_BAD) {
                w0 = vok[u] ? w0 : 0u;
                w1 = vok[u + 1] ? w1 : 0u;
            }
            // bytes (w0.0, w1.0, w0.1, w1.1) and (w0.2, w1.2, w0.3, w1.3)
            const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
            const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
            // element 4e4 + k: pair k of (lo.low, lo.high, hi.low, hi.high)
            if constexpr (DT == F16) {
                const half2_t v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false),
                                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true),
                                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false),
                                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true)};
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int r = 0; r < ROWS; ++r)
                        acc[r][4 * e4 + k] = __builtin_amdgcn_fdot2(
                            __builtin_bit_cast(half2_t, pp[r]), v[k], acc[r][4 * e4 + k], false);
            } else {
                const bf16x2_t v[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false),
                                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true),
                                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false),
                                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)};
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int r = 0; r < ROWS; ++r)
                        acc[r][4 * e4 + k] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(short2_t, pp[r]), __builtin_bit_cast(short2_t, v[k]),
                            acc[r][4 * e4 + k], false);
            }
        }
    }
}

// MASKED: q_len > 1, so rows of one sequence attend different position sets and
// every score gets its row's causal / window test (with one new row the attended
// union is exactly that row's set and no per-row test is needed).
template <int DT, int KT, int D, int ROWS, int CACHE, int U, bool MASKED, int NWAVES>
__global__ __launch_bounds__(NWAVES * 64, 1) void decode_valu_kernel(const DecodeParams p) {
    using G = Geo<KT, D>;
    constexpr int EPL = G::EPL, LPR = G::LPR, EB = G::EB;  // cache element geometry
    constexpr int EBQ = Elem<DT>::bytes;                   // query / output element bytes
    constexpr int THREADS = NWAVES * 64;
    constexpr int LGW = 64 / LPR;          // lane groups per wave
    constexpr int32_t TWW = LGW * U;       // positions per wave tile
    constexpr float NEG_INF = -__builtin_inff();

    const int wg = blockIdx.x;
    const int n_wg = gridDim.x;
    const FlatPlan fp = plan_flat<THREADS>(p, n_wg);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform, so tile loops branch on scalars
    const int lw = tid % 64;
    const int lane = lw % LPR;
    const int lgw = lw / LPR;  // lane group within the wave
    const int d0 = lane * EPL;

    __shared__ float sm_acc[NWAVES][ROWS][D];
    __shared__ float sm_ml[NWAVES][ROWS][2];
    __shared__ MergeSmem<ROWS, THREADS> msm;
    // the tile counter in word 0; lanes 1 .. 63 of the all-lane atomic below hit words
    // 1 .. 63 (adding 0), so one atomic never sends 64 lanes to one LDS bank
    __shared__ int s_tile_words[64];
    int& s_next_tile = s_tile_words[0];

    // Byte addresses: K row of (unit, slot idx) at kb + unit * unit_bytes + idx * tok_bytes
    // (unit = the pool block for paged caches, folded into kb otherwise); V at K + dv.
    const uint32_t tok_bytes = (uint32_t)(p.stride_tok * EB);
    const uint32_t unit_bytes = (uint32_t)(p.stride_seq * EB);
    const int64_t dv = reinterpret_cast<const char*>(p.v) - reinterpret_cast<const char*>(p.k);
    const float c = p.scale_log2;

    // Per-piece view: sequence, KV head, row block, attended span, work range and
    // the lane's K base address.
    struct Ctx {
        int b, kvh, rb;
        int32_t ja, jb, n_tiles;
        SeqSpan s;
        const char* kb;
        const char* klast;  // contiguous and ring caches: the lane's K chunk of the piece's last row
    };
    auto make_ctx = [&](const Piece& pc, const SeqSpan& s) __attribute__((always_inline)) {
        Ctx x;
        x.b = pc.b;
        x.kvh = pc.seg / p.row_blocks;
        x.rb = pc.seg - x.kvh * p.row_blocks;
        x.ja = pc.ja;
        x.jb = pc.jb;
        x.n_tiles = (pc.jb - pc.ja + TWW - 1) / TWW;
        x.s = s;
        x.kb = reinterpret_cast<const char*>(p.k) + ((int64_t)x.kvh * p.stride_head + d0) * EB;
        if constexpr (CACHE != PAGED) x.kb += (int64_t)x.b * p.stride_seq * EB;
        x.klast = x.kb;
        if constexpr (CACHE != PAGED) {
            const Loc L = locate<CACHE>(p, s, x.b, span_pos(s, pc.jb - 1));
            x.klast = x.kb + (uint64_t)(uint32_t)L.idx * tok_bytes;
        }
        return x;
    };
    // Query rows of a piece's KV head: row r = i * group + hg (new token i, head
    // kvh*group + hg); row_i = -1 for padding rows.
    using QF = QFrag<DT, KT>;
    auto load_q = [&](const Ctx& x, QF (&qv)[ROWS]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int rg = x.rb * ROWS + r;
            const bool ok = rg < p.rows;
            const int i = ok ? rg / p.group : 0;
            const int h = x.kvh * p.group + (ok ? rg - i * p.group : 0);
            const int64_t rid = ((int64_t)x.b * p.q_len + i) * p.num_q_heads + h;
#pragma unroll
            for (int n = 0; n < QF::N; ++n)
                qv[r].w[n] = ok ? load16(p.q, rid * D + d0 + n * (16 / EBQ), EBQ)
                                : u32x4{0, 0, 0, 0};
        }
    };

    // Wave tile t of a piece covers work indices ja + t * TWW ...: lane group g of the
    // wave takes ja + t * TWW + u * LGW + g (u < U), so each load instruction reads LGW
    // consecutive positions.  Loads are branch-free: a lane past the piece (or behind a
    // page-table entry outside the pool) loads a clamped, valid address and its data is
    // discarded by selects (score -> -inf, V -> 0).
    int32_t pos[U];
    bool val[U];
    const char* ka[U];
    int32_t blk[U];  // paged: page-table entries of the tile to address next
    auto fetch_pages = [&](const Ctx& x, int32_t t, int32_t (&dst)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j = min(x.ja + t * TWW + u * LGW + lgw, x.jb - 1);
            dst[u] = page_entry(p, x.b, span_pos(x.s, j));
        }
    };
    auto address = [&](const Ctx& x, int32_t t) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j = x.ja + t * TWW + u * LGW + lgw;
            val[u] = j < x.jb;
            pos[u] = span_pos(x.s, min(j, x.jb - 1));
            if constexpr (CACHE == PAGED) {
                const bool in_pool = (uint32_t)blk[u] < (uint32_t)p.num_blocks;
                val[u] = val[u] && in_pool;
                const uint32_t unit = in_pool ? (uint32_t)blk[u] : 0u;
                const uint32_t idx = (uint32_t)pos[u] & ((1u << p.log2_block) - 1);
                ka[u] = x.kb + (uint64_t)unit * unit_bytes + idx * tok_bytes;
            } else {
                const Loc L = locate<CACHE>(p, x.s, x.b, pos[u]);
                ka[u] = x.kb + (uint64_t)(uint32_t)L.idx * tok_bytes;
            }
        }
    };
    using KVT = typename KVec<KT>::T;
    // K and V words of the tile being computed and of the next one, in two buffers
    // whose roles alternate (the tile loop is unrolled by two), so that the next
    // tile's loads land in registers of their own and stay in flight across the
    // current tile's arithmetic: no register copies, no wait at the loop's end.
    KVT kwA[U], vwA[U], kwB[U], vwB[U];
    // Issue the loads of the wave's first tile of a piece (and the piece's Q rows).
    auto first_loads = [&](const Ctx& x, QF (&qv)[ROWS]) __attribute__((always_inline)) {
        load_q(x, qv);
        if (wave < x.n_tiles) {
            if constexpr (CACHE == PAGED) fetch_pages(x, wave, blk);
            address(x, wave);
#pragma unroll
            for (int u = 0; u < U; ++u) kwA[u] = load_stream<KVT>(ka[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) vwA[u] = load_stream<KVT>(ka[u] + dv);
        }
    };

    for_each_unit(p, fp, wg, n_wg, [&](int32_t ui) __attribute__((always_inline)) {
    if (p.k_new) append_unit_rows<CACHE, D, EB, THREADS>(p, fp, ui);
    // The next piece's Q rows and first wave tile are loaded before the current
    // piece's epilogue (merge across waves, stores, arrival), so they are in flight
    // while it runs.
    bool preloaded = false;
    QF qv[ROWS];
    for_each_piece_ahead(p, fp, ui, [&](const Piece& pc, const SeqSpan& s,
                                       auto&& next) __attribute__((always_inline)) {
        const Ctx x = make_ctx(pc, s);
        const int b = x.b, kvh = x.kvh, rb = x.rb;
        const int32_t n_tiles = x.n_tiles;
        if (tid == 0) s_next_tile = NWAVES;  // wave w starts with tile w
        __syncthreads();
        if (!preloaded) first_loads(x, qv);
        preloaded = false;
        // 8-bit caches: the K scale enters the exponent with the softmax scale (scores
        // stay raw code dot products), the V scale multiplies the piece's accumulator
        float cp = c, vsc = 1.0f;
        if constexpr (KT == FP8) {
            cp = c * p.k_scale[kvh];
            vsc = p.v_scale[kvh];
        }

        // MASKED: row r attends pos iff pos <= hi[r] and (pos < n_sink or pos >= lo[r]);
        // a tree mask (token-tree verification) instead lets row r see every position
        // before the new block and new position P0 + j iff bit j of tm[r] is set
        int32_t hi[ROWS], lo[ROWS];
        uint64_t tm[ROWS];
        const bool tree = p.mask_mode == MASK_TREE;
        const int32_t P0 = s.T - p.q_len;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int rg = rb * ROWS + r;
            const int i = rg < p.rows ? rg / p.group : p.q_len - 1;
            const int32_t P = P0 + i;
            hi[r] = tree ? s.T - 1 : P;
            lo[r] = p.mask_mode == MASK_SINK_WINDOW ? P - p.window + 1 : 0;
            tm[r] = tree ? p.tree_mask[(int64_t)b * p.q_len + i] : ~0ull;
        }
        const int32_t tree_from = tree ? P0 : 0x7fffffff;  // first position the tree masks
        float m[ROWS], l[ROWS], acc[ROWS][EPL];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            m[r] = NEG_INF;
            l[r] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[r][e] = 0.0f;
        }

        int32_t cur = wave;
        // the next tile for this wave (after tile `after`): one LDS atomic per tile,
        // requested a tile ahead (two for paged caches, whose page-table entries are
        // read as soon as the tile is granted); deterministic mode: every NWAVES-th tile,
        // a fixed summation order.  Every lane takes part in the atomic (lane 0 adds
        // 1 to the counter, lane l adds 0 to its own word l), so the loop holds no
        // lane-divergent branch; lane 0's result is the tile granted.
        auto grab = [&](int32_t after) __attribute__((always_inline)) -> int32_t {
            if (p.deterministic) return after + NWAVES;
            const int32_t t = __hip_atomic_fetch_add(&s_tile_words[lw], lw == 0 ? 1 : 0,
                                                     __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
            return __builtin_amdgcn_readfirstlane(t);
        };
        int32_t nxt = cur < n_tiles ? grab(cur) : n_tiles;
        if constexpr (CACHE == PAGED)
            if (nxt < n_tiles) fetch_pages(x, nxt, blk);
        // One tile: scores from kc; the next tile's loads into kn/vn (paged: first the
        // page-table entries of the tile after it, so that every wait in the loop is
        // for the oldest loads in flight); softmax update; P.V from vc.
        auto tile = [&](const KVT (&kc)[U], const KVT (&vc)[U], KVT (&kn)[U], KVT (&vn)[U])
                        __attribute__((always_inline)) {
            const bool more = nxt < n_tiles;
            // raw scores q.k; the softmax scale (times log2 e) is applied inside the
            // exp2 argument, so the running max m is kept in scaled units
            float sc[ROWS][U];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float x = group_sum<LPR>(dot_q<DT, KT>(qv[r], kc[u]));
                    bool ok = val[u];
                    if constexpr (MASKED)
                        ok = ok & (pos[u] <= hi[r]) & ((pos[u] < p.n_sink) | (pos[u] >= lo[r]));
                    sc[r][u] = ok ? x : NEG_INF;
                }
            }
            if constexpr (MASKED) {
                // the tree's bits, only on the (rare) tiles that reach the new block
                bool reach = false;
#pragma unroll
                for (int u = 0; u < U; ++u) reach |= pos[u] >= tree_from;
                if (__any(reach)) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int32_t rel = pos[u] - P0;
                        const uint64_t bit = rel >= 0 ? 1ull << (rel & 63) : 0ull;
#pragma unroll
                        for (int r = 0; r < ROWS; ++r)
                            if (rel >= 0 && !(tm[r] & bit)) sc[r][u] = NEG_INF;
                    }
                }
            }
            // a paged position behind an out-of-pool entry was read from block 0 and
            // may hold anything; every other discarded lane read an attended position
            bool vok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) vok[u] = val[u];
            // The next tile's loads are issued unconditionally, which keeps the loop
            // free of merges of loaded and not-loaded registers.  Past the last tile
            // they read one row (contiguous and ring caches: the piece's last) per load
            // instruction: streaming loads leave nothing in L2 for a re-read of the
            // whole tile to hit.
            if (more) {
                address(x, nxt);
            } else if constexpr (CACHE != PAGED) {
#pragma unroll
                for (int u = 0; u < U; ++u) ka[u] = x.klast;
            } else {
                // paged: the row lane 0 read (a valid address), one chunk per instruction.
                // Its offset from the cache base is broadcast, not the address itself, so
                // the loads keep the base's global provenance (an address rebuilt from an
                // integer would make them flat loads, which the compiler can only wait for
                // all at once).  readfirstlane returns a signed int: each half is widened
                // through uint32_t, so a low half with bit 31 set does not sign-extend.
                const uint64_t o0 = (uint64_t)(ka[0] - x.kb);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(o0 >> 32));
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)o0);
                const uint64_t o = ((uint64_t)hi << 32) | (uint64_t)lo;
#pragma unroll
                for (int u = 0; u < U; ++u) ka[u] = x.kb + o;
            }
            int32_t n2 = n_tiles;
            if constexpr (CACHE == PAGED) {
                if (more) n2 = grab(nxt);
                if (n2 < n_tiles) fetch_pages(x, n2, blk);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) kn[u] = load_stream<KVT>(ka[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) vn[u] = load_stream<KVT>(ka[u] + dv);
            float pw[ROWS][U];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                float mt = sc[r][0];
#pragma unroll
                for (int u = 1; u < U; ++u) mt = fmaxf(mt, sc[r][u]);
                const float m_top = fmaxf(m[r], mt * cp);  // cp > 0: max commutes with the scale
                const float m_new = m_top > m[r] + RESCALE_SLACK ? m_top : m[r];  // lazy
                const float m_use = m_new == NEG_INF ? 0.0f : m_new;
                if (__any(m_new != m[r])) {  // rescale only when some lane's reference moved
                    const float alpha = fast_exp2(m[r] - m_use);  // 0 while nothing was seen
                    l[r] *= alpha;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[r][e] *= alpha;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    pw[r][u] = fast_exp2(fmaf(sc[r][u], cp, -m_use));
                    l[r] += pw[r][u];
                }
                m[r] = m_new;
            }
            if constexpr (KT == FP8) {
                accumulate_fp8_pairs<DT, ROWS, U, CACHE == PAGED>(vc, vok, pw, acc);
            } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[EPL];
                unpack16<KT>(vc[u], vf);
                if constexpr (CACHE == PAGED) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) vf[e] = vok[u] ? vf[e] : 0.0f;
                }
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[r][e] = fmaf(pw[r][u], vf[e], acc[r][e]);
            }
            }
            cur = nxt;
            if constexpr (CACHE == PAGED) {
                nxt = n2;
            } else {
                if (cur < n_tiles) nxt = grab(cur);
            }
        };
        // Enter the tile loop with no vector memory operation in flight (the first
        // tile's loads, the previous piece's stores and the first page-table entries
        // complete here).  The compiler's wait counts in the loop hold on every path
        // into it, so they only need to cover the oldest loads in flight; with other
        // operations pending on entry they fall to zero and each tile would wait for
        // the next tile's loads.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unconstrained
        while (cur < n_tiles) {
            tile(kwA, vwA, kwB, vwB);
            if (cur >= n_tiles) break;
            tile(kwB, vwB, kwA, vwA);
        }

        Piece npc;
        SeqSpan ns;
        if (next(npc, ns)) {
            first_loads(make_ctx(npc, ns), qv);
            preloaded = true;
        }

        // Merge the lane groups of each wave (butterfly over lane offsets LPR .. 32).
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const float mo = __shfl_xor(m[r], off, 64);
                const float lo2 = __shfl_xor(l[r], off, 64);
                const float M = fmaxf(m[r], mo);
                const float Mu = M == NEG_INF ? 0.0f : M;
                const float a = fast_exp2(m[r] - Mu);
                const float cc = fast_exp2(mo - Mu);
                l[r] = l[r] * a + lo2 * cc;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float ao = __shfl_xor(acc[r][e], off, 64);
                    acc[r][e] = acc[r][e] * a + ao * cc;
                }
                m[r] = M;
            }
        }

        // Merge the waves through LDS.
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
        for (int idx = tid; idx < ROWS * D; idx += THREADS) {
            const int r = idx / D;
            const int d = idx - r * D;
            if (rb * ROWS + r >= p.rows) continue;
            float M = NEG_INF;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) M = fmaxf(M, sm_ml[w][r][0]);
            const float Mu = M == NEG_INF ? 0.0f : M;
            float L = 0.0f, A = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) {
                const float f = fast_exp2(sm_ml[w][r][0] - Mu);
                L += sm_ml[w][r][1] * f;
                A += sm_acc[w][r][d] * f;
            }
            A *= vsc;
            if (pc.nparts == 1) {
                const int64_t rid = row_id_of(p, b, kvh, rb * ROWS + r);
                store_elem<DT>(p.out, rid * D + d, L > 0.0f ? A / L : 0.0f);
            } else {
                const int64_t part = (int64_t)(pc.slot0 + pc.part) * ROWS + r;
                store_partial1<DT>(p, part * D + d, L > 0.0f ? A / L : 0.0f);  // normalised
                if (d == 0) {
                    store_partial(p.ws_ml + part * 2, M);
                    store_partial(p.ws_ml + part * 2 + 1, L);
                }
            }
        }
        if (pc.nparts > 1)
            arrive_and_merge<DT, D, ROWS, THREADS>(p, b, kvh, rb * ROWS, pc.unit, pc.slot0,
                                                   pc.nparts, msm);
        __syncthreads();  // LDS is reused by the next piece
    });
    });
    zero_empty_sequences<DT, THREADS, D>(p, wg, n_wg);
}

// ---------------------------------------------------------------- instance selection

// Positions per lane group per tile.
#ifndef KVATTN_VALU_U_SMALL
#define KVATTN_VALU_U_SMALL 4   // 1 or 2 rows
#endif
#ifndef KVATTN_VALU_U_MID
#define KVATTN_VALU_U_MID 4     // 4 rows
#endif
#ifndef KVATTN_VALU_U8_FACTOR
#define KVATTN_VALU_U8_FACTOR 1
#endif
#ifndef KVATTN_VALU_U_LARGE
#define KVATTN_VALU_U_LARGE 4   // 8 or 16 rows
#endif

// Kernel selection: one instance per (dtype, head_dim, row bucket, cache form,
// per-row mask); launches and occupancy queries go through the same choice.
// Waves per workgroup (one workgroup per compute unit): as many as the register
// budget of the row bucket allows.
#ifndef KVATTN_VALU_WAVES_SMALL
#define KVATTN_VALU_WAVES_SMALL 8   // 1 or 2 rows
#endif
constexpr int valu_waves(int rows_per_block) {
    return rows_per_block <= 2 ? KVATTN_VALU_WAVES_SMALL : (rows_per_block <= 4 ? 8 : 4);
}

template <int DT, int KT, int D, int ROWS, int CACHE>
inline const void* valu_kernel_t(bool masked) {
    // 8-bit caches with 1-2 rows: KVATTN_VALU_U8_FACTOR times the positions per
    // tile, so a tile moves as many bytes as a 16-bit one
    constexpr int U = (KT == FP8 && ROWS <= 2 ? KVATTN_VALU_U8_FACTOR : 1) *
                      (ROWS <= 2 ? KVATTN_VALU_U_SMALL
                                 : (ROWS <= 4 ? KVATTN_VALU_U_MID : KVATTN_VALU_U_LARGE));
    constexpr int NW = valu_waves(ROWS);
    return masked
               ? reinterpret_cast<const void*>(&decode_valu_kernel<DT, KT, D, ROWS, CACHE, U, true, NW>)
               : reinterpret_cast<const void*>(&decode_valu_kernel<DT, KT, D, ROWS, CACHE, U, false, NW>);
}

template <int DT, int KT, int D, int ROWS>
inline const void* valu_kernel_c(int cache_mode, bool masked) {
    switch (cache_mode) {
    case CONTIGUOUS: return valu_kernel_t<DT, KT, D, ROWS, CONTIGUOUS>(masked);
    case PAGED: return valu_kernel_t<DT, KT, D, ROWS, PAGED>(masked);
    default: return valu_kernel_t<DT, KT, D, ROWS, RING>(masked);
    }
}

template <int DT, int KT, int D>
inline const void* valu_kernel_r(int rows_per_block, int cache_mode, bool masked) {
    switch (rows_per_block) {
    case 1: return valu_kernel_c<DT, KT, D, 1>(cache_mode, masked);
    case 2: return valu_kernel_c<DT, KT, D, 2>(cache_mode, masked);
    case 4: return valu_kernel_c<DT, KT, D, 4>(cache_mode, masked);
    case 8: return valu_kernel_c<DT, KT, D, 8>(cache_mode, masked);
    default: return valu_kernel_c<DT, KT, D, 16>(cache_mode, masked);
    }
}

}  // namespace kvattn
