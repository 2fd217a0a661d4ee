// Split-KV decode on the matrix cores, for 16 to 64 query rows per KV head
// (speculative verification with grouped-query attention: q_len new tokens x
// the query heads that share one KV head).  Caches of the query's 16-bit type, or of
// 8-bit E4M3 codes converted exactly to it as they are loaded (instances of the two in
// decode_mfma.hip and decode_mfma_fp8.hip).
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
//                     position: the operand layout), Q^T fragments in LDS;
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
// The next tile's V is loaded as soon as this tile's V sits in LDS, its K as soon
// as S^T has consumed this tile's K, so both are in flight during the rest.  The
// four waves then merge through LDS and the workgroup writes the final rows (its
// sequence needs one split) or its partial (normalised rows, m, l); the last workgroup of the
// (sequence, KV head) merges the partials (split_merge.hpp).
#pragma once

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"
#include "split_merge.hpp"
#include "work_plan.hpp"
#include "fused_append.hpp"

namespace kvattn {
// Workgroups per CU the register budget is cut for (row tiles <= 3).
#ifndef KVATTN_MFMA_WG_PER_CU
#define KVATTN_MFMA_WG_PER_CU 1
#endif

// KT: element type of the caches, DT (16-bit) or FP8 (E4M3 codes, converted exactly to
// DT as they are loaded: every E4M3 value is a binary16 and a bfloat16 value; the K
// scale enters the exponent with the softmax scale, the V scale the accumulator).
template <int KT, int DT>
__device__ __forceinline__ u32x4 kv_words(const char* p) {
    if constexpr (KT == FP8) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = load_stream<u32x2>(p);  // codes of 8 consecutive elements
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t x = w[e];
            if constexpr (DT == F16) {
                r[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
                r[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
            } else {
                r[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
                r[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
            }
        }
        return r;
    } else {
        return load_stream<u32x4>(p);
    }
}

template <int DT, int KT, int D, int R, int CACHE>
__global__ __launch_bounds__(MFMA_THREADS, R <= 3 ? KVATTN_MFMA_WG_PER_CU : 1) void decode_mfma_kernel(const DecodeParams p) {
    using G = MfmaGeo<D, R>;
    constexpr int KS = G::KS, DT16 = G::DT16, VROW = G::VROW, CPR = G::CPR, PPI = G::PPI,
                  NV = G::NV;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr int NQ = R * 16;  // padded rows

    // V staging (per wave) during the loop, reused for the cross-wave merge after it;
    // the Q^T operand fragments, shared by the four waves.
    constexpr int SMEM_V = MFMA_WAVES * G::VBUF;
    // O merge buffer [waves][NQ][OROW] floats: rows padded by 4 floats so the 16 rows a
    // wave's lanes write at once start on 16 different 4-bank groups
    constexpr int OROW = D + 4;
    constexpr int SMEM_O = MFMA_WAVES * NQ * OROW * 4;
    constexpr int SMEM = SMEM_V > SMEM_O ? SMEM_V : SMEM_O;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    __shared__ u32x4 qsm[G::QFRAGS * 64];
    __shared__ float sm_m[MFMA_WAVES][NQ];
    __shared__ float sm_l[MFMA_WAVES][NQ];
    __shared__ float4 sm_wt[NQ];  // row n's weights of the four waves' accumulators
    __shared__ float2 sm_ml[NQ];  // row n's (max, sum) over the four waves

    // the tile counter in word 0; lanes 1 .. 63 of the all-lane atomic hit words 1 .. 63
    // (adding 0), so one atomic never sends 64 lanes to one LDS bank
    __shared__ int s_tile_words[64];
    int& s_next_tile = s_tile_words[0];

    const int wg = blockIdx.x;
    const int n_wg = gridDim.x;
    const FlatPlan fp = plan_flat<MFMA_THREADS>(p, n_wg);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform: scalar branches
    const int l = tid % 64;
    const int lr = l % 16;  // operand row / output column
    const int lq = l / 16;  // operand k-group / output row group

    for_each_unit(p, fp, wg, n_wg, [&](int32_t ui) __attribute__((always_inline)) {
    if (p.k_new) append_unit_rows<CACHE, D, Elem<KT>::bytes, MFMA_THREADS>(p, fp, ui);
    for_each_piece(p, fp, ui, [&](const Piece& pc, const SeqSpan& s) __attribute__((always_inline)) {
    const int b = pc.b;
    // more rows than one block holds (chunked prefill: hundreds of new rows) are cut
    // into blocks of NQ rows, one segment each
    const int kvh = pc.seg / p.row_blocks;
    const int row0 = (pc.seg - kvh * p.row_blocks) * NQ;
    const int32_t j0 = pc.ja;
    const int32_t j1 = pc.jb;

    char* vbuf = smem + wave * G::VBUF;
    constexpr int EB = Elem<KT>::bytes;  // bytes per cache element
    const char* kp = reinterpret_cast<const char*>(p.k);
    const char* vp = reinterpret_cast<const char*>(p.v);

    // Loads are branch-free: a position past the split is clamped to the split's last
    // one (an attended, finite row) and its scores are masked; a paged position behind
    // an out-of-pool entry reads block 0 and both its score and its V are discarded.
    // K in the A-operand lane mapping: position tile + tt*16 + lr, d chunk (ks*4+lq)*8.
    auto load_k = [&](int32_t tb, u32x4 (&kf)[2][KS]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int32_t j = min(tb + tt * 16 + lr, j1 - 1);
            Loc L = locate<CACHE>(p, s, b, span_pos(s, j));
            L.unit = L.unit >= 0 ? L.unit : 0;
            const int64_t off = row_offset<CACHE>(p, L, kvh) + lq * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[tt][ks] = kv_words<KT, DT>(kp + (off + ks * 32) * EB);
        }
    };
    // V coalesced: load v covers PPI whole rows, lane l -> row v*PPI + l/CPR, chunk l%CPR.
    bool vok[NV];
    auto load_v = [&](int32_t tb, u32x4 (&vf)[NV]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int32_t j = min(tb + v * PPI + l / CPR, j1 - 1);
            Loc L = locate<CACHE>(p, s, b, span_pos(s, j));
            vok[v] = L.unit >= 0;
            L.unit = L.unit >= 0 ? L.unit : 0;
            vf[v] = kv_words<KT, DT>(vp + (row_offset<CACHE>(p, L, kvh) + (l % CPR) * 8) * EB);
        }
    };

    // The first tile's K and V go in flight before the rest of the piece's setup (row
    // bounds, accumulators, Q): each wave's first load is then a few instructions
    // after the piece is known.
    const int32_t n_tiles = (j1 - j0 + TILE - 1) / TILE;
    u32x4 kc[2][KS], vr[NV];
    int32_t cur = wave;
    if (cur < n_tiles) {
        load_k(j0 + cur * TILE, kc);
        load_v(j0 + cur * TILE, vr);
    }
    // the thread index for everything that follows the first loads
    const int tp = opaque(tid);
    const int lrp = tp % 16, lqp = (tp % 64) / 16;

    // rows' new-token index (for the causal / window mask); padding rows act as the last
    int row_i[R];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        const int n = row0 + qt * 16 + lr;
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

    // Q^T operand fragments (LDS): fragment f = qt*KS + ks; lane l holds row
    // qt*16 + l%16, d chunk (ks*4 + l/16)*8.
    constexpr int QPT = (G::QFRAGS * 64 + MFMA_THREADS - 1) / MFMA_THREADS;
    u32x4 qreg[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int idx = tp + k * MFMA_THREADS;
        const int f = idx / 64, ll = idx % 64;
        const int qt = f / KS, ks = f % KS;
        const int n = row0 + qt * 16 + ll % 16;
        qreg[k] = u32x4{0, 0, 0, 0};
        if (idx < G::QFRAGS * 64 && n < p.rows) {
            const int i = n / p.group;
            const int h = kvh * p.group + (n - i * p.group);
            const int64_t off = (((int64_t)b * p.q_len + i) * p.num_q_heads + h) * D +
                                (ks * 4 + ll / 16) * 8;
            qreg[k] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) + off);
        }
    }

    // Waves take tiles of TILE positions from a counter in LDS (wave w starts with
    // tile w), so a wave the memory system serves faster takes more tiles; in
    // deterministic mode wave w takes tiles w, w + waves, ...  The next tile is
    // known one tile ahead, and the one after is requested at the top of each
    // iteration, so the LDS atomic's latency is not waited for.
    if (tid == 0) s_next_tile = MFMA_WAVES;
    // Every lane takes part in the atomic (lane 0 adds 1 to the counter, lane l adds 0
    // to its own word l): no lane-divergent branch in the tile loop.
    auto grab = [&](int32_t after) __attribute__((always_inline)) -> int32_t {
        if (p.deterministic) return after + MFMA_WAVES;
        const int32_t t = __hip_atomic_fetch_add(&s_tile_words[l], l == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(t);
    };

    // One register buffer each for K and V: the next tile's V is loaded as soon as
    // this tile's V sits in LDS, the next K as soon as S^T has consumed this K.  The
    // loads are issued unconditionally (past the last tile, positions clamp to the
    // piece's last one), so no path through the loop lacks them and the compiler's
    // waits stay partial: V staging waits for V only, S^T for K only.
    // Q staged from registers (the load counter is in order: this waits for the first
    // tile's loads as well, which the loop's first step needs anyway)
#pragma unroll
    for (int k = 0; k < QPT; ++k)
        if (tp + k * MFMA_THREADS < G::QFRAGS * 64) qsm[tp + k * MFMA_THREADS] = qreg[k];
    __syncthreads();  // Q^T and the tile counter are ready
    int32_t nxt = cur < n_tiles ? grab(cur) : n_tiles;

    // new row i sits at T - q_len + i; rows see positions <= their own
    const int32_t P0 = s.T - p.q_len;
    const bool sink_window = p.mask_mode == MASK_SINK_WINDOW;
    // tree mask (token-tree verification): a row sees every position before the new
    // block and new position P0 + j iff bit j of its word is set
    const bool tree = p.mask_mode == MASK_TREE;
    int32_t hi[R], lo[R];
    uint64_t tm[R];
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        hi[qt] = tree ? s.T - 1 : P0 + row_i[qt];
        lo[qt] = sink_window ? hi[qt] - p.window + 1 : 0;
        tm[qt] = tree ? p.tree_mask[(int64_t)b * p.q_len + row_i[qt]] : ~0ull;
    }
    // 8-bit caches: scores are raw code products, the K scale joins the softmax scale
    const float c = KT == FP8 ? p.scale_log2 * p.k_scale[kvh] : p.scale_log2;

    // enter the loop with no vector memory operation pending, so its head sees the
    // same state from every path
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unconstrained
    while (cur < n_tiles) {
        const int32_t tb = j0 + cur * TILE;
        const bool more = nxt < n_tiles;
        const int32_t n2 = more ? grab(nxt) : n_tiles;  // its value is used at the end
        // stage this tile's V rows in LDS: [position][d], padded rows, 16-byte writes;
        // note whether any row of the tile sits behind an out-of-pool page entry
        bool bad = false;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            u32x4 x = vr[v];
            if constexpr (CACHE == PAGED) {
                if (!vok[v]) x = u32x4{0, 0, 0, 0};
                bad = bad || !vok[v];
            }
            *reinterpret_cast<u32x4*>(vbuf + (v * PPI + l / CPR) * VROW + (l % CPR) * 16) = x;
        }
        load_v(j0 + nxt * TILE, vr);

        // S^T = K . Q^T
        f32x4 st[2][R];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int qt = 0; qt < R; ++qt) {
                f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mfma16x16x32<DT>(kc[tt][ks], qsm[(qt * KS + ks) * 64 + l], acc);
                st[tt][qt] = acc;
            }
        load_k(j0 + nxt * TILE, kc);

        // Mask only where it can bite: a partial tile, rows that do not all see the
        // tile's last position (q_len > 1), a tile reaching a tree's new block, the
        // window mask, or (paged) a bad entry.
        bool edge = (tb + TILE > j1) ||
                    ((p.q_len > 1 || tree) &&
                     (sink_window || span_pos(s, min(tb + TILE, j1) - 1) >= P0 + (tree ? 0 : 1)));
        if constexpr (CACHE == PAGED) edge = edge || __any(bad);
        if (edge) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t j = tb + tt * 16 + lq * 4 + e;
                    const int32_t pos = span_pos(s, min(j, j1 - 1));
                    bool pv = true;
                    if constexpr (CACHE == PAGED) {
                        const int32_t blk = page_entry(p, b, pos);
                        pv = (uint32_t)blk < (uint32_t)p.num_blocks;
                    }
                    const int32_t rel = pos - P0;
                    const uint64_t bit = rel >= 0 ? 1ull << (rel & 63) : 0ull;
#pragma unroll
                    for (int qt = 0; qt < R; ++qt) {
                        const bool ok = (j < j1) & pv & (pos <= hi[qt]) &
                                        ((pos < p.n_sink) | (pos >= lo[qt])) &
                                        ((rel < 0) | ((tm[qt] & bit) != 0));
                        st[tt][qt][e] = ok ? st[tt][qt][e] : NEG_INF;
                    }
                }
            }
        }

        // online softmax per row (row = lane column lr of each row tile); scores stay
        // raw, the scale enters through the exp2 argument
        uint32_t pf[R][4];
        // The weights are taken against the current reference at once, beside the
        // tile's maximum; only when some row's reference has to move (lazy rescaling:
        // rare after a piece's first tile) are they taken again against the new one.
        float pw[R][2][4], m_top[R];
        bool move = false;
#pragma unroll
        for (int qt = 0; qt < R; ++qt) {
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
            for (int qt = 0; qt < R; ++qt) {
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
        // P^T operand: k = 8*lq + e -> positions 4*lq+e (first half), 16+4*lq+e (second)
#pragma unroll
        for (int qt = 0; qt < R; ++qt) {
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

        // O^T += V^T . P^T.  V^T comes back from LDS with the gfx950 transposed read
        // (ds_read_b64_tr_b16): within each 16-lane group, lane j receives element j%4
        // of the rows that lanes j/4, j/4 + 4, j/4 + 8, j/4 + 12 address.  Lane i of
        // group g addresses the 4 d values dt*16 + 4*(i%4) .. +3 of position
        // 4g + i/4 (+16 for the second half), so lane j gets d = dt*16 + j at positions
        // 4g .. 4g + 3 (and 16 + 4g ..): the A operand in the P^T position order.
        __builtin_amdgcn_wave_barrier();
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef s16x4 __attribute__((address_space(3))) * lds_s16x4;
        const uint32_t vrow0 = (uint32_t)(size_t)vbuf + (lq * 4 + lr / 4) * VROW + (lr % 4) * 8;
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) {
            const uint32_t a0 = vrow0 + dt * 32;
            const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(size_t)a0);
            const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(size_t)(a0 + 16 * VROW));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w0 = __builtin_bit_cast(u32x2, h0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, h1);
            const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
#pragma unroll
            for (int qt = 0; qt < R; ++qt) {
                const u32x4 pb = {pf[qt][0], pf[qt][1], pf[qt][2], pf[qt][3]};
                o[dt][qt] = mfma16x16x32<DT>(va, pb, o[dt][qt]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        cur = nxt;
        nxt = n2;
    }

    // ---- merge the four waves: each wave leaves its row maxima and sums in LDS (one
    // barrier), then its unscaled O; meanwhile one thread per row works out the row's
    // weights w_w = 2^(m_w - M) / L (M the largest of the four running maxima, L the sum
    // of the l_w 2^(m_w - M)), so that after the second barrier every output element is
    // sum_w w_w O_w: four fused multiply-adds a wave, no exponentials
#pragma unroll
    for (int qt = 0; qt < R; ++qt) {
        const float lt = xsum_16_32(lsum[qt]);
        if (lqp == 0) {
            sm_m[wave][qt * 16 + lrp] = m[qt];
            sm_l[wave][qt * 16 + lrp] = lt;
        }
    }
    __syncthreads();  // every wave is done with its V staging area
    float* osum = reinterpret_cast<float*>(smem);  // [MFMA_WAVES][NQ][OROW]
    {
        float* slot = osum + wave * NQ * OROW;
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
            for (int qt = 0; qt < R; ++qt) {
                const f32x4 v = o[dt][qt];
                *reinterpret_cast<float4*>(slot + (qt * 16 + lrp) * OROW + dt * 16 + lqp * 4) =
                    float4{v[0], v[1], v[2], v[3]};
            }
    }
    static_assert(MFMA_WAVES == 4, "a float4 of weights per row");
    if (tp < NQ) {
        float mw[MFMA_WAVES], M = NEG_INF;
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w) {
            mw[w] = sm_m[w][tp];
            M = fmaxf(M, mw[w]);
        }
        const float Mu = M == NEG_INF ? 0.0f : M;
        float e[MFMA_WAVES], L = 0.0f;
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w) {
            e[w] = fast_exp2(mw[w] - Mu);  // 0 for a wave that saw nothing
            L += sm_l[w][tp] * e[w];
        }
        // 8-bit caches: P.V was taken on raw codes, the V scale multiplies the rows
        const float inv = L > 0.0f ? (KT == FP8 ? p.v_scale[kvh] : 1.0f) / L : 0.0f;
        sm_wt[tp] = float4{e[0] * inv, e[1] * inv, e[2] * inv, e[3] * inv};
        sm_ml[tp] = float2{M, L};
    }
    __syncthreads();
    // rows out, four d at a time: the final rows (one piece) or this piece's partial.
    // Every chunk's LDS words are read first, then combined: one LDS latency instead of
    // one per chunk (the accumulators are in LDS now, their registers free).
    constexpr int CH = NQ * D / 4 / MFMA_THREADS;  // chunks per thread
    static_assert(CH * MFMA_THREADS == NQ * D / 4, "whole chunks per thread");
    float4 cw[CH];
    float4 ca[CH][MFMA_WAVES];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int idx = tp + k * MFMA_THREADS;
        const int n = idx / (D / 4);
        const int d = (idx - n * (D / 4)) * 4;
        cw[k] = sm_wt[n];
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w)
            ca[k][w] = *reinterpret_cast<const float4*>(osum + (w * NQ + n) * OROW + d);
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int idx = tp + k * MFMA_THREADS;
        const int n = idx / (D / 4);
        const int d = (idx - n * (D / 4)) * 4;
        if (row0 + n >= p.rows) continue;
        const float wv[MFMA_WAVES] = {cw[k].x, cw[k].y, cw[k].z, cw[k].w};
        float4 A = float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < MFMA_WAVES; ++w) {
            const float4 a = ca[k][w];
            A.x = fmaf(wv[w], a.x, A.x);
            A.y = fmaf(wv[w], a.y, A.y);
            A.z = fmaf(wv[w], a.z, A.z);
            A.w = fmaf(wv[w], a.w, A.w);
        }
        if (pc.nparts == 1) {
            const int64_t rid = row_id_of(p, b, kvh, row0 + n);
            const uint2 w = {pack2<DT>(A.x, A.y), pack2<DT>(A.z, A.w)};
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + rid * D + d) = w;
        } else {  // normalised partial rows
            const int64_t part = (int64_t)(pc.slot0 + pc.part) * NQ + n;
            store_partial4<DT>(p, part * D + d, A);
            if (d == 0) {
                const float2 ml = sm_ml[n];
                store_partial_ml(p, part, ml.x, ml.y);
            }
        }
    }
    // the staging area is free again: the merge's scratch lives there
    static_assert(sizeof(MergeSmem<NQ, MFMA_THREADS, true>) <= SMEM, "merge scratch");
    __syncthreads();
    if (pc.nparts > 1) {
        auto& msm = *reinterpret_cast<MergeSmem<NQ, MFMA_THREADS, true>*>(smem);
        arrive_and_merge<DT, D, NQ, MFMA_THREADS>(p, b, kvh, row0, pc.unit, pc.slot0, pc.nparts,
                                                  msm);
        __syncthreads();  // LDS is reused by the next piece
    }
    });
    });
    zero_empty_sequences<DT, MFMA_THREADS, D>(p, wg, n_wg);
}

// Instance of the kernel for a cache form and a row-block size (16-row tiles).
template <int DT, int KT, int D, int R>
inline const void* mfma_kernel_c(int cache_mode) {
    switch (cache_mode) {
    case CONTIGUOUS: return reinterpret_cast<const void*>(&decode_mfma_kernel<DT, KT, D, R, CONTIGUOUS>);
    case PAGED: return reinterpret_cast<const void*>(&decode_mfma_kernel<DT, KT, D, R, PAGED>);
    default: return reinterpret_cast<const void*>(&decode_mfma_kernel<DT, KT, D, R, RING>);
    }
}

template <int DT, int KT, int D>
inline const void* mfma_kernel_r(int rows, int cache_mode) {
    switch (mfma_rows_per_block(rows) / 16) {
    case 1: return mfma_kernel_c<DT, KT, D, 1>(cache_mode);
    case 2: return mfma_kernel_c<DT, KT, D, 2>(cache_mode);
    case 3: return mfma_kernel_c<DT, KT, D, 3>(cache_mode);
    default: return mfma_kernel_c<DT, KT, D, 4>(cache_mode);
    }
}

}  // namespace kvattn
