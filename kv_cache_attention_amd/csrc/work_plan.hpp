// Balanced split-KV work decomposition, computed on the device from seq_lens.
//
// The work of a decode step is a list of segments: one per (sequence b, KV head,
// block of query rows), each holding the count_b positions sequence b attends
// (all KV heads and row blocks of a sequence have the same count).  Laid end to
// end in (b, KV head, row block) order they form one flat range of
// W = sum_b count_b * segs_per_seq position-units, cut into units for a grid
// sized by the host to what the GPU holds at once.  The head of the range is cut
// into one large unit per workgroup (units_per_wg of them), which each workgroup
// takes first; optionally (tail_pct > 0, a build setting that is off by default) the
// last tail_pct percent into about tail_units smaller units per workgroup, handed out
// by a device-wide queue to whichever workgroup is free.  Compute units are served by
// the memory system at rates that differ by several percent, so equal static shares
// end when the slowest finishes; a tail would let the faster ones take more of it,
// but each extra unit costs a piece epilogue and a ramp, which measured more than
// the spread it removed.
//
// A unit crosses segment boundaries: its pieces are processed one after the
// other.  A piece that is a whole segment writes the final rows; otherwise it
// writes a partial (normalised rows, running max and sum) and the last
// piece of the segment to finish merges them (split_merge.hpp).  Walking the
// pieces in flat order, both the unit index and the segment index never decrease
// and at least one grows at each step, so slot = unit + segment is a distinct
// workspace slot per piece; the pieces of one segment occupy consecutive slots.
// The slot count is bounded by units + segments.
//
// Nothing here needs the host to know the lengths: each workgroup reads seq_lens
// (a scan over the batch) before its first K/V load and keeps them - in the lanes of
// every wave for batches of up to 64 sequences (no LDS, no barrier), else in LDS
// (batches of up to kLenCache sequences) - so finding a unit's pieces costs no further
// memory round trip before the loads.
//
// Flat indices are 32-bit: the host launches over batch ranges whose flat range is
// at most kFlatMax (batch x segments x the longest attended set, whatever seq_lens
// holds), so every index, unit boundary and slot below fits with room to spare.  The
// arithmetic runs before a workgroup's first load, one wave per SIMD: 64-bit
// products, comparisons and divisions cost several instructions each there, and
// their registers pushed other values out to spill slots.
#pragma once

#include "device_common.hpp"

namespace kvattn {

constexpr int kLenCache = 1024;  // sequences whose lengths the plan keeps in LDS

// Per-thread view of the flat range after the scan over the batch: thread t owns
// sequences [b0, b0 + per) and their flat offsets [excl, excl + mine).
typedef const int32_t __attribute__((address_space(3)))* lds_i32_ptr;
struct FlatPlan {
    // LDS copy of seq_lens (batch <= kLenCache), typed as LDS so reads of it are LDS
    // reads (a generic pointer would make them flat loads, waited for with every load)
    lds_i32_ptr lens;
    bool has_lens;
    // batch <= 64: every wave holds the whole batch, sequence b in lane b - its length,
    // its flat work and its flat offset - so the plan needs no LDS and no barrier
    bool wl;
    int32_t lT, lw, lexcl;
    int32_t total;   // W
    int32_t big;     // positions per head unit
    int32_t n_big;   // head units: [u * big, (u + 1) * big) for u < n_big
    int32_t xb;      // n_big * big: where the tail starts (>= total: no tail)
    int32_t small;   // positions per tail unit
    int32_t n_units;
    int b0, per;
    int32_t excl, mine;
};

// Quotient of non-negative integers (an unsigned 32-bit division).
__device__ __forceinline__ int32_t div_nn(int32_t a, int32_t b) {
    return (int32_t)((uint32_t)a / (uint32_t)b);
}

// First flat index of unit u, and the unit holding flat index x (< total): the
// units partition the range in order, so both are monotone.
__device__ __forceinline__ int32_t unit_begin(const FlatPlan& f, int32_t u) {
    return u < f.n_big ? u * f.big : f.xb + (u - f.n_big) * f.small;
}
__device__ __forceinline__ int32_t unit_of(const FlatPlan& f, int32_t x) {
    return x < f.xb ? div_nn(x, f.big) : f.n_big + div_nn(x - f.xb, f.small);
}

// seq_lens[b] as the plan read it (b uniform across the wave).
__device__ __forceinline__ int32_t plan_len(const DecodeParams& p, const FlatPlan& f, int b) {
    if (f.wl) return __builtin_amdgcn_readlane(f.lT, b);
    return f.has_lens ? f.lens[b] : p.seq_lens[b];
}

// Span of sequence b, from the lengths the plan holds.
__device__ __forceinline__ SeqSpan plan_span(const DecodeParams& p, const FlatPlan& f, int b) {
    return seq_span_of(p, plan_len(p, f, b));
}

// Flat work of sequence b: attended positions x segments per sequence.
__device__ __forceinline__ int32_t seq_work(const DecodeParams& p, const FlatPlan& f, int b) {
    return plan_span(p, f, b).count * p.segs_per_seq;
}

template <int THREADS>
__device__ __forceinline__ FlatPlan plan_flat(const DecodeParams& p, int n_wg) {
    static_assert(THREADS % 64 == 0 && THREADS <= 1024, "whole waves");
    constexpr int NW = THREADS / 64;
    __shared__ int32_t s_part[NW];
    __shared__ int32_t s_lens[kLenCache];
    const int tid = threadIdx.x;
    FlatPlan f;
    f.has_lens = false;  // read from seq_lens while the plan is made
    f.lens = (lds_i32_ptr)s_lens;
    const int lane = tid & 63;
    int32_t total = 0;
    f.wl = p.batch <= 64;
    f.lT = f.lw = f.lexcl = 0;
    if (f.wl) {
        // one sequence per lane, the same in every wave: a scan over the wave
        const int32_t T = lane < p.batch ? p.seq_lens[lane] : 0;
        const int32_t w = lane < p.batch ? seq_span_of(p, T).count * p.segs_per_seq : 0;
        int32_t inc = w;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        f.lT = T;
        f.lw = w;
        f.lexcl = inc - w;
        total = __builtin_amdgcn_readlane(inc, 63);
        f.per = 0;
        f.b0 = 0;
        f.excl = 0;
        f.mine = 0;
    } else {
        f.per = (p.batch + THREADS - 1) / THREADS;  // sequences per thread
        f.b0 = tid * f.per;
        int32_t mine = 0;
        for (int k = 0; k < f.per; ++k) {
            const int b = f.b0 + k;
            if (b < p.batch) {
                const int32_t T = p.seq_lens[b];
                if (p.batch <= kLenCache) s_lens[b] = T;
                mine += seq_span_of(p, T).count * p.segs_per_seq;
            }
        }
        // inclusive scan over the wave, then across waves
        int32_t inc = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane == 63) s_part[tid >> 6] = inc;
        __syncthreads();  // s_part and s_lens are complete
        f.has_lens = p.batch <= kLenCache;
        int32_t before = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int32_t v = s_part[w];
            before += w < (tid >> 6) ? v : 0;
            total += v;
        }
        f.excl = before + inc - mine;
        f.mine = mine;
    }
    f.total = total;
    // units_per_wg = 0: units of exactly min_chunk positions (forced unit lengths)
    const int32_t units = n_wg * p.units_per_wg;
    int32_t usz = units > 0 ? div_nn(total + units - 1, units) : 0;
    if (usz < p.min_chunk) usz = p.min_chunk;
    usz = (usz + 15) & ~15;
    // uniform units of usz positions, unless the tail applies: every workgroup has
    // a head unit, and those (>= min_chunk) leave a tail to share
    f.big = usz;
    f.n_big = div_nn(total + usz - 1, usz);
    f.xb = f.n_big * usz;
    f.small = usz;
    if (p.tail_pct > 0 && units > 0 && f.n_big >= units) {
        int32_t big = (int32_t)(((int64_t)usz * (100 - p.tail_pct) / 100) & ~(int64_t)15);
        if (big < p.min_chunk) big = (p.min_chunk + 15) & ~15;
        if ((int64_t)units * big < total) {
            const int32_t rest = total - units * big;
            const int32_t tu = n_wg * p.tail_units;
            int32_t small = div_nn(rest + tu - 1, tu);
            if (small < p.min_chunk) small = p.min_chunk;
            f.big = big;
            f.n_big = units;
            f.xb = units * big;
            f.small = (small + 15) & ~15;
        }
    }
    f.n_units = f.xb >= total ? div_nn(total + f.big - 1, f.big)
                              : f.n_big + div_nn(total - f.xb + f.small - 1, f.small);
    return f;
}

// The sequence holding flat index x (< total) and its flat offset, found by the
// thread whose sequences hold x (sequences with no work hold no flat offset, so
// exactly one thread matches).  Every thread of the workgroup must call it.
struct SeqAt {
    int b;
    int32_t off;
};
__device__ __forceinline__ SeqAt seq_at(const DecodeParams& p, const FlatPlan& f, int32_t x) {
    if (f.wl) {  // the lane whose sequence holds x, found by a ballot in every wave
        const uint64_t hit = __ballot(f.lw > 0 && f.lexcl <= x && x < f.lexcl + f.lw);
        const int b = hit ? (int)__builtin_ctzll(hit) : 0;
        return SeqAt{b, __builtin_amdgcn_readlane(f.lexcl, b)};
    }
    __shared__ int32_t s_b;
    __shared__ int32_t s_off;
    __syncthreads();  // earlier readers of s_b / s_off are done
    if (f.excl <= x && x < f.excl + f.mine) {
        int32_t off = f.excl;
        for (int k = 0; k < f.per; ++k) {
            const int32_t w = seq_work(p, f, f.b0 + k);
            if (x < off + w) {
                s_b = f.b0 + k;
                s_off = off;
                break;
            }
            off += w;
        }
    }
    __syncthreads();
    return SeqAt{s_b, s_off};
}

// One piece of a unit: positions [ja, jb) of the attended list of segment
// `seg` (= kvh * row_blocks + row block) of sequence b.
struct Piece {
    int b;
    int seg;
    int32_t ja, jb;
    int32_t unit;   // segment id: b * segs_per_seq + seg (its arrival counter)
    int32_t slot0;  // workspace slot of the segment's first piece
    int nparts;     // pieces the segment is cut into (1: this piece writes the output)
    int part;       // this piece's index among them
};

// Calls f(piece, span, next) for each piece of unit u, in flat order.  next(np, ns)
// (at most one call, in every thread or in none) gives the unit's next piece and
// returns whether there is one, so a kernel can issue its first loads before the
// current piece's epilogue; the next piece is worked out only then, after the
// current piece's own first loads are in flight.
template <typename F>
__device__ __forceinline__ void for_each_piece_ahead(const DecodeParams& p, const FlatPlan& fp,
                                                     int32_t u, F&& f) {
    const int32_t x0 = unit_begin(fp, u);
    const int32_t x1 = min(unit_begin(fp, u + 1), fp.total);
    const SeqAt at = seq_at(p, fp, x0);
    int b = at.b;
    int32_t off_b = at.off;
    SeqSpan sb = plan_span(p, fp, b);
    // the piece that starts at flat index x (< x1)
    auto piece_at = [&](int32_t x, Piece& pc, SeqSpan& ps) __attribute__((always_inline)) {
        // sequences that hold nothing, or that x is already past, are skipped
        while (x >= off_b + sb.count * p.segs_per_seq) {
            off_b += sb.count * p.segs_per_seq;
            ++b;
            sb = plan_span(p, fp, b);
        }
        pc.b = b;
        pc.seg = (int)div_nn(x - off_b, sb.count);
        const int32_t seg0 = off_b + pc.seg * sb.count;
        pc.ja = x - seg0;
        pc.jb = min(sb.count, x1 - seg0);
        const int32_t first = unit_of(fp, seg0);
        const int32_t last = unit_of(fp, seg0 + sb.count - 1);
        pc.unit = b * p.segs_per_seq + pc.seg;
        pc.slot0 = first + pc.unit;
        pc.nparts = last - first + 1;
        pc.part = u - first;
        ps = sb;
        return seg0 + pc.jb;  // flat index just past the piece
    };
    if (x0 >= x1) return;
    Piece cur;
    SeqSpan cs;
    int32_t x = piece_at(x0, cur, cs);
    for (;;) {
        const bool more = x < x1;
        bool known = false;
        Piece nx = cur;
        SeqSpan ns = cs;
        int32_t xn = x;
        auto next = [&](Piece& np, SeqSpan& nps) __attribute__((always_inline)) {
            if (more && !known) xn = piece_at(x, nx, ns);
            known = true;
            np = nx;
            nps = ns;
            return more;
        };
        f(cur, cs, next);
        if (!more) break;
        if (!known) xn = piece_at(x, nx, ns);
        cur = nx;
        cs = ns;
        x = xn;
    }
}

// Calls f(piece, span) for each piece of unit u, in flat order.
template <typename F>
__device__ __forceinline__ void for_each_piece(const DecodeParams& p, const FlatPlan& fp,
                                               int32_t u, F&& f) {
    for_each_piece_ahead(p, fp, u,
                         [&](const Piece& pc, const SeqSpan& s, auto&&) __attribute__((always_inline)) {
                             f(pc, s);
                         });
}

// Runs body(u) for every unit this workgroup takes.  Workgroup w starts with unit
// w; when there are more units than workgroups, further units come from a
// device-wide counter (one atomic per unit, issued a unit ahead), so workgroups that
// the memory system serves faster take more.  In deterministic mode workgroup w takes
// units w, w + grid, ...  The last workgroup to leave puts the counter back to zero
// for the next call: every workgroup counts itself out only after its final take, so
// no take can follow the reset.  With no more units than workgroups (the usual plan)
// the counter is not touched at all: every workgroup hitting one address at launch
// and again at exit serialises for microseconds, and the loads that follow an atomic
// wait for it.
template <typename F>
__device__ __forceinline__ void for_each_unit(const DecodeParams& p, const FlatPlan& fp, int wg,
                                              int n_wg, F&& body) {
    __shared__ int32_t s_next_unit[2];  // by iteration parity: a slot is rewritten only
                                        // after a barrier that follows every read of it
    const bool queued = !p.deterministic && fp.n_units > n_wg;
    int32_t u = wg;
    for (int it = 0; u < fp.n_units; ++it) {
        int32_t next = 0;
        if (threadIdx.x == 0)  // issued now, its result is waited for only after the unit
            next = !queued ? u + n_wg
                           : n_wg + __hip_atomic_fetch_add(p.queue, 1, __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_AGENT);
        body(u);
        if (threadIdx.x == 0) s_next_unit[it & 1] = next;
        __syncthreads();
        u = s_next_unit[it & 1];
    }
    if (threadIdx.x == 0 && queued) {
        if (__hip_atomic_fetch_add(p.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            n_wg - 1) {
            __hip_atomic_store(p.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Rows of sequences that attend nothing (T = 0) are zeros; no piece covers them.
// Workgroup w takes sequences w, w + grid, ...
template <int DT, int THREADS, int D>
__device__ __forceinline__ void zero_empty_sequences(const DecodeParams& p, int wg, int n_wg) {
    for (int b = wg; b < p.batch; b += n_wg) {
        if (seq_span(p, b).count > 0) continue;
        const int64_t n = (int64_t)p.q_len * p.num_q_heads * D;  // elements of sequence b
        char* o = reinterpret_cast<char*>(p.out) + (int64_t)b * n * Elem<DT>::bytes;
        const int64_t n16 = n * Elem<DT>::bytes / 16;  // D * bytes is a multiple of 16
        for (int64_t i = threadIdx.x; i < n16; i += THREADS)
            reinterpret_cast<uint4*>(o)[i] = uint4{0, 0, 0, 0};
    }
}

}  // namespace kvattn
