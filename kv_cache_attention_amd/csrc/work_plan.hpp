// Balanced split-KV work decomposition, computed on the device from seq_lens.
//
// The work of a decode step is a list of segments: one per (sequence b, KV head,
// block of query rows), each holding the count_b positions sequence b attends
// (all KV heads and row blocks of a sequence have the same count).  Laid end to
// end in (b, KV head, row block) order they form one flat range of
// W = sum_b count_b * segs_per_seq position-units.  Workgroup w of the grid takes
// the slice [w * chunk, (w + 1) * chunk), chunk = max(ceil(W / grid), min_chunk):
// every workgroup streams the same number of K/V rows whatever the spread of
// sequence lengths, and the grid is sized by the host to what the GPU holds at
// once, so the whole step runs in a single resident round.
//
// A slice crosses segment boundaries: its pieces are processed one after the
// other.  A piece that is a whole segment writes the final rows; otherwise it
// writes a partial (unnormalised accumulator, running max and sum) and the last
// piece of the segment to finish merges them (split_merge.hpp).  Walking the
// pieces in flat order, both the workgroup index and the segment index never
// decrease and at least one grows at each step, so slot = workgroup + segment is
// a distinct workspace slot per piece; the pieces of one segment occupy
// consecutive slots.  The slot count is bounded by grid + segments.
//
// Nothing here needs the host to know the lengths: each workgroup reads seq_lens
// (a scan over the batch in LDS) before its first K/V load.
#pragma once

#include "device_common.hpp"

namespace kvattn {

struct WgRange {
    int64_t total;  // W
    int64_t chunk;
    int64_t x0, x1;  // this workgroup's flat slice (empty when x0 >= x1)
    int32_t b;       // sequence holding x0
    int64_t off_b;   // flat offset of sequence b
};

// Flat work of sequence b: attended positions x segments per sequence.
__device__ __forceinline__ int64_t seq_work(const DecodeParams& p, int b) {
    return (int64_t)seq_span(p, b).count * p.segs_per_seq;
}

template <int THREADS>
__device__ __forceinline__ WgRange plan_range(const DecodeParams& p, int wg, int n_wg) {
    static_assert(THREADS % 64 == 0 && THREADS <= 1024, "whole waves");
    constexpr int NW = THREADS / 64;
    __shared__ int64_t s_part[NW];
    __shared__ int32_t s_b;
    __shared__ int64_t s_off;
    const int tid = threadIdx.x;
    const int per = (p.batch + THREADS - 1) / THREADS;  // sequences per thread
    const int b0 = tid * per;
    int64_t mine = 0;
    for (int k = 0; k < per; ++k)
        if (b0 + k < p.batch) mine += seq_work(p, b0 + k);
    // inclusive scan over the wave, then across waves
    const int lane = tid & 63;
    int64_t inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const long long y = __shfl_up((long long)inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) s_part[tid >> 6] = inc;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int64_t v = s_part[w];
        before += w < (tid >> 6) ? v : 0;
        total += v;
    }
    const int64_t excl = before + inc - mine;  // flat offset of sequence b0

    WgRange r;
    r.total = total;
    int64_t chunk = (total + n_wg - 1) / n_wg;
    if (chunk < p.min_chunk) chunk = p.min_chunk;
    r.chunk = (chunk + 15) & ~(int64_t)15;
    r.x0 = (int64_t)wg * r.chunk;
    r.x1 = min(r.x0 + r.chunk, total);
    // the thread whose sequences hold x0 names the exact one (sequences with no
    // work hold no flat offset, so exactly one thread matches)
    if (r.x0 < total && excl <= r.x0 && r.x0 < excl + mine) {
        int64_t off = excl;
        for (int k = 0; k < per; ++k) {
            const int64_t w = seq_work(p, b0 + k);
            if (r.x0 < off + w) {
                s_b = b0 + k;
                s_off = off;
                break;
            }
            off += w;
        }
    }
    __syncthreads();
    r.b = r.x0 < total ? s_b : 0;
    r.off_b = r.x0 < total ? s_off : 0;
    return r;
}

// One piece of a slice: positions [ja, jb) of the attended list of segment
// `seg` (= kvh * row_blocks + row block) of sequence b.
struct Piece {
    int b;
    int seg;
    int32_t ja, jb;
    int64_t unit;   // segment id: b * segs_per_seq + seg (its arrival counter)
    int64_t slot0;  // workspace slot of the segment's first piece
    int nparts;     // pieces the segment is cut into (1: this piece writes the output)
    int part;       // this piece's index among them
};

// Calls f(piece, span) for each piece of the slice, in flat order.
template <typename F>
__device__ __forceinline__ void for_each_piece(const DecodeParams& p, const WgRange& r, int wg,
                                               F&& f) {
    if (r.x0 >= r.x1) return;
    int b = r.b;
    int64_t off_b = r.off_b;
    SeqSpan s = seq_span(p, b);
    int64_t x = r.x0;
    while (x < r.x1) {
        const int64_t wb = (int64_t)s.count * p.segs_per_seq;
        if (x >= off_b + wb) {  // past sequence b (or b holds nothing): next sequence
            off_b += wb;
            ++b;
            s = seq_span(p, b);
            continue;
        }
        Piece pc;
        pc.b = b;
        pc.seg = (int)((x - off_b) / s.count);
        const int64_t seg0 = off_b + (int64_t)pc.seg * s.count;
        pc.ja = (int32_t)(x - seg0);
        pc.jb = (int32_t)min<int64_t>(s.count, r.x1 - seg0);
        const int64_t first = seg0 / r.chunk;
        const int64_t last = (seg0 + s.count - 1) / r.chunk;
        pc.unit = (int64_t)b * p.segs_per_seq + pc.seg;
        pc.slot0 = first + pc.unit;
        pc.nparts = (int)(last - first + 1);
        pc.part = (int)(wg - first);
        f(pc, s);
        x = seg0 + pc.jb;
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
