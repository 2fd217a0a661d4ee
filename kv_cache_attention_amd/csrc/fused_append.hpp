// The KV append fused into the decode: a decode step writes the new tokens' keys and
// values back to the cache and attends over them (dothoosh.com speculative-decoding
// article, "The memory-bandwidth wall"), here in one launch.
//
// No grid-wide ordering is needed.  The new positions T - q_len .. T - 1 are the last
// ones of a sequence's attended list, and each is read only by the pieces that cover
// it; every workgroup, before the first load of a unit, writes the new rows that the
// unit's pieces read (K and V of the piece's KV head, from k_new / v_new) and waits
// until the stores are acknowledged, so its own later loads see them.  Pieces of
// other row blocks of the same (sequence, KV head) write the same rows again, with
// the same bytes.  No
// attended position shares a slot with a new one (a ring keeps n_sink + window +
// q_len - 1 <= capacity), so no other load of the step can see a slot change.  Rows
// without a slot (position < 0, past a contiguous or paged cache's capacity, a
// page-table entry outside the pool) are not written, as in the separate append.
#pragma once

#include "work_plan.hpp"

namespace kvattn {

// D: head_dim; EB: bytes per cache element (D * EB is a multiple of 16).  Every
// thread of the workgroup calls it; it returns after a workgroup barrier that follows
// the acknowledgement of every store.
template <int CACHE, int D, int EB, int THREADS>
__device__ __forceinline__ void append_unit_rows(const DecodeParams& p, const FlatPlan& fp,
                                                 int32_t u) {
    constexpr int RB = D * EB;    // bytes per row
    constexpr int CPR = RB / 16;  // 16-byte chunks per row
    static_assert(RB % 16 == 0, "rows of whole 16-byte chunks");
    char* kc = const_cast<char*>(reinterpret_cast<const char*>(p.k));
    char* vc = const_cast<char*>(reinterpret_cast<const char*>(p.v));
    for_each_piece(p, fp, u, [&](const Piece& pc, const SeqSpan& s) __attribute__((always_inline)) {
        int32_t T = plan_len(p, fp, pc.b);
        if (T < 0) T = 0;
        const int32_t tn = T - p.q_len;  // first new position
        // work index of the first new position (the new positions end the list)
        const int32_t jn = tn < s.sink ? max(tn, 0) : s.sink + max(tn - s.tail, 0);
        const int32_t j0 = max(pc.ja, jn);
        if (j0 >= pc.jb) return;
        const int kvh = pc.seg / p.row_blocks;
        const int n = (pc.jb - j0) * CPR;
        for (int c = threadIdx.x; c < n; c += THREADS) {
            const int32_t j = j0 + c / CPR;
            const int ch = c % CPR;
            const int32_t pos = span_pos(s, j);
            const Loc L = locate<CACHE>(p, s, pc.b, pos);
            if (L.unit < 0) continue;
            const int64_t src =
                (((int64_t)pc.b * p.q_len + (pos - tn)) * p.num_kv_heads + kvh) * RB + ch * 16;
            const int64_t dst = row_offset<CACHE>(p, L, kvh) * EB + ch * 16;
            const uint4 kx = *reinterpret_cast<const uint4*>(p.k_new + src);
            const uint4 vx = *reinterpret_cast<const uint4*>(p.v_new + src);
            *reinterpret_cast<uint4*>(kc + dst) = kx;
            *reinterpret_cast<uint4*>(vc + dst) = vx;
        }
    });
    // Every store is acknowledged (written to L2) before the barrier: a barrier alone
    // orders the instructions, not their completion, and the streaming K/V loads that
    // follow go to L2 and could reach it first.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

}  // namespace kvattn
