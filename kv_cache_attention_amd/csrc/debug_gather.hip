// Test entry: list, for every new row, the flat cache slots it attends, using the
// same span / locate / mask functions as the decode kernels.  One thread per row
// walks its positions in increasing order (a debug path, not a fast one).
#include "device_common.hpp"
#include "launch.hpp"

namespace kvattn {

template <int CACHE>
__global__ void debug_gather_kernel(const DecodeParams p, int max_slots, int32_t* slots_out,
                                    int32_t* counts_out) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;  // b * q_len + i
    if (row >= p.batch * p.q_len) return;
    const int b = row / p.q_len;
    const int i = row - b * p.q_len;
    const SeqSpan s = seq_span(p, b);
    int32_t n = 0;
    for (int32_t j = 0; j < s.count; ++j) {
        const int32_t pos = span_pos(s, j);
        if (!row_attends(p, s, b, i, pos)) continue;
        if (n < max_slots) {
            const Loc L = locate<CACHE>(p, s, b, pos);
            slots_out[(int64_t)row * max_slots + n] = (int32_t)flat_slot<CACHE>(p, L);
        }
        ++n;
    }
    counts_out[row] = n;
}

hipError_t launch_debug_gather(const DecodeParams& p, int max_slots, int32_t* slots_out,
                               int32_t* counts_out, hipStream_t st) {
    const int rows = p.batch * p.q_len;
    const dim3 grid((rows + 63) / 64), block(64);
    switch (p.cache_mode) {
    case CONTIGUOUS:
        hipLaunchKernelGGL(debug_gather_kernel<CONTIGUOUS>, grid, block, 0, st, p, max_slots,
                           slots_out, counts_out);
        break;
    case PAGED:
        hipLaunchKernelGGL(debug_gather_kernel<PAGED>, grid, block, 0, st, p, max_slots,
                           slots_out, counts_out);
        break;
    default:
        hipLaunchKernelGGL(debug_gather_kernel<RING>, grid, block, 0, st, p, max_slots,
                           slots_out, counts_out);
        break;
    }
    return hipGetLastError();
}

}  // namespace kvattn
