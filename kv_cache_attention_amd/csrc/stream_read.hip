// Measurement yardstick: a plain streaming read of a device buffer, every byte loaded
// once with 16-byte lane loads and folded into a register.  A decode step reads
// each attended K/V byte once, so its time is bounded below by bytes / bandwidth
// (dothoosh.com speculative-decoding article, "The memory-bandwidth wall"); this
// kernel measures the bandwidth a read-only stream actually reaches on the device,
// the practical ceiling beside the published HBM peak.
//
// Shape (the fastest of the read patterns measured on MI355X): one workgroup of 512
// threads per compute unit, each workgroup streaming its own contiguous share of the
// buffer with sixteen 16-byte nontemporal loads per thread in flight (128 KiB per
// compute unit); plain loads, per-wave shares, or more waves with shorter load
// trains each measured slower.  Nothing is written unless the fold hits one
// particular value (so the loads cannot be dropped and the write traffic is nil).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvattn {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t* __restrict__ buf,
                                                                  int64_t n16, int64_t chunk,
                                                                  uint32_t* sink) {
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < n16 ? c0 + chunk : n16;
    int64_t i = c0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * kReadThreads < c1; i += kReadUnroll * kReadThreads) {
        u32x4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = __builtin_nontemporal_load(buf + i + u * kReadThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < c1; i += kReadThreads) {
        const u32x4_t v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int num_cus,
                              hipStream_t st) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = num_cus > 0 ? num_cus : 1;
    const int64_t chunk = (n16 + grid - 1) / grid;  // 16-byte elements per workgroup
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0, st,
                       reinterpret_cast<const u32x4_t*>(buf), n16, chunk, sink);
    return hipGetLastError();
}

}  // namespace kvattn
