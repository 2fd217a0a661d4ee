// Matrix-core split-KV kernel for 16 or more query rows per KV head.
#include "device_common.hpp"
#include "launch.hpp"

namespace kvattn {

bool mfma_supported(int dtype, int head_dim, int rows) {
    (void)dtype; (void)head_dim; (void)rows;
    return false;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int dtype, int head_dim, hipStream_t st) {
    (void)p; (void)dtype; (void)head_dim; (void)st;
    return hipErrorNotSupported;
}

}  // namespace kvattn
