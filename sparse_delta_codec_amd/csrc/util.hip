// util.hip -- small fill kernels used instead of hipMemsetAsync, so the calls
// stay valid inside captured HIP graphs.
#include "device.hpp"

namespace pulse {

__global__ __launch_bounds__(256) void k_fill_zero(uint8_t *p, size_t nbytes) {
    const size_t nvec = nbytes / 16;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride)
        reinterpret_cast<uint4 *>(p)[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < (nbytes & 15)) p[nvec * 16 + threadIdx.x] = 0;
}

__global__ void k_write_count(int64_t *d, int64_t v) {
    if (threadIdx.x == 0) *d = v;
}

}  // namespace pulse

using namespace pulse;

extern "C" int pulse_launch_fill_zero(void *p, size_t nbytes, hipStream_t stream) {
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return -2;
    size_t blocks = (nbytes / 16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    k_fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<uint8_t *>(p), nbytes);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_write_count(int64_t *d, int64_t v, hipStream_t stream) {
    k_write_count<<<dim3(1), dim3(64), 0, stream>>>(d, v);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
