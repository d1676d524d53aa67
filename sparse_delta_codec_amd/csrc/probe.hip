// probe.hip -- achievable-bandwidth probes for the measurement (not part of the
// codec): plain streams over device buffers with 16-byte non-temporal loads
// and stores, in the read:write mixes the codec's kernels have, so that each
// kernel's rate can be set against what the memory system delivers for the
// same mix on the same GPU.  Built into its own library (libpulse_probe.so),
// which only the benchmark loads.
//
//   nread   number of source streams read (0..3), each of n 16-byte pieces
//   write   1: one destination stream of n pieces is written (the XOR of the
//           sources, or a constant when nread == 0); 0: nothing is written
//           but one piece per thread, and only when the XOR of everything it
//           read equals an impossible value (so the loads stay live)
// Every thread takes 4 consecutive pieces per step of a grid-stride loop, so a
// wave's loads cover 4 KiB of contiguous memory per stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4 __attribute__((ext_vector_type(4)));

template <int NR, bool WRITE>
__global__ __launch_bounds__(256) void k_probe(const v4 *__restrict__ a, const v4 *__restrict__ b,
                                               const v4 *__restrict__ c, v4 *__restrict__ out, int64_t n) {
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
    v4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x) * U + threadIdx.x; base < n; base += stride) {
        v4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            v[u] = v4{(uint32_t)i, 1u, 2u, 3u};
            if (i < n) {
                if (NR > 0) v[u] = __builtin_nontemporal_load(a + i);
                if (NR > 1) v[u] ^= __builtin_nontemporal_load(b + i);
                if (NR > 2) v[u] ^= __builtin_nontemporal_load(c + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x;
            if (WRITE) {
                if (i < n) __builtin_nontemporal_store(v[u], out + i);
            } else {
                acc ^= v[u];
            }
        }
    }
    if (!WRITE && acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0xF39CC060u && acc.w == 0x5CEDC834u)
        out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

// One probe launch on `stream`: 0 on success, -1 for bad arguments, -5 when
// the launch fails.  a, b, c, out: 16-byte aligned device buffers of n pieces
// (out: also when write == 0, it must hold one piece per launched thread).
extern "C" int probe_stream(const void *a, const void *b, const void *c, void *out, int64_t n, int32_t nread,
                            int32_t write, int32_t blocks, hipStream_t stream) {
    if (n <= 0 || nread < 0 || nread > 3 || blocks < 1 || !out || (nread == 0 && !write)) return -1;
    if ((nread > 0 && !a) || (nread > 1 && !b) || (nread > 2 && !c)) return -1;
    const v4 *pa = static_cast<const v4 *>(a), *pb = static_cast<const v4 *>(b), *pc = static_cast<const v4 *>(c);
    v4 *po = static_cast<v4 *>(out);
    const dim3 grid((unsigned)blocks), block(256);
    if (write) {
        if (nread == 0) k_probe<0, true><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
        else if (nread == 1) k_probe<1, true><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
        else if (nread == 2) k_probe<2, true><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
        else k_probe<3, true><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
    } else {
        if (nread == 1) k_probe<1, false><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
        else if (nread == 2) k_probe<2, false><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
        else k_probe<3, false><<<grid, block, 0, stream>>>(pa, pb, pc, po, n);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
