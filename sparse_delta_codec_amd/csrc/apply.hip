// apply.hip -- row a4 (patch scatter-apply) and the dense XOR apply of row a2/a6.
//
// Scatter: the receiver overrides the listed positions with the replacement
// bits; no floating-point addition, so no drift ("Taking Reinforcement Learning
// Cross Datacenter", Nan Jiang talk, 11:08-11:30; PULSE technical summary,
// "1. PULSESync", Ricostruzione).  Entries are read coalesced; because indices
// ascend, the 2-byte stores of one instruction land in a few neighbouring
// cache lines.
//
// XOR: dst ^= mask with 16-byte loads/stores ("GPU weight teleportation"
// write-up, "XOR masks").
#include "device.hpp"

namespace pulse {

// Lanes take consecutive entries (entry = base + q*64 + lane for q < 8), so
// one store instruction writes 64 consecutive entries of the ascending patch:
// a few neighbouring cache lines per instruction instead of one line per lane.
// Stores and loads share one in-order completion counter, so each iteration
// issues the next iteration's entry loads before its own stores: waiting for
// those loads then never waits for the stores (which only need to drain).
// Neither is masked: a load past the count reads the last entry and is
// dropped, a store that must not happen goes to the buffer's end and is
// dropped by the hardware, so the counter's waits stay exact.  (The view's
// byte size, 2 n, fits the 32-bit range field: n < 2^31.)
constexpr int kApPer = 8;

__global__ __launch_bounds__(256) void k_apply_patch(uint16_t *__restrict__ b, int64_t n,
                                                     const int32_t *__restrict__ idx,
                                                     const uint16_t *__restrict__ val,
                                                     const int64_t *__restrict__ d_count,
                                                     int64_t max_count, uint32_t *d_status) {
    int64_t count = *d_count;
    if (count > max_count) count = max_count;
    const int64_t per_wave = kApPer * kWave;
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / kWave) * per_wave;
    int64_t wb = ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave_id()) * per_wave;  // uniform
    bool bad = false;
    if (wb < count) {
        auto load = [&](int64_t base, int32_t (&ii)[kApPer], uint16_t (&vv)[kApPer]) {
#pragma unroll
            for (int q = 0; q < kApPer; ++q) {
                int64_t k = base + q * kWave + lane_id();
                k = k < count ? k : count - 1;
                ii[q] = idx[k];
                vv[q] = val[k];
            }
        };
        // the entries are waited for where they were loaded (before the
        // stores issued after them on the loop's back edge, none on entry),
        // so the loop head has nothing to wait for
        auto ready = [](int32_t (&ii)[kApPer], uint16_t (&vv)[kApPer]) {
#pragma unroll
            for (int q = 0; q < kApPer; ++q) asm volatile("" ::"v"(ii[q]), "v"((uint32_t)vv[q]));
        };
        const i32x4_t rsrc = buffer_rsrc(b, (uint32_t)(2 * n));
        const int32_t off_none = (int32_t)(uint32_t)(2 * n);
        int32_t ii[kApPer];
        uint16_t vv[kApPer];
        load(wb, ii, vv);
        ready(ii, vv);
        for (; wb < count; wb += stride) {
            int32_t ni[kApPer];
            uint16_t nv[kApPer];
            load(wb + stride < count ? wb + stride : wb, ni, nv);
#pragma unroll
            for (int q = 0; q < kApPer; ++q) {
                const int64_t k = wb + q * kWave + lane_id();
                const int32_t i = ii[q];
                const bool live = k < count;
                const bool in = i >= 0 && i < n;
                bad |= live && !in;
                // byte offset of element i: 2 i < 2^32 because n <= 2^31 - 1 (the
                // entry point's range check), computed unsigned so that
                // i >= 2^30 does not overflow a signed product
                const int32_t off = (int32_t)(2u * (uint32_t)i);
                raw_buffer_store_u16(vv[q], rsrc, live && in ? off : off_none, 0, 0);
            }
            ready(ni, nv);
#pragma unroll
            for (int q = 0; q < kApPer; ++q) {
                ii[q] = ni[q];
                vv[q] = nv[q];
            }
        }
    }
    if (__ballot(bad) && lane_id() == 0) or_agent32(d_status, 2u /*PULSE_DS_BADINDEX*/);
}

// ---- apply with the patch's tile index -----------------------------------------
// tile_first[t] is the first entry whose index is >= 16384 t (tile_first[ntiles]
// the count).  One workgroup per tile: a tile with many entries is read whole
// into LDS, its entries written there, and the tile written back with 16-byte
// stores, so no line of the view is left partially written; a tile with few
// entries (or the partial last tile) takes the entries' 2-byte stores.  Every
// write stays inside the workgroup's own tile; an entry outside it is skipped
// and reported (PULSE_DS_BADINDEX).
constexpr int kAtTile = 16384;
constexpr int64_t kAtDenseMin = 1024;  // entries per tile (6.25%) from which the tile is rewritten whole

__global__ __launch_bounds__(256) void k_apply_patch_tiled(uint16_t *__restrict__ b, int64_t n,
                                                           const int32_t *__restrict__ idx,
                                                           const uint16_t *__restrict__ val,
                                                           const int64_t *__restrict__ tile_first,
                                                           int64_t max_count, uint32_t *d_status) {
    __shared__ u32x4 img[kAtTile / 8];
    const int t = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int64_t e0 = tile * kAtTile;
    const int64_t len = n - e0 < kAtTile ? n - e0 : kAtTile;
    int64_t k0 = tile_first[tile], k1 = tile_first[tile + 1];
    k0 = k0 < 0 ? 0 : (k0 > max_count ? max_count : k0);
    k1 = k1 < k0 ? k0 : (k1 > max_count ? max_count : k1);
    bool bad = false;
    if (k1 - k0 < kAtDenseMin || len < kAtTile) {
        for (int64_t k = k0 + t; k < k1; k += 256) {
            const int64_t i = idx[k];
            if (i >= e0 && i < e0 + len) b[i] = val[k];
            else bad = true;
        }
    } else {
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const u32x4 *>(b + e0 + 8 * (t + 256 * i));
#pragma unroll
        for (int i = 0; i < 8; ++i) img[t + 256 * i] = v[i];
        __syncthreads();
        uint16_t *img16 = reinterpret_cast<uint16_t *>(img);
        for (int64_t k = k0 + t; k < k1; k += 256) {
            const int64_t i = (int64_t)idx[k] - e0;
            if (i >= 0 && i < kAtTile) img16[i] = val[k];
            else bad = true;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4 *>(b + e0 + 8 * (t + 256 * i)) = img[t + 256 * i];
    }
    if (__ballot(bad) && lane_id() == 0) or_agent32(d_status, 2u /*PULSE_DS_BADINDEX*/);
}

// The tile index of an ascending patch: entry k writes tile_first[t] = k for
// every tile t in (tile of entry k - 1, tile of entry k]; entry `count` (one
// past the last) closes the index up to ntiles.  Four entries per thread.
__global__ __launch_bounds__(256) void k_patch_tiles(const int32_t *__restrict__ idx, const int64_t *d_count,
                                                     int64_t max_count, int64_t n, int64_t *__restrict__ tile_first) {
    int64_t count = *d_count;
    if (count > max_count) count = max_count;
    if (count < 0) count = 0;
    const int64_t ntiles = (n + kAtTile - 1) / kAtTile;
    const int64_t k0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (k0 > count) return;
    auto tile_of = [&](int64_t k) -> int64_t {  // tile of entry k (count: ntiles; out-of-range clamped)
        if (k >= count) return ntiles;
        const int64_t i = idx[k];
        return i < 0 ? 0 : (i >= n ? ntiles - 1 : i / kAtTile);
    };
    int64_t prev = k0 > 0 ? tile_of(k0 - 1) : -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t k = k0 + j;
        if (k > count) break;
        const int64_t cur = tile_of(k);
        for (int64_t tt = prev + 1; tt <= cur && tt <= ntiles; ++tt) tile_first[tt] = k;
        prev = cur > prev ? cur : prev;
    }
}

__global__ __launch_bounds__(256) void k_xor_apply(uint8_t *__restrict__ dst,
                                                   const uint8_t *__restrict__ mask,
                                                   int64_t nbytes) {
    const int64_t nvec = nbytes / 16;
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
    const uint4 *m4 = reinterpret_cast<const uint4 *>(mask);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        uint4 d = d4[v];
        const uint4 m = m4[v];
        d.x ^= m.x; d.y ^= m.y; d.z ^= m.z; d.w ^= m.w;
        d4[v] = d;
    }
    if (blockIdx.x == 0 && threadIdx.x < (nbytes & 15)) {
        const int64_t i = nvec * 16 + threadIdx.x;
        dst[i] ^= mask[i];
    }
}

// Apply over a list of views: the patch stream of a list call, tensor s's
// entries being [seg_offsets[s], seg_offsets[s + 1]).  Each wave takes one
// contiguous range of 256-entry chunks, finds the tensor of its first entry by
// a binary search over seg_offsets and then walks forward; lanes whose entry
// lies past the current tensor step ahead on their own.
struct ViewDesc {  // the layout of pulse_view
    uint16_t *b;
    int64_t n;
};

__global__ __launch_bounds__(256) void k_apply_patch_segments(const ViewDesc *__restrict__ views, int32_t nseg,
                                                              const int32_t *__restrict__ idx,
                                                              const uint16_t *__restrict__ val,
                                                              const int64_t *__restrict__ seg_offsets,
                                                              int64_t max_count, uint32_t *d_status) {
    int64_t count = seg_offsets[nseg];
    if (count > max_count) count = max_count;
    const int64_t nchunks = (count + 255) / 256;
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x / kWave);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave_id();
    const int64_t c0 = nchunks * gw / nw, c1 = nchunks * (gw + 1) / nw;
    bool bad = false;
    if (c0 < c1) {
        // last tensor whose first entry is <= the range's first entry
        const int64_t k0 = c0 * 256;
        int32_t lo = 0, hi = nseg - 1;
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (seg_offsets[mid] <= k0) lo = mid;
            else hi = mid - 1;
        }
        int32_t s = lo;
        for (int64_t c = c0; c < c1; ++c) {
            int32_t ii[4];
            uint16_t vv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t k = c * 256 + q * kWave + lane_id();
                ii[q] = k < count ? idx[k] : -1;
                vv[q] = k < count ? val[k] : 0;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t k = c * 256 + q * kWave + lane_id();
                if (k >= count) break;
                int32_t sl = s;
                while (sl + 1 < nseg && k >= seg_offsets[sl + 1]) ++sl;
                const ViewDesc v = views[sl];
                const int64_t i = ii[q];
                if (i >= 0 && i < v.n) v.b[i] = vv[q];
                else bad = true;
            }
            const int64_t kn = (c + 1) * 256;
            while (s + 1 < nseg && seg_offsets[s + 1] <= kn) ++s;
        }
    }
    if (__ballot(bad) && lane_id() == 0) or_agent32(d_status, 2u /*PULSE_DS_BADINDEX*/);
}

}  // namespace pulse

using namespace pulse;

extern "C" int pulse_launch_apply_patch_segments(const void *views, int32_t nseg, const int32_t *idx,
                                                 const uint16_t *val, const int64_t *seg_offsets, int64_t max_count,
                                                 uint32_t *d_status, hipStream_t stream) {
    int64_t blocks = (max_count + 1023) / 1024;
    if (blocks > 256 * 32) blocks = 256 * 32;
    if (blocks < 1) blocks = 1;
    k_apply_patch_segments<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        static_cast<const ViewDesc *>(views), nseg, idx, val, seg_offsets, max_count, d_status);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_apply_patch(uint16_t *b, int64_t n, const int32_t *idx, const uint16_t *val,
                                        const int64_t *d_count, int64_t max_count, uint32_t *d_status,
                                        hipStream_t stream) {
    int64_t blocks = (max_count + 256 * kApPer - 1) / (256 * kApPer);
    if (blocks > 256 * 32) blocks = 256 * 32;
    if (blocks < 1) blocks = 1;
    k_apply_patch<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(b, n, idx, val, d_count, max_count, d_status);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_xor_apply(void *dst, const void *mask, int64_t nbytes, hipStream_t stream) {
    int64_t blocks = (nbytes / 16 + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (blocks < 1) blocks = 1;
    k_xor_apply<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<uint8_t *>(dst),
                                                                 static_cast<const uint8_t *>(mask), nbytes);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_apply_patch_tiled(uint16_t *b, int64_t n, const int32_t *idx, const uint16_t *val,
                                              const int64_t *tile_first, int64_t max_count, uint32_t *d_status,
                                              hipStream_t stream) {
    const int64_t ntiles = (n + kAtTile - 1) / kAtTile;
    k_apply_patch_tiled<<<dim3((unsigned)ntiles), dim3(256), 0, stream>>>(b, n, idx, val, tile_first, max_count,
                                                                         d_status);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_patch_tiles(const int32_t *idx, const int64_t *d_count, int64_t max_count, int64_t n,
                                        int64_t *tile_first, hipStream_t stream) {
    const int64_t threads = max_count / 4 + 1;
    k_patch_tiles<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(idx, d_count, max_count, n,
                                                                                     tile_first);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
