// patch_pack.hip -- compression of the patch stream: the form the patch takes
// before (and after) the LZ4 block codec.
//
// The sparse patches are compressed further with a generic lossless codec
// (PULSE technical summary, "1. PULSESync", Compressione).  Here that codec is
// this library's LZ4 block format, whose canonical parse only sees runs of one
// byte; an ascending (int32 index, BF16 value) patch has none.  So each index
// becomes its gap to the previous one (gap = idx[k] - idx[k-1] - 1, with
// idx[-1] = -1), and every group of 65536 entries is laid out as six byte
// planes (gap bytes 0..3, value bytes 0..1, little-endian), 64 KiB each: the
// high gap planes are long zero runs.  Entries past the count in the last
// group are zero.  Each plane is then exactly one 64 KiB LZ4 block.
//
// Pack: one thread per four consecutive entries, six 4-byte plane stores.
// Unpack: one 1024-thread workgroup per group, taken as a ticket; the indices
// are a prefix sum of gap + 1 over the whole patch, so each group's base comes
// from a decoupled look-back over the groups before it.  Wave w of the group
// owns entries [4096 w, 4096 w + 4096) in 16 rounds of 256 (4 per lane);
// pass 1 sums gap + 1, pass 2 reads the gap planes again (cache hits), scans
// each round and writes the indices and values with 16-byte and 8-byte stores.
#include "device.hpp"

namespace pulse {

constexpr int64_t PK_GROUP = 65536;
constexpr int PK_THREADS = 1024;
constexpr int PK_ROUNDS = 16;

// byte q of each of four plane words, as one little-endian word
__device__ __forceinline__ uint32_t gather_bytes(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3, int q) {
    const int s = 8 * q;
    return ((p0 >> s) & 0xFFu) | (((p1 >> s) & 0xFFu) << 8) | (((p2 >> s) & 0xFFu) << 16) |
           (((p3 >> s) & 0xFFu) << 24);
}

__global__ __launch_bounds__(256) void k_patch_pack(const int32_t *__restrict__ idx,
                                                    const uint16_t *__restrict__ val, int64_t count,
                                                    uint8_t *__restrict__ packed, int64_t nquads) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nquads) return;
    const int64_t k0 = 4 * t;
    const int64_t grp = k0 / PK_GROUP, j0 = k0 % PK_GROUP;
    int64_t i[4];
    uint32_t v[4];
    if (k0 + 3 < count) {
        const int4 q = *reinterpret_cast<const int4 *>(idx + k0);
        const ushort4 w = *reinterpret_cast<const ushort4 *>(val + k0);
        i[0] = q.x; i[1] = q.y; i[2] = q.z; i[3] = q.w;
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            i[q] = k0 + q < count ? idx[k0 + q] : 0;
            v[q] = k0 + q < count ? val[k0 + q] : 0u;
        }
    }
    int64_t prev = (k0 > 0 && k0 - 1 < count) ? (int64_t)idx[k0 - 1] : -1;
    uint32_t g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        g[q] = k0 + q < count ? (uint32_t)(i[q] - prev - 1) : 0u;
        prev = i[q];
    }
    uint8_t *base = packed + grp * 6 * PK_GROUP + j0;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        *reinterpret_cast<uint32_t *>(base + p * PK_GROUP) = gather_bytes(g[0], g[1], g[2], g[3], p);
    *reinterpret_cast<uint32_t *>(base + 4 * PK_GROUP) =
        (v[0] & 0xFFu) | ((v[1] & 0xFFu) << 8) | ((v[2] & 0xFFu) << 16) | ((v[3] & 0xFFu) << 24);
    *reinterpret_cast<uint32_t *>(base + 5 * PK_GROUP) = (v[0] >> 8) | ((v[1] >> 8) << 8) | ((v[2] >> 8) << 16) |
                                                        ((v[3] >> 8) << 24);
}

struct UnpackArgs {
    const uint8_t *packed;
    int64_t count;
    int32_t *idx;
    uint16_t *val;
    uint32_t *d_status;
    WsHeader *hdr;
    uint64_t *status;
    uint32_t ngroups;
};

constexpr uint64_t kGapCap = 0x80000000ull;  // every valid gap is below 2^31

__global__ __launch_bounds__(PK_THREADS) void k_patch_unpack(UnpackArgs a) {
    __shared__ uint32_t s_grp, s_tag;
    __shared__ uint64_t s_wtot[PK_THREADS / kWave];
    __shared__ uint64_t s_prefix;
    if (threadIdx.x == 0) {
        uint32_t grp, tag;
        ws_begin(a.hdr, a.ngroups, &grp, &tag);
        s_grp = grp;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t grp = s_grp, tag = s_tag;
    if (grp >= a.ngroups) {  // inconsistent workspace state: touch nothing
        if (threadIdx.x == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    const int w = wave_id(), l = lane_id();
    const uint8_t *pg = a.packed + (int64_t)grp * 6 * PK_GROUP;
    const int64_t e_grp = (int64_t)grp * PK_GROUP;
    bool bad = false;

    // gap + 1 of entry 4 l + q of round r (0 past the count); flags gaps that
    // no pack produces
    auto round_x = [&](int r, uint32_t xr[4]) {
        const int off = w * 4096 + r * 256 + 4 * l;
        const uint32_t p0 = *reinterpret_cast<const uint32_t *>(pg + off);
        const uint32_t p1 = *reinterpret_cast<const uint32_t *>(pg + PK_GROUP + off);
        const uint32_t p2 = *reinterpret_cast<const uint32_t *>(pg + 2 * PK_GROUP + off);
        const uint32_t p3 = *reinterpret_cast<const uint32_t *>(pg + 3 * PK_GROUP + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t g = gather_bytes(p0, p1, p2, p3, q);
            const bool valid = e_grp + off + q < a.count;
            bad |= valid && g >= kGapCap;
            xr[q] = valid ? (g >= kGapCap ? (uint32_t)kGapCap : g) + 1u : 0u;
        }
    };

    // pass 1: the wave's sum of gap + 1
    uint64_t lsum = 0;
#pragma unroll 4
    for (int r = 0; r < PK_ROUNDS; ++r) {
        uint32_t xr[4];
        round_x(r, xr);
        lsum += (uint64_t)xr[0] + xr[1] + xr[2] + xr[3];
    }
    const uint64_t wtot = wave_reduce_sum(lsum);
    if (l == 0) s_wtot[w] = wtot;
    __syncthreads();
    uint64_t gtot = 0, wpre = 0;
#pragma unroll
    for (int i = 0; i < PK_THREADS / kWave; ++i) {
        if (i < w) wpre += s_wtot[i];
        gtot += s_wtot[i];
    }
    if (w == 0) {
        bool failed = false;
        const uint64_t agg = gtot < (1ull << 38) ? gtot : (1ull << 38);  // only corrupt data gets near
        const uint64_t pre = lookback_wave(a.status, grp, tag, agg, &failed);
        if (l == 0) {
            if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
            s_prefix = pre;
        }
    }
    __syncthreads();

    // pass 2: indices = (sum of gap + 1 over the entries before) + gap
    uint64_t run = s_prefix + wpre;
#pragma unroll 2
    for (int r = 0; r < PK_ROUNDS; ++r) {
        const int off = w * 4096 + r * 256 + 4 * l;
        uint32_t xr[4];
        round_x(r, xr);  // read again (the group's planes were just read: cache hits)
        const uint64_t rs = (uint64_t)xr[0] + xr[1] + xr[2] + xr[3];
        const uint64_t incl = wave_incl_sum(rs);
        uint64_t c = run + incl - rs;
        int64_t iq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c += xr[q];
            iq[q] = (int64_t)c - 1;
        }
        const uint32_t v4 = *reinterpret_cast<const uint32_t *>(pg + 4 * PK_GROUP + off);
        const uint32_t v5 = *reinterpret_cast<const uint32_t *>(pg + 5 * PK_GROUP + off);
        const int64_t e0 = e_grp + off;
        if (e0 + 3 < a.count) {
#pragma unroll
            for (int q = 0; q < 4; ++q) bad |= iq[q] > 2147483647ll;
            *reinterpret_cast<int4 *>(a.idx + e0) = make_int4((int)iq[0], (int)iq[1], (int)iq[2], (int)iq[3]);
            *reinterpret_cast<ushort4 *>(a.val + e0) =
                make_ushort4((uint16_t)((v4 & 0xFFu) | ((v5 & 0xFFu) << 8)),
                             (uint16_t)(((v4 >> 8) & 0xFFu) | (((v5 >> 8) & 0xFFu) << 8)),
                             (uint16_t)(((v4 >> 16) & 0xFFu) | (((v5 >> 16) & 0xFFu) << 8)),
                             (uint16_t)((v4 >> 24) | ((v5 >> 24) << 8)));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (e0 + q < a.count) {
                    bad |= iq[q] > 2147483647ll;
                    a.idx[e0 + q] = (int32_t)iq[q];
                    a.val[e0 + q] = (uint16_t)(((v4 >> (8 * q)) & 0xFFu) | (((v5 >> (8 * q)) & 0xFFu) << 8));
                }
            }
        }
        run += __shfl(incl, kWave - 1, kWave);
    }
    if (__ballot(bad) && l == 0) or_agent32(a.d_status, 4u /*PULSE_DS_CORRUPT*/);
}

}  // namespace pulse

using namespace pulse;

extern "C" size_t pulse_patch_unpack_ws_bytes(int64_t count) {
    const int64_t ng = (count + PK_GROUP - 1) / PK_GROUP;
    return sizeof(WsHeader) + (size_t)(ng > 0 ? ng : 1) * sizeof(uint64_t);
}

extern "C" int64_t pulse_patch_packed_bytes_impl(int64_t count) {
    return (count + PK_GROUP - 1) / PK_GROUP * 6 * PK_GROUP;
}

extern "C" int pulse_launch_patch_pack(const int32_t *idx, const uint16_t *val, int64_t count, uint8_t *packed,
                                       hipStream_t stream) {
    const int64_t nquads = (count + PK_GROUP - 1) / PK_GROUP * (PK_GROUP / 4);
    const int64_t blocks = (nquads + 255) / 256;
    k_patch_pack<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(idx, val, count, packed, nquads);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_patch_unpack(const uint8_t *packed, int64_t count, int32_t *idx, uint16_t *val,
                                         uint32_t *d_status, void *ws, hipStream_t stream) {
    UnpackArgs a{};
    a.packed = packed;
    a.count = count;
    a.idx = idx;
    a.val = val;
    a.d_status = d_status;
    a.hdr = reinterpret_cast<WsHeader *>(ws);
    a.status = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(WsHeader));
    const int64_t ng = (count + PK_GROUP - 1) / PK_GROUP;
    a.ngroups = (uint32_t)ng;
    k_patch_unpack<<<dim3((unsigned)ng), dim3(PK_THREADS), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
