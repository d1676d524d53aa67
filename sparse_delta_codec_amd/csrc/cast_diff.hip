// cast_diff.hip -- rows a1 + a2 + a3: FP32 -> BF16 cast, bitwise diff against
// the previous served view, and compaction of the changed elements into an
// ascending (int32 index, BF16 value) patch, in one HBM pass.
//
// Sources: the served view is the master weights cast to the serving dtype,
// compared bitwise version to version ("Taking Reinforcement Learning Cross
// Datacenter", Nan Jiang talk, 10:49-11:08 and 12:12-12:44); the patch carries
// indices and new absolute values (PULSE technical summary, "1. PULSESync").
//
// Layout per tile (256 threads, 4096 elements): thread t owns four groups of
// four contiguous elements at tile_base + g*1024 + 4t, so each group is one
// float4 + one ushort4 load per lane and a wave reads 1 KiB / 512 B contiguous
// per instruction.  Changed-element counts of the four groups are packed in
// 16-bit fields of one u64 and scanned together; the tile total is placed by a
// decoupled look-back; entries are staged in LDS and written out contiguously.
#include "device.hpp"

namespace pulse {

constexpr int CD_THREADS = 256;
constexpr int CD_GROUPS = 4;
constexpr int CD_TILE = CD_THREADS * 4 * CD_GROUPS;  // 4096 elements

struct CastDiffArgs {
    const float *w_new;      // FROM_F32 source
    const uint16_t *b_in;    // !FROM_F32 source (new view)
    const uint16_t *b_old;
    uint16_t *b_new;
    uint16_t *mask;
    int32_t *idx;
    uint16_t *val;
    int64_t cap;
    int64_t *d_count;
    uint32_t *d_status;
    int64_t n;
    WsHeader *hdr;
    uint64_t *status;
    uint32_t ntiles;
};

template <bool FROM_F32>
__device__ __forceinline__ void load_new4(const CastDiffArgs &a, int64_t e, uint16_t out[4]) {
    if (e + 3 < a.n) {
        if constexpr (FROM_F32) {
            const float4 f = *reinterpret_cast<const float4 *>(a.w_new + e);
            out[0] = bf16_rne(__float_as_uint(f.x));
            out[1] = bf16_rne(__float_as_uint(f.y));
            out[2] = bf16_rne(__float_as_uint(f.z));
            out[3] = bf16_rne(__float_as_uint(f.w));
        } else {
            const ushort4 h = *reinterpret_cast<const ushort4 *>(a.b_in + e);
            out[0] = h.x; out[1] = h.y; out[2] = h.z; out[3] = h.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (e + k < a.n) {
                if constexpr (FROM_F32) out[k] = bf16_rne(__float_as_uint(a.w_new[e + k]));
                else out[k] = a.b_in[e + k];
            } else {
                out[k] = 0;
            }
        }
    }
}

__device__ __forceinline__ void load_old4(const uint16_t *p, int64_t e, int64_t n, uint16_t out[4]) {
    if (e + 3 < n) {
        const ushort4 h = *reinterpret_cast<const ushort4 *>(p + e);
        out[0] = h.x; out[1] = h.y; out[2] = h.z; out[3] = h.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = (e + k < n) ? p[e + k] : 0;
    }
}

__device__ __forceinline__ void store4(uint16_t *p, int64_t e, int64_t n, const uint16_t v[4]) {
    if (e + 3 < n) {
        *reinterpret_cast<ushort4 *>(p + e) = make_ushort4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e + k < n) p[e + k] = v[k];
    }
}

// ---- streaming variant: no compaction (pure cast, or cast + mask) -----------
template <bool HAS_OLD, bool W_NEW, bool W_MASK>
__global__ __launch_bounds__(256) void k_cast_stream(CastDiffArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
    for (int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; e < a.n; e += stride) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t eh = e + 4 * h;
            if (eh >= a.n) break;
            uint16_t nv[4], ov[4], mv[4];
            load_new4<true>(a, eh, nv);
            if constexpr (HAS_OLD && W_MASK) load_old4(a.b_old, eh, a.n, ov);  // before b_new may overwrite it
            if constexpr (W_NEW) store4(a.b_new, eh, a.n, nv);
            if constexpr (HAS_OLD && W_MASK) {
#pragma unroll
                for (int k = 0; k < 4; ++k) mv[k] = ov[k] ^ nv[k];
                store4(a.mask, eh, a.n, mv);
            }
        }
    }
}

// ---- single-pass compaction -------------------------------------------------
template <bool FROM_F32, bool W_NEW, bool W_MASK>
__global__ __launch_bounds__(CD_THREADS) void k_cast_compact(CastDiffArgs a) {
    __shared__ uint32_t s_tile, s_tag;
    __shared__ uint64_t s_scan[CD_THREADS / kWave];
    __shared__ uint64_t s_prefix;
    __shared__ uint16_t s_loc[CD_TILE];  // tile-local index of each entry
    __shared__ uint16_t s_val[CD_TILE];

    const int t = threadIdx.x;
    if (t == 0) {
        uint32_t tile, tag;
        ws_begin(a.hdr, &tile, &tag);
        s_tile = tile;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile, tag = s_tag;
    const int64_t base = (int64_t)tile * CD_TILE;

    uint16_t nv[CD_GROUPS][4];
    uint32_t chg[CD_GROUPS];
    uint64_t packed = 0;
#pragma unroll
    for (int g = 0; g < CD_GROUPS; ++g) {
        const int64_t e = base + g * (CD_THREADS * 4) + 4 * t;
        uint16_t ov[4];
        load_new4<FROM_F32>(a, e, nv[g]);
        load_old4(a.b_old, e, a.n, ov);
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e + k < a.n && nv[g][k] != ov[k]) m |= 1u << k;
        chg[g] = m;
        packed |= (uint64_t)__builtin_popcount(m) << (16 * g);
        if constexpr (W_NEW) store4(a.b_new, e, a.n, nv[g]);
        if constexpr (W_MASK) {
            uint16_t mv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) mv[k] = ov[k] ^ nv[g][k];
            store4(a.mask, e, a.n, mv);
        }
    }

    // exclusive scan of the four packed 16-bit counts (each field <= 1024)
    uint64_t totals;
    const uint64_t excl = block_excl_sum<CD_THREADS / kWave>(packed, s_scan, &totals);
    uint32_t gbase[CD_GROUPS];
    uint32_t run = 0;
#pragma unroll
    for (int g = 0; g < CD_GROUPS; ++g) {
        gbase[g] = run + (uint32_t)((excl >> (16 * g)) & 0xFFFF);
        run += (uint32_t)((totals >> (16 * g)) & 0xFFFF);
    }
    const uint32_t tile_count = run;

    // stage entries in LDS in ascending element order
#pragma unroll
    for (int g = 0; g < CD_GROUPS; ++g) {
        uint32_t m = chg[g], r = gbase[g];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (m & (1u << k)) {
                s_loc[r] = (uint16_t)(g * (CD_THREADS * 4) + 4 * t + k);
                s_val[r] = nv[g][k];
                ++r;
            }
        }
    }

    if (wave_id() == 0) {
        const uint64_t pre = lookback_wave(a.status, tile, tag, tile_count);
        if (lane_id() == 0) {
            s_prefix = pre;
            if (tile == a.ntiles - 1) *a.d_count = (int64_t)(pre + tile_count);
            if ((int64_t)(pre + tile_count) > a.cap) or_agent32(a.d_status, 1u /*PULSE_DS_CAPACITY*/);
            ws_end(a.hdr, a.ntiles);
        }
    }
    __syncthreads();
    const int64_t pre = (int64_t)s_prefix;
    for (uint32_t r = t; r < tile_count; r += CD_THREADS) {
        const int64_t pos = pre + r;
        if (pos < a.cap) {
            a.idx[pos] = (int32_t)(base + s_loc[r]);
            a.val[pos] = s_val[r];
        }
    }
}

}  // namespace pulse

using namespace pulse;

extern "C" int pulse_launch_cast_diff(const float *w_new, const uint16_t *b_in, const uint16_t *b_old,
                                      uint16_t *b_new, uint16_t *mask, int32_t *idx, uint16_t *val,
                                      int64_t cap, int64_t *d_count, uint32_t *d_status, int64_t n,
                                      void *ws, hipStream_t stream) {
    CastDiffArgs a{};
    a.w_new = w_new;
    a.b_in = b_in;
    a.b_old = b_old;
    a.b_new = b_new;
    a.mask = mask;
    a.idx = idx;
    a.val = val;
    a.cap = cap;
    a.d_count = d_count;
    a.d_status = d_status;
    a.n = n;
    const bool compact = idx != nullptr;
    if (!compact) {
        // streaming: grid sized to cover n with 8 elements per lane, capped
        int64_t blocks = (n + 256 * 8 - 1) / (256 * 8);
        if (blocks > 256 * 64) blocks = 256 * 64;
        if (blocks < 1) blocks = 1;
        const dim3 g((unsigned)blocks), b(256);
        if (b_old && mask && b_new) k_cast_stream<true, true, true><<<g, b, 0, stream>>>(a);
        else if (b_old && mask) k_cast_stream<true, false, true><<<g, b, 0, stream>>>(a);
        else k_cast_stream<false, true, false><<<g, b, 0, stream>>>(a);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
    a.hdr = reinterpret_cast<WsHeader *>(ws);
    a.status = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(WsHeader));
    const int64_t ntiles = (n + CD_TILE - 1) / CD_TILE;
    a.ntiles = (uint32_t)ntiles;
    const dim3 g((unsigned)ntiles), b(CD_THREADS);
    if (w_new) {
        if (b_new && mask) k_cast_compact<true, true, true><<<g, b, 0, stream>>>(a);
        else if (b_new) k_cast_compact<true, true, false><<<g, b, 0, stream>>>(a);
        else if (mask) k_cast_compact<true, false, true><<<g, b, 0, stream>>>(a);
        else k_cast_compact<true, false, false><<<g, b, 0, stream>>>(a);
    } else {
        k_cast_compact<false, false, false><<<g, b, 0, stream>>>(a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" size_t pulse_cast_diff_ws_bytes(int64_t n) {
    const int64_t ntiles = (n + CD_TILE - 1) / CD_TILE;
    return sizeof(WsHeader) + (size_t)(ntiles > 0 ? ntiles : 1) * sizeof(uint64_t);
}
