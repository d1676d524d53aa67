// cast_diff.hip -- rows a1 + a2 + a3: FP32 -> BF16 cast, bitwise diff against
// the previous served view, and compaction of the changed elements into an
// ascending (int32 index, BF16 value) patch, in one HBM pass.
//
// Sources: the served view is the master weights cast to the serving dtype,
// compared bitwise version to version ("Taking Reinforcement Learning Cross
// Datacenter", Nan Jiang talk, 10:49-11:08 and 12:12-12:44); the patch carries
// indices and new absolute values (PULSE technical summary, "1. PULSESync").
//
// One launch streams the tensor once; the patch is written in ascending index
// order by a single-pass decoupled look-back over 16384-element tiles, one
// workgroup per tile.  Tiles are handed out as tickets (one device-scope atomic
// when a workgroup starts), so no tile ever waits for one that has not been
// handed to a running workgroup, whatever else shares the GPU.
#include "device.hpp"

namespace pulse {

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
            const uint32_t p0 = cast_pair(f.x, f.y), p1 = cast_pair(f.z, f.w);
            out[0] = (uint16_t)p0;
            out[1] = (uint16_t)(p0 >> 16);
            out[2] = (uint16_t)p1;
            out[3] = (uint16_t)(p1 >> 16);
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
// Tile = 4 waves x 4096 elements.  Wave w owns [tile_base + 4096 w, +4096) as
// 16 groups of 256: lane l holds elements g*256 + 4l + k (one float4 + one
// ushort4 per group), so every load is 1 KiB / 512 B contiguous per wave.
// Pass 1 streams the tile (cast, compare, b_new / mask stores) keeping the
// changed flags (64 bits) and the new values (32 VGPRs) in registers; the
// wave totals give the tile total; one look-back places the tile; pass 2
// ranks each changed element with ballots (v_mbcnt) and stores it directly at
// its final position, lanes of a wave writing consecutive entries.
constexpr int CD_THREADS = 256;
constexpr int CD_GROUPS = 16;
constexpr int CD_WAVE_ELEMS = CD_GROUPS * 256;                    // 4096
constexpr int CD_TILE = (CD_THREADS / kWave) * CD_WAVE_ELEMS;   // 16384


// Pass 1 of one tile for one thread: loads, cast, compare, the b_new / mask
// stores; returns the changed flags (bit 4g+k: element g*256 + 4l + k) and
// keeps the new values in nvp (two BF16 per register).  FULL: the whole tile
// lies inside [0, n): the 8 groups of a half are loaded before any is used
// (float4 + 8 bytes per group), and every compare and store works on pairs of
// BF16 packed in 32 bits.
template <bool FULL, bool FROM_F32, bool W_NEW, bool W_MASK>
__device__ __forceinline__ uint64_t cd_pass1(const CastDiffArgs &a, int64_t wbase, int lo, uint32_t nvp[]) {
    uint64_t flags = 0;
    if constexpr (FULL) {
        const float *pw = a.w_new + wbase + lo;
        const uint16_t *pi = a.b_in + wbase + lo;
        const uint16_t *po = a.b_old + wbase + lo;
        uint16_t *pn = a.b_new + wbase + lo;
        uint16_t *pm = a.mask + wbase + lo;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 fv[8];
            u32x2 ov[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int off = (h * 8 + j) * 256;
                if constexpr (FROM_F32) fv[j] = *reinterpret_cast<const u32x4 *>(pw + off);
                else {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(pi + off);
                    fv[j] = u32x4{v.x, v.y, 0u, 0u};
                }
                ov[j] = *reinterpret_cast<const u32x2 *>(po + off);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int g = h * 8 + j;
                const int off = g * 256;
                uint32_t p0, p1;
                if constexpr (FROM_F32) {
                    p0 = cast_pair(__uint_as_float(fv[j].x), __uint_as_float(fv[j].y));
                    p1 = cast_pair(__uint_as_float(fv[j].z), __uint_as_float(fv[j].w));
                } else {
                    p0 = fv[j].x;
                    p1 = fv[j].y;
                }
                const uint32_t x0 = p0 ^ ov[j].x, x1 = p1 ^ ov[j].y;
                flags |= pair_flags(x0, x1) << (4 * g);
                nvp[2 * g] = p0;
                nvp[2 * g + 1] = p1;
                if constexpr (W_NEW) *reinterpret_cast<u32x2 *>(pn + off) = u32x2{p0, p1};
                if constexpr (W_MASK) *reinterpret_cast<u32x2 *>(pm + off) = u32x2{x0, x1};
            }
            sched_fence();  // eight groups of loads in flight at a time
        }
    } else {
        // the tile that extends past n: element by element
#pragma unroll 1
        for (int g = 0; g < CD_GROUPS; ++g) {
            const int64_t e = wbase + g * 256 + lo;
            uint16_t nv[4], ov[4];
            load_new4<FROM_F32>(a, e, nv);
            load_old4(a.b_old, e, a.n, ov);
            uint16_t mv[4];
            uint64_t f = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                mv[k] = ov[k] ^ nv[k];
                if (e + k < a.n && mv[k] != 0) f |= 1ull << k;
            }
            flags |= f << (4 * g);
            nvp[2 * g] = (uint32_t)nv[0] | ((uint32_t)nv[1] << 16);
            nvp[2 * g + 1] = (uint32_t)nv[2] | ((uint32_t)nv[3] << 16);
            if constexpr (W_NEW) store4(a.b_new, e, a.n, nv);
            if constexpr (W_MASK) store4(a.mask, e, a.n, mv);
        }
    }
    return flags;
}

constexpr int CD_SB = 512;  // patch entries staged per wave before a coalesced flush

struct CdShared {
    uint32_t wtot[CD_THREADS / kWave];
    uint64_t prefix;
    int32_t sbi[CD_THREADS / kWave][CD_SB];
    uint16_t sbv[CD_THREADS / kWave][CD_SB];
};

// Writes the wave's staged entries [0, nb) to the patch at out (lanes write
// consecutive entries: full-width stores) and empties the buffer.
__device__ __forceinline__ void cd_flush(const CastDiffArgs &a, const int32_t *sbi, const uint16_t *sbv, uint32_t &nb,
                                         int64_t &out) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the lanes' staged entries are visible to the wave
    for (uint32_t i = lane_id(); i < nb; i += kWave) {
        const int64_t pos = out + i;
        if (pos < a.cap) {
            a.idx[pos] = sbi[i];
            a.val[pos] = sbv[i];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // reads done before the buffer is refilled
    out += nb;
    nb = 0;
}

// Pass 2 of one wave: each changed element is ranked with ballots and staged
// in the wave's LDS buffer at its rank; the buffer goes out with coalesced
// stores (the wave's entries are one contiguous stretch of the patch, the
// first at position run).
__device__ __forceinline__ void cd_pass2(const CastDiffArgs &a, uint64_t flags, const uint32_t nvp[], int64_t wbase,
                                         int lo, int64_t run, int32_t *sbi, uint16_t *sbv) {
    uint32_t nb = 0;
#pragma unroll
    for (int g = 0; g < CD_GROUPS; ++g) {
        const uint32_t f = (uint32_t)(flags >> (4 * g)) & 0xFu;
        const uint64_t m0 = __ballot(f & 1u), m1 = __ballot(f & 2u), m2 = __ballot(f & 4u), m3 = __ballot(f & 8u);
        const uint32_t gtot = __builtin_popcountll(m0) + __builtin_popcountll(m1) + __builtin_popcountll(m2) +
                              __builtin_popcountll(m3);
        if (gtot == 0) continue;
        if (nb + gtot > (uint32_t)CD_SB) cd_flush(a, sbi, sbv, nb, run);
        uint32_t r = nb + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
        const int32_t e = (int32_t)(wbase + g * 256 + lo);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (f & (1u << k)) {
                sbi[r] = e + k;
                sbv[r] = (uint16_t)(nvp[2 * g + (k >> 1)] >> (16 * (k & 1)));
                ++r;
            }
        }
        nb += gtot;
    }
    if (nb) cd_flush(a, sbi, sbv, nb, run);
}

// Ranks and stages the wave's changed elements in its LDS buffer without
// storing them (the caller guarantees they fit); nb becomes their number.
__device__ __forceinline__ void cd_stage(uint64_t flags, const uint32_t nvp[], int64_t wbase, int lo, int32_t *sbi,
                                         uint16_t *sbv, uint32_t &nb) {
#pragma unroll
    for (int g = 0; g < CD_GROUPS; ++g) {
        const uint32_t f = (uint32_t)(flags >> (4 * g)) & 0xFu;
        const uint64_t m0 = __ballot(f & 1u), m1 = __ballot(f & 2u), m2 = __ballot(f & 4u), m3 = __ballot(f & 8u);
        const uint32_t gtot = __builtin_popcountll(m0) + __builtin_popcountll(m1) + __builtin_popcountll(m2) +
                              __builtin_popcountll(m3);
        if (gtot == 0) continue;
        uint32_t r = nb + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
        const int32_t e = (int32_t)(wbase + g * 256 + lo);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (f & (1u << k)) {
                sbi[r] = e + k;
                sbv[r] = (uint16_t)(nvp[2 * g + (k >> 1)] >> (16 * (k & 1)));
                ++r;
            }
        }
        nb += gtot;
    }
}

// One tile: pass 1, the tile total, its look-back, pass 2 (ranked stores).
template <bool FULL, bool FROM_F32, bool W_NEW, bool W_MASK>
__device__ __forceinline__ void cd_tile(const CastDiffArgs &a, uint32_t tile, uint32_t tag, CdShared &sh) {
    const int w = wave_id(), l = lane_id();
    const int64_t wbase = (int64_t)tile * CD_TILE + (int64_t)w * CD_WAVE_ELEMS;
    const int lo = 4 * l;
    uint32_t nvp[CD_GROUPS * 2];  // new values, two per register
    const uint64_t flags = cd_pass1<FULL, FROM_F32, W_NEW, W_MASK>(a, wbase, lo, nvp);

    const uint32_t wtot = wave_reduce_sum((uint32_t)__builtin_popcountll(flags));
    if (l == 0) sh.wtot[w] = wtot;
    __syncthreads();
    uint32_t tile_count = 0, wpre = 0;
#pragma unroll
    for (int i = 0; i < CD_THREADS / kWave; ++i) {
        if (i < w) wpre += sh.wtot[i];
        tile_count += sh.wtot[i];
    }
    uint32_t wmax = 0;
#pragma unroll
    for (int i = 0; i < CD_THREADS / kWave; ++i) wmax = sh.wtot[i] > wmax ? sh.wtot[i] : wmax;
    auto place = [&](uint64_t pre, bool failed) {  // lane 0 of wave 0
        if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        sh.prefix = pre;
        if (tile == a.ntiles - 1) *a.d_count = (int64_t)(pre + tile_count);
        if ((int64_t)(pre + tile_count) > a.cap) or_agent32(a.d_status, 1u /*PULSE_DS_CAPACITY*/);
    };
    if (wmax <= (uint32_t)CD_SB) {
        // every wave's entries fit its LDS buffer: publish the tile's count,
        // rank and stage while the predecessors' counts arrive, then store
        if (w == 0) lookback_publish(a.status, tile, tag, tile_count);
        uint32_t nb = 0;
        if (wtot != 0) cd_stage(flags, nvp, wbase, lo, sh.sbi[w], sh.sbv[w], nb);
        if (w == 0) {
            bool failed = false;
            const uint64_t pre = lookback_resolve(a.status, tile, tag, tile_count, &failed);
            if (l == 0) place(pre, failed);
        }
        __syncthreads();
        int64_t run = (int64_t)sh.prefix + wpre;
        if (nb) cd_flush(a, sh.sbi[w], sh.sbv[w], nb, run);
    } else {
        if (w == 0) {
            bool failed = false;
            const uint64_t pre = lookback_wave(a.status, tile, tag, tile_count, &failed);
            if (l == 0) place(pre, failed);
        }
        __syncthreads();
        if (tile_count != 0) cd_pass2(a, flags, nvp, wbase, lo, (int64_t)sh.prefix + wpre, sh.sbi[w], sh.sbv[w]);
    }
}

// One workgroup per tile, the tile taken as a ticket (one atomic) when the
// workgroup starts: a tile only waits on tiles of workgroups already running,
// so the kernel can share the GPU with any other.  The one tile that extends
// past n (always the last) goes through the checked path.
template <bool FROM_F32, bool W_NEW, bool W_MASK>
__global__ __launch_bounds__(CD_THREADS) void k_cast_compact(CastDiffArgs a) {
    __shared__ uint32_t s_tile, s_tag;
    __shared__ CdShared sh;
    if (threadIdx.x == 0) {
        uint32_t tile, tag;
        ws_begin(a.hdr, a.ntiles, &tile, &tag);
        s_tile = tile;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile, tag = s_tag;
    if (tile >= a.ntiles) {  // inconsistent workspace state: touch nothing
        if (threadIdx.x == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    const uint32_t nfull = (uint32_t)(a.n / CD_TILE);  // tiles entirely inside [0, n)
    if (tile < nfull) cd_tile<true, FROM_F32, W_NEW, W_MASK>(a, tile, tag, sh);
    else cd_tile<false, FROM_F32, W_NEW, W_MASK>(a, tile, tag, sh);
}

// ---- one launch over a list of tensors ---------------------------------------
// The host prepares the tiling metadata (each tensor's first tile, and the
// tensor of every tile), so one launch covers a whole list of tensors that
// live anywhere in memory ("GPU weight teleportation" write-up, "Moving the
// pipeline onto GPUs").  Tiles are tickets (one workgroup each, one atomic):
// a tile only waits on tiles of workgroups already running.  Indices are local
// to each tensor; the first tile of tensor s records its first entry.
struct SegDesc {  // the layout of pulse_segment
    const float *w_new;
    const uint16_t *b_old;
    uint16_t *b_new;
    int64_t n;
    int64_t tile0;
};

struct SegArgs {
    const SegDesc *segs;
    int32_t nseg;
    const uint32_t *tile_seg;
    uint32_t ntiles;
    int32_t *idx;
    uint16_t *val;
    int64_t cap;
    int64_t *seg_offsets;
    uint32_t *d_status;
    WsHeader *hdr;
    uint64_t *status;
};

template <bool W_NEW>
__global__ __launch_bounds__(CD_THREADS) void k_cast_compact_segments(SegArgs g) {
    __shared__ uint32_t s_tile, s_tag;
    __shared__ CdShared sh;
    if (threadIdx.x == 0) {
        uint32_t tile, tag;
        ws_begin(g.hdr, g.ntiles, &tile, &tag);
        s_tile = tile;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile, tag = s_tag;
    if (tile >= g.ntiles) {  // inconsistent workspace state: touch nothing
        if (threadIdx.x == 0) or_agent32(g.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    const uint32_t s = g.tile_seg[tile];
    SegDesc d{};
    if (s < (uint32_t)g.nseg) d = g.segs[s];
    const int64_t lt = (int64_t)tile - d.tile0;  // tile within the tensor
    const bool ok = s < (uint32_t)g.nseg && d.n >= 1 && d.n <= 2147483647ll && lt >= 0 && lt * CD_TILE < d.n &&
                    ((reinterpret_cast<uintptr_t>(d.w_new) | reinterpret_cast<uintptr_t>(d.b_old) |
                      reinterpret_cast<uintptr_t>(d.b_new)) & 15u) == 0 && (d.b_new != nullptr) == W_NEW;
    CastDiffArgs a{};
    a.w_new = d.w_new;
    a.b_old = d.b_old;
    a.b_new = d.b_new;
    a.idx = g.idx;
    a.val = g.val;
    a.cap = g.cap;
    a.d_status = g.d_status;
    a.n = d.n;
    const int w = wave_id(), l = lane_id();
    const int64_t wbase = lt * CD_TILE + (int64_t)w * CD_WAVE_ELEMS;
    const int lo = 4 * l;
    uint32_t nvp[CD_GROUPS * 2];
    uint64_t flags = 0;
    if (ok) {
        if ((lt + 1) * CD_TILE <= d.n) flags = cd_pass1<true, true, W_NEW, false>(a, wbase, lo, nvp);
        else flags = cd_pass1<false, true, W_NEW, false>(a, wbase, lo, nvp);
    }
    const uint32_t wtot = wave_reduce_sum((uint32_t)__builtin_popcountll(flags));
    if (l == 0) sh.wtot[w] = wtot;
    __syncthreads();
    uint32_t tile_count = 0, wpre = 0;
#pragma unroll
    for (int i = 0; i < CD_THREADS / kWave; ++i) {
        if (i < w) wpre += sh.wtot[i];
        tile_count += sh.wtot[i];
    }
    if (w == 0) {
        bool failed = false;
        const uint64_t pre = lookback_wave(g.status, tile, tag, tile_count, &failed);
        if (l == 0) {
            if (failed) or_agent32(g.d_status, 8u /*PULSE_DS_WORKSPACE*/);
            if (!ok) or_agent32(g.d_status, 0x10u /*PULSE_DS_BADSEGMENT*/);
            sh.prefix = pre;
            if (ok && lt == 0) g.seg_offsets[s] = (int64_t)pre;
            if (tile == g.ntiles - 1) g.seg_offsets[g.nseg] = (int64_t)(pre + tile_count);
            if ((int64_t)(pre + tile_count) > g.cap) or_agent32(g.d_status, 1u /*PULSE_DS_CAPACITY*/);
        }
    }
    __syncthreads();
    if (tile_count != 0) cd_pass2(a, flags, nvp, wbase, lo, (int64_t)sh.prefix + wpre, sh.sbi[w], sh.sbv[w]);
}

}  // namespace pulse

using namespace pulse;

extern "C" int pulse_launch_cast_diff_segments(const void *segs, int32_t nseg, const uint32_t *tile_seg,
                                               int64_t ntiles, int32_t *idx, uint16_t *val, int64_t cap,
                                               int64_t *seg_offsets, uint32_t *d_status, void *ws, int with_new,
                                               hipStream_t stream) {
    SegArgs g{};
    g.segs = static_cast<const SegDesc *>(segs);
    g.nseg = nseg;
    g.tile_seg = tile_seg;
    g.ntiles = (uint32_t)ntiles;
    g.idx = idx;
    g.val = val;
    g.cap = cap;
    g.seg_offsets = seg_offsets;
    g.d_status = d_status;
    g.hdr = reinterpret_cast<WsHeader *>(ws);
    g.status = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(WsHeader));
    if (with_new) k_cast_compact_segments<true><<<dim3((unsigned)ntiles), dim3(CD_THREADS), 0, stream>>>(g);
    else k_cast_compact_segments<false><<<dim3((unsigned)ntiles), dim3(CD_THREADS), 0, stream>>>(g);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

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
