// delta_compact.hip -- single-pass compaction of a per-element predicate into
// ascending (int32 index, value) entries, for two more views of the codec:
//
//  * FP8-view deltas: when the sampler serves FP8, the view to rebuild bit for
//    bit is the quantised one (E4M3 codes + per-block FP32 scales); its coarser
//    cells change fewer values per step ("Taking Reinforcement Learning Cross
//    Datacenter", Nan Jiang talk, 13:06-14:40; PULSE technical summary,
//    "Potenziale Futuro").  Codes are compared as bytes, scales as 32-bit
//    patterns; each changed position is sent with its new absolute value.
//  * PULSELoCo gate (PULSE technical summary, "2. PULSELoCo", Processo): an
//    FP32 pseudo-gradient plus the error-feedback buffer is sent only where
//    adding it to the shared checkpoint changes that entry's BF16 view; the
//    rest stays in the buffer for the next round.
//
// One 256-thread workgroup per tile of R rounds of 16384 elements (R = 4 for
// the one-byte codes, whose rounds are short, else 1); the tile is a ticket taken
// with one atomic when the workgroup starts, so a tile only ever waits for
// tiles whose workgroups are already running, whatever the device's residency
// (no co-residency assumption).  Pass 1 streams the tile with 16-byte loads
// and keeps the flags (64 per lane) and the values in registers; a one-wave
// decoupled look-back over epoch-tagged status words gives the tile's first
// entry; pass 2 ranks the flagged elements with ballots, stages each wave's
// entries in LDS at their ranks and writes them with coalesced stores.
//
// Lane l of wave w holds elements wbase + g*64*K + K*l + k (g < G, k < K,
// G*K = 64): K = 16 bytes per group for the codes, K = 4 words otherwise.
#include <type_traits>

#include "device.hpp"

namespace pulse {

enum DcMode { DC_U8 = 0, DC_U32 = 1, DC_GATE = 2 };

// K elements per lane and group, G groups, R rounds of DC_TILE elements a tile
template <int M> struct DcShape;
template <> struct DcShape<DC_U8> { static constexpr int K = 16, G = 4, R = 4; };
template <> struct DcShape<DC_U32> { static constexpr int K = 4, G = 16, R = 1; };
template <> struct DcShape<DC_GATE> { static constexpr int K = 4, G = 16, R = 1; };

struct DcArgs {
    const void *x0;  // U8 / U32: old view; GATE: checkpoint theta (float32)
    const void *x1;  // U8 / U32: new view; GATE: pseudo-gradient (float32)
    float *resid;    // GATE: error-feedback buffer, read then rewritten
    int32_t *idx;
    void *val;       // uint8 (U8) or 32-bit (U32, GATE) values
    int64_t cap;
    int64_t *d_count;
    uint32_t *d_status;
    int64_t n;
    WsHeader *hdr;
    uint64_t *status;
    uint32_t ntiles;
};

constexpr int DC_THREADS = 256;
constexpr int DC_WAVE_ELEMS = 4096;
constexpr int DC_TILE = (DC_THREADS / kWave) * DC_WAVE_ELEMS;  // 16384, one round
template <int M>
constexpr int64_t dc_tile_elems() { return (int64_t)DC_TILE * DcShape<M>::R; }
// entries staged per wave before a coalesced flush: at least one group's worth
// (64 lanes x K elements), which is what one group can add at once
template <int M>
constexpr int dc_sb() { return 64 * DcShape<M>::K > 512 ? 64 * DcShape<M>::K : 512; }

// bit k of the result is set iff byte k of x is non-zero
__device__ __forceinline__ uint32_t dc_nonzero_bytes(uint32_t x) {
    const uint32_t hi = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
    return (((hi >> 7) * 0x00204081u) >> 21) & 0xFu;
}

// The gate of one element: a = resid + delta; visible iff the BF16 view of
// theta + a differs from that of theta.  Float32 adds, round to nearest even.
__device__ __forceinline__ bool dc_gate(uint32_t th, uint32_t de, uint32_t re, uint32_t &a_bits) {
    const float a = __uint_as_float(re) + __uint_as_float(de);
    const float moved = __uint_as_float(th) + a;
    a_bits = __float_as_uint(a);
    const uint32_t pr = cast_pair(moved, __uint_as_float(th));  // both views in one conversion
    return (pr & 0xFFFFu) != (pr >> 16);
}

__device__ __forceinline__ uint32_t lanes_below_dc(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Pass 1 for one lane: flags (bit g*K + k) and the values kept for pass 2
// (U8: 16 words of packed codes; U32 / GATE: 64 words).
template <int M, bool FULL>
__device__ __forceinline__ uint64_t dc_pass1(const DcArgs &a, int64_t wbase, int l, uint32_t v[]) {
    constexpr int K = DcShape<M>::K, G = DcShape<M>::G;
    uint64_t flags = 0;
    if constexpr (M == DC_U8) {
        const uint8_t *po = static_cast<const uint8_t *>(a.x0) + wbase + K * l;
        const uint8_t *pn = static_cast<const uint8_t *>(a.x1) + wbase + K * l;
        if constexpr (FULL) {
            u32x4 o[G], w[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                o[g] = *reinterpret_cast<const u32x4 *>(po + g * 64 * K);
                w[g] = *reinterpret_cast<const u32x4 *>(pn + g * 64 * K);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    flags |= (uint64_t)dc_nonzero_bytes(o[g][d] ^ w[g][d]) << (g * K + 4 * d);
                    v[4 * g + d] = w[g][d];
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int64_t e = wbase + g * 64 * K + K * l + k;
                    if (e < a.n) {
                        const uint32_t ob = po[g * 64 * K + k], nb = pn[g * 64 * K + k];
                        if (ob != nb) flags |= 1ull << (g * K + k);
                        wd[k >> 2] |= nb << (8 * (k & 3));
                    }
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) v[4 * g + d] = wd[d];
            }
        }
    } else {
        const uint32_t *p0 = static_cast<const uint32_t *>(a.x0) + wbase + K * l;
        const uint32_t *p1 = static_cast<const uint32_t *>(a.x1) + wbase + K * l;
        const uint32_t *pr = reinterpret_cast<const uint32_t *>(a.resid) + wbase + K * l;
        if constexpr (FULL) {
            // four groups of loads in flight at a time
#pragma unroll
            for (int q = 0; q < G / 4; ++q) {
                u32x4 x0[4], x1[4], xr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int off = (4 * q + j) * 64 * K;
                    x0[j] = *reinterpret_cast<const u32x4 *>(p0 + off);
                    x1[j] = *reinterpret_cast<const u32x4 *>(p1 + off);
                    if constexpr (M == DC_GATE) xr[j] = *reinterpret_cast<const u32x4 *>(pr + off);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int g = 4 * q + j;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        bool f;
                        if constexpr (M == DC_GATE) {
                            f = dc_gate(x0[j][k], x1[j][k], xr[j][k], v[4 * g + k]);
                        } else {
                            f = x0[j][k] != x1[j][k];
                            v[4 * g + k] = x1[j][k];
                        }
                        flags |= (uint64_t)f << (g * K + k);
                    }
                }
                {
                    // this quarter's flags and values are final here
                    uint32_t lo = (uint32_t)flags, hi = (uint32_t)(flags >> 32);
                    asm volatile("" : "+v"(lo), "+v"(hi));
                    flags = ((uint64_t)hi << 32) | lo;
#pragma unroll
                    for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(v[16 * q + j]));
                }
                sched_fence();
            }
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t e = wbase + g * 64 * K + K * l + k;
                    uint32_t val = 0;
                    bool f = false;
                    if (e < a.n) {
                        const int off = g * 64 * K + k;
                        if constexpr (M == DC_GATE) {
                            f = dc_gate(p0[off], p1[off], pr[off], val);
                        } else {
                            val = p1[off];
                            f = p0[off] != val;
                        }
                    }
                    v[4 * g + k] = val;
                    flags |= (uint64_t)f << (g * K + k);
                }
                sched_fence();  // one group of loads at a time
            }
        }
    }
    return flags;
}

template <int M>
struct DcShared {
    uint32_t wtot[DcShape<M>::R][DC_THREADS / kWave];
    uint64_t prefix;
    int32_t sbi[DC_THREADS / kWave][dc_sb<M>()];
    typename std::conditional<M == DC_U8, uint8_t, uint32_t>::type sbv[DC_THREADS / kWave][dc_sb<M>()];
};

// Writes the wave's staged entries [0, nb) at patch position out and empties
// the buffer; lanes write consecutive entries.
template <int M, typename VT>
__device__ __forceinline__ void dc_flush(const DcArgs &a, const int32_t *sbi, const VT *sbv, uint32_t &nb,
                                         int64_t &out) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    VT *val = static_cast<VT *>(a.val);
    for (uint32_t i = lane_id(); i < nb; i += kWave) {
        const int64_t pos = out + i;
        if (pos < a.cap) {
            a.idx[pos] = sbi[i];
            val[pos] = sbv[i];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    out += nb;
    nb = 0;
}

template <int M, bool FULL>
__device__ __forceinline__ void dc_tile(const DcArgs &a, uint32_t tile, uint32_t tag, DcShared<M> &sh) {
    constexpr int K = DcShape<M>::K, G = DcShape<M>::G, R = DcShape<M>::R;
    const int w = wave_id(), l = lane_id();
    // round r of the tile: elements [tile * R + r) * DC_TILE, +DC_TILE), wave w
    // owning DC_WAVE_ELEMS of them; entries go out in element order
    int64_t wbase[R];
    uint32_t v[R][M == DC_U8 ? 16 : 64];
    uint64_t flags[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        wbase[r] = ((int64_t)tile * R + r) * DC_TILE + (int64_t)w * DC_WAVE_ELEMS;
        flags[r] = dc_pass1<M, FULL>(a, wbase[r], l, v[r]);
        // materialise the flags as one 64-bit word (otherwise the compiler keeps
        // each compare result live on its own until pass 2)
        uint32_t lo = (uint32_t)flags[r], hi = (uint32_t)(flags[r] >> 32);
        asm volatile("" : "+v"(lo), "+v"(hi));
        flags[r] = ((uint64_t)hi << 32) | lo;
        const uint32_t wtot = wave_reduce_sum((uint32_t)__builtin_popcountll(flags[r]));
        if (l == 0) sh.wtot[r][w] = wtot;
    }
    __syncthreads();
    uint32_t tile_count = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < DC_THREADS / kWave; ++i) tile_count += sh.wtot[r][i];
    if (w == 0) {
        bool failed = false;
        const uint64_t pre = lookback_wave(a.status, tile, tag, tile_count, &failed);
        if (l == 0) {
            if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
            sh.prefix = pre;
            if (tile == a.ntiles - 1) *a.d_count = (int64_t)(pre + tile_count);
            if ((int64_t)(pre + tile_count) > a.cap) or_agent32(a.d_status, 1u /*PULSE_DS_CAPACITY*/);
        }
    }
    __syncthreads();
    int32_t *sbi = sh.sbi[w];
    auto *sbv = sh.sbv[w];
    uint32_t before = 0;  // entries of the earlier rounds and of the lower waves of this one
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t rpre = 0, rtot = 0;
#pragma unroll
        for (int i = 0; i < DC_THREADS / kWave; ++i) {
            if (i < w) rpre += sh.wtot[r][i];
            rtot += sh.wtot[r][i];
        }
        int64_t run = (int64_t)sh.prefix + before + rpre;
        before += rtot;
        uint32_t nb = 0;
        if (rtot != 0 || M == DC_GATE) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint32_t f = (uint32_t)(flags[r] >> (g * K)) & ((1u << K) - 1u);
                uint64_t m[K];
                uint32_t gtot = 0;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    m[k] = __ballot((f >> k) & 1u);
                    gtot += __builtin_popcountll(m[k]);
                }
                uint32_t sent = 0;  // GATE: bit k set when element k went into the patch
                if (gtot != 0) {
                    if (nb + gtot > (uint32_t)dc_sb<M>()) dc_flush<M>(a, sbi, sbv, nb, run);
                    uint32_t q = nb;
#pragma unroll
                    for (int k = 0; k < K; ++k) q += lanes_below_dc(m[k]);
                    const int32_t e0 = (int32_t)(wbase[r] + g * 64 * K + K * l);
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        if (f & (1u << k)) {
                            sbi[q] = e0 + k;
                            if constexpr (M == DC_U8) sbv[q] = (uint8_t)(v[r][4 * g + (k >> 2)] >> (8 * (k & 3)));
                            else sbv[q] = v[r][4 * g + k];
                            if (run + q < a.cap) sent |= 1u << k;
                            ++q;
                        }
                    }
                    nb += gtot;
                }
                if constexpr (M == DC_GATE) {
                    // the buffer keeps everything that was not sent
                    uint32_t *pr = reinterpret_cast<uint32_t *>(a.resid) + wbase[r] + g * 64 * K + K * l;
                    u32x4 o;
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = (sent >> k) & 1u ? 0u : v[r][4 * g + k];
                    if constexpr (FULL) {
                        *reinterpret_cast<u32x4 *>(pr) = o;
                    } else {
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            if (wbase[r] + g * 64 * K + K * l + k < a.n) pr[k] = o[k];
                    }
                }
            }
            if (nb) dc_flush<M>(a, sbi, sbv, nb, run);
        }
    }
    __syncthreads();  // sh is reused by the next tile
}

template <int M>
__global__ __launch_bounds__(DC_THREADS) void k_delta_compact(DcArgs a) {
    __shared__ uint32_t s_tile, s_tag;
    __shared__ DcShared<M> sh;
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
    if (tile < (uint32_t)(a.n / dc_tile_elems<M>())) dc_tile<M, true>(a, tile, tag, sh);
    else dc_tile<M, false>(a, tile, tag, sh);
}

// ---- scatter of (index, value) entries: overwrite (codes, scales) or add ----
// Lanes take consecutive entries (entry = base + q*64 + lane, q < 4).
template <typename T, bool ADD>
__global__ __launch_bounds__(256) void k_scatter(T *__restrict__ b, int64_t n, const int32_t *__restrict__ idx,
                                                 const T *__restrict__ val, const int64_t *__restrict__ d_count,
                                                 int64_t max_count, uint32_t *d_status) {
    int64_t count = *d_count;
    if (count > max_count) count = max_count;
    const int64_t per_wave = 4 * kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
    bool bad = false;
    for (int64_t wb = ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave_id()) * per_wave; wb < count;
         wb += nwaves * per_wave) {
        int32_t ii[4];
        T vv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t k = wb + q * kWave + lane_id();
            ii[q] = k < count ? idx[k] : -1;
            vv[q] = k < count ? val[k] : T(0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t k = wb + q * kWave + lane_id();
            if (k >= count) break;
            const int64_t i = ii[q];
            if (i >= 0 && i < n) {
                if constexpr (ADD) b[i] = b[i] + vv[q];  // indices are unique within a patch
                else b[i] = vv[q];
            } else {
                bad = true;
            }
        }
    }
    if (__ballot(bad) && lane_id() == 0) or_agent32(d_status, 2u /*PULSE_DS_BADINDEX*/);
}

template <typename T, bool ADD>
int launch_scatter(T *b, int64_t n, const int32_t *idx, const T *val, const int64_t *d_count, int64_t max_count,
                   uint32_t *d_status, hipStream_t stream) {
    int64_t blocks = (max_count + 1023) / 1024;
    if (blocks > 256 * 32) blocks = 256 * 32;
    if (blocks < 1) blocks = 1;
    k_scatter<T, ADD><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(b, n, idx, val, d_count, max_count,
                                                                       d_status);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int M>
int launch_delta_compact(const void *x0, const void *x1, float *resid, int64_t n, int32_t *idx, void *val,
                         int64_t cap, int64_t *d_count, uint32_t *d_status, void *ws, hipStream_t stream) {
    DcArgs a{};
    a.x0 = x0;
    a.x1 = x1;
    a.resid = resid;
    a.idx = idx;
    a.val = val;
    a.cap = cap;
    a.d_count = d_count;
    a.d_status = d_status;
    a.n = n;
    a.hdr = reinterpret_cast<WsHeader *>(ws);
    a.status = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(WsHeader));
    const int64_t ntiles = (n + dc_tile_elems<M>() - 1) / dc_tile_elems<M>();
    a.ntiles = (uint32_t)ntiles;
    k_delta_compact<M><<<dim3((unsigned)ntiles), dim3(DC_THREADS), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace pulse

using namespace pulse;

extern "C" size_t pulse_delta_compact_ws_bytes(int64_t n) {
    const int64_t ntiles = (n + DC_TILE - 1) / DC_TILE;
    return sizeof(WsHeader) + (size_t)(ntiles > 0 ? ntiles : 1) * sizeof(uint64_t);
}

// FP8-view delta: the codes, then the scales, on one workspace (the second
// launch starts after the first has re-armed the workspace for the next call).
extern "C" int pulse_launch_fp8_delta(const uint8_t *codes_old, const uint8_t *codes_new, int64_t n_codes,
                                      const float *scales_old, const float *scales_new, int64_t n_scales,
                                      int32_t *code_idx, uint8_t *code_val, int64_t code_cap,
                                      int64_t *d_code_count, int32_t *scale_idx, float *scale_val,
                                      int64_t scale_cap, int64_t *d_scale_count, uint32_t *d_status, void *ws,
                                      hipStream_t stream) {
    int rc = launch_delta_compact<DC_U8>(codes_old, codes_new, nullptr, n_codes, code_idx, code_val, code_cap,
                                         d_code_count, d_status, ws, stream);
    if (rc) return rc;
    return launch_delta_compact<DC_U32>(scales_old, scales_new, nullptr, n_scales, scale_idx, scale_val,
                                        scale_cap, d_scale_count, d_status, ws, stream);
}

extern "C" int pulse_launch_fp8_apply(uint8_t *codes, int64_t n_codes, float *scales, int64_t n_scales,
                                      const int32_t *code_idx, const uint8_t *code_val,
                                      const int64_t *d_code_count, int64_t max_code_count,
                                      const int32_t *scale_idx, const float *scale_val,
                                      const int64_t *d_scale_count, int64_t max_scale_count, uint32_t *d_status,
                                      hipStream_t stream) {
    if (max_code_count > 0) {
        const int rc = launch_scatter<uint8_t, false>(codes, n_codes, code_idx, code_val, d_code_count,
                                                      max_code_count, d_status, stream);
        if (rc) return rc;
    }
    if (max_scale_count > 0)
        return launch_scatter<uint32_t, false>(reinterpret_cast<uint32_t *>(scales), n_scales, scale_idx,
                                               reinterpret_cast<const uint32_t *>(scale_val), d_scale_count,
                                               max_scale_count, d_status, stream);
    return 0;
}

extern "C" int pulse_launch_loco_gate(const float *theta, const float *delta, float *resid, int64_t n,
                                      int32_t *idx, float *val, int64_t cap, int64_t *d_count, uint32_t *d_status,
                                      void *ws, hipStream_t stream) {
    return launch_delta_compact<DC_GATE>(theta, delta, resid, n, idx, val, cap, d_count, d_status, ws, stream);
}

extern "C" int pulse_launch_loco_accumulate(float *acc, int64_t n, const int32_t *idx, const float *val,
                                            const int64_t *d_count, int64_t max_count, uint32_t *d_status,
                                            hipStream_t stream) {
    return launch_scatter<float, true>(acc, n, idx, val, d_count, max_count, d_status, stream);
}
