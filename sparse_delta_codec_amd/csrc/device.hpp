// device.hpp -- gfx950 building blocks shared by the codec kernels:
// wave64 scans/reductions, agent-scope status words and the decoupled
// look-back prefix (Merrill & Garland, "Single-pass Parallel Prefix Scan with
// Decoupled Look-back", 2016) used to place per-tile outputs in order.
#pragma once

#include <limits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pulse {

// ---- raw buffer stores ------------------------------------------------------
// A buffer resource (CDNA3/4 layout: 48-bit base, stride 0, num_records in
// bytes, word 3 = 0x00020000 for the gfx9 family) and the raw 16-bit buffer
// store.  A raw buffer store whose offset is at or past num_records is
// dropped by the hardware, so a lane that must not write is given the offset
// num_records instead of being masked off: every store instruction is then
// issued, and the memory counter's waits for earlier loads stay exact.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

__device__ void raw_buffer_store_u16(uint16_t v, i32x4_t rsrc, int32_t voffset, int32_t soffset,
                                     int32_t aux) __asm("llvm.amdgcn.raw.buffer.store.i16");

__device__ __forceinline__ i32x4_t buffer_rsrc(const void *p, uint32_t num_bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4_t r;
    r.x = (int32_t)(uint32_t)a;
    r.y = (int32_t)(uint32_t)((a >> 32) & 0xFFFFu);
    r.z = (int32_t)num_bytes;
    r.w = 0x00020000;
    return r;
}


constexpr int kWave = 64;

// native 16-byte vector: copies stay in registers (HIP's uint4 struct copies
// can turn into memcpy through the stack)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---- wave-level scans and reductions -----------------------------------------
// 32-bit scans use DPP (data-parallel primitives of the GFX9 ISA): row shifts
// inside each 16-lane row, then the row broadcasts of lane 15 and lane 31, one
// VALU operation per step and no LDS; wider types use ds_bpermute shuffles.
// Lanes whose DPP source does not exist keep `old` (bound_ctrl off).
template <int CTRL, int ROWM, int BANKM, typename T>
__device__ __forceinline__ T dpp_mov(T old, T v) {
    static_assert(sizeof(T) == 4, "32-bit DPP move");
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                            CTRL, ROWM, BANKM, false));
}
namespace dppc {
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowShl1 = 0x101, kRowShl2 = 0x102, kRowShl4 = 0x104, kRowShl8 = 0x108;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138, kWaveShl1 = 0x130;
}  // namespace dppc

template <typename T>
__device__ __forceinline__ T wave_incl_sum(T v) {
    if constexpr (sizeof(T) == 4) {
        using namespace dppc;
        v += dpp_mov<kRowShr1, 0xf, 0xf>(T(0), v);
        v += dpp_mov<kRowShr2, 0xf, 0xf>(T(0), v);
        v += dpp_mov<kRowShr4, 0xf, 0xe>(T(0), v);
        v += dpp_mov<kRowShr8, 0xf, 0xc>(T(0), v);
        v += dpp_mov<kRowBcast15, 0xa, 0xf>(T(0), v);
        v += dpp_mov<kRowBcast31, 0xc, 0xf>(T(0), v);
        return v;
    } else {
        const int lane = lane_id();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            T o = __shfl_up(v, d, kWave);
            if (lane >= d) v += o;
        }
        return v;
    }
}

template <typename T>
__device__ __forceinline__ T wave_incl_max(T v) {
    if constexpr (sizeof(T) == 4) {
        using namespace dppc;
        const T id = std::numeric_limits<T>::lowest();
        T o;
        o = dpp_mov<kRowShr1, 0xf, 0xf>(id, v); v = o > v ? o : v;
        o = dpp_mov<kRowShr2, 0xf, 0xf>(id, v); v = o > v ? o : v;
        o = dpp_mov<kRowShr4, 0xf, 0xe>(id, v); v = o > v ? o : v;
        o = dpp_mov<kRowShr8, 0xf, 0xc>(id, v); v = o > v ? o : v;
        o = dpp_mov<kRowBcast15, 0xa, 0xf>(id, v); v = o > v ? o : v;
        o = dpp_mov<kRowBcast31, 0xc, 0xf>(id, v); v = o > v ? o : v;
        return v;
    } else {
        const int lane = lane_id();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            T o = __shfl_up(v, d, kWave);
            if (lane >= d) v = o > v ? o : v;
        }
        return v;
    }
}

// inclusive scan from the top lane down: lane l gets min(v[l..63])
template <typename T>
__device__ __forceinline__ T wave_incl_min_rev(T v) {
    if constexpr (sizeof(T) == 4) {
        using namespace dppc;
        const T id = std::numeric_limits<T>::max();
        T o;
        o = dpp_mov<kRowShl1, 0xf, 0xf>(id, v); v = o < v ? o : v;
        o = dpp_mov<kRowShl2, 0xf, 0xf>(id, v); v = o < v ? o : v;
        o = dpp_mov<kRowShl4, 0xf, 0x7>(id, v); v = o < v ? o : v;
        o = dpp_mov<kRowShl8, 0xf, 0x3>(id, v); v = o < v ? o : v;
        // lane 16 r now holds the minimum of row r; add the rows above
        const T r1 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
        const T r2 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        const T r3 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
        const T s2 = r2 < r3 ? r2 : r3;
        const T s1 = r1 < s2 ? r1 : s2;
        const int row = lane_id() >> 4;
        const T above = row == 0 ? s1 : (row == 1 ? s2 : (row == 2 ? r3 : id));
        return above < v ? above : v;
    } else {
        const int lane = lane_id();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            T o = __shfl_down(v, d, kWave);
            if (lane + d < kWave) v = o < v ? o : v;
        }
        return v;
    }
}

template <typename T>
__device__ __forceinline__ T wave_reduce_max(T v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
        T o = __shfl_xor(v, d, kWave);
        v = o > v ? o : v;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_reduce_sum(T v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses,
// not for its global loads, so loads issued before it stay in flight across it
// (__syncthreads would drain them).  The memory clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Scheduling fence: the instruction scheduler moves nothing across it (no
// instruction is emitted), e.g. to keep loads in the order their waits assume.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---- block-level scans (NW waves); `sh` holds NW entries, one barrier pair ---
// exclusive sum; returns the thread's exclusive prefix, *total the block sum
template <int NW, typename T>
__device__ __forceinline__ T block_excl_sum(T v, T *sh, T *total) {
    T incl = wave_incl_sum(v);
    if (lane_id() == kWave - 1) sh[wave_id()] = incl;
    __syncthreads();
    T base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        T x = sh[w];
        if (w < wave_id()) base += x;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// exclusive max over lower threads (identity `lo`), *total = block max
template <int NW, typename T>
__device__ __forceinline__ T block_excl_max(T v, T lo, T *sh, T *total) {
    T incl = wave_incl_max(v);
    T excl;
    if constexpr (sizeof(T) == 4) {
        excl = dpp_mov<dppc::kWaveShr1, 0xf, 0xf>(lo, incl);
    } else {
        excl = __shfl_up(incl, 1, kWave);
        if (lane_id() == 0) excl = lo;
    }
    if (lane_id() == kWave - 1) sh[wave_id()] = incl;
    __syncthreads();
    T base = lo, tot = lo;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        T x = sh[w];
        if (w < wave_id()) base = x > base ? x : base;
        tot = x > tot ? x : tot;
    }
    __syncthreads();
    *total = tot;
    return excl > base ? excl : base;
}

// exclusive min over higher threads (identity `hi`)
template <int NW, typename T>
__device__ __forceinline__ T block_excl_min_rev(T v, T hi, T *sh) {
    T incl = wave_incl_min_rev(v);
    T excl;
    if constexpr (sizeof(T) == 4) {
        excl = dpp_mov<dppc::kWaveShl1, 0xf, 0xf>(hi, incl);
    } else {
        excl = __shfl_down(incl, 1, kWave);
        if (lane_id() == kWave - 1) excl = hi;
    }
    if (lane_id() == 0) sh[wave_id()] = incl;
    __syncthreads();
    T base = hi;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        T x = sh[w];
        if (w > wave_id()) base = x < base ? x : base;
    }
    __syncthreads();
    return excl < base ? excl : base;
}

// ---- agent-scope (whole-device) atomics --------------------------------------
// MI355X has one L2 per XCD; agent-scope atomic loads/stores make the status
// words coherent across the eight XCDs.
__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent32(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_agent32(uint32_t *p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- workspace layout shared by every single-pass (look-back) kernel --------
// [0, 256): header; [256, ...): one 64-bit status word per tile.
// status word: [63:40] epoch tag (never 0), [39] inclusive flag, [38:0] value.
// The ticket is the one hot atomic (all tiles of a call hit it); the state every
// tile reads and the op counters sit on their own 128-byte lines so those
// accesses do not queue behind the ticket atomics.
struct WsHeader {
    uint64_t ticket;  // tiles handed out on this workspace so far (never reset)
    uint64_t pad0[15];
    uint64_t state;   // [63:40] epoch (calls completed), [39:0] ticket at the start of this call
    uint64_t pad1[7];
    uint32_t aux;     // per-op counter (decode: slow-block count)
    uint32_t aux2;    // per-op counter (decode: slow-kernel blocks finished)
    uint32_t aux3;    // per-op counter (decode: blocks for the wave walk)
    uint32_t pad2[13];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

constexpr uint32_t kTagMod = 0xFFFFFFu;
constexpr uint64_t kValueMask = (1ull << 39) - 1;
constexpr uint64_t kInclusive = 1ull << 39;
constexpr uint64_t kBaseMask = (1ull << 40) - 1;

__device__ __forceinline__ uint64_t make_status(uint32_t tag, bool inclusive, uint64_t v) {
    return ((uint64_t)tag << 40) | (inclusive ? kInclusive : 0ull) | (v & kValueMask);
}

__device__ __forceinline__ uint64_t add_agent64(uint64_t *p, uint64_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-call prologue, thread 0 only: a dynamic tile id (ticket order == start
// order, so every tile this one waits on is already resident) and this call's
// epoch tag, with one atomic per tile.  The call state is read before the
// ticket is taken (the ticket address depends on it, so the load has returned
// first); the tile that takes the call's last ticket therefore re-arms the
// state only after every tile of the call has read it.
__device__ __forceinline__ void ws_begin(WsHeader *h, uint32_t ntiles, uint32_t *tile, uint32_t *tag) {
    const uint64_t st = ld_agent(&h->state);
    uint64_t *tp = &h->ticket + (st == ~0ull ? 1 : 0);  // never taken: state is never all ones
    const uint64_t t = add_agent64(tp, 1ull);
    const uint64_t tl = (t - st) & kBaseMask;
    const uint32_t ep = (uint32_t)(st >> 40);
    *tile = (uint32_t)tl;
    *tag = ep % kTagMod + 1u;
    if (tl == (uint64_t)ntiles - 1)
        st_agent(&h->state, ((uint64_t)((ep + 1u) % kTagMod) << 40) | ((t + 1) & kBaseMask));
}

// Decoupled look-back, executed by one full wave (all 64 lanes) of the tile.
// Publishes the tile's aggregate, sums predecessors' aggregates until one with
// an inclusive prefix is found, publishes the tile's inclusive prefix and
// returns the exclusive prefix (identical in every lane).
// MAX = true combines with max instead of +.
// The wait for a predecessor is bounded: a predecessor that never publishes
// can only come from a workspace whose state is inconsistent (not initialised,
// or shared by concurrent calls).  Past the budget the wave gives up, sets
// *failed (the caller reports it) and still publishes, so its successors end
// too and the kernel always terminates.
constexpr uint32_t kSpinLimit = 1u << 20;

// The two halves of the look-back, for callers that overlap other work with
// the wait: publish the tile's aggregate (tile 0: its inclusive value) ...
__device__ __forceinline__ void lookback_publish(uint64_t *status, uint32_t tile, uint32_t tag,
                                                 uint64_t aggregate) {
    if (lane_id() == 0) st_agent(&status[tile], make_status(tag, tile == 0, aggregate));
}

// The first window of a look-back, read ahead of time: lane l reads the status
// word of tile - 1 - l.  A wave that issues it early and resolves later (with
// `first`) has the round trip overlap its other work.
__device__ __forceinline__ uint64_t lookback_prefetch(const uint64_t *status, uint32_t tile) {
    const int64_t p = (int64_t)tile - 1 - lane_id();
    return p >= 0 ? ld_agent(&status[p]) : 0ull;
}

// ... then, by the same full wave, wait for the predecessors, publish the
// inclusive prefix and return the exclusive one.  `first`, when given, is the
// wave's lookback_prefetch of this tile, used as the first poll.
template <bool MAX = false>
__device__ __forceinline__ uint64_t lookback_resolve(uint64_t *status, uint32_t tile, uint32_t tag,
                                                     uint64_t aggregate, bool *failed,
                                                     const uint64_t *first = nullptr) {
    const int lane = lane_id();
    uint32_t spins = 0;
    if (tile == 0) return 0;

    uint64_t prefix = 0;
    int64_t j = (int64_t)tile - 1;  // newest predecessor the window starts at
    bool use_first = first != nullptr;
    while (true) {
        const int64_t p = j - lane;
        uint64_t w = 0;
        bool valid, incl;
        while (true) {
            if (use_first) w = *first;
            else if (p >= 0) w = ld_agent(&status[p]);
            use_first = false;
            valid = p < 0 || (uint32_t)(w >> 40) == tag;
            incl = p >= 0 && valid && (w & kInclusive);
            const uint64_t vmask = __ballot(valid);
            const uint64_t imask = __ballot(incl);
            if (imask) {
                const int stop = __builtin_ctzll(imask);
                const uint64_t need = (stop == 63) ? ~0ull : ((2ull << stop) - 1);
                if ((vmask & need) == need) break;
            } else if (vmask == ~0ull) {
                break;
            }
            if (++spins > kSpinLimit) {
                *failed = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (*failed) break;
        const uint64_t imask = __ballot(incl);
        uint64_t mine = (p >= 0) ? (w & kValueMask) : 0;
        const int stop = imask ? __builtin_ctzll(imask) : kWave;
        if (lane > stop) mine = 0;
        if constexpr (MAX) {
            const uint64_t r = wave_reduce_max(mine);
            prefix = r > prefix ? r : prefix;
        } else {
            prefix += wave_reduce_sum(mine);
        }
        if (imask) break;
        j -= kWave;
        if (j < 0) break;  // (never reached: tile 0 is always inclusive)
    }
    uint64_t incl_v;
    if constexpr (MAX) incl_v = aggregate > prefix ? aggregate : prefix;
    else incl_v = prefix + aggregate;
    if (lane == 0) st_agent(&status[tile], make_status(tag, true, incl_v));
    return prefix;
}

template <bool MAX = false>
__device__ __forceinline__ uint64_t lookback_wave(uint64_t *status, uint32_t tile, uint32_t tag,
                                                  uint64_t aggregate, bool *failed) {
    lookback_publish(status, tile, tag, aggregate);
    return lookback_resolve<MAX>(status, tile, tag, aggregate, failed);
}

// Bytes [o, o + 16) of the 32 bytes A (low) then B, for o in 1 .. 16.
__device__ __forceinline__ u32x4 take16(const u32x4 &A, const u32x4 &B, int o) {
    const uint32_t w[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
    const int wq = o >> 2, bs = o & 3;
    if (o == 16) return B;
    if (wq == 0)
        return u32x4{__builtin_amdgcn_alignbyte(w[1], w[0], bs), __builtin_amdgcn_alignbyte(w[2], w[1], bs),
                     __builtin_amdgcn_alignbyte(w[3], w[2], bs), __builtin_amdgcn_alignbyte(w[4], w[3], bs)};
    if (wq == 1)
        return u32x4{__builtin_amdgcn_alignbyte(w[2], w[1], bs), __builtin_amdgcn_alignbyte(w[3], w[2], bs),
                     __builtin_amdgcn_alignbyte(w[4], w[3], bs), __builtin_amdgcn_alignbyte(w[5], w[4], bs)};
    if (wq == 2)
        return u32x4{__builtin_amdgcn_alignbyte(w[3], w[2], bs), __builtin_amdgcn_alignbyte(w[4], w[3], bs),
                     __builtin_amdgcn_alignbyte(w[5], w[4], bs), __builtin_amdgcn_alignbyte(w[6], w[5], bs)};
    return u32x4{__builtin_amdgcn_alignbyte(w[4], w[3], bs), __builtin_amdgcn_alignbyte(w[5], w[4], bs),
                 __builtin_amdgcn_alignbyte(w[6], w[5], bs), __builtin_amdgcn_alignbyte(w[7], w[6], bs)};
}

__device__ __forceinline__ uint16_t bf16_rne(uint32_t x) {
    // nearest BF16, ties to even; NaN -> quiet NaN with sign and top payload
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
    return (uint16_t)((x + 0x7FFFu + ((x >> 16) & 1u)) >> 16);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// lanes below this one whose bit is set in m (rank of the lane among them)
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// two FP32 masters to two BF16 packed low-first in 32 bits: one
// v_cvt_pk_bf16_f32.  gfx950's conversion rounds to nearest, ties to even,
// keeps subnormals (this library is built with FP32 denormals on) and quiets a
// NaN by setting the top mantissa bit while keeping the sign and the upper
// payload: it equals bf16_rne on every one of the 2^32 FP32 patterns, which a
// full sweep on the device confirmed.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cast_pair(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{x, y}), bf16x2_t));
}

// changed flags of four BF16 (two XOR words): bit k for element k
__device__ __forceinline__ uint64_t pair_flags(uint32_t x0, uint32_t x1) {
    return (uint64_t)((x0 & 0xFFFFu) != 0) | ((uint64_t)((x0 >> 16) != 0) << 1) |
           ((uint64_t)((x1 & 0xFFFFu) != 0) << 2) | ((uint64_t)((x1 >> 16) != 0) << 3);
}

}  // namespace pulse
