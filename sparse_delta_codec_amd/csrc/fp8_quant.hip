// fp8_quant.hip -- row a7: projection fusion (stacking) + BF16 -> FP8-E4M3
// quantisation per 128x128 block with FP32 scales.
//
// The sender rebuilds the full weight, fuses projections and quantises BF16
// training weights for FP8 inference ("Weight transfer for RL post-training in
// under 2 seconds", opening paragraph and "Potok zadan").  Format: OCP E4M3
// "fn" (bias 7, largest finite 448, no Inf).  Per block: amax = max |x|,
// s = amax / 448 (IEEE float32 division; 1 when amax == 0), code =
// E4M3(fl32(x / s)), round to nearest even (fl32(x / s) <= 448 * (1 + 2^-23)
// always, which rounds to the largest finite code).
//
// One workgroup per (expert, block row, block column).  Thread t covers
// columns [8*(t%16), +8) of rows t/16 + 16*i, i = 0..7: every load instruction
// of a wave reads four complete 256-byte block rows, every store writes four
// 128-byte code rows.  The block is read once (kept in registers between the
// amax reduction and the quantisation).
#include "device.hpp"

#include <algorithm>
#include <utility>
#include <vector>

namespace pulse {

constexpr int FQ_MAXSRC = 8;

struct QuantArgs {
    const uint16_t *src[FQ_MAXSRC];
    int64_t row0[FQ_MAXSRC + 1];  // first stacked row of each source, row0[nsrc] = R
    int64_t bstride[FQ_MAXSRC];
    int32_t nsrc;
    int64_t cols;
    int64_t R;
    int64_t nbc;
    uint8_t *codes;
    float *scales;
};

// One 128x128 block (row block br, column block bc, matrix e) of a stacked
// matrix whose source s holds rows [row0[s], row0[s + 1]); by the whole
// 256-thread workgroup.
struct QBlock {
    const uint16_t *const *src;
    const int64_t *row0;
    const int64_t *bstride;  // per-source matrix stride (elements), or NULL
    int32_t nsrc;
    int64_t cols, R, nbc;
    uint8_t *codes;
    float *scales;
};

// Thread t of the 256-thread workgroup holds v[i] = columns [8 (t % 16), +8)
// of row t / 16 + 16 i of a 128x128 block (ok[i]: the piece lies inside the
// matrix).  Block amax, the scale (written by thread 0 to *scale) and the
// codes of the thread's pieces (piece i to codes_row0 + (t / 16 + 16 i) * cols,
// codes_row0 being the code of the block's first row at the thread's first
// column).  s_red[w * red_stride], w < 4: LDS words for the waves' maxima,
// free when the call starts.
template <bool STREAM = false>
__device__ __forceinline__ void quant_regs(const uint4 (&v)[8], const bool (&ok)[8], uint32_t *s_red,
                                           int red_stride, uint8_t *codes_row0, int64_t cols, float *scale) {
    const int t = threadIdx.x;
    const int rg = t >> 4;
    uint32_t amax = 0;  // max |x| as BF16 magnitude bits (ordered like the values)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!ok[i]) continue;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
            amax = lo > amax ? lo : amax;
            amax = hi > amax ? hi : amax;
        }
    }
    amax = wave_reduce_max(amax);
    if (lane_id() == 0) s_red[wave_id() * red_stride] = amax;
    __syncthreads();
    amax = s_red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) amax = s_red[w * red_stride] > amax ? s_red[w * red_stride] : amax;

    const float amax_f = __uint_as_float(amax << 16);
    const float s = amax == 0 ? 1.0f : amax_f / 448.0f;  // IEEE division
    if (t == 0) *scale = s;

    // q = fl32(|x| / s) without a division per element: with y = fl32(1/ss)
    // (IEEE, once), q0 = fl32(xs*y), r = xs - ss*q0 (exact with an FMA) and
    // q = fl32(q0 + r*y) is the correctly rounded quotient (Markstein, "Computation
    // of elementary functions on the IBM RISC System/6000 processor", 1990)
    // while xs and the remainder stay normal; both operands are scaled by 2^40
    // when s < 2^60 (the quotient is unchanged) so that they do.  Checked on
    // every finite BF16 amax against every BF16 magnitude up to it: the E4M3
    // codes equal those of the IEEE quotient (differences are confined to
    // subnormal quotients, all of which encode to 0).
    const bool up = s < 1.152921504606846976e18f;  // 2^60
    const float ss = up ? s * 1099511627776.0f : s;  // 2^40
    const float xm = up ? 1099511627776.0f : 1.0f;
    const float y = 1.0f / ss;  // IEEE division
    auto quot = [&](uint32_t xbits) {  // xbits: |x| as float32 bits
        const float xs = __uint_as_float(xbits) * xm;
        const float q0 = xs * y;
        const float rm = __builtin_fmaf(-q0, ss, xs);
        return __builtin_fmaf(rm, y, q0);
    };

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!ok[i]) continue;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t packed[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w0 = w[2 * h], w1 = w[2 * h + 1];
            // magnitudes (the hardware conversion rounds to nearest even and is
            // exact against the E4M3 definition for |q| <= 448.5), signs after
            int c = __builtin_amdgcn_cvt_pk_fp8_f32(quot((w0 << 16) & 0x7FFF0000u), quot(w0 & 0x7FFF0000u), 0, false);
            c = __builtin_amdgcn_cvt_pk_fp8_f32(quot((w1 << 16) & 0x7FFF0000u), quot(w1 & 0x7FFF0000u), c, true);
            const uint32_t sg = ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) |
                                (w1 & 0x80000000u);
            packed[h] = (uint32_t)c | sg;
        }
        uint8_t *dst = codes_row0 + (int64_t)(rg + 16 * i) * cols;
        if (STREAM)  // written once, not read again here: kept out of the caches
            __builtin_nontemporal_store(u32x2{packed[0], packed[1]}, reinterpret_cast<u32x2 *>(dst));
        else
            *reinterpret_cast<uint2 *>(dst) = make_uint2(packed[0], packed[1]);
    }
}

template <int MAXS>
__device__ __forceinline__ void quant_block(const QBlock &a, int64_t br, int64_t bc, int64_t e, uint32_t *s_red) {
    const int t = threadIdx.x;
    const int rg = t >> 4, seg = t & 15;
    const int64_t col = bc * 128 + seg * 8;
    const bool col_ok = col < a.cols;  // cols is a multiple of 8

    uint4 v[8];
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = br * 128 + rg + 16 * i;
        ok[i] = col_ok && r < a.R;
        v[i] = make_uint4(0, 0, 0, 0);
        if (ok[i]) {
            int s = 0;
#pragma unroll
            for (int k = 1; k < MAXS; ++k)
                if (k < a.nsrc && r >= a.row0[k]) s = k;
            const uint16_t *p = a.src[s] + (a.bstride ? e * a.bstride[s] : 0) + (r - a.row0[s]) * a.cols + col;
            v[i] = *reinterpret_cast<const uint4 *>(p);
        }
    }
    quant_regs(v, ok, s_red, 1, a.codes + (e * a.R + br * 128) * a.cols + col, a.cols,
               a.scales + (e * ((a.R + 127) / 128) + br) * a.nbc + bc);
}

__global__ __launch_bounds__(256) void k_fp8_block_quant(QuantArgs a) {
    __shared__ uint32_t s_red[4];
    const QBlock q{a.src, a.row0, a.bstride, a.nsrc, a.cols, a.R, a.nbc, a.codes, a.scales};
    quant_block<FQ_MAXSRC>(q, blockIdx.y, blockIdx.x, blockIdx.z, s_red);
}

// ---- several stacked groups in one launch -------------------------------------
// The launch covers the blocks of up to FQ_MAXG groups back to back (group g's
// blocks are [block0[g], block0[g + 1]), row-block major), so small groups
// (a layer's [q;k;v] or o) share the GPU with the others instead of running
// as launches too small to fill it.
constexpr int FQ_MAXG = 8;
constexpr int FQ_GSRC = 4;

struct QGroup {
    const uint16_t *src[FQ_GSRC];
    int64_t row0[FQ_GSRC + 1];
    int64_t cols, R, nbc;
    uint8_t *codes;
    float *scales;
    int32_t nsrc;
};

struct QuantGroupsArgs {
    QGroup g[FQ_MAXG];
    int64_t block0[FQ_MAXG + 1];
    int32_t ng;
};

__global__ __launch_bounds__(256) void k_fp8_block_quant_groups(QuantGroupsArgs a) {
    __shared__ uint32_t s_red[4];
    const int64_t blk = blockIdx.x;
    int g = 0;  // the group of this block (uniform)
#pragma unroll
    for (int i = 1; i < FQ_MAXG; ++i)
        if (i < a.ng && blk >= a.block0[i]) g = i;
    const QGroup &G = a.g[g];  // read in place from the argument block
    const int64_t lb = blk - a.block0[g];
    const QBlock q{G.src, G.row0, nullptr, G.nsrc, G.cols, G.R, G.nbc, G.codes, G.scales};
    quant_block<FQ_GSRC>(q, lb / G.nbc, lb % G.nbc, 0, s_red);
}

// ---- the receiver's pass: patch apply and FP8 quantisation in one read ----------
// The receiver overrides the patch's positions in its BF16 view and quantises
// the new view for FP8 serving.  Done apart, the apply's 2-byte stores leave
// three quarters of the view's 32-byte sectors partially written and the
// quantisation reads the whole view again; here one workgroup per 128x128
// block reads the block once into an LDS image, writes the block's entries
// there, stores back the 16-byte pieces that changed and quantises from the
// patched values.  A group is a stack of sources that are row-major matrices
// inside the view (FP8 groups), or a source that is only patched (norms,
// biases).  The entries of a block row are found through the patch's segment
// index seg_first[s] = first entry with index >= 128 s; the groups' sources
// tile the view, so every entry inside it is applied by exactly one workgroup.
constexpr int kSegLog = 7;

struct AQGroupDev {
    int64_t off[FQ_GSRC];  // element offset of each source in the view
    int64_t row0[FQ_GSRC + 1];
    int64_t cols, R, nbc;
    uint8_t *codes;  // [R][cols], or unused when quant == 0
    float *scales;   // [ceil(R/128)][nbc]
    int32_t nsrc;
    int32_t quant;
};

struct AQPlanHeader {
    int64_t n, ngroups, nblocks, reserved;
};

// plan: header, block0[ngroups + 1] (rounded up to 16 bytes), groups[ngroups]
__host__ __device__ inline int64_t aq_groups_offset(int64_t ng) {
    return (int64_t)sizeof(AQPlanHeader) + ((8 * (ng + 1) + 15) / 16) * 16;
}

// Segment index of an ascending patch: seg_first[s] for s in (segment of
// entry k - 1, segment of entry k] is k (entry `count` closes the index up to
// nseg).  Eight consecutive entries a lane (two 16-byte loads); a gap of more
// than 8 segments (a long unchanged run) is filled by the whole wave, 64
// stores an instruction.  An index outside [0, n), or one not above its
// predecessor, sets PULSE_DS_BADINDEX.
constexpr int kSegPer = 8;
constexpr int kAqXcds = 8;            // the XCDs workgroups are dispatched to in turn
constexpr int kAqTicketStride = 32;   // uint32 words between the per-XCD counters (128 bytes)

__global__ __launch_bounds__(256) void k_patch_segments(const int32_t *__restrict__ idx, const int64_t *d_count,
                                                        int64_t max_count, int64_t n, int32_t *__restrict__ seg_first,
                                                        uint32_t *d_status, uint32_t *tickets) {
    // the receiver pass that follows on the stream takes its blocks from
    // these counters (one per XCD, each on its own 128-byte line)
    if (blockIdx.x == 0 && threadIdx.x < kAqXcds) tickets[threadIdx.x * kAqTicketStride] = 0u;
    int64_t count = *d_count;
    if (count > max_count) count = max_count;
    if (count < 0) count = 0;
    const int64_t nseg = (n + 127) >> kSegLog;
    auto seg_of = [&](int64_t i) -> int64_t { return i < 0 ? 0 : (i >= n ? nseg : i >> kSegLog); };
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * kSegPer;
    bool bad = false;
    // base is uniform across the wave, so every lane runs every iteration
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + wave_id() * kWave) * kSegPer; base <= count;
         base += stride) {
        const int64_t k0 = base + lane_id() * kSegPer;
        int64_t iv[kSegPer + 1];  // entries k0 - 1 .. k0 + 7 (n past the count)
        iv[0] = k0 > 0 && k0 - 1 < count ? (int64_t)idx[k0 - 1] : -1;
        if (k0 + kSegPer <= count && (reinterpret_cast<uintptr_t>(idx + k0) & 15) == 0) {
            const int4 a = *reinterpret_cast<const int4 *>(idx + k0);
            const int4 c = *reinterpret_cast<const int4 *>(idx + k0 + 4);
            iv[1] = a.x; iv[2] = a.y; iv[3] = a.z; iv[4] = a.w;
            iv[5] = c.x; iv[6] = c.y; iv[7] = c.z; iv[8] = c.w;
        } else {
#pragma unroll
            for (int j = 0; j < kSegPer; ++j) iv[j + 1] = k0 + j < count ? (int64_t)idx[k0 + j] : n;
        }
#pragma unroll
        for (int j = 0; j < kSegPer; ++j) {
            const int64_t k = k0 + j;
            int64_t a = 0, z = -1;  // the segments [a, z] take the value k
            if (k <= count) {
                const int64_t i = iv[j + 1], ip = iv[j];
                if (k < count) bad |= i < 0 || i >= n || (k > 0 && i <= ip);
                a = (k == 0 ? -1 : seg_of(ip)) + 1;
                z = seg_of(i);
            }
            const bool wide = z - a >= 8;
            if (!wide)
                for (int64_t s = a; s <= z; ++s) seg_first[s] = (int32_t)k;
            uint64_t m = __ballot(wide);
            while (m) {
                const int l = __builtin_ctzll(m);
                m &= m - 1;
                const int64_t la = __shfl((long long)a, l), lz = __shfl((long long)z, l);
                const int32_t lk = (int32_t)(base + l * kSegPer + j);
                for (int64_t s = la + lane_id(); s <= lz; s += kWave) seg_first[s] = lk;
            }
        }
    }
    if (__ballot(bad) && lane_id() == 0) or_agent32(d_status, 2u /*PULSE_DS_BADINDEX*/);
}

// One block's description, uniform across the workgroup, held in plain
// scalars (a struct kept in a loop is left in private memory, and selects
// among its fields become indexed loads from there).  Every offset and size
// inside a view is below 2^31 (int32 patch indices), so 32 bits suffice.
#define AQ_FIELDS(X)                                                                                                  \
    X(int32_t, o0) X(int32_t, o1) X(int32_t, o2) X(int32_t, o3) X(int32_t, r1) X(int32_t, r2) X(int32_t, r3)        \
    X(int32_t, cols) X(int32_t, R) X(int32_t, nbc) X(int32_t, br) X(int32_t, bc) X(int32_t, quant)                   \
    X(uint8_t *, codes) X(float *, scales)

// The block blk of the plan: its group (last g with block0[g] <= blk) and its
// place in it.
#define AQ_LOCATE(P, blk)                                                                                             \
    do {                                                                                                              \
        const int64_t *block0_ = reinterpret_cast<const int64_t *>(plan + sizeof(AQPlanHeader));                     \
        int64_t lo_ = 0, hi_ = ng - 1;                                                                                \
        while (lo_ < hi_) {                                                                                           \
            const int64_t mid_ = (lo_ + hi_ + 1) >> 1;                                                                \
            if (block0_[mid_] <= (blk)) lo_ = mid_;                                                                   \
            else hi_ = mid_ - 1;                                                                                      \
        }                                                                                                             \
        const AQGroupDev &G_ = reinterpret_cast<const AQGroupDev *>(plan + aq_groups_offset(ng))[lo_];               \
        P##o0 = (int32_t)G_.off[0];                                                                                   \
        P##o1 = (int32_t)G_.off[1];                                                                                   \
        P##o2 = (int32_t)G_.off[2];                                                                                   \
        P##o3 = (int32_t)G_.off[3];                                                                                   \
        P##r1 = (int32_t)G_.row0[1];                                                                                  \
        P##r2 = (int32_t)G_.row0[2];                                                                                  \
        P##r3 = (int32_t)G_.row0[3];                                                                                  \
        P##cols = (int32_t)G_.cols;                                                                                   \
        P##R = (int32_t)G_.R;                                                                                         \
        P##nbc = (int32_t)G_.nbc;                                                                                     \
        const int32_t lb_ = (int32_t)((blk) - block0_[lo_]);                                                          \
        P##br = lb_ / P##nbc;                                                                                         \
        P##bc = lb_ - P##br * P##nbc;                                                                                 \
        P##quant = G_.quant;                                                                                          \
        P##codes = G_.codes;                                                                                          \
        P##scales = G_.scales;                                                                                        \
    } while (0)

// View index of (row r < R, column c) of a stack of up to four sources; a
// source past nsrc starts at row R (as the plan sets it), so it is never
// picked.  Selects only: no indexed load, no branch.
__device__ __forceinline__ int32_t aq_elem(int32_t o0, int32_t o1, int32_t o2, int32_t o3, int32_t r1, int32_t r2,
                                           int32_t r3, int32_t cols, int32_t r, int32_t c) {
    const bool in1 = r >= r1, in2 = r >= r2, in3 = r >= r3;
    const int32_t o = in3 ? o3 : (in2 ? o2 : (in1 ? o1 : o0));
    const int32_t r0 = in3 ? r3 : (in2 ? r2 : (in1 ? r1 : 0));
    return o + (r - r0) * cols + c;
}

// Persistent workgroups.  Each XCD (workgroups go to the 8 XCDs in turn)
// takes a contiguous range of blocks, and its workgroups take the blocks of
// that range one at a time from a counter of their own XCD (a ticket, taken
// one block ahead).  The blocks an XCD works on at any moment are thus a
// compact window of about as many consecutive blocks as it holds
// workgroups: neighbouring column blocks of the same rows, whose entries lie
// in the same 128-byte lines of the patch (a block row uses some 60 bytes of
// its row's lines).  The window's lines, about 1 MB, stay in the XCD's 4 MB
// L2 while its neighbours read them; a workgroup walking its own strided runs
// of blocks would instead keep some 8 MB of lines open and fetch each line
// several times.  The view, the write-back and the codes are streamed
// (non-temporal) so they do not evict those lines.  A workgroup looks up the
// next block's entry range while it patches and quantises the current block,
// so a block's own loads (the view and the entries) go out together.  Blocks
// are independent of one another, so the order in which workgroups take them
// is free.
constexpr int kAqMaxGroups = 128 * 8;  // 4 workgroups on each of the 256 CUs

__global__ __launch_bounds__(256, 4) void k_apply_quant(uint16_t *__restrict__ b, int64_t n,
                                                       const int32_t *__restrict__ idx,
                                                       const uint16_t *__restrict__ val,
                                                       const int64_t *__restrict__ d_count, int64_t max_count,
                                                       const int32_t *__restrict__ seg_first,
                                                       const uint8_t *__restrict__ plan, int64_t nblk,
                                                       uint32_t *d_status, uint32_t *tickets) {
    static_assert(FQ_GSRC == 4, "four sources a group");
    __shared__ u32x4 img[128 * 16];  // the block, 256 bytes a row
    __shared__ uint32_t s_next;      // the ticket of the workgroup's next block
    __shared__ uint2 dirty[128 * 16 / 8];  // a byte per 16-byte piece: 1 once an entry landed in it
    const AQPlanHeader *hdr = reinterpret_cast<const AQPlanHeader *>(plan);
    const int t = threadIdx.x;
    if (hdr->n != n || hdr->nblocks != nblk) {  // a plan made for another view
        if (blockIdx.x == 0 && t == 0) or_agent32(d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    const int64_t ng = hdr->ngroups;
    const int64_t x = blockIdx.x % kAqXcds, q = nblk / kAqXcds, rem = nblk % kAqXcds;
    const int64_t x0 = x * q + (x < rem ? x : rem), x1 = x0 + q + (x < rem ? 1 : 0);
    uint32_t *const ticket = tickets + x * kAqTicketStride;
    if (t == 0) s_next = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int64_t blk = x0 + (int64_t)s_next;
    __syncthreads();  // every thread has read s_next before it holds the next ticket
    if (blk >= x1) return;

    int32_t count;
    {
        int64_t c = *d_count;
        c = c > max_count ? max_count : c;
        count = (int32_t)(c < 0 ? 0 : c);
    }
    // Lanes t = 2 rl, 2 rl + 1 hold the entry range of block row rl (looked up
    // a block ahead).  The entries are loaded 16 lanes a row, one entry a lane:
    // lane l of wave w takes entry (l % 16) of rows 32 w + 4 j + l / 16,
    // j < 8, so one load instruction reads four rows' runs of the patch.
    const int rl = t >> 1;
    const int rg = t >> 4, seg = t & 15; // view: rows rg + 16 i, columns [8 seg, +8)
    const int lane = t & 63, l16 = lane & 15;
    const int erow0 = (t >> 6) * 32 + (lane >> 4);  // + 4 j: the rows whose entries this lane loads

#define AQ_DECL(T, f) T c_##f; T n_##f;
    AQ_FIELDS(AQ_DECL)
#undef AQ_DECL
#define ELEM(P, r, c) aq_elem(P##o0, P##o1, P##o2, P##o3, P##r1, P##r2, P##r3, P##cols, (r), (c))
    // the entry range of row rl of a block: its first element and the index
    // words around it
#define LOOKUP(P, e, sf0, sf1)                                                                                        \
    do {                                                                                                              \
        const int32_t len_ = P##cols - P##bc * 128 < 128 ? P##cols - P##bc * 128 : 128;                              \
        e = ELEM(P, P##br * 128 + rl < P##R ? P##br * 128 + rl : P##R - 1, P##bc * 128);                               \
        sf0 = seg_first[e >> kSegLog];                                                                                \
        sf1 = seg_first[((e + len_ - 1) >> kSegLog) + 1];                                                             \
    } while (0)

    AQ_LOCATE(c_, blk);
    int32_t e, sf0, sf1;
    LOOKUP(c_, e, sf0, sf1);

    for (;;) {
        // the next block's ticket: taken now, published in LDS just before the
        // first barrier (its round trip overlaps the block's loads)
        uint32_t next_ticket = 0;
        if (t == 0) next_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int32_t col = c_bc * 128 + seg * 8;
        const bool col_ok = col < c_cols;
        const int32_t len = c_cols - c_bc * 128 < 128 ? c_cols - c_bc * 128 : 128;
        // The block's pieces: a piece outside the matrix reads the last row or
        // the first column instead (never written back nor quantised), so the
        // loads are unconditional and all in flight at once.
        uint4 v[8];
        bool ok[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int32_t r = c_br * 128 + rg + 16 * i;
            ok[i] = col_ok && r < c_R;
            const u32x4 w = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(b + ELEM(c_, r < c_R ? r : c_R - 1, col_ok ? col : 0)));
        v[i] = make_uint4(w.x, w.y, w.z, w.w);
        }
        // every row's first 16 entries; past a row's last entry a lane reads
        // entry 0 (the patch buffer holds at least one) and drops it
        const bool row_ok = c_br * 128 + rl < c_R;
        int32_t k0 = row_ok ? sf0 : 0, k1 = row_ok ? sf1 : 0;
        k0 = k0 < 0 ? 0 : (k0 > count ? count : k0);
        k1 = k1 < k0 ? k0 : (k1 > count ? count : k1);
        int32_t ii[8];
        uint16_t vv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int src = 8 * j + 2 * (lane >> 4);  // the lane holding row erow0 + 4 j's range
            const int32_t a0 = __shfl(k0, src), a1 = __shfl(k1, src);
            const int32_t kk = a0 + l16;
            const int32_t kc = kk < a1 ? kk : 0;
            const int32_t xi = idx[kc];
            const uint16_t yv = val[kc];
            ii[j] = kk < a1 ? xi : -1;
            vv[j] = yv;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) img[(rg + 16 * i) * 16 + seg] = u32x4{v[i].x, v[i].y, v[i].z, v[i].w};
        dirty[t] = uint2{0u, 0u};
        if (t == 0) s_next = next_ticket;
        __syncthreads();

        // the next block and its entry range (the current one again at the end)
        const int64_t nb = x0 + (int64_t)s_next;
        const bool more = nb < x1;
        AQ_LOCATE(n_, more ? nb : blk);
        int32_t ne, nsf0, nsf1;
        LOOKUP(n_, ne, nsf0, nsf1);

        uint16_t *img16 = reinterpret_cast<uint16_t *>(img);
        uint8_t *dirty8 = reinterpret_cast<uint8_t *>(dirty);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = erow0 + 4 * j;  // block row
            const int32_t er = __shfl(e, 8 * j + 2 * (lane >> 4));
            const int32_t rel = ii[j] - er;
            if (ii[j] >= 0 && rel >= 0 && rel < len) {
                img16[r * 128 + rel] = vv[j];
                dirty8[r * 16 + (rel >> 3)] = 1;
            }
        }
        // rows with more than 16 entries: the two lanes of the row take the
        // rest in turn
        for (int32_t k = k0 + 16 + (t & 1); k < k1; k += 2) {
            const int32_t rel = idx[k] - e;
            if (rel >= 0 && rel < len) {
                img16[rl * 128 + rel] = val[k];
                dirty8[rl * 16 + (rel >> 3)] = 1;
            }
        }
        __syncthreads();

        // the patched block: the 64-byte lines that received an entry are
        // written back (the others hold the view's own bytes), and the whole
        // block is quantised
        uint4 u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 w = img[(rg + 16 * i) * 16 + seg];
            u[i] = make_uint4(w.x, w.y, w.z, w.w);
            // a 64-byte line of the row (four 16-byte pieces, four neighbouring
            // lanes) is written whole when an entry landed in any of its
            // pieces, else not at all: no partially written lines
            uint32_t dl = dirty8[(rg + 16 * i) * 16 + seg];
            dl |= dpp_mov<0xB1, 0xf, 0xf>(0u, dl);  // quad_perm [1,0,3,2]
            dl |= dpp_mov<0x4E, 0xf, 0xf>(0u, dl);  // quad_perm [2,3,0,1]
            if (ok[i] && dl)
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(b + ELEM(c_, c_br * 128 + rg + 16 * i, col)));
        }
        if (c_quant) {
            __syncthreads();  // the image is read; its first words hold the waves' maxima
            quant_regs<true>(u, ok, reinterpret_cast<uint32_t *>(img), 1,
                             c_codes + (int64_t)c_br * 128 * c_cols + col, c_cols,
                             c_scales + (int64_t)c_br * c_nbc + c_bc);
        }
        if (!more) break;
        __syncthreads();  // the image (and the maxima) read, s_next read, before the next block starts
        blk = nb;
#define AQ_NEXT(T, f) c_##f = n_##f;
        AQ_FIELDS(AQ_NEXT)
#undef AQ_NEXT
        e = ne;
        sf0 = nsf0;
        sf1 = nsf1;
    }
#undef LOOKUP
#undef ELEM
}
#undef AQ_LOCATE
#undef AQ_FIELDS

}  // namespace pulse

using namespace pulse;

extern "C" int pulse_launch_fp8_block_quant(const uint16_t *const *srcs, const int64_t *src_rows, int32_t nsrc,
                                            int64_t cols, int64_t batch, const int64_t *src_batch_stride,
                                            uint8_t *codes, float *scales, hipStream_t stream) {
    QuantArgs a{};
    int64_t R = 0;
    for (int i = 0; i < nsrc; ++i) {
        a.src[i] = srcs[i];
        a.row0[i] = R;
        a.bstride[i] = src_batch_stride ? src_batch_stride[i] : 0;
        R += src_rows[i];
    }
    for (int i = nsrc; i <= FQ_MAXSRC; ++i) a.row0[i] = R;
    a.nsrc = nsrc;
    a.cols = cols;
    a.R = R;
    a.nbc = (cols + 127) / 128;
    a.codes = codes;
    a.scales = scales;
    const dim3 g((unsigned)a.nbc, (unsigned)((R + 127) / 128), (unsigned)batch);
    k_fp8_block_quant<<<g, dim3(256), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// groups: (host) descriptors in the layout of pulse_quant_group
struct QGroupHost {
    const uint16_t *src[4];
    int64_t rows[4];
    int32_t nsrc;
    int32_t pad;
    int64_t cols;
    uint8_t *codes;
    float *scales;
};

extern "C" int pulse_launch_fp8_block_quant_groups(const void *groups, int32_t ngroups, hipStream_t stream) {
    const QGroupHost *h = static_cast<const QGroupHost *>(groups);
    QuantGroupsArgs a{};
    int64_t total = 0;
    for (int g = 0; g < ngroups; ++g) {
        QGroup &G = a.g[g];
        int64_t R = 0;
        for (int i = 0; i < FQ_GSRC; ++i) {
            G.src[i] = i < h[g].nsrc ? h[g].src[i] : h[g].src[0];
            G.row0[i] = R;
            if (i < h[g].nsrc) R += h[g].rows[i];
        }
        G.row0[FQ_GSRC] = R;
        for (int i = h[g].nsrc; i < FQ_GSRC; ++i) G.row0[i] = R;
        G.cols = h[g].cols;
        G.R = R;
        G.nbc = (h[g].cols + 127) / 128;
        G.codes = h[g].codes;
        G.scales = h[g].scales;
        G.nsrc = h[g].nsrc;
        a.block0[g] = total;
        total += ((R + 127) / 128) * G.nbc;
    }
    for (int g = ngroups; g <= FQ_MAXG; ++g) a.block0[g] = total;
    for (int g = ngroups; g < FQ_MAXG; ++g) a.g[g] = a.g[0];
    a.ng = ngroups;
    if (total > 0x7FFFFFFF) return -3;
    k_fp8_block_quant_groups<<<dim3((unsigned)total), dim3(256), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ---- the receiver's pass ------------------------------------------------------
struct AQGroupHost {  // the layout of pulse_aq_group
    int64_t src_offset[4];
    int64_t rows[4];
    int32_t nsrc;
    int32_t quantise;
    int64_t cols;
    uint8_t *codes;
    float *scales;
};

extern "C" int64_t pulse_apply_quant_plan_size(int32_t ngroups) {
    if (ngroups < 1) return 0;
    return aq_groups_offset(ngroups) + (int64_t)ngroups * (int64_t)sizeof(AQGroupDev);
}

// Checks the groups (-1 bad value, -2 misaligned) and that their sources tile
// [0, n); writes the plan to device memory (synchronously).
extern "C" int pulse_build_apply_quant_plan(const void *groups, int32_t ngroups, int64_t n, void *plan,
                                            int64_t plan_bytes, int64_t *nblocks) {
    const AQGroupHost *h = static_cast<const AQGroupHost *>(groups);
    const int64_t need = pulse_apply_quant_plan_size(ngroups);
    if (need == 0 || !groups || !plan || !nblocks || n < 1) return -1;
    if (plan_bytes < need) return -4;
    std::vector<uint8_t> host((size_t)need, 0);
    AQPlanHeader *hdr = reinterpret_cast<AQPlanHeader *>(host.data());
    int64_t *block0 = reinterpret_cast<int64_t *>(host.data() + sizeof(AQPlanHeader));
    AQGroupDev *gd = reinterpret_cast<AQGroupDev *>(host.data() + aq_groups_offset(ngroups));
    std::vector<std::pair<int64_t, int64_t>> spans;  // (offset, length) of every source
    int64_t total = 0;
    for (int g = 0; g < ngroups; ++g) {
        const AQGroupHost &q = h[g];
        if (q.nsrc < 1 || q.nsrc > FQ_GSRC || q.cols < 8 || q.cols % 8 != 0) return -1;
        if (q.quantise != 0 && q.quantise != 1) return -1;
        if (q.quantise && (!q.codes || !q.scales)) return -1;
        if (q.quantise && (reinterpret_cast<uintptr_t>(q.codes) % 8 != 0 ||
                           reinterpret_cast<uintptr_t>(q.scales) % 4 != 0))
            return -2;
        AQGroupDev &G = gd[g];
        int64_t R = 0;
        for (int i = 0; i < q.nsrc; ++i) {
            if (q.rows[i] < 1 || q.src_offset[i] < 0) return -1;
            if (q.src_offset[i] % 8 != 0) return -2;
            if (q.rows[i] > n / q.cols || q.src_offset[i] > n - q.rows[i] * q.cols) return -1;
            spans.emplace_back(q.src_offset[i], q.rows[i] * q.cols);
            G.off[i] = q.src_offset[i];
            G.row0[i] = R;
            R += q.rows[i];
        }
        for (int i = q.nsrc; i < FQ_GSRC; ++i) {
            G.off[i] = G.off[0];
            G.row0[i] = R;
        }
        G.row0[FQ_GSRC] = R;
        G.cols = q.cols;
        G.R = R;
        G.nbc = (q.cols + 127) / 128;
        G.codes = q.codes;
        G.scales = q.scales;
        G.nsrc = q.nsrc;
        G.quant = q.quantise;
        block0[g] = total;
        total += ((R + 127) / 128) * G.nbc;
    }
    block0[ngroups] = total;
    if (total > 0x7FFFFFFF) return -3;
    std::sort(spans.begin(), spans.end());
    int64_t end = 0;
    for (const auto &sp : spans) {
        if (sp.first != end) return -1;  // a gap or an overlap
        end += sp.second;
    }
    if (end != n) return -1;
    hdr->n = n;
    hdr->ngroups = ngroups;
    hdr->nblocks = total;
    if (hipMemcpy(plan, host.data(), (size_t)need, hipMemcpyHostToDevice) != hipSuccess) return -5;
    *nblocks = total;
    return 0;
}

// Workspace of the receiver's pass: the segment index (one int32 per 128
// elements and the closing one), then the per-XCD block counters on lines of
// their own.
static int64_t aq_ticket_offset(int64_t n) { return (((n + 127) / 128 + 1) * 4 + 255) / 256 * 256; }

extern "C" size_t pulse_apply_quant_ws_bytes(int64_t n) {
    return (size_t)(aq_ticket_offset(n) + kAqXcds * kAqTicketStride * 4);
}

extern "C" int pulse_launch_apply_quant(uint16_t *b, int64_t n, const int32_t *idx, const uint16_t *val,
                                        const int64_t *d_count, int64_t max_count, const void *plan, int64_t nblocks,
                                        uint32_t *d_status, void *ws, hipStream_t stream) {
    int32_t *seg_first = static_cast<int32_t *>(ws);
    uint32_t *tickets = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + aq_ticket_offset(n));
    int64_t blocks = (max_count + 1 + 256 * kSegPer - 1) / (256 * kSegPer);
    if (blocks > 256 * 8) blocks = 256 * 8;
    k_patch_segments<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(idx, d_count, max_count, n, seg_first,
                                                                       d_status, tickets);
    if (hipGetLastError() != hipSuccess) return -5;
    if (nblocks < 1) return 0;
    // as many workgroups as the GPU holds at once (4 a CU), no more than blocks
    int64_t per = (nblocks + kAqXcds - 1) / kAqXcds;
    if (per > kAqMaxGroups / kAqXcds) per = kAqMaxGroups / kAqXcds;
    k_apply_quant<<<dim3((unsigned)(kAqXcds * per)), dim3(256), 0, stream>>>(
        b, n, idx, val, d_count, max_count, seg_first, static_cast<const uint8_t *>(plan), nblocks, d_status,
        tickets);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
