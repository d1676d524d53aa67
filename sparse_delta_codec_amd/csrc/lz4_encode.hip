// lz4_encode.hip -- row a5: LZ4 block encoding of the XOR mask.
//
// The pages pick LZ4 because it codes long runs in few commands and RL masks
// are long zero runs ("GPU weight teleportation" write-up, "Moving the
// pipeline onto GPUs"; the masks are mostly zero, "XOR masks").  The byte
// format is the public LZ4 block format.  LZ4 encodings are not unique; this
// encoder emits the canonical "offset-1 run" parse: every maximal run of one
// byte value [s, e) with i = s+1, j = min(e, n-5), j-i >= 4 and i <= n-12 is
// one sequence (literals since the previous such run, then a match of offset 1
// and length j-i); the rest of the block is the final literal run.  Because a
// run's sequence depends only on its own (s, e, n), a block is parsed in
// parallel and the output is bit-for-bit deterministic.
//
// One workgroup of 1024 threads (16 waves) per block, the block taken as a
// ticket (one atomic) when the workgroup starts, so a block only ever waits
// for blocks already handed to running workgroups (the encoder can share the
// GPU with any other kernel); thread t owns the block bytes [t*CH, (t+1)*CH), CH = block_bytes / 1024 (64
// for 64 KiB blocks, so a chunk's run boundaries fit one 64-bit mask):
//  1. coalesced 16-byte loads (the XOR of two sources when given) into a 64 KiB
//     LDS image whose 16-byte pieces are XOR-swizzled per chunk, so both the
//     coalesced writes and each thread's reads of its own chunk are free of
//     bank conflicts;
//  2. per thread: SWAR run-boundary bitmask of its chunk (1 bit per byte);
//  3. one in-order pass over the chunk's runs (a run is complete when the next
//     boundary is found) gives the thread's first/last qualifying run and the
//     bytes of its sequences; block scans (next boundary after the chunk,
//     last qualifying j before it, first qualifying i after it, byte offsets);
//  4. decoupled look-back over blocks gives the block's payload offset;
//  5. emission: each thread writes its sequences' headers and the literal bytes
//     of its own chunk into a 14 KiB LDS window, relative to the block's
//     start, while wave 0 waits for the predecessors' sizes; the window is
//     then copied out with 16-byte stores.  Every block of a sparse mask fits
//     one window; a larger encoding takes several window passes, each thread
//     emitting only in the passes its bytes reach.  A block with no
//     qualifying run at all (incompressible bytes) is one literal sequence and
//     skips the window: its bytes go from the image straight to the payload.
//
// The fused sender pass (pulse_cast_diff_lz4) runs the same block encoder on a
// mask it makes itself: step 1 becomes the FP32 -> BF16 cast of the block's
// 32768 masters (64 KiB blocks), the compare with the old view, the store of
// the new view and of old ^ new into the LDS image, so the mask never leaves
// the chip and neither view is read twice.  The changed elements of the
// block are ranked as they are found (ballots, in index order) and staged in
// the output window, which is idle until step 5; a second look-back over the
// blocks' patch counts, resolved while the block is analysed, places them in
// the ascending (index, new value) patch.
#include "../../include/pulse.h"
#include "device.hpp"

#include <mutex>

extern "C" int pulse_launch_fill_zero(void *, size_t, hipStream_t);

namespace pulse {

constexpr int LZE_THREADS = 1024;
constexpr int LZE_MAX_BLOCK = 65536;
constexpr int LZE_WIN = 14336;  // output staging window
constexpr int32_t LZE_INF = 0x7FFFFFFF;

struct Lz4EncArgs {
    const uint8_t *src;
    const uint8_t *src_xor;
    int64_t nbytes;
    int32_t block_bytes;
    uint8_t *payload;
    int64_t cap;
    uint32_t *comp_sizes;
    uint64_t *comp_offsets;
    uint64_t *d_total;
    uint32_t *d_status;
    WsHeader *hdr;
    uint64_t *status;
    uint32_t nblocks;
};

// extra length bytes of a length nibble: 0 below 15, else (v - 15) / 255 + 1,
// which is (v + 240) / 255 for every v >= 0; the multiply-shift divides
// exactly for v + 240 < 66299 (lengths here are at most 65536)
__device__ __forceinline__ int32_t ext_bytes(int32_t v) {
    return (int32_t)((uint32_t)__umul24((uint32_t)v + 240u, 0x8081u) >> 23);
}

__device__ __forceinline__ int32_t seq_bytes(int32_t ll, int32_t ml) {
    return 1 + ext_bytes(ll) + ll + 2 + ext_bytes(ml - 4);
}

// LDS image of a block: chunk c (CH = 2^CHLOG bytes, NPC = CH/16 pieces) at
// c*CH, its 16-byte piece k stored at slot k ^ ((c >> (4 - log2 NPC)) & (NPC-1)):
// any 16 consecutive lanes, whether writing consecutive pieces or reading the
// same piece of their own chunks, hit 16 distinct 16-byte bank groups.
template <int CHLOG>
__device__ __forceinline__ int32_t img_addr(int32_t p) {
    constexpr int NPCLOG = CHLOG - 4;
    const int32_t c = p >> CHLOG;
    const int32_t k = (p >> 4) & ((1 << NPCLOG) - 1);
    const int32_t sw = (c >> (4 - NPCLOG)) & ((1 << NPCLOG) - 1);
    return (c << CHLOG) + ((k ^ sw) << 4) + (p & 15);
}

// Starts (chunk bit u = position cs + u) of the runs that become sequences:
// no run boundary among the next four positions (the run is >= 5 bytes, so
// j - i >= 4) and s <= len - 13 (so i <= len - 12; the end-of-block clamp
// j = min(e, len - 5) then never shortens the match below 4).  hi: boundary
// bits of the positions just past the chunk (only next_after can be one).
template <int CH>
__device__ __forceinline__ uint64_t qualifying_starts(uint64_t m, uint64_t hi, int32_t cs, int32_t len) {
    uint64_t y;
    if constexpr (CH == 64) {
        y = (m >> 1) | (m >> 2) | (m >> 3) | (m >> 4) | (hi << 63) | (hi << 62) | (hi << 61) | (hi << 60);
    } else {
        const uint64_t M = m | (hi << CH);
        y = (M >> 1) | (M >> 2) | (M >> 3) | (M >> 4);
    }
    uint64_t q = m & ~y;
    const int32_t lim = len - 13 - cs;  // largest qualifying bit
    if (lim < 0) q = 0;
    else if (lim < 63) q &= (2ull << lim) - 1;
    return q;
}

// End of the run starting at chunk bit u: the next boundary in the chunk, or
// the first one after it.
__device__ __forceinline__ int32_t run_end(uint64_t m, int u, int32_t cs, int32_t next_after) {
    const uint64_t after = u >= 63 ? 0ull : (m >> (u + 1));
    return after ? cs + u + 1 + (int32_t)__builtin_ctzll(after) : next_after;
}

// Output byte x of the window pass that holds bytes [wb, wb + LZE_WIN) lives
// at win[x - wb]; a byte outside the pass goes to a guard byte past the window
// (never copied out).
__device__ __forceinline__ void win_put(uint8_t *win, int32_t wb, int32_t x, uint32_t v) {
    const uint32_t r = (uint32_t)(x - wb);
    win[r < (uint32_t)LZE_WIN ? r : (uint32_t)(LZE_WIN + 16)] = (uint8_t)v;
}

// extra length bytes of a nibble capped at 15: 255s then a byte < 255
__device__ __forceinline__ int32_t put_len(uint8_t *win, int32_t wb, int32_t x, int32_t v) {
    int32_t rem = v - 15;
    for (; rem >= 255; rem -= 255) win_put(win, wb, x++, 255u);
    win_put(win, wb, x++, (uint32_t)rem);
    return x;
}

// Emission of one thread's sequences and of the literal bytes of its own
// chunk, as far as they fall in the window pass [wb, wb + LZE_WIN).  Byte p
// of the chunk sits at p ^ sw16 in the swizzled image (the swizzle only
// permutes the chunk's 16-byte pieces).
template <int CHLOG>
__device__ __forceinline__ void emit_chunk(uint8_t *win, int32_t wb, const uint8_t *s_img, uint64_t Q, uint64_t m,
                                           int32_t cs, int32_t chunk_end, int32_t next_after, int32_t len,
                                           int32_t carry_j, int32_t pos0, int32_t next_qi, int32_t sw16) {
    // chunk bytes [lo, hi) to output bytes base + p, clipped to the pass
    auto lits = [&](int32_t base, int32_t lo, int32_t hi) {
        const int32_t d = base - wb;
        lo = lo > -d ? lo : -d;
        hi = hi < LZE_WIN - d ? hi : LZE_WIN - d;
        for (int32_t p = lo; p < hi; ++p) win[d + p] = s_img[p ^ sw16];
    };
    int32_t la = carry_j, pos = pos0;
    while (Q) {
        const int u = __builtin_ctzll(Q);
        Q &= Q - 1;
        const int32_t s = cs + u, e = run_end(m, u, cs, next_after);
        const int32_t i = s + 1, j = e < len - 5 ? e : len - 5;
        const int32_t ll = i - la, ml = j - i;
        const int32_t h = 1 + ext_bytes(ll);
        win_put(win, wb, pos, (uint32_t)(((ll >= 15 ? 15 : ll) << 4) | (ml - 4 >= 15 ? 15 : ml - 4)));
        if (ll >= 15) put_len(win, wb, pos + 1, ll);
        lits(pos + h - la, la > cs ? la : cs, i);
        int32_t q = pos + h + ll;
        win_put(win, wb, q, 1u);
        win_put(win, wb, q + 1, 0u);
        q += 2;
        if (ml - 4 >= 15) q = put_len(win, wb, q, ml - 4);
        pos = q;
        la = j;
    }
    // literals of this chunk that belong to the next sequence after it
    const int32_t lo = la > cs ? la : cs;
    if (lo < chunk_end) {
        const int32_t ll = (next_qi != LZE_INF ? next_qi : len) - la;
        lits(pos + 1 + ext_bytes(ll) - la, lo, chunk_end);
    }
}

constexpr int LZE_NW = LZE_THREADS / kWave;


struct EncShared {
    uint8_t img[LZE_MAX_BLOCK];
    uint8_t win[LZE_WIN + 48];  // window byte x at win[16 + x]; guards around it
    // one slot set per block scan; a set is written again only in the next
    // block, after barriers every wave has passed, so each scan needs one barrier
    int32_t scan[4][LZE_NW];
    uint64_t off;
    uint32_t pw[LZE_NW];  // fused pass: changed elements of each wave
    uint64_t poff;        // fused pass: the block's first patch entry
    uint32_t comp;        // plain encoder: the size of a block left to enc_gather
};

// ---- fused sender pass: cast + diff + compaction feeding the block encoder ----
struct FusedArgs {
    const float *w_new;    // [n] FP32 masters
    const uint16_t *b_old; // [n] previous view
    uint16_t *b_new;       // [n] new view, or NULL (may equal b_old)
    int32_t *idx;          // patch, or NULL (then val, d_count, pstatus unused)
    uint16_t *val;
    int64_t cap;
    int64_t *d_count;
    uint64_t *pstatus;     // look-back words over the blocks' patch counts
    int64_t n;
    int64_t *tile_first;   // first patch entry of each 16384-element tile [ntiles + 1], or NULL
    int64_t ntiles;
};

constexpr int kPatchTile = 16384;  // elements per tile of the patch's tile index

// entries staged per wave in the output window: (offset in block, value) as
// one 32-bit word; a wave with more falls back to direct stores
constexpr int LZF_STAGE = (LZE_WIN + 48) / 4 / LZE_NW;

// Step 1 of the fused pass for one wave: wave wv owns the block's elements
// [wv * NG * 256, +NG * 256) as NG groups of 256, lane l holding elements
// 256 g + 4 l + k (a 16-byte load of masters and an 8-byte load of the old
// view per group, 1 KiB / 512 B contiguous per wave).  fused_load issues the
// loads; fused_consume casts, compares, stores the new view, puts old ^ new
// into the image and, with PATCH, ranks each changed element among the
// wave's (ballots, index order) and stages it.  Between the two the loads
// stay in flight while the workgroup finishes its previous block.  The masters
// and the two views are streamed (non-temporal: each byte is touched once),
// which leaves the L2 to the status words and the payload window.
template <int CHLOG>
struct FusedGeom {
    static constexpr int BLK_E = (1 << CHLOG) * LZE_THREADS / 2;  // elements per block
    static constexpr int NG = BLK_E / (LZE_NW * 256);              // groups per wave
};

template <int CHLOG, int G0, int GN>
__device__ __forceinline__ void fused_load(const FusedArgs &f, int64_t blk_e0, u32x4 *fv, u32x2 *ov, int tid) {
    constexpr int BLK_E = FusedGeom<CHLOG>::BLK_E, NG = FusedGeom<CHLOG>::NG;
    const int wv = tid / kWave, ln = tid % kWave;
    const int32_t w0 = wv * NG * 256 + 4 * ln;
    if (blk_e0 + BLK_E <= f.n) {
#pragma unroll
        for (int j = 0; j < GN; ++j) {
            const int64_t e = blk_e0 + w0 + (G0 + j) * 256;
            fv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(f.w_new + e));
            ov[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(f.b_old + e));
        }
    } else {  // the call's last block: elements past n read as zero
#pragma unroll
        for (int j = 0; j < GN; ++j) {
            const int64_t e = blk_e0 + w0 + (G0 + j) * 256;
            uint32_t fw[4], ow[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool in = e + k < f.n;
                fw[k] = in ? __float_as_uint(f.w_new[e + k]) : 0u;
                ow[k >> 1] |= (in ? (uint32_t)f.b_old[e + k] : 0u) << (16 * (k & 1));
            }
            fv[j] = u32x4{fw[0], fw[1], fw[2], fw[3]};
            ov[j] = u32x2{ow[0], ow[1]};
        }
    }
}

template <int CHLOG, bool PATCH, int G0, int GN>
__device__ __forceinline__ uint32_t fused_consume(const FusedArgs &f, int64_t blk_e0, const u32x4 *fv,
                                                  const u32x2 *ov, uint8_t *s_img, uint32_t *stg, int tid,
                                                  uint32_t nb) {
    constexpr int BLK_E = FusedGeom<CHLOG>::BLK_E, NG = FusedGeom<CHLOG>::NG;
    const int wv = tid / kWave, ln = tid % kWave;
    const int32_t w0 = wv * NG * 256 + 4 * ln;
    const bool full = blk_e0 + BLK_E <= f.n;
#pragma unroll
    for (int j = 0; j < GN; ++j) {
        const int32_t eo = w0 + (G0 + j) * 256;
        const int64_t e = blk_e0 + eo;
        const uint32_t p0 = cast_pair(__uint_as_float(fv[j].x), __uint_as_float(fv[j].y));
        const uint32_t p1 = cast_pair(__uint_as_float(fv[j].z), __uint_as_float(fv[j].w));
        const uint32_t x0 = p0 ^ ov[j].x, x1 = p1 ^ ov[j].y;  // zero past n
        if (f.b_new) {
            if (full) {
                __builtin_nontemporal_store(u32x2{p0, p1}, reinterpret_cast<u32x2 *>(f.b_new + e));
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (e + k < f.n) f.b_new[e + k] = (uint16_t)((k < 2 ? p0 : p1) >> (16 * (k & 1)));
            }
        }
        *reinterpret_cast<u32x2 *>(s_img + img_addr<CHLOG>(2 * eo)) = u32x2{x0, x1};
        if constexpr (PATCH) {
            const uint32_t fl = (uint32_t)pair_flags(x0, x1);
            const uint64_t m0 = __ballot(fl & 1u), m1 = __ballot(fl & 2u), m2 = __ballot(fl & 4u),
                           m3 = __ballot(fl & 8u);
            const uint32_t gtot = __builtin_popcountll(m0) + __builtin_popcountll(m1) +
                                  __builtin_popcountll(m2) + __builtin_popcountll(m3);
            uint32_t r = nb + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (fl & (1u << k)) {
                    if (r < (uint32_t)LZF_STAGE)
                        stg[r] = (uint32_t)(eo + k) | (((k < 2 ? p0 : p1) >> (16 * (k & 1))) << 16);
                    ++r;
                }
            }
            nb += gtot;
        }
    }
    return nb;
}

// Patch stores of a block whose waves could not all stage their entries: the
// flags come back from the image, the values from the masters (the old view
// may already be overwritten by the new one).
template <int CHLOG>
__device__ __forceinline__ void fused_patch_direct(const FusedArgs &f, int64_t blk_e0, const uint8_t *s_img,
                                                   int64_t run, int tid) {
    constexpr int BLK_E = (1 << CHLOG) * LZE_THREADS / 2;
    constexpr int NG = BLK_E / (LZE_NW * 256);
    const int wv = tid / kWave, ln = tid % kWave;
    const int32_t w0 = wv * NG * 256 + 4 * ln;
#pragma unroll 1
    for (int g = 0; g < NG; ++g) {
        const int32_t eo = w0 + g * 256;
        const u32x2 x = *reinterpret_cast<const u32x2 *>(s_img + img_addr<CHLOG>(2 * eo));
        const uint32_t fl = (uint32_t)pair_flags(x.x, x.y);
        const uint64_t m0 = __ballot(fl & 1u), m1 = __ballot(fl & 2u), m2 = __ballot(fl & 4u), m3 = __ballot(fl & 8u);
        const uint32_t gtot = __builtin_popcountll(m0) + __builtin_popcountll(m1) + __builtin_popcountll(m2) +
                              __builtin_popcountll(m3);
        int64_t r = run + lanes_below(m0) + lanes_below(m1) + lanes_below(m2) + lanes_below(m3);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (fl & (1u << k)) {
                const int64_t e = blk_e0 + eo + k;
                if (r < f.cap) {
                    f.idx[r] = (int32_t)e;
                    f.val[r] = bf16_rne(__float_as_uint(f.w_new[e]));
                }
                ++r;
            }
        }
        run += gtot;
    }
}

// Step 1 of the plain encoder: the block's bytes (or the XOR of two sources)
// into the image, with coalesced 16-byte loads.
template <int CHLOG>
__device__ __forceinline__ void enc_load(const Lz4EncArgs &a, uint32_t b, uint8_t *s_img) {
    const int t = threadIdx.x;
    const int64_t blk_base = (int64_t)b * a.block_bytes;
    const int32_t len = (int32_t)((a.nbytes - blk_base) < a.block_bytes ? (a.nbytes - blk_base) : a.block_bytes);
    const int32_t npieces = a.block_bytes / 16;
    for (int32_t q = t; q < npieces; q += LZE_THREADS) {
        const int32_t off = q * 16;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (off + 16 <= len) {
            v = *reinterpret_cast<const uint4 *>(a.src + blk_base + off);
            if (a.src_xor) {
                const uint4 x = *reinterpret_cast<const uint4 *>(a.src_xor + blk_base + off);
                v.x ^= x.x; v.y ^= x.y; v.z ^= x.z; v.w ^= x.w;
            }
        } else if (off < len) {
            uint32_t w[4] = {0, 0, 0, 0};
            for (int k = 0; k < len - off; ++k) {
                uint32_t byte = a.src[blk_base + off + k];
                if (a.src_xor) byte ^= a.src_xor[blk_base + off + k];
                w[k >> 2] |= byte << (8 * (k & 3));
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *reinterpret_cast<uint4 *>(s_img + img_addr<CHLOG>(off)) = v;
    }
}

// ---- large blocks of few sequences: emission by output piece ---------------
// A block whose encoding is larger than the window (nearly incompressible
// bytes with a few runs, such as the sign-and-exponent plane of a packed
// patch) would take several window passes, each copying its literals byte by
// byte.  With fewer than LZE_GCAP sequences the plain encoder places it (its
// size and offset, in enc_rest) and then writes it by output piece
// (enc_gather): the sequences go into a table in the window (output start, run
// start i, match end j), and each thread builds whole aligned 16-byte pieces
// of the payload: a piece inside one literal run is 16 image bytes (from two
// image pieces), any other piece is put together byte by byte from its
// sequences' token, length bytes, literals and offset.
constexpr int LZE_GCAP = (LZE_WIN + 48) / 8;

struct GatherTab {
    const uint2 *tab;  // entry k < nseq: (output start, i | j << 16); entry nseq: (output start, 0)
    int32_t nseq, len;
    // the last entry whose output starts at or before o
    __device__ __forceinline__ int32_t find(int32_t o) const {
        int32_t lo = 0, hi = nseq;
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if ((int32_t)tab[mid].x <= o) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    }
    // entry k: output start O, literal run [la, i) of the input, match [i, j),
    // token and literal-length bytes h
    __device__ __forceinline__ void get(int32_t k, int32_t &O, int32_t &la, int32_t &i, int32_t &j,
                                       int32_t &h) const {
        O = (int32_t)tab[k].x;
        la = k == 0 ? 0 : (int32_t)(tab[k - 1].y >> 16);
        const bool fin = k == nseq;
        i = fin ? len : (int32_t)(tab[k].y & 0xFFFFu);
        j = fin ? len : (int32_t)(tab[k].y >> 16);
        h = 1 + ext_bytes(i - la);
    }
};

// Output byte o of entry k (o inside the entry's bytes)
template <int CHLOG>
__device__ __forceinline__ uint32_t gather_byte(const GatherTab &g, const uint8_t *s_img, int32_t k, int32_t o) {
    int32_t O, la, i, j, h;
    g.get(k, O, la, i, j, h);
    const int32_t ll = i - la, ml = j - i, rel = o - O;
    if (rel == 0) return (uint32_t)(((ll >= 15 ? 15 : ll) << 4) | (k == g.nseq ? 0 : (ml - 4 >= 15 ? 15 : ml - 4)));
    if (rel < h) return rel < h - 1 ? 255u : (uint32_t)(ll - 15 - 255 * (h - 2));
    if (rel < h + ll) return s_img[img_addr<CHLOG>(la + rel - h)];
    const int32_t e = rel - h - ll;  // the offset bytes, then the match length bytes
    if (e < 2) return e == 0 ? 1u : 0u;
    const int32_t em = ext_bytes(ml - 4);
    return e - 2 < em - 1 ? 255u : (uint32_t)(ml - 4 - 15 - 255 * (em - 1));
}

// Writes block b, placed by enc_rest (sh.off, sh.comp), by output piece.  The
// run analysis of enc_rest's steps 2 and 3 is made again here from the image
// (still whole: nothing was emitted), so that none of enc_rest's state has to
// outlive it.
template <int CHLOG>
__device__ __forceinline__ void enc_gather(const Lz4EncArgs &a, uint32_t b, EncShared &sh, int t) {
    constexpr int32_t CH = 1 << CHLOG;
    const uint8_t *const s_img = sh.img;
    const int wv = __builtin_amdgcn_readfirstlane(t / kWave), ln = t % kWave;
    const int64_t blk_base = (int64_t)b * a.block_bytes;
    const int32_t len = (int32_t)((a.nbytes - blk_base) < a.block_bytes ? (a.nbytes - blk_base) : a.block_bytes);
    const uint32_t off_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sh.off >> 32));
    const uint32_t off_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sh.off);
    const uint64_t off = ((uint64_t)off_hi << 32) | off_lo;
    const int32_t comp = __builtin_amdgcn_readfirstlane((int)sh.comp);
    if ((int64_t)(off + comp) > a.cap) return;

    // the run boundaries of this thread's chunk (as in enc_rest, step 2)
    const int32_t cs = t * CH;
    const int32_t cl = len - cs < 0 ? 0 : (len - cs < CH ? len - cs : CH);
    constexpr int NW = (CH + 31) / 32;
    uint32_t mw[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) mw[i] = 0;
    if (cl > 0) {
        uint32_t prev = (t > 0) ? ((uint32_t)s_img[img_addr<CHLOG>(cs - 1)] << 24) : 0u;
#pragma unroll
        for (int32_t q = 0; q < CH; q += 16) {
            const uint4 v = *reinterpret_cast<const uint4 *>(s_img + img_addr<CHLOG>(cs + q));
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                uint32_t h[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t x = d[k + e] ^ __builtin_amdgcn_alignbyte(d[k + e], prev, 3);
                    prev = d[k + e];
                    h[e] = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
                }
                const uint32_t byte8 = (((h[0] >> 4) | h[1]) * 0x00204081u) >> 24;
                const int p0 = q + 4 * k;
                mw[p0 >> 5] |= byte8 << (p0 & 31);
            }
        }
        if (t == 0) mw[0] |= 1u;
        if (cl < CH) {
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const int32_t lo = 32 * i;
                mw[i] &= cl <= lo ? 0u : (cl - lo >= 32 ? ~0u : ((1u << (cl - lo)) - 1u));
            }
        }
    }
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) m |= (uint64_t)mw[i] << (32 * i);
    int32_t next_after;
    {
        const int32_t first_b = m ? cs + __builtin_ctzll(m) : len;
        const int32_t inc = wave_incl_min_rev(first_b);
        const int32_t exc = dpp_mov<dppc::kWaveShl1, 0xf, 0xf>(len, inc);
        if (ln == 0) sh.scan[0][wv] = inc;
        __syncthreads();
        int32_t above = len;
#pragma unroll
        for (int w = 0; w < LZE_NW; ++w) {
            const int32_t x = sh.scan[0][w];
            if (w > wv) above = x < above ? x : above;
        }
        next_after = exc < above ? exc : above;
    }
    // the qualifying runs (step 3): this thread's last match end, then the
    // previous one (exclusive maximum) as the start of its first literal run
    uint64_t hi = 0;
    {
        const int32_t d = next_after - (cs + CH);
        if (next_after < len && d >= 0 && d < 4) hi = 1ull << d;
    }
    const uint64_t Q = cl > 0 ? qualifying_starts<CH>(m, hi, cs, len) : 0ull;
    int32_t last_qj = 0;
    for (uint64_t q = Q; q;) {
        const int u = 63 - __builtin_clzll(q);  // the last qualifying run
        const int32_t e = run_end(m, u, cs, next_after);
        last_qj = e < len - 5 ? e : len - 5;
        break;
    }
    int32_t carry_j;
    {
        const int32_t inc_j = wave_incl_max(last_qj);
        const int32_t exc_j = dpp_mov<dppc::kWaveShr1, 0xf, 0xf>(0, inc_j);
        if (ln == kWave - 1) sh.scan[1][wv] = inc_j;
        __syncthreads();
        int32_t below = 0;
#pragma unroll
        for (int w = 0; w < LZE_NW; ++w) {
            const int32_t xj = sh.scan[1][w];
            if (w < wv) below = xj > below ? xj : below;
        }
        carry_j = exc_j > below ? exc_j : below;
    }
    // this thread's sequence bytes and count, and their exclusive sums
    int32_t tot = 0;
    {
        int32_t la = carry_j;
        for (uint64_t q = Q; q;) {
            const int u = __builtin_ctzll(q);
            q &= q - 1;
            const int32_t e = run_end(m, u, cs, next_after);
            const int32_t i = cs + u + 1, j = e < len - 5 ? e : len - 5;
            tot += seq_bytes(i - la, j - i);
            la = j;
        }
    }
    int32_t pos0, rank0, nseq, qsum;
    {
        const uint32_t v = (uint32_t)tot | ((uint32_t)__builtin_popcountll(Q) << 18);
        const uint32_t inc = wave_incl_sum(v);
        if (ln == kWave - 1) sh.scan[3][wv] = (int32_t)inc;
        __syncthreads();
        uint32_t below = 0, all = 0;
#pragma unroll
        for (int w = 0; w < LZE_NW; ++w) {
            const uint32_t x = (uint32_t)sh.scan[3][w];
            if (w < wv) below += x;
            all += x;
        }
        const uint32_t ex = below + inc - v;
        pos0 = (int32_t)(ex & 0x3FFFFu);
        rank0 = (int32_t)(ex >> 18);
        qsum = __builtin_amdgcn_readfirstlane((int)(all & 0x3FFFFu));
        nseq = __builtin_amdgcn_readfirstlane((int)(all >> 18));
    }
    // the table (enc_rest placed the block only with nseq < LZE_GCAP)
    uint2 *const tab = reinterpret_cast<uint2 *>(sh.win);
    {
        int32_t r = rank0, pos = pos0, la = carry_j;
        for (uint64_t q = Q; q;) {
            const int u = __builtin_ctzll(q);
            q &= q - 1;
            const int32_t e = run_end(m, u, cs, next_after);
            const int32_t i = cs + u + 1, j = e < len - 5 ? e : len - 5;
            if (r < LZE_GCAP - 1) tab[r] = make_uint2((uint32_t)pos, (uint32_t)i | ((uint32_t)j << 16));
            ++r;
            pos += seq_bytes(i - la, j - i);
            la = j;
        }
        if (t == 0 && nseq < LZE_GCAP) tab[nseq] = make_uint2((uint32_t)qsum, 0u);
    }
    __syncthreads();
    if (nseq >= LZE_GCAP) return;  // (never: enc_rest counted the same runs)
    const GatherTab g{tab, nseq, len};
    uint8_t *const dst = a.payload + off;
    // aligned payload piece u holds output bytes [16 u - shift, +16)
    const int32_t shift = (int32_t)((uintptr_t)dst & 15);
    uint8_t *const base = dst - shift;
    const int32_t npc = (shift + comp + 15) >> 4;
    for (int32_t u = t; u < npc; u += LZE_THREADS) {
        const int32_t o0 = 16 * u - shift;
        int32_t k = g.find(o0 > 0 ? o0 : 0);
        int32_t O, la, i, j, h;
        g.get(k, O, la, i, j, h);
        if (o0 >= O + h && o0 + 16 <= O + h + (i - la)) {  // inside one literal run
            const int32_t p = la + (o0 - O - h), q = p >> 4, r = p & 15;
            const u32x4 A = *reinterpret_cast<const u32x4 *>(s_img + img_addr<CHLOG>(q << 4));
            if (r) {
                const u32x4 B = *reinterpret_cast<const u32x4 *>(s_img + img_addr<CHLOG>((q + 1) << 4));
                *reinterpret_cast<u32x4 *>(base + 16 * u) = take16(A, B, r);
            } else {
                *reinterpret_cast<u32x4 *>(base + 16 * u) = A;
            }
        } else if (o0 >= 0 && o0 + 16 <= comp) {
            uint64_t lo = 0, hi8 = 0;  // (no indexed array: it would live in scratch)
            for (int32_t x = 0; x < 16; ++x) {
                while (k < nseq && (int32_t)tab[k + 1].x <= o0 + x) ++k;
                const uint64_t v = gather_byte<CHLOG>(g, s_img, k, o0 + x);
                if (x < 8) lo |= v << (8 * x);
                else hi8 |= v << (8 * (x - 8));
            }
            *reinterpret_cast<u32x4 *>(base + 16 * u) =
                u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi8, (uint32_t)(hi8 >> 32)};
        } else {  // the block's first or last piece, shared with its neighbours
            for (int32_t x = 0; x < 16; ++x) {
                const int32_t o = o0 + x;
                if (o < 0 || o >= comp) continue;
                while (k < nseq && (int32_t)tab[k + 1].x <= o) ++k;
                base[16 * u + x] = (uint8_t)gather_byte<CHLOG>(g, s_img, k, o);
            }
        }
    }
}

// Steps 2-5 of block b, by the whole workgroup, once the image is complete
// (and, for the fused pass, the patch counts of the waves are in sh.pw and
// their entries staged).  Ends with the block's output written, or, for the
// plain encoder, returns true with the block placed (sh.off, sh.comp) but not
// written: a block larger than the window with few sequences, which
// enc_gather then writes by output piece.
template <int CHLOG, bool PATCH = false>
__device__ __forceinline__ bool enc_rest(const Lz4EncArgs &a, const FusedArgs &f, uint32_t b, uint32_t tag,
                                         EncShared &sh, int t) {
    constexpr int32_t CH = 1 << CHLOG;
    uint8_t *const s_img = sh.img;
    uint8_t *const s_win = sh.win;
    // the wave index is the same in every lane: held in a scalar register, the
    // per-wave comparisons of the block scans stay scalar
    const int wv = __builtin_amdgcn_readfirstlane(t / kWave), ln = t % kWave;
    const int64_t blk_base = (int64_t)b * a.block_bytes;
    const int32_t len = (int32_t)((a.nbytes - blk_base) < a.block_bytes ? (a.nbytes - blk_base) : a.block_bytes);
    [[maybe_unused]] uint32_t *const stg = reinterpret_cast<uint32_t *>(s_win) + wv * LZF_STAGE;
    [[maybe_unused]] const int64_t blk_e0 = blk_base / 2;
    // the block's patch count goes out at once, so later blocks' look-backs
    // can sum it while this block is still being analysed
    // and wave 1 places it among the others later (step 3), when the
    // predecessors' counts are long published
    uint32_t p_count = 0;
    if constexpr (PATCH) {
        const uint32_t x = ln < LZE_NW ? sh.pw[ln] : 0u;
        p_count = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(x), LZE_NW - 1);
        if (wv == 1) lookback_publish(f.pstatus, b, tag, (uint64_t)p_count);
    }

    // 2. run-boundary bitmask of this thread's chunk
    const int32_t cs = t * CH;
    const int32_t cl = len - cs < 0 ? 0 : (len - cs < CH ? len - cs : CH);
    // byte p differs from byte p - 1: the high bit of each byte of
    // ((x & 0x7F..) + 0x7F..) | x, x = d ^ (d << 8 | previous byte); the flags
    // of two dwords (bits 7, 15, 23, 31 of each, the first shifted down by 4)
    // are gathered into 8 bits by one multiply: no two of the shifted copies
    // land on the same bit, so no carries
    constexpr int NW = (CH + 31) / 32;
    uint32_t mw[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) mw[i] = 0;
    if (cl > 0) {
        uint32_t prev = (t > 0) ? ((uint32_t)s_img[img_addr<CHLOG>(cs - 1)] << 24) : 0u;
#pragma unroll
        for (int32_t q = 0; q < CH; q += 16) {
            const uint4 v = *reinterpret_cast<const uint4 *>(s_img + img_addr<CHLOG>(cs + q));
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                uint32_t h[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t x = d[k + e] ^ __builtin_amdgcn_alignbyte(d[k + e], prev, 3);
                    prev = d[k + e];
                    h[e] = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
                }
                const uint32_t byte8 = (((h[0] >> 4) | h[1]) * 0x00204081u) >> 24;
                const int p0 = q + 4 * k;
                mw[p0 >> 5] |= byte8 << (p0 & 31);
            }
        }
        if (t == 0) mw[0] |= 1u;  // a run starts at the block start
        if (cl < CH) {            // the block's last, partial chunk
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const int32_t lo = 32 * i;
                mw[i] &= cl <= lo ? 0u : (cl - lo >= 32 ? ~0u : ((1u << (cl - lo)) - 1u));
            }
        }
    }
    uint64_t m = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) m |= (uint64_t)mw[i] << (32 * i);

    // first run boundary at or after the next chunk: exclusive minimum over
    // the higher threads
    int32_t next_after;
    {
        const int32_t first_b = m ? cs + __builtin_ctzll(m) : len;
        const int32_t inc = wave_incl_min_rev(first_b);
        const int32_t exc = dpp_mov<dppc::kWaveShl1, 0xf, 0xf>(len, inc);
        if (ln == 0) sh.scan[0][wv] = inc;
        __syncthreads();
        int32_t above = len;
#pragma unroll
        for (int w = 0; w < LZE_NW; ++w) {
            const int32_t x = sh.scan[0][w];
            if (w > wv) above = x < above ? x : above;
        }
        next_after = exc < above ? exc : above;
    }

    // the first poll of the patch look-back goes out now; wave 1 reads it
    // after its run analysis
    uint64_t p_first = 0;
    if (PATCH && wv == 1) p_first = lookback_prefetch(f.pstatus, b);

    // 3. the runs that become sequences (bit-parallel), then one pass over
    //    them: first one (i1, its match length), last j, and the bytes of the
    //    sequences after the first
    uint64_t hi = 0;
    {
        const int32_t d = next_after - (cs + CH);
        if (next_after < len && d >= 0 && d < 4) hi = 1ull << d;
    }
    const uint64_t Q = cl > 0 ? qualifying_starts<CH>(m, hi, cs, len) : 0ull;
    int32_t first_qi = LZE_INF, first_ml = 0, last_qj = 0, rest = 0;
    for (uint64_t q = Q; q;) {
        const int u = __builtin_ctzll(q);
        q &= q - 1;
        const int32_t e = run_end(m, u, cs, next_after);
        const int32_t i = cs + u + 1, j = e < len - 5 ? e : len - 5;
        if (first_qi == LZE_INF) {
            first_qi = i;
            first_ml = j - i;
        } else {
            rest += seq_bytes(i - last_qj, j - i);
        }
        last_qj = j;
    }
    // the last j before this chunk (exclusive maximum, 0 if none) and the
    // first qualifying i after it (exclusive minimum over the higher threads),
    // under one barrier
    int32_t carry_j, next_qi, a_final;
    {
        const int32_t inc_j = wave_incl_max(last_qj);
        const int32_t exc_j = dpp_mov<dppc::kWaveShr1, 0xf, 0xf>(0, inc_j);
        const int32_t inc_i = wave_incl_min_rev(first_qi);
        const int32_t exc_i = dpp_mov<dppc::kWaveShl1, 0xf, 0xf>(LZE_INF, inc_i);
        if (ln == kWave - 1) sh.scan[1][wv] = inc_j;
        if (ln == 0) sh.scan[2][wv] = inc_i;
        if constexpr (PATCH) {
            if (wv == 1) {
                bool failed = false;
                const uint64_t pre = lookback_resolve(f.pstatus, b, tag, (uint64_t)p_count, &failed, &p_first);
                if (ln == 0) {
                    if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
                    sh.poff = pre;
                    if (b == a.nblocks - 1) *f.d_count = (int64_t)(pre + p_count);
                    if ((int64_t)(pre + p_count) > f.cap) or_agent32(a.d_status, 1u /*PULSE_DS_CAPACITY*/);
                }
                if (f.tile_first) {
                    // the tile index: every tile that starts in this block starts
                    // at a wave boundary, so its first entry is the block's place
                    // plus the counts of the waves before it
                    constexpr int BLK_E = FusedGeom<CHLOG>::BLK_E, WAVE_E = FusedGeom<CHLOG>::NG * 256;
                    const uint32_t x = ln < LZE_NW ? sh.pw[ln] : 0u;
                    const uint32_t incl = wave_incl_sum(x);
                    const int64_t t1 = (blk_e0 + BLK_E + kPatchTile - 1) / kPatchTile;
                    for (int64_t tt = (blk_e0 + kPatchTile - 1) / kPatchTile; tt < t1 && tt < f.ntiles; ++tt) {
                        const int wj = (int)((tt * kPatchTile - blk_e0) / WAVE_E);
                        const uint32_t before = wj > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)incl, wj - 1) : 0u;
                        if (ln == 0) f.tile_first[tt] = (int64_t)(pre + before);
                    }
                    if (b == a.nblocks - 1 && ln == 0) f.tile_first[f.ntiles] = (int64_t)(pre + p_count);
                }
            }
        }
        __syncthreads();
        int32_t below = 0, all = 0, above = LZE_INF;
#pragma unroll
        for (int w = 0; w < LZE_NW; ++w) {
            const int32_t xj = sh.scan[1][w], xi = sh.scan[2][w];
            if (w < wv) below = xj > below ? xj : below;
            all = xj > all ? xj : all;
            if (w > wv) above = xi < above ? xi : above;
        }
        carry_j = exc_j > below ? exc_j : below;
        next_qi = exc_i < above ? exc_i : above;
        a_final = __builtin_amdgcn_readfirstlane(all);  // uniform: keep it in a scalar register
    }
    // the fused pass's patch, placed by wave 1 before the barrier above: the
    // staged entries go out with coalesced stores (the window is next written
    // by the emission, after the next barrier)
    if constexpr (PATCH) {
        // the waves' counts in lanes 0..15: prefix, own count and maximum by
        // DPP scans, read back as scalars
        const uint32_t x = ln < LZE_NW ? sh.pw[ln] : 0u;
        const uint32_t incl = wave_incl_sum(x), mx = wave_incl_max(x);
        const uint32_t p_mine = (uint32_t)__builtin_amdgcn_readlane((int)x, wv);
        const uint32_t p_wpre = (uint32_t)__builtin_amdgcn_readlane((int)incl, wv) - p_mine;
        const uint32_t p_wmax = (uint32_t)__builtin_amdgcn_readlane((int)mx, LZE_NW - 1);
        const uint32_t po_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sh.poff >> 32));
        const uint32_t po_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sh.poff);
        const int64_t run = (int64_t)(((uint64_t)po_hi << 32) | po_lo) + p_wpre;
        if (p_wmax <= (uint32_t)LZF_STAGE) {
            for (uint32_t i = ln; i < p_mine; i += kWave) {
                const int64_t pos = run + i;
                if (pos < f.cap) {
                    const uint32_t v = stg[i];
                    f.idx[pos] = (int32_t)(blk_e0 + (v & 0xFFFFu));
                    f.val[pos] = (uint16_t)(v >> 16);
                }
            }
        } else {
            fused_patch_direct<CHLOG>(f, blk_e0, s_img, run, t);
        }
    }
    const int32_t tot = first_qi == LZE_INF ? 0 : seq_bytes(first_qi - carry_j, first_ml) + rest;
    // byte offset of this thread's sequences (exclusive sum) and the block's
    // sequence bytes
    int32_t pos0, qsum;
    {
        const int32_t inc = wave_incl_sum(tot);
        if (ln == kWave - 1) sh.scan[3][wv] = inc;
        __syncthreads();
        int32_t below = 0, all = 0;
#pragma unroll
        for (int w = 0; w < LZE_NW; ++w) {
            const int32_t x = sh.scan[3][w];
            if (w < wv) below += x;
            all += x;
        }
        pos0 = below + inc - tot;
        qsum = __builtin_amdgcn_readfirstlane(all);
    }
    const int32_t ll_final = len - a_final;
    const int32_t comp = qsum + 1 + ext_bytes(ll_final) + ll_final;

    // A block without a qualifying run (incompressible bytes, such as the
    // value planes of a packed patch) is one literal sequence: its token and
    // length bytes, then the block's bytes as they are.  Those go from the
    // image straight to the payload with 16-byte stores (each output piece
    // from two image pieces), instead of through the window byte by byte.
    // a block larger than the window: its sequences are counted (slot set 0
    // of the scans is free again), and with fewer than LZE_GCAP it is left to
    // enc_gather once placed
    [[maybe_unused]] bool defer = false;  // (uniform)
    if constexpr (!PATCH) {
        if (qsum != 0 && comp > LZE_WIN) {
            const int32_t c = __builtin_popcountll(Q);
            const int32_t ci = wave_incl_sum(c);
            if (ln == kWave - 1) sh.scan[0][wv] = ci;
            __syncthreads();
            int32_t nseq = 0;
#pragma unroll
            for (int w = 0; w < LZE_NW; ++w) nseq += sh.scan[0][w];
            defer = __builtin_amdgcn_readfirstlane(nseq) < LZE_GCAP;
        }
    }
    if (qsum == 0 || defer) {
        if (wv == 0) {
            lookback_publish(a.status, b, tag, (uint64_t)comp);
            bool failed = false;
            const uint64_t off = lookback_resolve(a.status, b, tag, (uint64_t)comp, &failed);
            if (ln == 0) {
                if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
                sh.off = off;
                sh.comp = (uint32_t)comp;
                a.comp_sizes[b] = (uint32_t)comp;
                a.comp_offsets[b] = off;
                if (b == a.nblocks - 1) *a.d_total = off + comp;
                if ((int64_t)(off + comp) > a.cap) or_agent32(a.d_status, 1u /*PULSE_DS_CAPACITY*/);
            }
        }
        __syncthreads();
        if (defer) return true;
        const uint32_t off_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sh.off >> 32));
        const uint32_t off_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sh.off);
        const uint64_t off = ((uint64_t)off_hi << 32) | off_lo;
        if ((int64_t)(off + comp) > a.cap) return false;
        uint8_t *const dst = a.payload + off;
        const int32_t h = 1 + ext_bytes(len);  // token and length bytes
        if (t < h) {
            uint32_t v;
            if (t == 0) v = (uint32_t)((len >= 15 ? 15 : len) << 4);
            else if (t < h - 1) v = 255u;
            else v = (uint32_t)(len - 15 - 255 * (h - 2));
            dst[t] = (uint8_t)v;
        }
        // literal byte p goes to body + p; aligned piece u of the body's
        // span covers literal bytes [16 u - shift, +16)
        uint8_t *const body = dst + h;
        const int32_t shift = (int32_t)((uintptr_t)body & 15);
        uint8_t *const base = body - shift;
        const int32_t npc = (shift + len + 15) >> 4;
        auto piece = [&](int32_t k) {  // image piece k (bytes [16 k, +16))
            return *reinterpret_cast<const u32x4 *>(s_img + img_addr<CHLOG>(k << 4));
        };
        for (int32_t u = t; u < npc; u += LZE_THREADS) {
            const int32_t p0 = 16 * u - shift;
            if (p0 >= 0 && p0 + 16 <= len) {
                const u32x4 r = shift == 0 ? piece(u) : take16(piece(u - 1), piece(u), 16 - shift);
                *reinterpret_cast<u32x4 *>(base + 16 * u) = r;
            } else {
                for (int32_t j = 0; j < 16; ++j) {
                    const int32_t p = p0 + j;
                    if (p >= 0 && p < len) base[16 * u + j] = s_img[img_addr<CHLOG>(p)];
                }
            }
        }
        return false;
    }

    // 4 + 5. place the block and emit it.  Wave 0 publishes the block's size;
    // every wave emits into the LDS window (relative to the block's start),
    // and only then does wave 0 wait for the predecessors' sizes, so the wait
    // overlaps the emission.  A block whose encoding is larger than the window
    // (incompressible data) is emitted in several window passes; a thread
    // skips a pass that none of its bytes fall in.
    const int32_t sw16 = ((t >> (4 - (CHLOG - 4))) & ((1 << (CHLOG - 4)) - 1)) << 4;
    if (wv == 0) lookback_publish(a.status, b, tag, (uint64_t)comp);
    // output bytes this thread writes: inside [pos0, whi)
    int32_t whi = pos0 + tot;
    {
        const int32_t la = Q ? last_qj : carry_j;
        if ((la > cs ? la : cs) < cs + cl) {
            const int32_t ll = (next_qi != LZE_INF ? next_qi : len) - la;
            whi += 1 + ext_bytes(ll) + (cs + cl - la);
        }
    }
    uint8_t *const win = s_win + 16;
    for (int32_t wb = 0; wb < comp; wb += LZE_WIN) {
        if (whi > pos0 && pos0 < wb + LZE_WIN && whi > wb)
            emit_chunk<CHLOG>(win, wb, s_img, Q, m, cs, cs + cl, next_after, len, carry_j, pos0, next_qi, sw16);
        if (t == 0) {  // the final literal run's token and length bytes
            win_put(win, wb, qsum, (uint32_t)((ll_final >= 15 ? 15 : ll_final) << 4));
            if (ll_final >= 15) put_len(win, wb, qsum + 1, ll_final);
        }
        if (wb == 0 && wv == 0) {
            bool failed = false;
            const uint64_t off = lookback_resolve(a.status, b, tag, (uint64_t)comp, &failed);
            if (ln == 0) {
                if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
                sh.off = off;
                a.comp_sizes[b] = (uint32_t)comp;
                a.comp_offsets[b] = off;
                if (b == a.nblocks - 1) *a.d_total = off + comp;
                if ((int64_t)(off + comp) > a.cap) or_agent32(a.d_status, 1u /*PULSE_DS_CAPACITY*/);
            }
        }
        __syncthreads();
        // readfirstlane returns int: each half goes through uint32_t, so the
        // low half is not sign-extended into the high one
        const uint32_t off_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sh.off >> 32));
        const uint32_t off_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sh.off);
        const uint64_t off = ((uint64_t)off_hi << 32) | off_lo;
        if ((int64_t)(off + comp) > a.cap) return false;
        const int32_t n = comp - wb < LZE_WIN ? comp - wb : LZE_WIN;
        uint8_t *dst = a.payload + off + wb;
        // copy the pass out with 16-byte stores to aligned addresses (bytes
        // for the first and last piece, shared with the neighbouring bytes):
        // aligned piece u covers pass bytes [16 u - shift, +16), which sit at
        // s_win [16 u + 16 - shift, +16), inside the aligned pair 16 u, 16 u + 16
        const int32_t shift = (int32_t)((uintptr_t)dst & 15);
        const int32_t end = shift + n;
        uint8_t *base = dst - shift;
        const int o = 16 - shift;  // 1 .. 16, the same for the whole block
        for (int32_t q = 16 * t; q < end; q += 16 * LZE_THREADS) {
            if (q >= shift && q + 16 <= end) {
                const u32x4 A = *reinterpret_cast<const u32x4 *>(s_win + q);
                const u32x4 B = *reinterpret_cast<const u32x4 *>(s_win + q + 16);
                const u32x4 r = take16(A, B, o);
                *reinterpret_cast<u32x4 *>(base + q) = r;
            } else {
                for (int32_t x = (q > shift ? q : shift); x < q + 16 && x < end; ++x) base[x] = s_win[16 + x - shift];
            }
        }
        if (wb + LZE_WIN < comp) __syncthreads();  // the next pass rewrites the window
    }
    return false;
}

template <int CHLOG>
__global__ __launch_bounds__(LZE_THREADS, 8) void k_lz4_encode(Lz4EncArgs a) {
    __shared__ __align__(16) EncShared sh;
    __shared__ uint32_t s_b, s_tag;
    if (threadIdx.x == 0) {
        uint32_t b, tag;
        ws_begin(a.hdr, a.nblocks, &b, &tag);
        s_b = b;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t b = s_b, tag = s_tag;
    if (b >= a.nblocks) {  // inconsistent workspace state: touch nothing
        if (threadIdx.x == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    enc_load<CHLOG>(a, b, sh.img);
    __syncthreads();
    if (enc_rest<CHLOG>(a, FusedArgs{}, b, tag, sh, threadIdx.x)) enc_gather<CHLOG>(a, b, sh, threadIdx.x);
}

// The fused pass: one 1024-thread workgroup per 64 KiB mask block (32768
// elements), the block taken as a ticket when the workgroup starts; two
// workgroups share a CU, so one's loads overlap the other's analysis.
template <int CHLOG, bool PATCH>
__global__ __launch_bounds__(LZE_THREADS, 8) void k_cast_diff_lz4(Lz4EncArgs a, FusedArgs f) {
    constexpr int BLK_E = FusedGeom<CHLOG>::BLK_E, NG = FusedGeom<CHLOG>::NG;
    __shared__ __align__(16) EncShared sh;
    __shared__ uint32_t s_b, s_tag;
    const int t = threadIdx.x;
    if (t == 0) {
        uint32_t b, tag;
        ws_begin(a.hdr, a.nblocks, &b, &tag);
        s_b = b;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t b = s_b, tag = s_tag;
    if (b >= a.nblocks) {  // inconsistent workspace state: touch nothing
        if (t == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    // step 1 in rounds of (up to) four groups: loads in flight, then consumed
    constexpr int GI = NG < 4 ? NG : 4;
    uint32_t *const stg = reinterpret_cast<uint32_t *>(sh.win) + (t / kWave) * LZF_STAGE;
    uint32_t nw = 0;
    {
        u32x4 fv[GI];
        u32x2 ov[GI];
        fused_load<CHLOG, 0, GI>(f, (int64_t)b * BLK_E, fv, ov, t);
        nw = fused_consume<CHLOG, PATCH, 0, GI>(f, (int64_t)b * BLK_E, fv, ov, sh.img, stg, t, nw);
    }
    if constexpr (NG > GI) {
        sched_fence();
        u32x4 fv[NG - GI];
        u32x2 ov[NG - GI];
        fused_load<CHLOG, GI, NG - GI>(f, (int64_t)b * BLK_E, fv, ov, t);
        nw = fused_consume<CHLOG, PATCH, GI, NG - GI>(f, (int64_t)b * BLK_E, fv, ov, sh.img, stg, t, nw);
    }
    sched_fence();  // keeps the later steps' code out of step 1
    if (PATCH && (t % kWave) == 0) sh.pw[t / kWave] = nw;
    __syncthreads();
    if (enc_rest<CHLOG, PATCH>(a, f, b, tag, sh, t)) {
        if constexpr (!PATCH) enc_gather<CHLOG>(a, b, sh, t);
    }
}

}  // namespace pulse

using namespace pulse;

extern "C" size_t pulse_lz4_encode_ws_bytes(int64_t nbytes, int32_t block_bytes) {
    const int64_t nb = block_bytes > 0 ? (nbytes + block_bytes - 1) / block_bytes : 0;
    return sizeof(WsHeader) + (size_t)(nb > 0 ? nb : 1) * sizeof(uint64_t);
}

extern "C" int pulse_launch_lz4_encode(const void *src, const void *src_xor, int64_t nbytes,
                                       int32_t block_bytes, uint8_t *payload, int64_t cap,
                                       uint32_t *comp_sizes, uint64_t *comp_offsets, uint64_t *d_total,
                                       uint32_t *d_status, void *ws, hipStream_t stream) {
    Lz4EncArgs a{};
    a.src = static_cast<const uint8_t *>(src);
    a.src_xor = static_cast<const uint8_t *>(src_xor);
    a.nbytes = nbytes;
    a.block_bytes = block_bytes;
    a.payload = payload;
    a.cap = cap;
    a.comp_sizes = comp_sizes;
    a.comp_offsets = comp_offsets;
    a.d_total = d_total;
    a.d_status = d_status;
    a.hdr = reinterpret_cast<WsHeader *>(ws);
    a.status = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(WsHeader));
    const int64_t nb = (nbytes + block_bytes - 1) / block_bytes;
    a.nblocks = (uint32_t)nb;
    const dim3 grid((unsigned)nb), block(LZE_THREADS);
    if (block_bytes == 65536) k_lz4_encode<6><<<grid, block, 0, stream>>>(a);
    else if (block_bytes == 32768) k_lz4_encode<5><<<grid, block, 0, stream>>>(a);
    else k_lz4_encode<4><<<grid, block, 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Workspace of the fused pass: the header, the blocks' payload-size words, then
// their patch-count words.
extern "C" size_t pulse_cast_diff_lz4_ws_bytes(int64_t n, int32_t block_bytes) {
    const int64_t nb = block_bytes > 0 ? (2 * n + block_bytes - 1) / block_bytes : 0;
    return sizeof(WsHeader) + 2 * (size_t)(nb > 0 ? nb : 1) * sizeof(uint64_t);
}

extern "C" int pulse_launch_cast_diff_lz4(const float *w_new, const uint16_t *b_old, uint16_t *b_new, int32_t *idx,
                                          uint16_t *val, int64_t cap, int64_t *d_count, int64_t n,
                                          int32_t block_bytes, uint8_t *payload, int64_t payload_cap,
                                          uint32_t *comp_sizes, uint64_t *comp_offsets, uint64_t *d_total,
                                          uint32_t *d_status, int64_t *tile_first, void *ws, hipStream_t stream) {
    const int64_t nbytes = 2 * n;
    const int64_t nb = (nbytes + block_bytes - 1) / block_bytes;
    Lz4EncArgs a{};
    a.src = nullptr;
    a.src_xor = nullptr;
    a.nbytes = nbytes;
    a.block_bytes = block_bytes;
    a.payload = payload;
    a.cap = payload_cap;
    a.comp_sizes = comp_sizes;
    a.comp_offsets = comp_offsets;
    a.d_total = d_total;
    a.d_status = d_status;
    a.hdr = reinterpret_cast<WsHeader *>(ws);
    a.status = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + sizeof(WsHeader));
    a.nblocks = (uint32_t)nb;
    FusedArgs f{};
    f.w_new = w_new;
    f.b_old = b_old;
    f.b_new = b_new;
    f.idx = idx;
    f.val = val;
    f.cap = cap;
    f.d_count = d_count;
    f.pstatus = a.status + nb;
    f.n = n;
    f.tile_first = idx ? tile_first : nullptr;
    f.ntiles = (n + kPatchTile - 1) / kPatchTile;
    const dim3 grid((unsigned)nb), block(LZE_THREADS);
    const bool patch = idx != nullptr;
    if (block_bytes == 65536) {
        if (patch) k_cast_diff_lz4<6, true><<<grid, block, 0, stream>>>(a, f);
        else k_cast_diff_lz4<6, false><<<grid, block, 0, stream>>>(a, f);
    } else if (block_bytes == 32768) {
        if (patch) k_cast_diff_lz4<5, true><<<grid, block, 0, stream>>>(a, f);
        else k_cast_diff_lz4<5, false><<<grid, block, 0, stream>>>(a, f);
    } else {
        if (patch) k_cast_diff_lz4<4, true><<<grid, block, 0, stream>>>(a, f);
        else k_cast_diff_lz4<4, false><<<grid, block, 0, stream>>>(a, f);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ---- scratch of the allocation-free fused pass ------------------------------
// pulse_cast_diff_lz4_noalloc takes its workspace from this array instead of
// the caller: the header and two look-back words per mask block for up to
// kNoAllocMaxBlocks blocks, enough for every n <= 2^31 - 1 at every block size
// (4 MiB + 256 bytes).  Each GPU the library runs on holds its own copy until
// the process ends.  On the host the array's name is only a stand-in for the
// symbol, never a device address: host code uses the address that
// hipGetSymbolAddress returns for the current device, once per device.
constexpr int64_t kNoAllocMaxBlocks = 262144;
constexpr size_t kNoAllocScratchBytes = sizeof(pulse::WsHeader) + 2 * (size_t)kNoAllocMaxBlocks * sizeof(uint64_t);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes == PULSE_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

namespace {
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kNoAllocMaxDevices];  // device address of `scratch`, per device
}  // namespace

extern "C" size_t pulse_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

// The current device's scratch address.  On a device's first call the symbol
// is looked up (with that device current) and the array is cleared by a fill
// kernel on `stream`, ahead of the kernels of that call; the epoch-tagged
// look-back words need no clearing after that.  nullptr on failure.
extern "C" void *pulse_noalloc_scratch(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        if (pulse_launch_fill_zero(p, kNoAllocScratchBytes, stream) != 0) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}
