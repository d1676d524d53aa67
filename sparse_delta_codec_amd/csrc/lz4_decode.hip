// lz4_decode.hip -- row a6: LZ4 block decode with in-place XOR (or store).
//
// The sampler XORs the decoded mask into its old weights and obtains exactly
// the new ones ("GPU weight teleportation" write-up, "XOR masks"); the decoded
// mask is applied in place in HBM, and receiver-side work dominates that
// pipeline ("Moving the pipeline onto GPUs").  The byte format is the public
// LZ4 block format; any valid block is accepted, not only the canonical parse.
//
// A block's token chain is serial, while applying it is a dense stream (a
// sparse mask still changes nearly every cache line of dst).  Four kernels:
//  K1 k_lz4_parse   one LANE per block, 64 blocks per wave.  Checks the block
//                   table (inside the payload, no block starting before the
//                   end of an earlier one: a prefix max over blocks by
//                   decoupled look-back), then walks each block's token chain
//                   from a 256-byte LDS ring of its compressed bytes that the
//                   wave refills with coalesced loads when lanes run out.  A
//                   block in the form the canonical encoder writes (every match
//                   has offset 1 and follows >= 1 literal) is validated in full
//                   and every 16th sequence start (input, output position) is
//                   recorded as a checkpoint; any other block is handed to K3.
//                   A block with a length chain longer than the ring (a run
//                   of one byte over most of the block), a literal run
//                   longer than 2,055 bytes, or a compressed size over 3/4 of
//                   its length is listed for K1L.
//  K1L k_lz4_long   one WAVE per listed block: the same walk and checks
//                   straight from global memory, a KiB per coalesced load.
//  K2 k_lz4_fast    one WORKGROUP per checkpointed block: stages its compressed
//                   bytes in LDS, starts the loads of its dst range (XOR mode),
//                   rebuilds the block in a zeroed LDS image with one thread
//                   per 16-sequence segment (long literal runs and non-zero
//                   fills are deferred and copied a wave per run in 16-byte
//                   pieces), then
//                   XORs (or stores) the image with 16-byte accesses; chunks
//                   whose mask bytes are all zero are not written back.  A
//                   block that is one literal run of its full length (the
//                   shape incompressible data takes) skips the image: its
//                   length bytes are checked in parallel and its literals
//                   stream from the payload to dst with 16-byte accesses.
//  K3 k_lz4_slow    every other block: serial, fully validating parse by one
//                   thread over LDS-staged input, cooperative copies into a
//                   64 KiB LDS image, then a coalesced XOR / store.
// No byte of a block's dst range is written unless the whole block is valid.
#include "device.hpp"

namespace pulse {

constexpr uint32_t BI_BAD = 0x80000000u;
constexpr uint32_t BI_SLOW = 0x40000000u;
constexpr uint32_t BI_LIT = 0x20000000u;  // one literal run the size of the block (length bytes checked by K2)
constexpr uint32_t BI_NSEQ = 0x1FFFFFFFu;

// Checkpoints: one per 2^L sequences, L = ck_log(S) in 0 .. 4 chosen from the
// block's compressed size S.  A sequence that is not the last one takes >= 3
// compressed bytes (token, 2-byte offset), so a block holds at most
// floor(S / (3 * 2^L)) + 1 checkpoints: L is the smallest value that keeps
// this at or under kCkSeg + 1 (one segment per K2 thread), up to 16
// sequences a checkpoint for large blocks.  A sparse mask's small blocks thus
// get short segments: their few sequences are rebuilt by many threads instead
// of a few walking long ones.  A block with L = 4 that compresses to more
// than half its length (ck_direct: long literal runs of nearly incompressible
// bytes) and holds at most kCkDirect sequences also gets one checkpoint per
// sequence, in the kCkDirect slots after its 16-sequence ones (from
// ck_direct_slot(S)): it is rebuilt one sequence per thread.  Block b's
// checkpoints start at off_b / kCkBytes + (kCkSeg + 2) b, which keeps the
// blocks' regions disjoint (room for floor(S / kCkBytes) + kCkSeg + 2 entries).
constexpr uint32_t kCkEvery = 16;             // the largest interval
constexpr uint64_t kCkBytes = 3 * kCkEvery;
constexpr uint32_t kCkSeg = 256;
constexpr uint32_t kCkDirect = 128;
__device__ __forceinline__ uint32_t ck_log(uint32_t S) {
    uint32_t L = 0;
    while (L < 4 && S > ((3u * kCkSeg) << L)) ++L;
    return L;
}
__device__ __forceinline__ bool ck_direct(uint32_t S, uint32_t len, uint32_t nseq) {
    return ck_log(S) == 4 && 2 * S > len && nseq <= kCkDirect;
}
__device__ __forceinline__ uint32_t ck_direct_slot(uint32_t S) { return S / (uint32_t)kCkBytes + 2; }

struct Lz4DecArgs {
    const uint8_t *payload;
    int64_t payload_bytes;
    const uint64_t *offs;
    const uint32_t *sizes;
    int64_t nblocks;
    int32_t block_bytes;
    int64_t nbytes;
    uint8_t *dst;
    int32_t mode;  // 0 store, 1 xor
    uint32_t *d_status;
    WsHeader *hdr;
    uint64_t *status;    // look-back words of K1 (one per K1 workgroup)
    uint32_t *binfo;     // per block: BI_BAD | BI_SLOW | number of sequences
    uint32_t *slow_list; // blocks for K3
    uint32_t *long_list; // blocks for K1L
    uint2 *ckpt;         // checkpoints (input position, output position)
    uint32_t k1_tiles;
};

__device__ __forceinline__ int64_t ck_base(uint64_t off, int64_t b) {
    return (int64_t)(off / kCkBytes) + (int64_t)(kCkSeg + 2) * b;
}

__device__ __forceinline__ uint32_t block_len(const Lz4DecArgs &a, int64_t b) {
    const int64_t rest = a.nbytes - b * (int64_t)a.block_bytes;
    return (uint32_t)(rest < a.block_bytes ? rest : a.block_bytes);
}

// byte i (0 .. 15) of a 16-byte window held as two little-endian 64-bit halves
__device__ __forceinline__ uint32_t win_byte(uint64_t lo, uint64_t hi, uint32_t i) {
    return (uint32_t)((i < 8 ? lo : hi) >> (8 * (i & 7))) & 0xFFu;
}

// ---- K1 ----------------------------------------------------------------------
// Bytes of compressed stream held per lane.  The parse runs beside the
// receiver's pass and shares the CUs' LDS with it: 256 bytes (17 KB a wave)
// take twice the refills of 512 but leave the other kernel twice the room,
// and the step is faster for it.
constexpr int K1_RING = 256;
// The K1_LOOK bytes after the ring are loaded with it: a sequence that starts
// in the ring is read whole from one window (no step near the ring's end has
// to go byte by byte), and a lane stalls only once its position leaves the ring.
constexpr int K1_LOOK = 32;
// Rings sit K1_STRIDE bytes apart: lanes refilled together read at nearly the
// same ring offsets, and with a power-of-two stride those reads would all fall
// in one LDS bank; 16 more bytes per ring move each lane four banks along.
constexpr int K1_STRIDE = K1_RING + K1_LOOK + 16;
constexpr int K1_PIECES = K1_RING / 16;        // 16-byte pieces per ring
constexpr int K1_RPI = kWave / K1_PIECES;      // rings filled by one load instruction
constexpr int K1_BATCH = 8;                    // loads in flight per lane
constexpr int K1_RPB = K1_RPI * K1_BATCH;      // rings per batch
static_assert(kWave % K1_PIECES == 0 && kWave % K1_RPB == 0 && K1_RPB < 64, "ring geometry");

// Refills the rings of the lanes that ask with the K1_RING bytes starting at
// their position `ip` in the block rounded down to a 16-byte aligned address;
// rb becomes the ring's start relative to the block.  Lanes fetch one piece
// each, K1_BATCH loads in flight before the LDS writes; a lane without a piece
// to fetch reloads the aligned piece holding payload byte 0 and drops it into
// its spill slot past the rings.  Pieces starting past the payload end are not
// fetched: an aligned 16-byte load that starts inside the payload never leaves
// the page holding its first byte.
__device__ __forceinline__ void ring_refill(uint8_t *rings, const uint8_t *pay, int64_t pay_bytes, int64_t boff,
                                            int32_t &rb, bool need, uint32_t ip) {
    const int64_t mis = (int64_t)(reinterpret_cast<uintptr_t>(pay) & 15);
    int64_t rbo = 0;
    if (need) {
        rbo = ((boff + ip + mis) & ~(int64_t)15) - mis;  // pay + rbo is 16-byte aligned
        rb = (int32_t)(rbo - boff);
    }
    const uint64_t nmask = __ballot(need);
    const int lane = lane_id();
    const int k = lane % K1_PIECES, r = lane / K1_PIECES;
    // the lane's own lookahead pieces, in flight with the batches below
    u32x4 la[K1_LOOK / 16];
    bool lok[K1_LOOK / 16];
#pragma unroll
    for (int u = 0; u < K1_LOOK / 16; ++u) {
        const int64_t o = rbo + K1_RING + 16 * u;
        lok[u] = need && o < pay_bytes;
        la[u] = *reinterpret_cast<const u32x4 *>(pay + (lok[u] ? o : -mis));
    }
#pragma unroll
    for (int g = 0; g < kWave; g += K1_RPB) {
        if (((nmask >> g) & ((1ull << K1_RPB) - 1)) == 0) continue;
        u32x4 v[K1_BATCH];
        bool ok[K1_BATCH];
#pragma unroll
        for (int u = 0; u < K1_BATCH; ++u) {
            const int j = g + u * K1_RPI + r;
            const int64_t o = __shfl(rbo, j, kWave) + 16 * k;
            ok[u] = ((nmask >> j) & 1ull) && o < pay_bytes;
            v[u] = *reinterpret_cast<const u32x4 *>(pay + (ok[u] ? o : -mis));
        }
        // unconditional stores keep all loads of the batch ahead of the first write
#pragma unroll
        for (int u = 0; u < K1_BATCH; ++u) {
            const int j = g + u * K1_RPI + r;
            uint8_t *to = ok[u] ? rings + j * K1_STRIDE + 16 * k : rings + kWave * K1_STRIDE + 16 * lane;
            *reinterpret_cast<u32x4 *>(to) = v[u];
        }
    }
#pragma unroll
    for (int u = 0; u < K1_LOOK / 16; ++u) {
        uint8_t *to = lok[u] ? rings + lane * K1_STRIDE + K1_RING + 16 * u : rings + kWave * K1_STRIDE + 16 * lane;
        *reinterpret_cast<u32x4 *>(to) = la[u];
    }
    __syncthreads();  // one-wave workgroup: the refilled rings are visible to their owners
}

// Byte reader over a block's compressed bytes (block byte x at base + mis + x,
// base 16-byte aligned, in LDS or global memory) that holds two consecutive
// aligned 16-byte pieces and loads the next two together when a byte past
// them is read: a length chain, or the offset, match bytes and next token
// after a skipped literal run, costs one round trip per 32 bytes.  Only pieces
// holding a byte of the block are loaded (such a piece never leaves that
// byte's page).
struct Win32 {
    const uint8_t *base;
    uint32_t mis, end, cur;  // end: pieces holding a byte of the block
    uint64_t q0, q1, q2, q3; // block bytes from piece cur on, eight per word
    __device__ __forceinline__ Win32(const uint8_t *b, uint32_t m, uint32_t S)
        : base(b), mis(m), end((m + S + 15) >> 4), cur(0xFFFFFFFEu), q0(0), q1(0), q2(0), q3(0) {}
    // position of block byte x in the window, loading the window if needed
    __device__ __forceinline__ uint32_t at(uint32_t x) {
        const uint32_t p = mis + x, k = p >> 4;
        if (k - cur > 1u) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(base + 16 * (size_t)k);
            u32x4 b = {0u, 0u, 0u, 0u};  // (not read when the block ends in piece k)
            if (k + 1 < end) b = *reinterpret_cast<const u32x4 *>(base + 16 * (size_t)k + 16);
            q0 = ((uint64_t)a.y << 32) | a.x;
            q1 = ((uint64_t)a.w << 32) | a.z;
            q2 = ((uint64_t)b.y << 32) | b.x;
            q3 = ((uint64_t)b.w << 32) | b.z;
            cur = k;
        }
        return p - 16 * cur;
    }
    // the eight bytes of the window word holding window byte o (branch-free)
    __device__ __forceinline__ uint64_t word(uint32_t o) const {
        const uint64_t lo = (o & 16u) ? q2 : q0, hi = (o & 16u) ? q3 : q1;
        return (o & 8u) ? hi : lo;
    }
    __device__ __forceinline__ uint32_t operator[](uint32_t x) {
        const uint32_t o = at(x);
        return (uint32_t)(word(o) >> (8 * (o & 7u))) & 0xFFu;
    }
    // block bytes x .. x + 7 are all 255 and start a window word (x + 8 <= S)
    __device__ __forceinline__ bool ff8(uint32_t x) {
        if ((mis + x) & 7u) return false;
        return word(at(x)) == ~0ull;
    }
};

// Byte reader for a walk that a whole wave does together (every lane holds the
// same position): lane l holds the aligned 16-byte piece cur + l, so the wave
// holds 1 KiB of the block (byte x at base + mis + x, base 16-byte aligned),
// loaded with one coalesced access whenever a byte past it is read: a jump
// over a literal run costs one round trip, a length chain one per KiB.  A byte
// is taken from the lane holding it by readlane, so the walk's state stays in
// scalar registers.  Only pieces holding a byte of the block are loaded.
struct WinWave {
    const uint8_t *base;
    uint32_t mis, end, cur;  // end: pieces holding a byte of the block
    u32x4 v;                 // piece cur + lane
    __device__ __forceinline__ WinWave(const uint8_t *b, uint32_t m, uint32_t S)
        : base(b), mis(m), end((m + S + 15) >> 4), cur(0xFFFFFFC0u), v{0u, 0u, 0u, 0u} {}
    // the block's aligned dword holding block byte x (x < S)
    __device__ __forceinline__ uint32_t dword_at(uint32_t x) {
        const uint32_t p = mis + x, k = p >> 4;
        if (k - cur >= (uint32_t)kWave) {
            const uint32_t c = k + (uint32_t)lane_id();
            v = c < end ? *reinterpret_cast<const u32x4 *>(base + 16 * (size_t)c) : u32x4{0u, 0u, 0u, 0u};
            cur = k;
        }
        const uint32_t r = p - 16 * cur, w = (r >> 2) & 3u;
        const uint32_t d = w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
        return (uint32_t)__builtin_amdgcn_readlane((int)d, (int)(r >> 4));
    }
    __device__ __forceinline__ uint32_t operator[](uint32_t x) {
        return (dword_at(x) >> (8 * ((mis + x) & 3u))) & 0xFFu;
    }
    // block bytes x .. x + 7 are all 255 and start an aligned dword pair (x + 8 <= S)
    __device__ __forceinline__ bool ff8(uint32_t x) {
        if ((mis + x) & 7u) return false;
        return (dword_at(x) & dword_at(x + 4)) == ~0u;
    }
};

// Adds to n the length bytes starting at block byte q (bytes added while they
// are 255, eight at a time where they fill an aligned word); q moves past them.
// False when they run past the block (S bytes) or n passes len.
template <class Win>
__device__ __forceinline__ bool win_chain(Win &src, uint32_t S, uint32_t len, uint32_t &q, uint32_t &n) {
    uint32_t x;
    do {
        if (q >= S) return false;
        if (S - q >= 8 && src.ff8(q)) {
            n += 8 * 255;
            q += 8;
            x = 255;
        } else {
            x = src[q++];
            n += x;
        }
        if (n > len) return false;
    } while (x == 255);
    return true;
}

// Lane state of the walk, one word (bit flags in a VGPR keep divergent joins
// free of per-flag lane-mask bookkeeping).
constexpr uint32_t F_DONE = 1u, F_BAD = 2u, F_SLOW = 4u, F_STALL = 8u, F_OFF = 16u, F_LIT = 32u, F_LONG = 64u,
                   F_DCK = 128u;
// A literal run longer than this (a length chain of more than eight bytes)
// ends the ring walk with F_LONG: such runs belong to almost incompressible
// blocks of few sequences, where each run would cost the ring walk a refill.
constexpr uint32_t K1_LIT_MAX = 15 + 8 * 255;
constexpr int32_t K1_NO_RING = -(1 << 30);  // ring start before the first refill
// Sequences the walk's fast step takes per iteration, and the last ring offset
// at which a later one of them may start (its 20-byte window then ends inside
// the ring and its lookahead).
constexpr int K1_SEQ = 4;
constexpr int K1_SEQ_MAX = K1_RING + K1_LOOK - 20;

// Reads a length extension (bytes added while they are 255) starting at
// block position q into n.  r0: ring index of the step's first byte; a chain
// that leaves a ring refilled at that step cannot be read from the ring at all
// (F_LONG: the block is walked again by k1_walk_long), nor can a length above
// cap (<= len) that is not above len.
__device__ __forceinline__ uint32_t read_ext(const uint8_t *ring, int32_t rb, uint32_t S, uint32_t len,
                                             uint32_t cap, uint32_t r0, uint32_t &q, uint32_t &n) {
    while (true) {
        if (q >= S) return F_BAD | F_DONE;
        const uint32_t rq = q - (uint32_t)rb;
        if (rq >= (uint32_t)(K1_RING + K1_LOOK)) return r0 < 16 ? (F_LONG | F_DONE) : F_STALL;
        const uint32_t x = ring[rq];
        ++q;
        n += x;
        if (n > cap) return n > len ? (F_BAD | F_DONE) : (F_LONG | F_DONE);
        if (x != 255) return 0;
    }
}

// The checks of one canonical sequence whose token (literal length ll, match
// code mc, compressed size seq_in) starts the 16-byte window w0..w3 (little
// endian): 1 to 12 literals, offset 1, at most one match-length byte, at most
// `room` compressed bytes and `out` decoded bytes.  True, with the match
// length, when the window holds such a sequence.
__device__ __forceinline__ bool k1_fast_check(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t ll,
                                              uint32_t mc, uint32_t seq_in, uint32_t room, uint32_t out,
                                              uint32_t &ml) {
    // the offset and the first match-length byte: window bytes lc + 1 .. lc + 3
    // (lc <= 12), taken by one byte-align from the dword pair holding them
    const uint32_t p = (ll <= 12 ? ll : 12u) + 1u, k = p >> 2;
    const uint32_t a0 = (k & 1u) ? w1 : w0, a1 = (k & 1u) ? w3 : w2;
    const uint32_t b0 = (k & 1u) ? w2 : w1;
    const uint32_t lo = (k & 2u) ? a1 : a0, hi = (k & 2u) ? w3 : b0;
    const uint32_t v = __builtin_amdgcn_alignbyte(hi, lo, p & 3u);
    const uint32_t mo = v & 0xFFFFu, x = (v >> 16) & 0xFFu;
    ml = mc + 4 + (mc == 15 ? x : 0u);
    return (ll - 1u < 12u) & (mo == 1) & ((mc != 15) | (x != 255)) & (seq_in <= room) & (ll + ml <= out);
}

struct WalkResult {
    uint32_t nseq, flags;
};

// One lane's walk over its block (S compressed bytes, len decoded bytes).
// Each step consumes one sequence: the token (with literal-length bytes and
// the skipped literals), then the offset (with match-length bytes).  A step
// whose bytes lie past the ring stalls the lane until the wave's next refill.
// The block is handed to K3 (F_SLOW) at the first sequence not in canonical
// form.  A length chain longer than the ring (a run of one byte over most of a
// 64 KiB block), or a literal run longer than K1_LIT_MAX, ends the ring walk
// with F_LONG; such blocks are few and have few sequences, and k1_walk_long
// walks them again from global memory.
__device__ __forceinline__ WalkResult k1_walk(uint8_t *rings, const uint8_t *ring, bool active, const uint8_t *pay,
                                              int64_t pay_bytes, int64_t boff, uint32_t S, uint32_t len, uint2 *ck,
                                              uint32_t ckl) {
    int32_t rb = K1_NO_RING;  // empty ring: every position maps past it
    uint32_t ip = 0, op = 0, tok = 0, nseq = 0;
    const uint32_t ckm = (1u << ckl) - 1u;
    uint32_t f = active ? 0u : F_DONE;
    while (__ballot(!(f & F_DONE))) {
        f &= ~F_STALL;
        while (true) {
            const bool run = !(f & (F_DONE | F_STALL));
            if (!__ballot(run)) break;
            // fast step, without branches: up to K1_SEQ whole canonical
            // sequences (each 1 to 12 literals, offset 1, at most one
            // match-length byte, inside the block and the output), each read
            // from a 20-byte window of the ring and its lookahead; everything
            // the general step would check holds.  The first starts in the
            // ring (a lane past the ring stalls here), each later one at most
            // K1_SEQ_MAX bytes into it, so every window ends inside the ring
            // and its lookahead.  A lane that cannot take one (or is not
            // running) reads the ring's first bytes and takes none.
            bool took;
            {
                const uint32_t r = ip - (uint32_t)rb;
                const bool tryf = run && !(f & F_OFF) && ip < S;
                const bool st = tryf && r >= (uint32_t)K1_RING;
                f |= st ? F_STALL : 0u;
                bool go = tryf && !st;
                uint32_t rj = go ? r : 0u;
                took = false;
                const uint32_t *d = reinterpret_cast<const uint32_t *>(ring + (rj & ~3u));
                uint32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3], d4 = d[4];
#pragma unroll
                for (int j = 0; j < K1_SEQ; ++j) {
                    const uint32_t sh = rj & 3u;
                    const uint32_t w0 = __builtin_amdgcn_alignbyte(d1, d0, sh),
                                   w1 = __builtin_amdgcn_alignbyte(d2, d1, sh),
                                   w2 = __builtin_amdgcn_alignbyte(d3, d2, sh),
                                   w3 = __builtin_amdgcn_alignbyte(d4, d3, sh);
                    // the next sequence's position depends on the token alone:
                    // its window is read before this sequence is checked
                    const uint32_t ll = (w0 >> 4) & 15u, mc = w0 & 15u;
                    const uint32_t seq_in = 3u + ll + (mc == 15u ? 1u : 0u);
                    const uint32_t rn = rj + (seq_in <= 16u ? seq_in : 16u);
                    const uint32_t rjn = rn <= (uint32_t)K1_SEQ_MAX ? rn : 0u;
                    if (j + 1 < K1_SEQ) {
                        const uint32_t *dn = reinterpret_cast<const uint32_t *>(ring + (rjn & ~3u));
                        d0 = dn[0], d1 = dn[1], d2 = dn[2], d3 = dn[3], d4 = dn[4];
                    }
                    uint32_t ml;
                    const bool fj = k1_fast_check(w0, w1, w2, w3, ll, mc, seq_in, S - ip, len - op, ml) & go;
                    const bool ckw = fj & ((nseq & ckm) == 0);  // one condition: one masked store
                    if (ckw) ck[nseq >> ckl] = make_uint2(ip, op);
                    nseq += fj ? 1u : 0u;
                    ip += fj ? seq_in : 0u;
                    op += fj ? ll + ml : 0u;
                    if (j == 0) took = fj;
                    go = fj && rn <= (uint32_t)K1_SEQ_MAX;
                    rj = rjn;
                }
            }
            if (run) {
                if (!took && !(f & (F_OFF | F_STALL))) {
                    const uint32_t r = ip - (uint32_t)rb;
                    if (ip >= S) {
                        f |= F_BAD | F_DONE;
                    } else if (r >= (uint32_t)K1_RING) {
                        f |= F_STALL;
                    } else {
                        tok = ring[r];
                        uint32_t q = ip + 1, ll = tok >> 4, e = 0;
                        if (ll == 15) e = read_ext(ring, rb, S, len, len < K1_LIT_MAX ? len : K1_LIT_MAX, r, q, ll);
                        if (!e && (ll > S - q || ll > len - op)) e = F_BAD | F_DONE;
                        if (e) {
                            f |= e;
                        } else {
                            if ((nseq & ckm) == 0) ck[nseq >> ckl] = make_uint2(ip, op);
                            ++nseq;
                            ip = q + ll;
                            op += ll;
                            if (ip == S) f |= F_DONE | (op != len ? F_BAD : 0u);
                            else if (ll == 0) f |= F_SLOW | F_DONE;  // a match right after a match
                            else f |= F_OFF;
                        }
                    }
                }
                if (!took && (f & (F_OFF | F_DONE | F_STALL)) == F_OFF) {
                    const uint32_t r = ip - (uint32_t)rb;
                    if (S - ip < 2) {
                        f |= F_BAD | F_DONE;
                    } else if (r >= (uint32_t)(K1_RING + K1_LOOK - 2)) {
                        f |= F_STALL;
                    } else {
                        const uint32_t mo = (uint32_t)ring[r] | ((uint32_t)ring[r + 1] << 8);
                        const uint32_t x0 = ring[r + 2];  // first match-length byte, if there is one
                        uint32_t q = ip + 2, ml = (tok & 15) + 4, e = 0;
                        if ((tok & 15) == 15) {
                            if (q < S && x0 != 255) {
                                ++q;
                                ml += x0;
                                if (ml > len) e = F_BAD | F_DONE;
                            } else {
                                e = read_ext(ring, rb, S, len, len, r, q, ml);
                            }
                        }
                        if (!e) {
                            if (mo == 0 || mo > op || ml > len - op) e = F_BAD | F_DONE;
                            else if (mo != 1) e = F_SLOW | F_DONE;
                        }
                        if (e) {
                            f |= e;
                        } else {
                            op += ml;
                            ip = q;
                            f &= ~F_OFF;
                        }
                    }
                }
            }
        }
        if (!__ballot(!(f & F_DONE))) break;
        ring_refill(rings, pay, pay_bytes, boff, rb, (f & (F_STALL | F_DONE)) == F_STALL, ip);
    }
    return WalkResult{nseq, f};
}


// The walk of one block straight from global memory, for the blocks with a
// length chain longer than the ring or a literal run longer than K1_LIT_MAX:
// the same checks, flags and checkpoints as the ring walk (a sequence that is
// not canonical: F_SLOW), by a whole wave (K1L) reading the block a KiB at a
// time.  dck (or null): the block's direct checkpoint slots, filled for its
// first kCkDirect sequences; a valid block of at most kCkDirect sequences then
// has them all (F_DCK).  Only the lanes with `wr` store checkpoints.
__device__ __forceinline__ WalkResult k1_walk_long(const uint8_t *pay, int64_t boff, uint32_t S, uint32_t len,
                                                   uint2 *ck, uint32_t ckl, uint2 *dck, bool wr) {
    const uint8_t *blk = pay + boff;
    const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(blk) & 15);
    WinWave src(blk - mis, mis, S);
    uint32_t ip = 0, op = 0, nseq = 0;
    const WalkResult bad{0u, F_BAD | F_DONE};
    while (true) {
        if (ip >= S) return bad;
        const uint32_t tok = src[ip];
        uint32_t q = ip + 1, ll = tok >> 4;
        if (ll == 15 && !win_chain(src, S, len, q, ll)) return bad;
        if (ll > S - q || ll > len - op) return bad;
        if (wr && (nseq & ((1u << ckl) - 1u)) == 0) ck[nseq >> ckl] = make_uint2(ip, op);
        if (wr && dck && nseq < kCkDirect) dck[nseq] = make_uint2(ip, op);
        ++nseq;
        ip = q + ll;
        op += ll;
        if (ip == S) {
            if (op != len) return bad;
            return WalkResult{nseq, F_DONE | (dck && nseq <= kCkDirect ? F_DCK : 0u)};
        }
        if (ll == 0) return WalkResult{nseq, F_SLOW | F_DONE};  // a match right after a match
        if (S - ip < 2) return bad;
        const uint32_t mo = src[ip] | (src[ip + 1] << 8);
        if (mo == 0 || mo > op) return bad;
        if (mo != 1) return WalkResult{nseq, F_SLOW | F_DONE};
        q = ip + 2;
        uint32_t ml = (tok & 15) + 4;
        if ((tok & 15) == 15 && !win_chain(src, S, len, q, ml)) return bad;
        if (ml > len - op) return bad;
        op += ml;
        ip = q;
    }
}

// The direct checkpoints of a validated block (see ck_direct): its sequence
// starts walked again from global memory, 32 bytes at a time.
__device__ __forceinline__ void k1_direct_ck(const uint8_t *pay, int64_t boff, uint32_t S, uint32_t nseq,
                                             uint2 *dck) {
    const uint8_t *blk = pay + boff;
    const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(blk) & 15);
    Win32 src(blk - mis, mis, S);
    uint32_t ip = 0, op = 0;
    for (uint32_t k = 0; k < nseq; ++k) {
        dck[k] = make_uint2(ip, op);
        const uint32_t tok = src[ip];
        uint32_t q = ip + 1, ll = tok >> 4;
        if (ll == 15) win_chain(src, S, ~0u, q, ll);  // (validated: it ends inside the block)
        q += ll;
        op += ll;
        if (k + 1 == nseq) break;  // the final sequence has no match
        q += 2;
        uint32_t ml = (tok & 15) + 4;
        if ((tok & 15) == 15) win_chain(src, S, ~0u, q, ml);
        op += ml;
        ip = q;
    }
}

__global__ __launch_bounds__(64) void k_lz4_parse(Lz4DecArgs a) {
    __shared__ __align__(16) uint8_t s_rings[kWave * K1_STRIDE + kWave * 16];  // rings, then spill slots
    __shared__ uint32_t s_tile, s_tag;
    __shared__ uint64_t s_scan[1];
    const int lane = lane_id();
    if (lane == 0) {
        uint32_t tile, tag;
        ws_begin(a.hdr, a.k1_tiles, &tile, &tag);
        s_tile = tile;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile, tag = s_tag;
    if (tile >= a.k1_tiles) {  // inconsistent workspace state: touch nothing
        if (lane == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    const int64_t b = (int64_t)tile * 64 + lane;
    const bool live = b < a.nblocks;

    // table checks: inside the payload, not before the end of any earlier block
    uint64_t off = 0, S = 0;
    bool bad = !live;
    if (live) {
        off = a.offs[b];
        S = a.sizes[b];
        bad = off > (uint64_t)a.payload_bytes || S > (uint64_t)a.payload_bytes - off || S == 0;
    }
    const uint64_t lim = (uint64_t)a.payload_bytes + 1;  // ends are compared against offsets <= payload
    uint64_t end = 0;
    if (live) {
        const uint64_t e = off + S < off ? ~0ull : off + S;
        end = e < lim ? e : lim;
    }
    uint64_t tile_max;
    const uint64_t in_tile = block_excl_max<1>(end, (uint64_t)0, s_scan, &tile_max);
    bool failed = false;
    const uint64_t pre = lookback_wave<true>(a.status, tile, tag, tile_max, &failed);
    if (failed && lane == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
    const uint64_t before = in_tile > pre ? in_tile : pre;
    if (live && b > 0 && off < before) bad = true;

    const uint32_t len = live ? block_len(a, b) : 0;
    uint2 *ck = a.ckpt + (live ? ck_base(off, b) : 0);
    // a block that compresses to more than 3/4 of its length (nearly
    // incompressible bytes: few, long literal runs, each a ring refill) is not
    // walked here
    const bool dense = live && !bad && 4 * S > 3 * (uint64_t)len;
    WalkResult w = k1_walk(s_rings, s_rings + lane * K1_STRIDE, !bad && !dense, a.payload, a.payload_bytes,
                           (int64_t)off, (uint32_t)S, len, ck, ck_log((uint32_t)S));
    // such a block, and one the ring cannot walk, is listed for K1L, which
    // walks it with a whole wave and writes its block info
    const bool lng = dense || (live && !bad && (w.flags & F_LONG) != 0);
    if (lng) {
        const uint32_t k = add_agent32(&a.hdr->aux3, 1u);
        if (k < a.nblocks) a.long_list[k] = (uint32_t)b;
    }
    // a valid block of one sequence is one literal run: K2 copies it as such
    if (w.nseq == 1 && !(w.flags & (F_BAD | F_SLOW))) w.flags |= F_LIT;
    // a large, literal-heavy block of few sequences: one checkpoint per sequence
    // (written here unless the walk from global memory wrote them)
    const bool direct = !bad && !lng && !(w.flags & (F_BAD | F_SLOW | F_LIT | F_DCK)) &&
                        ck_direct((uint32_t)S, len, w.nseq);
    if (__ballot(direct)) {
        if (direct) k1_direct_ck(a.payload, (int64_t)off, (uint32_t)S, w.nseq, ck + ck_direct_slot((uint32_t)S));
    }
    const uint32_t nseq = w.nseq;
    const bool slow = (w.flags & F_SLOW) != 0;
    bad = bad || (w.flags & F_BAD) != 0;
    if (live && !lng) {
        if (bad) {
            a.binfo[b] = BI_BAD;
            or_agent32(a.d_status, 4u /*PULSE_DS_CORRUPT*/);
        } else if (slow) {
            a.binfo[b] = BI_SLOW;
            const uint32_t k = add_agent32(&a.hdr->aux, 1u);
            if (k < a.nblocks) a.slow_list[k] = (uint32_t)b;
        } else {
            a.binfo[b] = nseq | ((w.flags & F_LIT) ? BI_LIT : 0u);
        }
    }
}

// ---- K1L ---------------------------------------------------------------------
// The blocks K1 listed (compressed to more than 3/4 of their length, a literal
// run longer than K1_LIT_MAX, or a length chain longer than the ring: the
// nearly incompressible blocks of few, long sequences), one wave per block:
// the wave walks the block from global memory a KiB at a time, so each jump
// over a literal run is one coalesced round trip, and the blocks are walked
// side by side on many SIMDs instead of in one lane each.  Then the block's
// info, as K1 writes it for the others.  Four waves per workgroup, each on
// its own blocks.
constexpr int K1L_THREADS = 256;
constexpr int K1L_GROUPS = 2048;

__global__ __launch_bounds__(K1L_THREADS) void k_lz4_long(Lz4DecArgs a) {
    constexpr uint32_t NW = K1L_THREADS / kWave;
    uint32_t count = ld_agent32(&a.hdr->aux3);
    if (count > a.nblocks) count = (uint32_t)a.nblocks;
    const bool lead = lane_id() == 0;
    const uint32_t wv = threadIdx.x / kWave;
    for (uint32_t i = blockIdx.x * NW + wv; i < count; i += gridDim.x * NW) {
        const uint32_t bu = a.long_list[i];
        if (bu >= a.nblocks) continue;  // (a workspace whose last parse had no apply)
        const int64_t b = bu;
        const uint64_t off = a.offs[b];
        const uint32_t S = a.sizes[b];
        const uint32_t len = block_len(a, b);
        uint2 *ck = a.ckpt + ck_base(off, b);
        const bool dsz = ck_direct(S, len, 0);  // the size test of ck_direct
        WalkResult w = k1_walk_long(a.payload, (int64_t)off, S, len, ck, ck_log(S),
                                    dsz ? ck + ck_direct_slot(S) : nullptr, lead);
        if (w.nseq == 1 && !(w.flags & (F_BAD | F_SLOW))) w.flags |= F_LIT;
        if (lead) {
            if (w.flags & F_BAD) {
                a.binfo[b] = BI_BAD;
                or_agent32(a.d_status, 4u /*PULSE_DS_CORRUPT*/);
            } else if (w.flags & F_SLOW) {
                a.binfo[b] = BI_SLOW;
                const uint32_t k = add_agent32(&a.hdr->aux, 1u);
                if (k < a.nblocks) a.slow_list[k] = (uint32_t)b;
            } else {
                a.binfo[b] = w.nseq | ((w.flags & F_LIT) ? BI_LIT : 0u);
            }
        }
    }
}

// ---- K2 ----------------------------------------------------------------------
constexpr int K2_THREADS = 256;
constexpr int K2_STAGE = 14336;  // compressed bytes staged in LDS (image + stage: 2 workgroups per CU)
constexpr int K2_SPT = (K2_STAGE / 16 + K2_THREADS - 1) / K2_THREADS;
constexpr uint32_t K2_LONG = 32;  // literal runs and fills longer than this are deferred
constexpr int K2_QCAP = 128;
constexpr uint32_t K2_FILL = 0x80000000u;

struct K2Queue {
    uint32_t op[K2_QCAP], n[K2_QCAP], src[K2_QCAP];  // src: input position, or K2_FILL | byte
    uint32_t count;
};

__device__ __forceinline__ bool k2_defer(K2Queue &qu, uint32_t op, uint32_t n, uint32_t src) {
    const uint32_t e = atomicAdd(&qu.count, 1u);
    if (e >= (uint32_t)K2_QCAP) return false;
    qu.op[e] = op;
    qu.n[e] = n;
    qu.src[e] = src;
    return true;
}

// The sum of a validated length chain starting at src[q] (bytes added while
// they are 255); q moves past it.  GROUP (the LDS stage): past eight bytes of
// 255, four bytes are tested per round trip while they are all 255 (shorter
// chains, the common ones, and the global-memory variant keep the byte loop,
// which their hot paths run faster).
template <bool GROUP, typename Src>
__device__ __forceinline__ uint32_t k2_chain(Src &src, uint32_t S, uint32_t &q) {
    uint32_t x, n = 0, k = 0;
    do {
        x = src[q++];
        n += x;
        ++k;
    } while (x == 255 && k < 8);
    if (x != 255) return n;
    while (GROUP && q + 4 <= S && (src[q] & src[q + 1] & src[q + 2] & src[q + 3]) == 255u) {
        q += 4;
        n += 4 * 255;
    }
    do {
        x = src[q++];
        n += x;
    } while (x == 255);
    return n;
}

// One sequence of a validated canonical block: literal bytes into the zeroed
// image, then the offset-1 fill when it repeats a non-zero byte; runs longer
// than K2_LONG are queued for the whole workgroup.  Returns false at the final
// sequence.
template <bool GROUP, typename Src>
__device__ __forceinline__ bool k2_seq_bytes(Src &src, uint32_t S, uint32_t &ip, uint32_t &op, uint8_t *img,
                                             K2Queue &qu) {
    const uint32_t tok = src[ip];
    uint32_t q = ip + 1, ll = tok >> 4;
    if (ll == 15) ll += k2_chain<GROUP>(src, S, q);
    uint32_t last = 0;
    if (ll > K2_LONG) {
        last = src[q + ll - 1];
        if (!k2_defer(qu, op, ll, q))
            for (uint32_t i = 0; i < ll; ++i) img[op + i] = src[q + i];
    } else {
        for (uint32_t i = 0; i < ll; ++i) {
            last = src[q + i];
            if (last) img[op + i] = (uint8_t)last;
        }
    }
    q += ll;
    op += ll;
    if (q >= S) return false;  // the final sequence
    q += 2;                    // offset 1
    uint32_t ml = (tok & 15) + 4;
    if ((tok & 15) == 15) ml += k2_chain<GROUP>(src, S, q);
    if (last) {
        if (ml <= K2_LONG || !k2_defer(qu, op, ml, K2_FILL | last))
            for (uint32_t i = 0; i < ml; ++i) img[op + i] = (uint8_t)last;
    }
    op += ml;
    ip = q;
    return true;
}

// Rebuild of one segment of 2^ckl sequences (starting at checkpoint c) from
// global memory (block byte x at base + mis + x, base 16-byte aligned).
__device__ __forceinline__ void k2_segment(const uint8_t *base, uint32_t mis, uint32_t S, uint32_t nseq, uint32_t s,
                                           uint32_t ckl, uint2 c, uint8_t *img, K2Queue &qu) {
    uint32_t ip = c.x, op = c.y;
    const uint32_t rest = nseq - (s << ckl);
    const uint32_t kend = rest < (1u << ckl) ? rest : (1u << ckl);
    const uint8_t *src = base + mis;
    for (uint32_t k = 0; k < kend; ++k)
        if (!k2_seq_bytes<false>(src, S, ip, op, img, qu)) break;
}

// The same from the LDS stage (the block's bytes start at stage + mis).  The
// common sequence of a sparse mask -- 1 to 12 literals ending in a zero byte
// (the first byte of the zero run the match repeats, so no fill), offset 1, at
// most one match-length byte -- is decoded from one 16-byte window (five
// aligned dwords joined by byte-align shifts): one LDS round trip; only the
// non-zero literal bytes are written (the image is zeroed).  Any other
// sequence goes byte by byte, and the next one is tried on the fast path again.
__device__ __forceinline__ void k2_segment_lds(const uint8_t *stage, uint32_t mis, uint32_t S, uint32_t nseq,
                                               uint32_t s, uint32_t ckl, uint2 c, uint8_t *img, K2Queue &qu) {
    uint32_t ip = c.x, op = c.y;
    const uint32_t rest = nseq - (s << ckl);
    const uint32_t kend = rest < (1u << ckl) ? rest : (1u << ckl);
    const uint8_t *src = stage + mis;
    for (uint32_t k = 0; k < kend; ++k) {
        const uint32_t P = mis + ip;
        const uint32_t *d = reinterpret_cast<const uint32_t *>(stage + (P & ~3u));
        const uint32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3], d4 = d[4];  // (past the block: padding, unused)
        const uint32_t sh = P & 3u;
        const uint32_t w0 = __builtin_amdgcn_alignbyte(d1, d0, sh), w1 = __builtin_amdgcn_alignbyte(d2, d1, sh);
        const uint32_t w2 = __builtin_amdgcn_alignbyte(d3, d2, sh), w3 = __builtin_amdgcn_alignbyte(d4, d3, sh);
        const uint64_t lo = ((uint64_t)w1 << 32) | w0, hi = ((uint64_t)w3 << 32) | w2;  // bytes ip .. ip+15
        const uint32_t ll = (w0 >> 4) & 15u, mc = w0 & 15u;
        const uint32_t lc = ll <= 12 ? ll : 12u;
        const uint32_t lastb = win_byte(lo, hi, lc);  // literal byte ll
        const uint32_t x = win_byte(lo, hi, lc + 3);  // byte 3 + ll
        // (bitwise, not short-circuit: one branch)
        const uint32_t fast = (uint32_t)(ll - 1u < 12u) & (uint32_t)(lastb == 0) & (uint32_t)(ip + 1 + ll < S) &
                              (uint32_t)((mc != 15) | (x != 255));
        if (fast) {
            // non-zero literal bytes 1 .. ll-1: high bit of each byte of
            // ((w & 0x7F..) + 0x7F..) | w, two words' flags gathered per multiply
            uint32_t h[4];
            const uint32_t wv[4] = {w0, w1, w2, w3};
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (((wv[e] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | wv[e]) & 0x80808080u;
            const uint32_t nz16 = ((((h[0] >> 4) | h[1]) * 0x00204081u) >> 24) |
                                  (((((h[2] >> 4) | h[3]) * 0x00204081u) >> 24) << 8);
            uint32_t nz = nz16 & ((1u << ll) - 2u);
            while (nz) {
                const uint32_t i = (uint32_t)__builtin_ctz(nz);
                nz &= nz - 1;
                img[op + i - 1] = (uint8_t)win_byte(lo, hi, i);
            }
            const uint32_t ext = mc == 15 ? 1u : 0u;
            op += ll + mc + 4 + (ext ? x : 0u);
            ip += 3 + ll + ext;
        } else if (!k2_seq_bytes<true>(src, S, ip, op, img, qu)) {
            break;
        }
    }
}

// Thread t rebuilds segments t, t + 256, ...; the first from the checkpoint c0
// loaded early (no loop around it, so nothing waits for the dst loads).
// The block's bytes are at src + mis (src 16-byte aligned): the LDS stage when
// STAGED, else global memory.
template <bool STAGED>
__device__ __forceinline__ void k2_segments(const uint8_t *src, uint32_t mis, uint32_t S, uint32_t nseq,
                                            uint32_t ckl, const uint2 *ck, uint2 c0, uint8_t *img, K2Queue &qu) {
    const uint32_t nseg = (nseq + (1u << ckl) - 1) >> ckl;
    const uint32_t t = threadIdx.x;
    if constexpr (STAGED) {
        if (t < nseg) k2_segment_lds(src, mis, S, nseq, t, ckl, c0, img, qu);
        for (uint32_t s = t + K2_THREADS; s < nseg; s += K2_THREADS)
            k2_segment_lds(src, mis, S, nseq, s, ckl, ck[s], img, qu);
    } else {
        if (t < nseg) k2_segment(src, mis, S, nseq, t, ckl, c0, img, qu);
        for (uint32_t s = t + K2_THREADS; s < nseg; s += K2_THREADS)
            k2_segment(src, mis, S, nseq, s, ckl, ck[s], img, qu);
    }
}

// The queued runs, one wave per run: a literal run is copied from the
// compressed bytes (block byte 0 at src, LDS or global memory) and a fill
// writes its byte, both as 16-byte image pieces (each from two aligned source
// pieces); the pieces at the run's two ends, shared with its neighbours, go
// byte by byte.  Each lane has up to four pieces in flight.
__device__ __forceinline__ void k2_deferred(const uint8_t *src, uint8_t *img, const K2Queue &qu) {
    constexpr int NWV = K2_THREADS / kWave, U = 4;
    const uint32_t nq = qu.count < (uint32_t)K2_QCAP ? qu.count : (uint32_t)K2_QCAP;
    const uint32_t ln = threadIdx.x & (kWave - 1);
    for (uint32_t e = threadIdx.x / kWave; e < nq; e += NWV) {
        const uint32_t o = qu.op[e], n = qu.n[e], sv = qu.src[e];
        const uint32_t p0 = o >> 4, p1 = (o + n - 1) >> 4;  // image pieces the run touches
        const bool fill = (sv & K2_FILL) != 0;
        const uint8_t *g = src + (fill ? 0u : sv);           // source of image byte o
        const uint32_t gm = (uint32_t)((reinterpret_cast<uintptr_t>(g) - o) & 15u);
        const uint32_t fb = (sv & 0xFFu) * 0x01010101u;
        for (uint32_t p = p0 + ln; p <= p1; p += U * kWave) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t pp = p + (uint32_t)(u * kWave);
                v[u] = u32x4{fb, fb, fb, fb};
                if (!fill && pp <= p1 && 16 * pp >= o && 16 * pp + 16 <= o + n) {
                    const u32x4 *a4 = reinterpret_cast<const u32x4 *>(g + (16 * pp - o) - gm);
                    v[u] = a4[0];
                    if (gm) v[u] = take16(v[u], a4[1], (int)gm);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t pp = p + (uint32_t)(u * kWave);
                if (pp > p1) continue;
                if (16 * pp >= o && 16 * pp + 16 <= o + n) {
                    *reinterpret_cast<u32x4 *>(img + 16 * pp) = v[u];
                } else {
                    const uint32_t lo = 16 * pp > o ? 16 * pp : o, hi = 16 * pp + 16 < o + n ? 16 * pp + 16 : o + n;
                    for (uint32_t x = lo; x < hi; ++x) img[x] = fill ? (uint8_t)sv : (uint8_t)g[x - o];
                }
            }
        }
    }
}

// byte r (0 .. 31) of the 32 bytes A (low) then B, branch-free
__device__ __forceinline__ uint32_t byte32(const u32x4 &A, const u32x4 &B, uint32_t r) {
    const uint64_t a0 = ((uint64_t)A.y << 32) | A.x, a1 = ((uint64_t)A.w << 32) | A.z;
    const uint64_t b0 = ((uint64_t)B.y << 32) | B.x, b1 = ((uint64_t)B.w << 32) | B.z;
    const uint64_t lo = (r & 16u) ? b0 : a0, hi = (r & 16u) ? b1 : a1;
    return (uint32_t)(((r & 8u) ? hi : lo) >> (8 * (r & 7u))) & 0xFFu;
}

// The queued runs of a block read from global memory (block byte 0 at src),
// one wave per run, as k2_deferred does from the LDS stage, but with every
// load of a lane's pieces issued before any is used: for each of its image
// pieces a lane loads the one or two aligned 16-byte pieces holding the
// source of the piece's bytes in the run (a lane past the run reloads the
// run's first), so a round of four pieces per lane costs one memory round
// trip.  Whole pieces are shifted into place (the shift is the same for all of
// a run's pieces) and stored with 16-byte writes; a run's two end pieces,
// shared with its neighbours, are written byte by byte from the registers.
__device__ __forceinline__ void k2_deferred_global(const uint8_t *src, uint8_t *img, const K2Queue &qu) {
    constexpr int NWV = K2_THREADS / kWave, U = 4;
    const uint32_t nq = qu.count < (uint32_t)K2_QCAP ? qu.count : (uint32_t)K2_QCAP;
    const uint32_t ln = threadIdx.x & (kWave - 1);
    for (uint32_t e = threadIdx.x / kWave; e < nq; e += NWV) {
        // the run, the same in every lane of the wave
        const uint32_t o = (uint32_t)__builtin_amdgcn_readfirstlane((int)qu.op[e]);
        const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane((int)qu.n[e]);
        const uint32_t sv = (uint32_t)__builtin_amdgcn_readfirstlane((int)qu.src[e]);
        const uint32_t p0 = o >> 4, p1 = (o + n - 1) >> 4;  // image pieces the run touches
        if (sv & K2_FILL) {
            const uint32_t fb = (sv & 0xFFu) * 0x01010101u;
            for (uint32_t pp = p0 + ln; pp <= p1; pp += kWave) {
                if (16 * pp >= o && 16 * pp + 16 <= o + n) {
                    *reinterpret_cast<u32x4 *>(img + 16 * pp) = u32x4{fb, fb, fb, fb};
                } else {
                    const uint32_t lo = 16 * pp > o ? 16 * pp : o, hi = 16 * pp + 16 < o + n ? 16 * pp + 16 : o + n;
                    for (uint32_t x = lo; x < hi; ++x) img[x] = (uint8_t)sv;
                }
            }
            continue;
        }
        const uint8_t *g = src + sv;  // source of image byte o
        const uint8_t *glast = g + (n - 1);
        const uint32_t gm = (uint32_t)((reinterpret_cast<uintptr_t>(g) - o) & 15u);  // shift of every whole piece
        for (uint32_t p = p0 + ln; p <= p1; p += U * kWave) {
            u32x4 A[U], B[U];
            const uint8_t *base[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t pp = p + (uint32_t)(u * kWave);
                const uint32_t lo = pp <= p1 && 16 * pp > o ? 16 * pp : o;
                const uint8_t *s0 = g + (lo - o);
                base[u] = s0 - (reinterpret_cast<uintptr_t>(s0) & 15u);
                const uint8_t *bb = base[u] + 16 <= glast ? base[u] + 16 : base[u];
                A[u] = *reinterpret_cast<const u32x4 *>(base[u]);
                B[u] = *reinterpret_cast<const u32x4 *>(bb);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t pp = p + (uint32_t)(u * kWave);
                if (pp > p1) continue;
                if (16 * pp >= o && 16 * pp + 16 <= o + n) {
                    *reinterpret_cast<u32x4 *>(img + 16 * pp) = gm ? take16(A[u], B[u], (int)gm) : A[u];
                } else {
                    const uint32_t lo = 16 * pp > o ? 16 * pp : o, hi = 16 * pp + 16 < o + n ? 16 * pp + 16 : o + n;
                    for (uint32_t x = lo; x < hi; ++x)
                        img[x] = (uint8_t)byte32(A[u], B[u], (uint32_t)((g + (x - o)) - base[u]));
                }
            }
        }
    }
}

// One block of K2.  STAGED: the compressed bytes fit the LDS stage (else they
// are read from global memory); the two variants share no code path, so the
// waits of the staged one never count the other's byte loads.
template <int IMG, bool XOR, bool STAGED>
__device__ __forceinline__ void k2_block(const Lz4DecArgs &a, int64_t b, uint32_t nseq, uint64_t off, uint32_t S,
                                         uint8_t *s_img, uint8_t *s_stage, K2Queue &s_q) {
    constexpr int CPT = IMG / (16 * K2_THREADS);  // 16-byte chunks per thread
    const int t = threadIdx.x;
    const uint32_t len = block_len(a, b);
    const uint8_t *in = a.payload + off;
    const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(in) & 15);
    const uint32_t nfull = len >> 4, nchunk = (len + 15) >> 4;
    uint4 *dst4 = reinterpret_cast<uint4 *>(a.dst + b * (int64_t)a.block_bytes);
    uint4 *img4 = reinterpret_cast<uint4 *>(s_img);

    // compressed bytes and the first checkpoint, then dst: waiting for the
    // former leaves the dst loads in flight.  The view is read and written
    // once per call, so its accesses are non-temporal (they would otherwise
    // push the next blocks' compressed bytes out of the L2).  The stage loads are unconditional
    // (a thread past the block reloads its first piece) so that none of them
    // waits behind a branch.
    u32x4 sv[K2_SPT];
    const uint32_t nsc = STAGED ? (S + mis + 15) >> 4 : 0;
    if constexpr (STAGED) {
        const u32x4 *in4 = reinterpret_cast<const u32x4 *>(in - mis);
#pragma unroll
        for (int k = 0; k < K2_SPT; ++k) {
            const uint32_t c = t + K2_THREADS * k;
            sv[k] = in4[c < nsc ? c : 0u];
        }
    }
    const uint2 *ck = a.ckpt + ck_base(off, b);
    uint32_t ckl = ck_log(S);
    if (ck_direct(S, len, nseq)) {  // one checkpoint per sequence
        ck += ck_direct_slot(S);
        ckl = 0;
    }
    const uint32_t nseg = (nseq + (1u << ckl) - 1) >> ckl;
    const uint2 c0 = ck[(uint32_t)t < nseg ? t : 0];
    sched_fence();
    u32x4 dv[CPT];
    if constexpr (XOR) {
        const u32x4 *d4 = reinterpret_cast<const u32x4 *>(dst4);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const uint32_t c = t + K2_THREADS * k;
            dv[k] = __builtin_nontemporal_load(d4 + (c < nfull ? c : 0u));  // (past the block: a reload, never used)
        }
    }
    if (t == 0) s_q.count = 0;
    if constexpr (STAGED) {
        // pieces past the block land in the thread's own first image chunk,
        // which the same thread zeroes right after
#pragma unroll
        for (int k = 0; k < K2_SPT; ++k) {
            const uint32_t c = t + K2_THREADS * k;
            u32x4 *to = reinterpret_cast<u32x4 *>(c < nsc ? reinterpret_cast<uint4 *>(s_stage) + c : img4 + t);
            *to = sv[k];
        }
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const uint32_t c = t + K2_THREADS * k;
        if (c < nchunk) img4[c] = make_uint4(0, 0, 0, 0);
    }
    lds_barrier();

    if constexpr (STAGED) {
        k2_segments<true>(static_cast<const uint8_t *>(s_stage), mis, S, nseq, ckl, ck, c0, s_img, s_q);
        lds_barrier();
        k2_deferred(static_cast<const uint8_t *>(s_stage + mis), s_img, s_q);
    } else {
        k2_segments<false>(in - mis, mis, S, nseq, ckl, ck, c0, s_img, s_q);
        lds_barrier();
        k2_deferred_global(in, s_img, s_q);
    }
    lds_barrier();

#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const uint32_t c = t + K2_THREADS * k;
        const u32x4 v = reinterpret_cast<const u32x4 *>(s_img)[c < nchunk ? c : 0];
        if constexpr (XOR) {
            // a 64-byte line (four 16-byte chunks, four neighbouring lanes) is
            // written whole when any of its chunks changes, else not at all:
            // no partially written lines
            uint32_t nz = (v.x | v.y | v.z | v.w) != 0u ? 1u : 0u;
            nz |= dpp_mov<0xB1, 0xf, 0xf>(0u, nz);  // quad_perm [1,0,3,2]
            nz |= dpp_mov<0x4E, 0xf, 0xf>(0u, nz);  // quad_perm [2,3,0,1]
            if (c < nfull && nz) __builtin_nontemporal_store(dv[k] ^ v, reinterpret_cast<u32x4 *>(dst4) + c);
        } else {
            if (c < nfull) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst4) + c);
        }
    }
    if (nfull < nchunk && (uint32_t)t == nfull % K2_THREADS) {  // ragged tail of the last block
        uint8_t *d = reinterpret_cast<uint8_t *>(dst4 + nfull);
        const uint8_t *v = s_img + 16 * nfull;
        for (uint32_t x = 0; x < (len & 15); ++x) d[x] = XOR ? (uint8_t)(d[x] ^ v[x]) : v[x];
    }
}

// A block K1 found to be one literal run of its full length L (validated in
// full, or, for a chain longer than K1's ring, only its token and its size
// S = L + h checked): its h - 1 length bytes are checked here in parallel
// (255s, then the remainder), and the literals go to dst with
// 16-byte streams (XORed in, or stored), each dst piece from two aligned
// pieces of the payload.  A block whose length bytes say otherwise may still
// be a valid block of another shape: it is handed to K3, which decodes and
// checks any block.
template <bool XOR>
__device__ __forceinline__ void k2_literal_block(const Lz4DecArgs &a, int64_t b, uint64_t off, uint32_t S,
                                                 uint32_t *s_flag) {
    const int t = threadIdx.x;
    const uint32_t len = block_len(a, b);
    const uint8_t *in = a.payload + off;
    const uint32_t h = S - len;
    if (t == 0) *s_flag = 0u;
    __syncthreads();
    for (uint32_t x = (uint32_t)t + 1; x < h; x += K2_THREADS) {
        const uint32_t want = x < h - 1 ? 255u : len - 15 - 255 * (h - 2);
        if (in[x] != want) *s_flag = 1u;
    }
    __syncthreads();
    if (*s_flag) {
        if (t == 0) {
            const uint32_t k = add_agent32(&a.hdr->aux, 1u);
            if (k < a.nblocks) a.slow_list[k] = (uint32_t)b;
        }
        return;
    }
    const uint8_t *src = in + h;
    const uint32_t mis = (uint32_t)__builtin_amdgcn_readfirstlane((int)(reinterpret_cast<uintptr_t>(src) & 15));
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src - mis);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(a.dst + b * (int64_t)a.block_bytes);
    const uint32_t nfull = len >> 4;
    // four dst pieces per thread and round, every load of a round issued
    // before any is used (a piece past the block reloads the round's first)
    constexpr int U = 4;
    for (uint32_t c0 = t; c0 < nfull; c0 += U * K2_THREADS) {
        u32x4 A[U], B[U], D[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = c0 + (uint32_t)(u * K2_THREADS), cc = c < nfull ? c : c0;
            // (the second piece holds the last bytes of dst piece cc when
            // mis > 0: it starts inside the block's data, so it never leaves
            // the data's page)
            A[u] = s4[cc];
            B[u] = s4[mis ? cc + 1 : cc];
            if constexpr (XOR) D[u] = __builtin_nontemporal_load(d4 + cc);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = c0 + (uint32_t)(u * K2_THREADS);
            if (c >= nfull) break;
            u32x4 v = mis ? take16(A[u], B[u], (int)mis) : A[u];
            if constexpr (XOR) v ^= D[u];
            __builtin_nontemporal_store(v, d4 + c);
        }
    }
    if (t == 0) {  // ragged tail of the last block
        uint8_t *d = reinterpret_cast<uint8_t *>(d4 + nfull);
        const uint8_t *v = src + 16 * nfull;
        for (uint32_t x = 0; x < (len & 15); ++x) d[x] = XOR ? (uint8_t)(d[x] ^ v[x]) : v[x];
    }
}

// IMG: image bytes, >= block_bytes (one instantiation per supported size class);
// XOR: mode 1.  Both are compile-time so that every load is issued on one path
// and the waits for the stage loads leave the dst loads in flight.
template <int IMG, bool XOR>
__global__ __launch_bounds__(K2_THREADS) void k_lz4_fast(Lz4DecArgs a) {
    __shared__ __align__(16) uint8_t s_img[IMG];
    __shared__ __align__(16) uint8_t s_stage[K2_STAGE + 32];  // (+32: the 16-byte windows may read past the data)
    __shared__ K2Queue s_q;
    const int64_t b = blockIdx.x;
    const uint32_t info = a.binfo[b];
    if (info & (BI_BAD | BI_SLOW)) return;
    const uint64_t off = a.offs[b];
    const uint32_t S = a.sizes[b];
    if (info & BI_LIT) {
        k2_literal_block<XOR>(a, b, off, S, &s_q.count);
        return;
    }
    const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(a.payload + off) & 15);
    if (S + mis <= (uint32_t)K2_STAGE) k2_block<IMG, XOR, true>(a, b, info & BI_NSEQ, off, S, s_img, s_stage, s_q);
    else k2_block<IMG, XOR, false>(a, b, info & BI_NSEQ, off, S, s_img, s_stage, s_q);
}

// ---- K3 ----------------------------------------------------------------------
constexpr int K3_THREADS = 256;
constexpr int K3_STAGE = 66 * 1024;  // holds any block up to the LZ4 bound of 64 KiB

__global__ __launch_bounds__(K3_THREADS) void k_lz4_slow(Lz4DecArgs a) {
    __shared__ __align__(16) uint8_t s_dec[65536];
    __shared__ __align__(16) uint8_t s_in[K3_STAGE];
    __shared__ uint32_t s_h[6];
    const int t = threadIdx.x;
    uint32_t count = ld_agent32(&a.hdr->aux);
    if (count > a.nblocks) count = (uint32_t)a.nblocks;
    for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
        const int64_t b = a.slow_list[i];
        const uint64_t off = a.offs[b];
        const uint32_t S = a.sizes[b];
        const uint32_t len = block_len(a, b);
        const uint8_t *in = a.payload + off;
        const uint32_t mis = (uint32_t)(reinterpret_cast<uintptr_t>(in) & 15);
        const bool staged = S + mis <= (uint32_t)K3_STAGE;
        if (staged) {
            const uint4 *in4 = reinterpret_cast<const uint4 *>(in - mis);
            for (uint32_t c = t; c < (S + mis + 15) >> 4; c += K3_THREADS)
                reinterpret_cast<uint4 *>(s_in)[c] = in4[c];
        }
        __syncthreads();
        const uint8_t *src = staged ? static_cast<const uint8_t *>(s_in + mis) : in;
        uint32_t ip = 0, op = 0;
        bool bad = false;
        while (true) {
            if (t == 0) {
                // one sequence, with every check of the block format
                uint32_t lit = 0, ll = 0, mo = 0, ml = 0, fin = 0, err = 0;
                if (ip >= S) err = 1;
                const uint32_t tok = err ? 0u : src[ip++];
                ll = tok >> 4;
                if (!err && ll == 15) {
                    while (true) {
                        if (ip >= S) { err = 1; break; }
                        const uint32_t x = src[ip++];
                        ll += x;
                        if (ll > len) { err = 1; break; }
                        if (x != 255) break;
                    }
                }
                if (!err && (ll > S - ip || ll > len - op)) err = 1;
                if (!err) {
                    lit = ip;
                    ip += ll;
                    if (ip == S) {
                        fin = 1;
                        if (op + ll != len) err = 1;
                    } else if (S - ip < 2) {
                        err = 1;
                    } else {
                        mo = (uint32_t)src[ip] | ((uint32_t)src[ip + 1] << 8);
                        ip += 2;
                        if (mo == 0 || mo > op + ll) err = 1;
                        ml = (tok & 15) + 4;
                        if (!err && (tok & 15) == 15) {
                            while (true) {
                                if (ip >= S) { err = 1; break; }
                                const uint32_t x = src[ip++];
                                ml += x;
                                if (ml > len) { err = 1; break; }
                                if (x != 255) break;
                            }
                        }
                        if (!err && ml > len - op - ll) err = 1;
                    }
                }
                s_h[0] = lit;
                s_h[1] = ll;
                s_h[2] = mo;
                s_h[3] = ml;
                s_h[4] = fin;
                s_h[5] = err;
            }
            __syncthreads();
            const uint32_t lit = s_h[0], ll = s_h[1], mo = s_h[2], ml = s_h[3], fin = s_h[4], err = s_h[5];
            __syncthreads();
            if (err) {
                bad = true;
                break;
            }
            for (uint32_t x = t; x < ll; x += K3_THREADS) s_dec[op + x] = src[lit + x];
            __syncthreads();
            op += ll;
            if (fin) break;
            // forward copy with overlap: byte x of the match repeats the mo bytes before it
            for (uint32_t x = t; x < ml; x += K3_THREADS) s_dec[op + x] = s_dec[op - mo + (x % mo)];
            __syncthreads();
            op += ml;
        }
        if (bad) {
            if (t == 0) or_agent32(a.d_status, 4u /*PULSE_DS_CORRUPT*/);
        } else {
            uint8_t *dstb = a.dst + b * (int64_t)a.block_bytes;
            for (uint32_t q = 16 * t; q < len; q += 16 * K3_THREADS) {
                if (q + 16 <= len) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(s_dec + q);
                    if (a.mode == 1) {
                        uint4 d = *reinterpret_cast<const uint4 *>(dstb + q);
                        d.x ^= v.x; d.y ^= v.y; d.z ^= v.z; d.w ^= v.w;
                        *reinterpret_cast<uint4 *>(dstb + q) = d;
                    } else {
                        *reinterpret_cast<uint4 *>(dstb + q) = v;
                    }
                } else {
                    for (uint32_t x = q; x < len; ++x)
                        dstb[x] = a.mode == 1 ? (uint8_t)(dstb[x] ^ s_dec[x]) : s_dec[x];
                }
            }
        }
        __syncthreads();
    }
    if (t == 0) {
        const uint32_t d = add_agent32(&a.hdr->aux2, 1u);
        if (d == gridDim.x - 1) {
            st_agent32(&a.hdr->aux, 0u);
            st_agent32(&a.hdr->aux2, 0u);
            st_agent32(&a.hdr->aux3, 0u);
        }
    }
}

}  // namespace pulse

using namespace pulse;

namespace {
// The regions of a decode workspace are a function of its size alone, so the
// look-back status words of one call never overlap the per-block data another
// call of a different size left behind (a stale word must never carry a
// matching epoch tag).  Status: 1 word per KiB; block info, slow list and
// long list: ws/8 bytes each; checkpoints: the rest.
struct DecLayout {
    size_t status, binfo, slow, longl, ckpt;
    size_t status_words, blocks, ck_entries;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
DecLayout dec_layout(size_t ws) {
    DecLayout L;
    L.status = sizeof(WsHeader);
    L.status_words = ws >> 10;
    L.binfo = al256(L.status + 8 * L.status_words);
    L.blocks = ws >> 5;
    L.slow = al256(L.binfo + 4 * L.blocks);
    L.longl = al256(L.slow + 4 * L.blocks);
    L.ckpt = al256(L.longl + 4 * L.blocks);
    L.ck_entries = ws > L.ckpt ? (ws - L.ckpt) / sizeof(uint2) : 0;
    return L;
}
size_t ck_needed(int64_t nblocks, int64_t payload_bytes) {
    return (size_t)payload_bytes / kCkBytes + (size_t)(kCkSeg + 2) * (size_t)nblocks + 2;
}
bool dec_fits(size_t ws, int64_t nblocks, int64_t payload_bytes) {
    const DecLayout L = dec_layout(ws);
    const size_t k1 = (size_t)(nblocks + 63) / 64;
    return ws >= L.ckpt && k1 <= L.status_words && (size_t)nblocks <= L.blocks &&
           ck_needed(nblocks, payload_bytes) <= L.ck_entries;
}

template <int IMG>
void launch_fast(const Lz4DecArgs &a, hipStream_t stream) {
    if (a.mode == 1) k_lz4_fast<IMG, true><<<dim3((unsigned)a.nblocks), dim3(K2_THREADS), 0, stream>>>(a);
    else k_lz4_fast<IMG, false><<<dim3((unsigned)a.nblocks), dim3(K2_THREADS), 0, stream>>>(a);
}
}  // namespace

extern "C" size_t pulse_lz4_decode_ws_bytes(int64_t nblocks, int64_t payload_bytes) {
    if (nblocks < 0 || payload_bytes < 0) return 0;
    size_t ws = al256(4096 + 40 * (size_t)nblocks + 8 * ck_needed(nblocks, payload_bytes) * 4 / 3);
    while (!dec_fits(ws, nblocks, payload_bytes)) ws = al256(ws + ws / 8 + 256);
    return ws;
}

extern "C" int pulse_lz4_decode_ws_fits(size_t ws, int64_t nblocks, int64_t payload_bytes) {
    return dec_fits(ws, nblocks, payload_bytes) ? 1 : 0;
}

namespace {
Lz4DecArgs dec_args(const uint8_t *payload, int64_t payload_bytes, const uint64_t *offs, const uint32_t *sizes,
                    int64_t nblocks, int32_t block_bytes, int64_t nbytes, void *dst, int32_t mode,
                    uint32_t *d_status, void *ws, size_t ws_bytes) {
    const DecLayout L = dec_layout(ws_bytes);
    char *w = static_cast<char *>(ws);
    Lz4DecArgs a{};
    a.payload = payload;
    a.payload_bytes = payload_bytes;
    a.offs = offs;
    a.sizes = sizes;
    a.nblocks = nblocks;
    a.block_bytes = block_bytes;
    a.nbytes = nbytes;
    a.dst = static_cast<uint8_t *>(dst);
    a.mode = mode;
    a.d_status = d_status;
    a.hdr = reinterpret_cast<WsHeader *>(w);
    a.status = reinterpret_cast<uint64_t *>(w + L.status);
    a.binfo = reinterpret_cast<uint32_t *>(w + L.binfo);
    a.slow_list = reinterpret_cast<uint32_t *>(w + L.slow);
    a.long_list = reinterpret_cast<uint32_t *>(w + L.longl);
    a.ckpt = reinterpret_cast<uint2 *>(w + L.ckpt);
    a.k1_tiles = (uint32_t)((nblocks + 63) / 64);
    return a;
}
}  // namespace

// K1 and K1L: validate the block table and parse every block into the
// workspace (per-block info, checkpoints, the list of blocks for K3).
extern "C" int pulse_launch_lz4_decode_parse(const uint8_t *payload, int64_t payload_bytes, const uint64_t *offs,
                                             const uint32_t *sizes, int64_t nblocks, int32_t block_bytes,
                                             int64_t nbytes, uint32_t *d_status, void *ws, size_t ws_bytes,
                                             hipStream_t stream) {
    const Lz4DecArgs a = dec_args(payload, payload_bytes, offs, sizes, nblocks, block_bytes, nbytes, nullptr, 0,
                                  d_status, ws, ws_bytes);
    k_lz4_parse<<<dim3(a.k1_tiles), dim3(64), 0, stream>>>(a);
    const int64_t nw = K1L_THREADS / kWave, gl = (nblocks + nw - 1) / nw < K1L_GROUPS ? (nblocks + nw - 1) / nw : K1L_GROUPS;
    if (gl > 0) k_lz4_long<<<dim3((unsigned)gl), dim3(K1L_THREADS), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// K2 and K3 over what the parse left in the workspace; K3's last workgroup
// clears the workspace's slow-block counters, so the next parse starts clean.
extern "C" int pulse_launch_lz4_decode_apply(const uint8_t *payload, int64_t payload_bytes, const uint64_t *offs,
                                             const uint32_t *sizes, int64_t nblocks, int32_t block_bytes,
                                             int64_t nbytes, void *dst, int32_t mode, uint32_t *d_status, void *ws,
                                             size_t ws_bytes, hipStream_t stream) {
    const Lz4DecArgs a = dec_args(payload, payload_bytes, offs, sizes, nblocks, block_bytes, nbytes, dst, mode,
                                  d_status, ws, ws_bytes);
    if (block_bytes <= 16384) launch_fast<16384>(a, stream);
    else if (block_bytes <= 32768) launch_fast<32768>(a, stream);
    else launch_fast<65536>(a, stream);
    const int64_t g3 = nblocks < 512 ? nblocks : 512;
    k_lz4_slow<<<dim3((unsigned)g3), dim3(K3_THREADS), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int pulse_launch_lz4_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *offs,
                                       const uint32_t *sizes, int64_t nblocks, int32_t block_bytes,
                                       int64_t nbytes, void *dst, int32_t mode, uint32_t *d_status, void *ws,
                                       size_t ws_bytes, hipStream_t stream) {
    const int rc = pulse_launch_lz4_decode_parse(payload, payload_bytes, offs, sizes, nblocks, block_bytes, nbytes,
                                                 d_status, ws, ws_bytes, stream);
    if (rc != 0) return rc;
    return pulse_launch_lz4_decode_apply(payload, payload_bytes, offs, sizes, nblocks, block_bytes, nbytes, dst,
                                         mode, d_status, ws, ws_bytes, stream);
}
