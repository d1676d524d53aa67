// lz4_decode.hip -- row a6: LZ4 block decode with in-place XOR (or store).
//
// The sampler XORs the decoded mask into its old weights and obtains exactly
// the new ones ("GPU weight teleportation" write-up, "XOR masks"); the decoded
// mask is applied in place in HBM, and receiver-side work dominates that
// pipeline ("Moving the pipeline onto GPUs").  The byte format is the public
// LZ4 block format; any valid block is accepted, not only the canonical parse.
//
// The token chain of a block is inherently serial, so it is split from the
// data movement:
//  K1 k_lz4_parse   one LANE per block: checks the block table (inside the
//                   payload, no block starting before the end of an earlier
//                   one -- a prefix max over blocks by decoupled look-back),
//                   walks the token chain with a 16-byte register window,
//                   validates it, and records token positions in a bitmap
//                   (1 bit per compressed byte, disjoint per block).  64 blocks
//                   are parsed per wave, so the serial chains run in parallel.
//  K2 k_lz4_decode  one WORKGROUP per block: bitmap -> token list (popcount
//                   scan) -> per-sequence headers, one thread each -> output
//                   offsets (block scan) -> each thread rebuilds 16-byte output
//                   chunks directly from the compressed bytes and XORs them into
//                   dst with coalesced 16-byte accesses (all-zero chunks are
//                   skipped in XOR mode).  Valid when every match copies from
//                   its own sequence's literals (offset <= literal length),
//                   which holds for every block the canonical encoder writes.
//  K3 k_lz4_slow    general path for the other blocks: sequential parse by one
//                   thread, cooperative copies into a 64 KiB LDS image, then a
//                   coalesced XOR/store.
// K1 validates a block completely before K2/K3 write any byte of its range.
#include "device.hpp"

namespace pulse {

constexpr uint32_t BI_BAD = 0x80000000u;
constexpr uint32_t BI_SLOW = 0x40000000u;
constexpr uint32_t BI_NSEQ = 0x3FFFFFFFu;

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
    uint64_t *status;  // look-back words of K1 (one per K1 workgroup)
    uint32_t *binfo;   // per block: BI_BAD | BI_SLOW | number of sequences
    uint32_t *slow_list;
    uint32_t *bitmap;
    uint32_t k1_tiles;
};

// ---- K1 ----------------------------------------------------------------------
// Reads byte i of a block through an aligned 16-byte window; an aligned 16-byte
// load that contains a byte of the payload never leaves that byte's 4 KiB page.
struct Window {
    uintptr_t base;  // address of byte 0 of the block
    uintptr_t cur;   // aligned address held in w, or 1 (none)
    uint4 w;
    __device__ __forceinline__ uint32_t get(int64_t i) {
        const uintptr_t a = base + (uintptr_t)i;
        const uintptr_t al = a & ~(uintptr_t)15;
        if (al != cur) {
            w = *reinterpret_cast<const uint4 *>(al);
            cur = al;
        }
        const uint32_t k = (uint32_t)(a - al);
        const uint32_t d = (k < 8) ? ((k < 4) ? w.x : w.y) : ((k < 12) ? w.z : w.w);
        return (d >> (8 * (k & 3))) & 0xFFu;
    }
};

struct BitWriter {
    uint32_t *words;   // this block's bitmap words
    int64_t cur;       // word being filled
    uint32_t bits;
    __device__ __forceinline__ void mark(int64_t pos) {
        const int64_t w = pos >> 5;
        if (w != cur) {
            words[cur] = bits;
            for (int64_t z = cur + 1; z < w; ++z) words[z] = 0u;
            cur = w;
            bits = 0u;
        }
        bits |= 1u << (pos & 31);
    }
    __device__ __forceinline__ void finish(int64_t nwords) {
        words[cur] = bits;
        for (int64_t z = cur + 1; z < nwords; ++z) words[z] = 0u;
    }
};

__global__ __launch_bounds__(256) void k_lz4_parse(Lz4DecArgs a) {
    __shared__ uint32_t s_tile, s_tag;
    __shared__ uint64_t s_scan[4];
    __shared__ uint64_t s_pre;
    const int t = threadIdx.x;
    if (t == 0) {
        uint32_t tile, tag;
        ws_begin(a.hdr, a.k1_tiles, &tile, &tag);
        s_tile = tile;
        s_tag = tag;
    }
    __syncthreads();
    const uint32_t tile = s_tile, tag = s_tag;
    if (tile >= a.k1_tiles) {  // inconsistent workspace state: touch nothing
        if (t == 0) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
        return;
    }
    const int64_t b = (int64_t)tile * 256 + t;
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
    const uint64_t in_tile = block_excl_max<4>(end, (uint64_t)0, s_scan, &tile_max);
    if (wave_id() == 0) {
        bool failed = false;
        const uint64_t pre = lookback_wave<true>(a.status, tile, tag, tile_max, &failed);
        if (lane_id() == 0) {
            if (failed) or_agent32(a.d_status, 8u /*PULSE_DS_WORKSPACE*/);
            s_pre = pre;
        }
    }
    __syncthreads();
    const uint64_t before = in_tile > s_pre ? in_tile : s_pre;
    if (live && b > 0 && off < before) bad = true;
    if (!live) return;

    const int64_t len = (a.nbytes - b * (int64_t)a.block_bytes) < a.block_bytes
                            ? (a.nbytes - b * (int64_t)a.block_bytes)
                            : a.block_bytes;
    uint32_t nseq = 0;
    bool slow = false;
    if (!bad) {
        Window win{(uintptr_t)(a.payload + off), (uintptr_t)1, make_uint4(0, 0, 0, 0)};
        BitWriter bw{a.bitmap + (off >> 5) + b, 0, 0u};
        const int64_t Sb = (int64_t)S;
        int64_t ip = 0, op = 0;
        while (true) {
            if (ip >= Sb) { bad = true; break; }
            bw.mark(ip);
            const uint32_t tok = win.get(ip++);
            int64_t ll = tok >> 4;
            if (ll == 15) {
                uint32_t x;
                do {
                    if (ip >= Sb) { bad = true; break; }
                    x = win.get(ip++);
                    ll += x;
                } while (x == 255 && ll <= len);
                if (bad) break;
            }
            if (ll > Sb - ip || ll > len - op) { bad = true; break; }
            ip += ll;
            op += ll;
            ++nseq;
            if (ip == Sb) {
                if (op != len) bad = true;
                break;
            }
            if (Sb - ip < 2) { bad = true; break; }
            const int64_t mo = (int64_t)win.get(ip) | ((int64_t)win.get(ip + 1) << 8);
            ip += 2;
            if (mo == 0 || mo > op) { bad = true; break; }
            int64_t ml = (tok & 15) + 4;
            if ((tok & 15) == 15) {
                uint32_t x;
                do {
                    if (ip >= Sb) { bad = true; break; }
                    x = win.get(ip++);
                    ml += x;
                } while (x == 255 && ml <= len);
                if (bad) break;
            }
            if (ml > len - op) { bad = true; break; }
            if (mo > ll) slow = true;  // the match reaches outside its own literals
            op += ml;
        }
        if (!bad) bw.finish((Sb + 31) >> 5);
    }
    if (bad) {
        a.binfo[b] = BI_BAD;
        or_agent32(a.d_status, 4u /*PULSE_DS_CORRUPT*/);
    } else if (slow) {
        a.binfo[b] = BI_SLOW | nseq;
        const uint32_t k = add_agent32(&a.hdr->aux, 1u);
        if (k < a.nblocks) a.slow_list[k] = (uint32_t)b;
    } else {
        a.binfo[b] = nseq;
    }
}

// ---- K2 ----------------------------------------------------------------------
constexpr int LZD_THREADS = 256;
constexpr int LZD_BATCH = 2048;

struct SeqHdr {
    uint32_t lit;   // literal start in the compressed block
    uint32_t ll;    // literal length
    uint32_t mo;    // match offset (0: final sequence)
    uint32_t len;   // literal + match length
    uint32_t next;  // position after the sequence
};

__device__ __forceinline__ SeqHdr parse_seq(const uint8_t *in, uint32_t p, uint32_t S) {
    SeqHdr h;
    const uint32_t tok = in[p];
    uint32_t q = p + 1;
    uint32_t ll = tok >> 4;
    if (ll == 15) {
        uint32_t x;
        do {
            x = in[q++];
            ll += x;
        } while (x == 255);
    }
    h.lit = q;
    h.ll = ll;
    q += ll;
    if (q >= S) {
        h.mo = 0;
        h.len = ll;
        h.next = q;
        return h;
    }
    h.mo = (uint32_t)in[q] | ((uint32_t)in[q + 1] << 8);
    q += 2;
    uint32_t ml = (tok & 15) + 4;
    if ((tok & 15) == 15) {
        uint32_t x;
        do {
            x = in[q++];
            ml += x;
        } while (x == 255);
    }
    h.len = ll + ml;
    h.next = q;
    return h;
}

__global__ __launch_bounds__(LZD_THREADS) void k_lz4_decode(Lz4DecArgs a) {
    __shared__ uint32_t s_lit[LZD_BATCH];  // token positions, then literal starts
    __shared__ uint32_t s_ll[LZD_BATCH];
    __shared__ uint16_t s_mo[LZD_BATCH];
    __shared__ uint32_t s_out[LZD_BATCH + 1];
    __shared__ __align__(16) uint8_t s_slot[LZD_THREADS * 16];
    __shared__ uint32_t s_scan[LZD_THREADS / kWave];

    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const uint32_t info = a.binfo[b];
    if (info & (BI_BAD | BI_SLOW)) return;
    const uint32_t nseq = info & BI_NSEQ;
    const uint64_t off = a.offs[b];
    const uint32_t S = a.sizes[b];
    const uint8_t *in = a.payload + off;
    const int64_t blk = b * (int64_t)a.block_bytes;
    const uint32_t len = (uint32_t)((a.nbytes - blk) < a.block_bytes ? (a.nbytes - blk) : a.block_bytes);
    const uint32_t *words = a.bitmap + (off >> 5) + b;
    const uint32_t nwords = (S + 31) >> 5;
    const uint32_t wpt = (nwords + LZD_THREADS - 1) / LZD_THREADS;
    uint8_t *slot = s_slot + t * 16;
    uint8_t *dstb = a.dst + blk;

    uint32_t out_carry = 0;
    for (uint32_t bs = 0; bs < nseq; bs += LZD_BATCH) {
        const uint32_t nb = (nseq - bs) < (uint32_t)LZD_BATCH ? (nseq - bs) : (uint32_t)LZD_BATCH;

        // (1) token positions of ranks [bs, bs + nb)
        const uint32_t w0 = t * wpt, w1 = (w0 + wpt) < nwords ? (w0 + wpt) : nwords;
        uint32_t cnt = 0;
        for (uint32_t w = w0; w < w1; ++w) cnt += __builtin_popcount(words[w]);
        uint32_t ntok;
        uint32_t r = block_excl_sum<LZD_THREADS / kWave>(cnt, s_scan, &ntok);
        for (uint32_t w = w0; w < w1 && r < bs + nb; ++w) {
            uint32_t x = words[w];
            while (x) {
                const uint32_t bit = __builtin_ctz(x);
                x &= x - 1;
                if (r >= bs && r < bs + nb) s_lit[r - bs] = (w << 5) + bit;
                ++r;
            }
        }
        __syncthreads();

        // (2) headers: thread t owns sequences [t*spt, (t+1)*spt)
        const uint32_t spt = (nb + LZD_THREADS - 1) / LZD_THREADS;
        const uint32_t k0 = t * spt, k1 = (k0 + spt) < nb ? (k0 + spt) : nb;
        uint32_t mysum = 0;
        for (uint32_t k = k0; k < k1; ++k) {
            const SeqHdr h = parse_seq(in, s_lit[k], S);
            s_lit[k] = h.lit;
            s_ll[k] = h.ll;
            s_mo[k] = (uint16_t)h.mo;
            s_out[k] = mysum;  // local offset for now
            mysum += h.len;
        }
        uint32_t btot;
        const uint32_t base = block_excl_sum<LZD_THREADS / kWave>(mysum, s_scan, &btot);
        for (uint32_t k = k0; k < k1; ++k) s_out[k] += out_carry + base;
        if (t == 0) s_out[nb] = out_carry + btot;
        __syncthreads();

        // (3) rebuild the output chunks of [lo, hi) and apply them
        const uint32_t lo = out_carry, hi = out_carry + btot;
        if (hi > lo) {
            for (uint32_t c = (lo >> 4) + t; c <= ((hi - 1) >> 4); c += LZD_THREADS) {
                const uint32_t q = c << 4;
                uint32_t p = q > lo ? q : lo;
                const uint32_t pend = (q + 16) < hi ? (q + 16) : hi;
                // largest k with s_out[k] <= p
                uint32_t kl = 0, kh = nb - 1;
                while (kl < kh) {
                    const uint32_t mid = (kl + kh + 1) >> 1;
                    if (s_out[mid] <= p) kl = mid;
                    else kh = mid - 1;
                }
                uint32_t k = kl;
                *reinterpret_cast<uint4 *>(slot) = make_uint4(0, 0, 0, 0);
                while (p < pend) {
                    while (s_out[k + 1] <= p) ++k;
                    const uint32_t sb = s_out[k], ll = s_ll[k], litend = sb + ll;
                    if (p < litend) {
                        const uint32_t e = pend < litend ? pend : litend;
                        const uint8_t *src = in + s_lit[k] + (p - sb);
                        for (; p < e; ++p, ++src) slot[p - q] = *src;
                    } else {
                        const uint32_t send = s_out[k + 1];
                        const uint32_t e = pend < send ? pend : send;
                        const uint32_t mo = s_mo[k];
                        // byte m of the match = literal (ll - mo + m % mo) of this sequence
                        const uint8_t *src = in + s_lit[k] + ll - mo;
                        if (mo == 1) {
                            const uint8_t v = *src;
                            if (v)
                                for (; p < e; ++p) slot[p - q] = v;
                            p = e;
                        } else {
                            for (; p < e; ++p) slot[p - q] = src[(p - litend) % mo];
                        }
                    }
                }
                const uint4 v = *reinterpret_cast<const uint4 *>(slot);
                const bool zero = (v.x | v.y | v.z | v.w) == 0u;
                if (a.mode == 1) {
                    if (zero) continue;
                    if (q + 16 <= len) {
                        uint4 d = *reinterpret_cast<const uint4 *>(dstb + q);
                        d.x ^= v.x; d.y ^= v.y; d.z ^= v.z; d.w ^= v.w;
                        *reinterpret_cast<uint4 *>(dstb + q) = d;
                    } else {
                        for (uint32_t x = q; x < len; ++x) dstb[x] ^= slot[x - q];
                    }
                } else {
                    if (q >= lo && q + 16 <= hi) {
                        *reinterpret_cast<uint4 *>(dstb + q) = v;
                    } else {
                        const uint32_t x0 = q > lo ? q : lo;
                        for (uint32_t x = x0; x < pend; ++x) dstb[x] = slot[x - q];
                    }
                }
            }
        }
        out_carry = hi;
        __syncthreads();
    }
}

// ---- K3 ----------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lz4_slow(Lz4DecArgs a) {
    __shared__ __align__(16) uint8_t s_dec[65536];
    __shared__ uint32_t s_h[5];
    const int t = threadIdx.x;
    uint32_t count = ld_agent32(&a.hdr->aux);
    if (count > a.nblocks) count = (uint32_t)a.nblocks;
    for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
        const int64_t b = a.slow_list[i];
        const uint64_t off = a.offs[b];
        const uint32_t S = a.sizes[b];
        const uint8_t *in = a.payload + off;
        const int64_t blk = b * (int64_t)a.block_bytes;
        const uint32_t len = (uint32_t)((a.nbytes - blk) < a.block_bytes ? (a.nbytes - blk) : a.block_bytes);
        uint32_t ip = 0, op = 0;
        while (true) {
            // the stream was fully validated by k_lz4_parse
            if (t == 0) {
                const SeqHdr h = parse_seq(in, ip, S);
                s_h[0] = h.lit;
                s_h[1] = h.ll;
                s_h[2] = h.mo;
                s_h[3] = h.next;
                s_h[4] = h.len - h.ll;
            }
            __syncthreads();
            const uint32_t lit = s_h[0], ll = s_h[1], mo = s_h[2], next = s_h[3], ml = s_h[4];
            for (uint32_t x = t; x < ll; x += 256) s_dec[op + x] = in[lit + x];
            __syncthreads();
            op += ll;
            if (mo == 0) break;
            // forward copy with overlap: byte x of the match repeats the mo bytes before it
            for (uint32_t x = t; x < ml; x += 256) s_dec[op + x] = s_dec[op - mo + (x % mo)];
            __syncthreads();
            op += ml;
            ip = next;
        }
        __syncthreads();
        for (uint32_t q = 16 * t; q < len; q += 16 * 256) {
            if (q + 16 <= len) {
                const uint4 v = *reinterpret_cast<const uint4 *>(s_dec + q);
                if (a.mode == 1) {
                    uint4 d = *reinterpret_cast<const uint4 *>(a.dst + blk + q);
                    d.x ^= v.x; d.y ^= v.y; d.z ^= v.z; d.w ^= v.w;
                    *reinterpret_cast<uint4 *>(a.dst + blk + q) = d;
                } else {
                    *reinterpret_cast<uint4 *>(a.dst + blk + q) = v;
                }
            } else {
                for (uint32_t x = q; x < len; ++x)
                    a.dst[blk + x] = a.mode == 1 ? (uint8_t)(a.dst[blk + x] ^ s_dec[x]) : s_dec[x];
            }
        }
        __syncthreads();
    }
    if (t == 0) {
        const uint32_t d = add_agent32(&a.hdr->aux2, 1u);
        if (d == gridDim.x - 1) {
            st_agent32(&a.hdr->aux, 0u);
            st_agent32(&a.hdr->aux2, 0u);
        }
    }
}

}  // namespace pulse

using namespace pulse;

namespace {
// The regions of a decode workspace are a function of its size alone, so the
// look-back status words of one call never overlap the per-block data another
// call of a different size left behind (a stale word must never carry a
// matching epoch tag).  Status: 1 word per KiB; block info and slow list:
// ws/8 bytes each; bitmap: the rest.
struct DecLayout {
    size_t status, binfo, slow, bitmap;
    size_t status_words, blocks, bitmap_words;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
DecLayout dec_layout(size_t ws) {
    DecLayout L;
    L.status = sizeof(WsHeader);
    L.status_words = ws >> 10;
    L.binfo = al256(L.status + 8 * L.status_words);
    L.blocks = ws >> 5;
    L.slow = al256(L.binfo + 4 * L.blocks);
    L.bitmap = al256(L.slow + 4 * L.blocks);
    L.bitmap_words = ws > L.bitmap ? (ws - L.bitmap) / 4 : 0;
    return L;
}
bool dec_fits(size_t ws, int64_t nblocks, int64_t payload_bytes) {
    const DecLayout L = dec_layout(ws);
    const size_t k1 = (size_t)(nblocks + 255) / 256;
    const size_t words = (size_t)(payload_bytes >> 5) + (size_t)nblocks + 2;
    return ws >= L.bitmap && k1 <= L.status_words && (size_t)nblocks <= L.blocks && words <= L.bitmap_words;
}
}  // namespace

extern "C" size_t pulse_lz4_decode_ws_bytes(int64_t nblocks, int64_t payload_bytes) {
    if (nblocks < 0 || payload_bytes < 0) return 0;
    const size_t words = (size_t)(payload_bytes >> 5) + (size_t)nblocks + 2;
    size_t ws = al256(4096 + 32 * (size_t)nblocks + (4 * words) * 4 / 3);
    while (!dec_fits(ws, nblocks, payload_bytes)) ws = al256(ws + ws / 8 + 256);
    return ws;
}

extern "C" int pulse_lz4_decode_ws_fits(size_t ws, int64_t nblocks, int64_t payload_bytes) {
    return dec_fits(ws, nblocks, payload_bytes) ? 1 : 0;
}

extern "C" int pulse_launch_lz4_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *offs,
                                       const uint32_t *sizes, int64_t nblocks, int32_t block_bytes,
                                       int64_t nbytes, void *dst, int32_t mode, uint32_t *d_status, void *ws,
                                       size_t ws_bytes, hipStream_t stream) {
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
    a.bitmap = reinterpret_cast<uint32_t *>(w + L.bitmap);
    const int64_t k1 = (nblocks + 255) / 256;
    a.k1_tiles = (uint32_t)k1;
    k_lz4_parse<<<dim3((unsigned)k1), dim3(256), 0, stream>>>(a);
    k_lz4_decode<<<dim3((unsigned)nblocks), dim3(LZD_THREADS), 0, stream>>>(a);
    const int64_t g3 = nblocks < 512 ? nblocks : 512;
    k_lz4_slow<<<dim3((unsigned)g3), dim3(256), 0, stream>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
