/*
 * oracle.c -- plain, slow CPU oracle of the trainer->sampler weight-delta codec.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke entry point
 * and the bench's CPU-baseline leg use it; the HIP library never does, and the
 * two share no code.  Built with plain gcc -O2, no intrinsics, no threads, no
 * FP contraction (see oracle/_build.py).  Source key in oracle.h.
 *
 * Parity status of each function (what pins it lives in tests/test_oracle_*.py):
 *   oracle_bf16_rne         pinned: worked values of the pages, torch's CPU cast,
 *                           textbook nearest-value in binary64.  NaN results are
 *                           our own reading (quiet bit set): parity unpinned.
 *   oracle_cast_diff/compact pinned: numpy flatnonzero, exhaustive tiny inputs.
 *   oracle_apply_patch      pinned: apply(old, patch) == new, version chains,
 *                           numpy's fancy assignment on entries in any order.
 *   oracle_lz4_encode_*     pinned: closed-form block sizes and bytes, an
 *                           independent decoder, brute force on tiny inputs.
 *   oracle_lz4_decode_*     pinned: spec-valid random streams with known output,
 *                           corrupt streams.
 *   oracle_e4m3_rne, oracle_fp8_block_quant
 *                           pinned: torch.float8_e4m3fn, nearest-of-set search,
 *                           closed forms for constant blocks, stacking invariant;
 *                           block by block against numpy's float32 division and
 *                           torch's E4M3 on ragged edge blocks, stacks whose
 *                           sources end inside a 128-row band, and batches read
 *                           at an expert stride larger than the stack.
 *   oracle_fp8_delta, oracle_fp8_apply_delta
 *                           pinned: numpy flatnonzero over the codes and the scale
 *                           bit patterns; apply(quant(old), delta) == quant(new).
 *   oracle_patch_pack, oracle_patch_unpack
 *                           pinned: numpy diff + little-endian byte views; round
 *                           trips; constant planes give 6 x 267 B (the closed form
 *                           of a constant 64 KiB block); index overflow rejected.
 *   oracle_cast_diff_segments, oracle_apply_patch_segments
 *                           pinned: torch's cast + numpy flatnonzero per tensor,
 *                           concatenated; apply over the list rebuilds every view.
 *   oracle_loco_gate, oracle_loco_accumulate
 *                           pinned: torch's float32 add and BF16 cast, the exact
 *                           conservation resid' + sent == resid + delta, closed
 *                           forms for constant updates near 1 (sent every 4th
 *                           round upward, every 2nd downward), numpy add.at.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* a1  FP32 -> BF16, round to nearest, ties to even.                         */
/* The served view is the master weight cast to the dtype the rollout engine  */
/* serves [Jiang talk, 10:49-10:56; Jiang report, "Sparse Patch ..."]; a value */
/* only changes once an update crosses the nearest rounding boundary, half a  */
/* BF16 ulp [Jiang talk, 07:24-08:07; PULSE summary, "Osservazione Centrale"]. */
/* ------------------------------------------------------------------------ */
uint16_t oracle_bf16_rne(uint32_t x)
{
    uint32_t hi = x >> 16;    /* BF16 pattern of x truncated toward zero      */
    uint32_t lo = x & 0xFFFFu; /* distance to it, in 2^-16 of one BF16 ulp     */

    if ((x & 0x7FFFFFFFu) > 0x7F800000u) /* NaN: keep sign and payload, quiet */
        return (uint16_t)(hi | 0x0040u);

    /* BF16 and FP32 share sign/exponent layout, so within one sign the bit
     * patterns are ordered like the magnitudes and hi+1 is the next BF16 away
     * from zero (the carry into the exponent gives the next binade, or Inf).
     * Nearest: above the midpoint go up; exactly at it pick the even one. */
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

void oracle_cast_bf16(const float *w, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bits;
        memcpy(&bits, &w[i], 4);
        out[i] = oracle_bf16_rne(bits);
    }
}

/* ------------------------------------------------------------------------ */
/* a2 + a3  bitwise compare of consecutive served versions and the sparse     */
/* patch of (index, new absolute value) [PULSE summary, "1. PULSESync" --     */
/* Processo / Ricostruzione; Jiang talk, 10:56-11:30 and 12:12-12:44].        */
/* ------------------------------------------------------------------------ */
static void compact_pair(const uint16_t *b_old, const uint16_t *b_new, int32_t *patch_idx,
                         uint16_t *patch_val, int64_t cap, int64_t *count,
                         uint32_t *status, int64_t n)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (b_old[i] != b_new[i]) { /* compared as 16-bit patterns */
            if (m < cap) {
                if (patch_idx) patch_idx[m] = (int32_t)i;
                if (patch_val) patch_val[m] = b_new[i]; /* absolute, not a difference */
            }
            ++m;
        }
    }
    if (m > cap && status) *status |= ORACLE_CAPACITY;
    if (count) *count = m;
}

void oracle_cast_diff(const float *w_new, const uint16_t *b_old, uint16_t *b_new,
                      uint16_t *xor_mask, int32_t *patch_idx, uint16_t *patch_val,
                      int64_t patch_cap, int64_t *count, uint32_t *status, int64_t n)
{
    uint16_t *cast = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
    oracle_cast_bf16(w_new, cast, n);
    if (b_new) memcpy(b_new, cast, (size_t)n * sizeof(uint16_t));
    if (b_old) {
        if (xor_mask)
            for (int64_t i = 0; i < n; ++i) xor_mask[i] = (uint16_t)(b_old[i] ^ cast[i]);
        if (patch_idx || patch_val || count)
            compact_pair(b_old, cast, patch_idx, patch_val, patch_cap, count, status, n);
    }
    free(cast);
}

void oracle_compact(const uint16_t *b_old, const uint16_t *b_new, int32_t *patch_idx,
                    uint16_t *patch_val, int64_t patch_cap, int64_t *count,
                    uint32_t *status, int64_t n)
{
    compact_pair(b_old, b_new, patch_idx, patch_val, patch_cap, count, status, n);
}

/* ------------------------------------------------------------------------ */
/* a4  selective override: the receiver writes the replacement bits at the    */
/* listed positions; no floating-point addition, hence no drift [Jiang talk,  */
/* 11:08-11:30; PULSE summary, "1. PULSESync" -- Ricostruzione].              */
/* ------------------------------------------------------------------------ */
void oracle_apply_patch(uint16_t *b, int64_t n, const int32_t *patch_idx,
                        const uint16_t *patch_val, int64_t count, uint32_t *status)
{
    for (int64_t k = 0; k < count; ++k) {
        int64_t i = patch_idx[k];
        if (i < 0 || i >= n) {
            if (status) *status |= ORACLE_BADINDEX;
            continue;
        }
        b[i] = patch_val[k];
    }
}

/* a2/a6: the sampler XORs the mask into its old weights [Teleport, "XOR masks"]. */
void oracle_xor_apply(uint8_t *dst, const uint8_t *mask, int64_t nbytes)
{
    for (int64_t i = 0; i < nbytes; ++i) dst[i] = (uint8_t)(dst[i] ^ mask[i]);
}

/* ------------------------------------------------------------------------ */
/* a5  LZ4 block encoding of the XOR mask.  The write-up picks LZ4 because it  */
/* codes long runs in few commands and RL masks are long zero runs [Teleport,  */
/* "Moving the pipeline onto GPUs"]; the byte format is the public [LZ4 spec]. */
/*                                                                            */
/* LZ4 encodings are not unique, so the encoding is fixed by a canonical      */
/* parse (our reading): cut the block b[0,n) into maximal runs of one byte     */
/* value [s,e).  Run r gives i=s+1, j=min(e,n-5), L=j-i; it qualifies when     */
/* L >= 4 and i <= n-12.  Each qualifying run, in order, becomes one sequence: */
/* literals b[a,i) (a = previous qualifying j, or 0), match offset 1, length L. */
/* A final sequence carries the literals b[a,n).                              */
/* ------------------------------------------------------------------------ */
static int64_t put_len_ext(uint8_t *out, int64_t o, int64_t v)
{
    /* v >= 15 was capped at 15 in the token nibble; the rest follows as 255s
     * and a final byte < 255 */
    int64_t rem = v - 15;
    while (rem >= 255) {
        out[o++] = 255;
        rem -= 255;
    }
    out[o++] = (uint8_t)rem;
    return o;
}

static int64_t put_sequence(uint8_t *out, int64_t o, const uint8_t *lit, int64_t ll,
                            int has_match, int64_t ml)
{
    uint8_t tok = (uint8_t)((ll >= 15 ? 15 : ll) << 4);
    if (has_match) tok |= (uint8_t)(ml - 4 >= 15 ? 15 : ml - 4);
    out[o++] = tok;
    if (ll >= 15) o = put_len_ext(out, o, ll);
    for (int64_t k = 0; k < ll; ++k) out[o++] = lit[k];
    if (has_match) {
        out[o++] = 1; /* offset 1, little endian */
        out[o++] = 0;
        if (ml - 4 >= 15) o = put_len_ext(out, o, ml - 4);
    }
    return o;
}

int64_t oracle_lz4_encode_block(const uint8_t *b, int64_t n, uint8_t *out)
{
    int64_t o = 0;
    int64_t a = 0; /* first byte not yet covered by an emitted sequence */
    int64_t s = 0;
    while (s < n) {
        int64_t e = s + 1;
        while (e < n && b[e] == b[s]) ++e; /* maximal run [s, e) */
        int64_t i = s + 1;
        int64_t j = e < n - 5 ? e : n - 5;
        if (j - i >= 4 && i <= n - 12) {
            o = put_sequence(out, o, b + a, i - a, 1, j - i);
            a = j;
        }
        s = e;
    }
    return put_sequence(out, o, b + a, n - a, 0, 0);
}

void oracle_lz4_encode_blocks(const uint8_t *src, const uint8_t *src_xor, int64_t nbytes,
                              int32_t block_bytes, uint8_t *payload, int64_t payload_cap,
                              uint32_t *comp_sizes, uint64_t *comp_offsets,
                              uint64_t *total, uint32_t *status)
{
    int64_t nb = (nbytes + block_bytes - 1) / block_bytes;
    uint8_t *blk = (uint8_t *)malloc((size_t)block_bytes);
    uint8_t *enc = (uint8_t *)malloc((size_t)block_bytes + (size_t)block_bytes / 255 + 64);
    uint64_t off = 0;
    for (int64_t bi = 0; bi < nb; ++bi) {
        int64_t base = bi * (int64_t)block_bytes;
        int64_t n = nbytes - base < block_bytes ? nbytes - base : block_bytes;
        for (int64_t k = 0; k < n; ++k)
            blk[k] = (uint8_t)(src[base + k] ^ (src_xor ? src_xor[base + k] : 0));
        int64_t sz = oracle_lz4_encode_block(blk, n, enc);
        comp_sizes[bi] = (uint32_t)sz;
        comp_offsets[bi] = off;
        if ((int64_t)off + sz <= payload_cap) {
            if (payload) memcpy(payload + off, enc, (size_t)sz);
        } else if (status) {
            *status |= ORACLE_CAPACITY;
        }
        off += (uint64_t)sz;
    }
    if (total) *total = off;
    free(blk);
    free(enc);
}

/* ------------------------------------------------------------------------ */
/* a6  LZ4 block decoding [LZ4 spec], validated before anything is written:   */
/* the sampler ends up with exactly the new weights [Teleport, "XOR masks"],  */
/* so a block that does not decode cleanly must not touch them.  Malformed:   */
/* a length running past the input, offset 0 or beyond the bytes produced so  */
/* far, output beyond out_size, or input ending anywhere but after a literal  */
/* run with exactly out_size bytes produced; over a payload also a block     */
/* outside [0, payload_bytes) or starting before the end of an earlier block  */
/* (our readings).                                                            */
/* ------------------------------------------------------------------------ */
static int read_len_ext(const uint8_t *in, int64_t comp_size, int64_t *ip, int64_t *len)
{
    for (;;) {
        if (*ip >= comp_size) return -1;
        uint8_t x = in[(*ip)++];
        *len += x;
        if (*len > ((int64_t)1 << 40)) return -1;
        if (x != 255) return 0;
    }
}

int oracle_lz4_decode_block(const uint8_t *in, int64_t comp_size, uint8_t *out,
                            int64_t out_size)
{
    int64_t ip = 0, op = 0;
    for (;;) {
        if (ip >= comp_size) return -1;
        uint8_t tok = in[ip++];
        int64_t ll = tok >> 4;
        if (ll == 15 && read_len_ext(in, comp_size, &ip, &ll)) return -1;
        if (ll > comp_size - ip || ll > out_size - op) return -1;
        for (int64_t k = 0; k < ll; ++k) out[op++] = in[ip++];
        if (ip == comp_size) return op == out_size ? 0 : -1; /* last sequence */
        if (comp_size - ip < 2) return -1;
        int64_t offset = (int64_t)in[ip] | ((int64_t)in[ip + 1] << 8);
        ip += 2;
        if (offset == 0 || offset > op) return -1;
        int64_t ml = (tok & 15) + 4;
        if ((tok & 15) == 15 && read_len_ext(in, comp_size, &ip, &ml)) return -1;
        if (ml > out_size - op) return -1;
        for (int64_t k = 0; k < ml; ++k, ++op) out[op] = out[op - offset]; /* forward, overlap replicates */
    }
}

void oracle_lz4_decode_blocks(const uint8_t *payload, int64_t payload_bytes,
                              const uint64_t *comp_offsets, const uint32_t *comp_sizes,
                              int64_t nblocks, int32_t block_bytes, int64_t nbytes,
                              uint8_t *dst, int32_t mode, uint32_t *status)
{
    uint8_t *blk = (uint8_t *)malloc((size_t)block_bytes);
    uint64_t end_so_far = 0; /* furthest end of any earlier block in the payload */
    for (int64_t bi = 0; bi < nblocks; ++bi) {
        int64_t base = bi * (int64_t)block_bytes;
        if (base >= nbytes) break;
        int64_t n = nbytes - base < block_bytes ? nbytes - base : block_bytes;
        uint64_t off = comp_offsets[bi];
        uint64_t sz = comp_sizes[bi];
        uint64_t end = off + sz < off ? UINT64_MAX : off + sz;
        /* the payload is the blocks' encodings end to end in block order, the
         * offsets being the exclusive scan of the sizes; a table in which a
         * block starts before the end of an earlier one describes no such
         * payload, and the block is malformed (our reading of that layout) */
        int bad = off > (uint64_t)payload_bytes || sz > (uint64_t)payload_bytes - off ||
                  (bi > 0 && off < end_so_far);
        if (end > end_so_far) end_so_far = end;
        if (!bad) bad = oracle_lz4_decode_block(payload + off, (int64_t)sz, blk, n) != 0;
        if (bad) {
            if (status) *status |= ORACLE_CORRUPT;
            continue;
        }
        for (int64_t k = 0; k < n; ++k)
            dst[base + k] = mode ? (uint8_t)(dst[base + k] ^ blk[k]) : blk[k];
    }
    free(blk);
}

/* ------------------------------------------------------------------------ */
/* a7  FP8 serving: projection fusion then quantisation [Perplexity, "Potok   */
/* zadan" -- preparing parameters: full weight, projection fusion, quantise]. */
/* Format per [OCP FP8] E4M3 "fn": bias 7, largest finite 448, no Inf,        */
/* subnormals k * 2^-9.  Block shape, scale rule and rounding are readings.   */
/* ------------------------------------------------------------------------ */
uint8_t oracle_e4m3_rne(float q)
{
    uint32_t bits;
    memcpy(&bits, &q, 4);
    uint8_t sign = (uint8_t)((bits >> 24) & 0x80u);
    if (isnan(q)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)q);
    if (a == 0.0) return sign;                     /* +0 -> 0x00, -0 -> 0x80 */
    if (a >= 448.0) return (uint8_t)(sign | 0x7E); /* nearest or saturated */

    /* spacing of E4M3 values around a: 2^-9 below 2^-6, else 2^(e-3) */
    int e;
    frexp(a, &e);       /* a = f * 2^e, f in [0.5, 1) */
    int exp2 = e - 1;   /* a in [2^exp2, 2^(exp2+1)) */
    double step = exp2 < -6 ? ldexp(1.0, -9) : ldexp(1.0, exp2 - 3);
    double k = a / step; /* exact: step is a power of two */
    double fl = floor(k);
    double frac = k - fl;
    int64_t kk = (int64_t)fl;
    if (frac > 0.5 || (frac == 0.5 && (kk & 1))) kk += 1;

    int code;
    if (exp2 < -6) {
        code = (int)kk; /* subnormal codes 0..8; 8 is the smallest normal */
    } else {
        /* value = kk * 2^(exp2-3) with kk in [8, 16]; code = (E << 3) | m,
         * E = exp2 + 7, m = kk - 8 (kk == 16 lands on the next binade) */
        code = (exp2 + 7) * 8 + (int)(kk - 8);
    }
    if (code > 0x7E) code = 0x7E;
    return (uint8_t)(sign | code);
}

static float bf16_to_float(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

void oracle_fp8_block_quant(const uint16_t *const *srcs, const int64_t *src_rows,
                            int32_t nsrc, int64_t cols, int64_t batch,
                            const int64_t *src_batch_stride, uint8_t *codes, float *scales)
{
    int64_t R = 0;
    for (int32_t i = 0; i < nsrc; ++i) R += src_rows[i];
    int64_t nbr = (R + 127) / 128, nbc = (cols + 127) / 128;

    /* the stacked matrix, built explicitly: [src0; src1; ...] along rows */
    uint16_t *stk = (uint16_t *)malloc((size_t)(R > 0 ? R : 1) * (size_t)(cols > 0 ? cols : 1) * 2);
    for (int64_t e = 0; e < batch; ++e) {
        int64_t r0 = 0;
        for (int32_t i = 0; i < nsrc; ++i) {
            const uint16_t *s = srcs[i] + (src_batch_stride ? e * src_batch_stride[i] : 0);
            memcpy(stk + r0 * cols, s, (size_t)(src_rows[i] * cols) * 2);
            r0 += src_rows[i];
        }
        uint8_t *ce = codes + e * R * cols;
        float *se = scales + e * nbr * nbc;
        for (int64_t br = 0; br < nbr; ++br) {
            for (int64_t bc = 0; bc < nbc; ++bc) {
                int64_t rlo = br * 128, rhi = rlo + 128 < R ? rlo + 128 : R;
                int64_t clo = bc * 128, chi = clo + 128 < cols ? clo + 128 : cols;
                float amax = 0.0f;
                for (int64_t r = rlo; r < rhi; ++r)
                    for (int64_t c = clo; c < chi; ++c) {
                        float v = fabsf(bf16_to_float(stk[r * cols + c]));
                        if (v > amax) amax = v;
                    }
                float s = amax == 0.0f ? 1.0f : amax / 448.0f;
                se[br * nbc + bc] = s;
                for (int64_t r = rlo; r < rhi; ++r)
                    for (int64_t c = clo; c < chi; ++c) {
                        float q = bf16_to_float(stk[r * cols + c]) / s; /* IEEE division */
                        ce[r * cols + c] = oracle_e4m3_rne(q);
                    }
            }
        }
    }
    free(stk);
}

/* ------------------------------------------------------------------------ */
/* f1  deltas of the FP8 served view.  When the rollout engine serves FP8,    */
/* the view that must match bit for bit is the quantised one, and its coarser */
/* cells change fewer values per step [Jiang talk, 13:06-14:40; PULSE summary,*/
/* "Potenziale Futuro"].  Two quantised versions (codes and per-block scales) */
/* are compared bitwise, exactly like the BF16 views; each changed position   */
/* becomes an (index, new absolute value) entry, ascending.                   */
/* ------------------------------------------------------------------------ */
void oracle_fp8_delta(const uint8_t *codes_old, const uint8_t *codes_new, int64_t n_codes,
                      const float *scales_old, const float *scales_new, int64_t n_scales,
                      int32_t *code_idx, uint8_t *code_val, int64_t code_cap, int64_t *code_count,
                      int32_t *scale_idx, float *scale_val, int64_t scale_cap, int64_t *scale_count,
                      uint32_t *status)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n_codes; ++i) {
        if (codes_old[i] != codes_new[i]) {
            if (m < code_cap) {
                code_idx[m] = (int32_t)i;
                code_val[m] = codes_new[i];
            }
            ++m;
        }
    }
    if (m > code_cap && status) *status |= ORACLE_CAPACITY;
    *code_count = m;

    m = 0;
    for (int64_t i = 0; i < n_scales; ++i) {
        uint32_t a, b; /* compared as 32-bit patterns */
        memcpy(&a, &scales_old[i], 4);
        memcpy(&b, &scales_new[i], 4);
        if (a != b) {
            if (m < scale_cap) {
                scale_idx[m] = (int32_t)i;
                scale_val[m] = scales_new[i];
            }
            ++m;
        }
    }
    if (m > scale_cap && status) *status |= ORACLE_CAPACITY;
    *scale_count = m;
}

void oracle_fp8_apply_delta(uint8_t *codes, int64_t n_codes, float *scales, int64_t n_scales,
                            const int32_t *code_idx, const uint8_t *code_val, int64_t code_count,
                            const int32_t *scale_idx, const float *scale_val, int64_t scale_count,
                            uint32_t *status)
{
    for (int64_t k = 0; k < code_count; ++k) {
        int64_t i = code_idx[k];
        if (i < 0 || i >= n_codes) {
            if (status) *status |= ORACLE_BADINDEX;
            continue;
        }
        codes[i] = code_val[k];
    }
    for (int64_t k = 0; k < scale_count; ++k) {
        int64_t i = scale_idx[k];
        if (i < 0 || i >= n_scales) {
            if (status) *status |= ORACLE_BADINDEX;
            continue;
        }
        scales[i] = scale_val[k];
    }
}

/* ------------------------------------------------------------------------ */
/* f3  PULSELoCo: the compute-visibility gate on FP32 pseudo-gradients with   */
/* an FP32 error-feedback buffer [PULSE summary, "2. PULSELoCo" -- Processo]. */
/* A worker's pseudo-gradient is its parameter update over H local steps;     */
/* added to what was held back before, an entry is sent only if applying it  */
/* to the shared checkpoint would change that entry's BF16 view; otherwise it */
/* stays in the buffer and is looked at again next round.                     */
/* ------------------------------------------------------------------------ */
void oracle_loco_gate(const float *theta, const float *delta, float *resid, int64_t n,
                      int32_t *idx, float *val, int64_t cap, int64_t *count, uint32_t *status)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        float a = resid[i] + delta[i];   /* accumulated update, FP32 */
        float moved = theta[i] + a;      /* the checkpoint entry after it */
        uint32_t tb, mb;
        memcpy(&tb, &theta[i], 4);
        memcpy(&mb, &moved, 4);
        if (oracle_bf16_rne(mb) != oracle_bf16_rne(tb)) { /* visible: send it */
            if (m < cap) {
                idx[m] = (int32_t)i;
                val[m] = a;
                resid[i] = 0.0f;
            } else {
                resid[i] = a; /* no room to send it: it is not sent, so it stays */
            }
            ++m;
        } else {
            resid[i] = a; /* held back for the next round */
        }
    }
    if (m > cap && status) *status |= ORACLE_CAPACITY;
    *count = m;
}

/* The receiving trainer sums the workers' sparse updates: acc[idx[k]] += val[k]. */
void oracle_loco_accumulate(float *acc, int64_t n, const int32_t *idx, const float *val,
                            int64_t count, uint32_t *status)
{
    for (int64_t k = 0; k < count; ++k) {
        int64_t i = idx[k];
        if (i < 0 || i >= n) {
            if (status) *status |= ORACLE_BADINDEX;
            continue;
        }
        acc[i] = acc[i] + val[k];
    }
}

/* ------------------------------------------------------------------------ */
/* f2  compression of the patch stream.  The sparse patches are compressed    */
/* further with a generic lossless codec [PULSE summary, "1. PULSESync" --    */
/* Compressione].  Reading: the codec is this codec's LZ4 block format (the   */
/* canonical parse, 64 KiB blocks), and the patch is first put in a form whose */
/* redundancy a run-based parse can see: each index becomes its gap to the    */
/* previous one, gap = idx[k] - idx[k-1] - 1 (idx[-1] = -1), and every group   */
/* of ORACLE_PACK_GROUP entries is laid out as six byte planes (gap bytes 0-3, */
/* value bytes 0-1, little-endian), each plane ORACLE_PACK_GROUP bytes long;  */
/* entries past the count in the last group are zero.                         */
/* ------------------------------------------------------------------------ */
int64_t oracle_patch_packed_bytes(int64_t count)
{
    return (count + ORACLE_PACK_GROUP - 1) / ORACLE_PACK_GROUP * 6 * ORACLE_PACK_GROUP;
}

void oracle_patch_pack(const int32_t *idx, const uint16_t *val, int64_t count, uint8_t *packed)
{
    const int64_t G = ORACLE_PACK_GROUP;
    int64_t groups = (count + G - 1) / G;
    for (int64_t g = 0; g < groups; ++g) {
        uint8_t *base = packed + g * 6 * G;
        for (int64_t j = 0; j < G; ++j) {
            int64_t k = g * G + j;
            uint32_t gap = 0;
            uint16_t v = 0;
            if (k < count) {
                int64_t prev = k > 0 ? (int64_t)idx[k - 1] : -1;
                gap = (uint32_t)((int64_t)idx[k] - prev - 1);
                v = val[k];
            }
            for (int p = 0; p < 4; ++p) base[p * G + j] = (uint8_t)(gap >> (8 * p));
            base[4 * G + j] = (uint8_t)(v & 0xFFu);
            base[5 * G + j] = (uint8_t)(v >> 8);
        }
    }
}

/* Inverse of oracle_patch_pack: idx[k] = idx[k-1] + 1 + gap.  Returns 0, or -1
 * when an index would pass INT32_MAX (such data cannot come from a pack). */
int oracle_patch_unpack(const uint8_t *packed, int64_t count, int32_t *idx, uint16_t *val)
{
    const int64_t G = ORACLE_PACK_GROUP;
    int64_t prev = -1;
    for (int64_t k = 0; k < count; ++k) {
        const uint8_t *base = packed + (k / G) * 6 * G;
        int64_t j = k % G;
        uint32_t gap = 0;
        for (int p = 0; p < 4; ++p) gap |= (uint32_t)base[p * G + j] << (8 * p);
        int64_t i = prev + 1 + (int64_t)gap;
        if (i > 2147483647LL) return -1;
        idx[k] = (int32_t)i;
        val[k] = (uint16_t)(base[4 * G + j] | (base[5 * G + j] << 8));
        prev = i;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* f4  one call over a list of tensors.  The tiling and address-mapping       */
/* metadata is prepared on the CPU so that one kernel launch covers the whole */
/* model [Teleport, "Moving the pipeline onto GPUs"].  What it computes is    */
/* exactly the per-tensor rows a1-a4: for each tensor in list order, the cast */
/* / diff / compaction with indices local to the tensor; the entries of all   */
/* tensors form one stream, seg_offsets[s] being tensor s's first entry and   */
/* seg_offsets[nseg] the total.                                               */
/* ------------------------------------------------------------------------ */
void oracle_cast_diff_segments(const float *const *w_new, const uint16_t *const *b_old,
                               uint16_t *const *b_new, const int64_t *n, int32_t nseg,
                               int32_t *idx, uint16_t *val, int64_t cap, int64_t *seg_offsets,
                               uint32_t *status)
{
    int64_t m = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        seg_offsets[s] = m;
        for (int64_t i = 0; i < n[s]; ++i) {
            uint32_t bits;
            memcpy(&bits, &w_new[s][i], 4);
            uint16_t v = oracle_bf16_rne(bits);
            if (b_new && b_new[s]) b_new[s][i] = v;
            if (v != b_old[s][i]) {
                if (m < cap) {
                    idx[m] = (int32_t)i; /* local to the tensor */
                    val[m] = v;
                }
                ++m;
            }
        }
    }
    seg_offsets[nseg] = m;
    if (m > cap && status) *status |= ORACLE_CAPACITY;
}

void oracle_apply_patch_segments(uint16_t *const *views, const int64_t *n, int32_t nseg,
                                 const int32_t *idx, const uint16_t *val,
                                 const int64_t *seg_offsets, uint32_t *status)
{
    for (int32_t s = 0; s < nseg; ++s)
        oracle_apply_patch(views[s], n[s], idx + seg_offsets[s], val + seg_offsets[s],
                           seg_offsets[s + 1] - seg_offsets[s], status);
}

