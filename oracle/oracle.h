/*
 * oracle.h -- plain, slow CPU oracle of the trainer->sampler weight-delta codec.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke entry
 * point and the bench's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never calls
 * it.  Every function is a straight loop over the definition it cites; nothing
 * is blocked, fused, vectorised or reordered.
 *
 * Sources (the pages this codec is defined by):
 *  [Jiang talk]    "Taking Reinforcement Learning Cross Datacenter -- Nan Jiang,
 *                  Modal" (transcript, timecodes given as mm:ss).
 *  [Jiang report]  the Korean written report of the same talk (section titles).
 *  [PULSE summary] gist.science technical summary of arXiv 2602.03839 "PULSE"
 *                  (sections "Osservazione Centrale", "1. PULSESync", ...).
 *  [Teleport]      "GPU weight teleportation syncs RL samplers in under 4 s with
 *                  0.23 s pauses" (Turkish write-up of the humansand.ai post;
 *                  sections "XOR masks", "Moving the pipeline onto GPUs").
 *  [Perplexity]    "Weight transfer for RL post-training in under 2 seconds"
 *                  (Polish translation; sections "Potok zadan", "Czysta separacja").
 * Facts not on the pages: the public LZ4 Block Format description [LZ4 spec],
 * the OCP 8-bit floating point spec, E4M3 [OCP FP8], IEEE-754 binary32.
 *
 * Status bits (OR-ed into *status; the caller clears it):
 *   ORACLE_CAPACITY 1  more entries / bytes than the capacity; counts stay exact
 *   ORACLE_BADINDEX 2  apply: entries with index >= n were skipped
 *   ORACLE_CORRUPT  4  lz4 decode: a malformed block; its destination untouched
 */
#ifndef SDC_ORACLE_H
#define SDC_ORACLE_H
#include <stdint.h>

#define ORACLE_CAPACITY 1u
#define ORACLE_BADINDEX 2u
#define ORACLE_CORRUPT 4u
#define ORACLE_PACK_GROUP 65536

#ifdef __cplusplus
extern "C" {
#endif

/* a1: nearest BF16 to an FP32 bit pattern, ties to even. */
uint16_t oracle_bf16_rne(uint32_t f32_bits);
void oracle_cast_bf16(const float *w, uint16_t *out, int64_t n);

/* a1+a2+a3: cast w_new, compare with b_old bitwise, emit the outputs that are
 * non-NULL: the new view, the XOR mask, and the (ascending index, new value)
 * patch with its exact count. */
void oracle_cast_diff(const float *w_new, const uint16_t *b_old, uint16_t *b_new,
                      uint16_t *xor_mask, int32_t *patch_idx, uint16_t *patch_val,
                      int64_t patch_cap, int64_t *count, uint32_t *status, int64_t n);

/* a3 on two existing BF16 views. */
void oracle_compact(const uint16_t *b_old, const uint16_t *b_new, int32_t *patch_idx,
                    uint16_t *patch_val, int64_t patch_cap, int64_t *count,
                    uint32_t *status, int64_t n);

/* a4: b[idx[k]] = val[k] for k < count; entries with idx outside [0, n) skipped. */
void oracle_apply_patch(uint16_t *b, int64_t n, const int32_t *patch_idx,
                        const uint16_t *patch_val, int64_t count, uint32_t *status);

/* a2/a6: dst ^= mask over nbytes bytes. */
void oracle_xor_apply(uint8_t *dst, const uint8_t *mask, int64_t nbytes);

/* a5: canonical "offset-1 run" LZ4 block encoding of one block of n bytes.
 * out must hold at least lz4 worst case (n + n/255 + 16) bytes.  Returns the
 * compressed size. */
int64_t oracle_lz4_encode_block(const uint8_t *src, int64_t n, uint8_t *out);

/* a5 over a buffer: independent blocks of block_bytes (last one short), each
 * encoded canonically, concatenated.  Encoded bytes are src[i] ^ src_xor[i]
 * when src_xor is non-NULL.  comp_sizes/comp_offsets get one entry per block,
 * *total the exact sum.  A block that does not fit entirely under payload_cap
 * is not written and sets ORACLE_CAPACITY. */
void oracle_lz4_encode_blocks(const uint8_t *src, const uint8_t *src_xor, int64_t nbytes,
                              int32_t block_bytes, uint8_t *payload, int64_t payload_cap,
                              uint32_t *comp_sizes, uint64_t *comp_offsets,
                              uint64_t *total, uint32_t *status);

/* a6: decode one LZ4 block of comp_size bytes that must expand to exactly
 * out_size bytes.  Returns 0 when well formed (out filled), -1 when malformed
 * (out contents unspecified). */
int oracle_lz4_decode_block(const uint8_t *in, int64_t comp_size, uint8_t *out,
                            int64_t out_size);

/* a6 over a payload: mode 0 stores the decoded bytes into dst, mode 1 XORs them
 * into dst.  A malformed block (including one whose bytes lie outside
 * [0, payload_bytes) or that starts before the end of an earlier block) leaves
 * its dst range untouched and sets ORACLE_CORRUPT. */
void oracle_lz4_decode_blocks(const uint8_t *payload, int64_t payload_bytes,
                              const uint64_t *comp_offsets, const uint32_t *comp_sizes,
                              int64_t nblocks, int32_t block_bytes, int64_t nbytes,
                              uint8_t *dst, int32_t mode, uint32_t *status);

/* a7: OCP E4M3 ("fn") code of an FP32 value: nearest finite value, ties to the
 * even code, magnitudes beyond the largest finite value (448) saturate. */
uint8_t oracle_e4m3_rne(float q);

/* a7: stack nsrc sources [rows_i, cols] along rows, then quantise each 128x128
 * block: amax, s = amax/448 (1 when amax == 0), code = e4m3(x / s).
 * srcs[i] + e*src_batch_stride[i] is source i of batch entry e.
 * codes: [batch][sum rows][cols]; scales: [batch][ceil(R/128)][ceil(cols/128)]. */
void oracle_fp8_block_quant(const uint16_t *const *srcs, const int64_t *src_rows,
                            int32_t nsrc, int64_t cols, int64_t batch,
                            const int64_t *src_batch_stride, uint8_t *codes, float *scales);

/* f1: FP8-view deltas.  Codes compared as bytes, scales as 32-bit patterns;
 * each changed position gives an ascending (index, new value) entry; counts
 * exact, entries beyond a capacity not written (ORACLE_CAPACITY). */
void oracle_fp8_delta(const uint8_t *codes_old, const uint8_t *codes_new, int64_t n_codes,
                      const float *scales_old, const float *scales_new, int64_t n_scales,
                      int32_t *code_idx, uint8_t *code_val, int64_t code_cap, int64_t *code_count,
                      int32_t *scale_idx, float *scale_val, int64_t scale_cap, int64_t *scale_count,
                      uint32_t *status);
/* f1: codes[code_idx[k]] = code_val[k], scales[scale_idx[k]] = scale_val[k]. */
void oracle_fp8_apply_delta(uint8_t *codes, int64_t n_codes, float *scales, int64_t n_scales,
                            const int32_t *code_idx, const uint8_t *code_val, int64_t code_count,
                            const int32_t *scale_idx, const float *scale_val, int64_t scale_count,
                            uint32_t *status);
/* f3: a = resid + delta; sent (index, a) and resid = 0 where
 * bf16(theta + a) != bf16(theta), else resid = a.  All float32.  Visible
 * entries beyond the capacity are counted but not sent: resid = a. */
void oracle_loco_gate(const float *theta, const float *delta, float *resid, int64_t n,
                      int32_t *idx, float *val, int64_t cap, int64_t *count, uint32_t *status);
/* f3: acc[idx[k]] += val[k] (float32) for k < count. */
void oracle_loco_accumulate(float *acc, int64_t n, const int32_t *idx, const float *val,
                            int64_t count, uint32_t *status);
/* f2: bytes of the packed form of a patch of `count` entries (whole groups). */
int64_t oracle_patch_packed_bytes(int64_t count);
/* f2: gaps and byte planes, ORACLE_PACK_GROUP entries per group (see oracle.c). */
void oracle_patch_pack(const int32_t *idx, const uint16_t *val, int64_t count, uint8_t *packed);
/* f2: inverse; 0, or -1 when an index would pass INT32_MAX. */
int oracle_patch_unpack(const uint8_t *packed, int64_t count, int32_t *idx, uint16_t *val);
/* f4: cast/diff/compact over a list of tensors, indices local to each tensor,
 * one entry stream; seg_offsets [nseg + 1].  b_new may be NULL (or hold NULLs). */
void oracle_cast_diff_segments(const float *const *w_new, const uint16_t *const *b_old,
                               uint16_t *const *b_new, const int64_t *n, int32_t nseg,
                               int32_t *idx, uint16_t *val, int64_t cap, int64_t *seg_offsets,
                               uint32_t *status);
/* f4: apply each tensor's slice of the stream to its view. */
void oracle_apply_patch_segments(uint16_t *const *views, const int64_t *n, int32_t nseg,
                                 const int32_t *idx, const uint16_t *val,
                                 const int64_t *seg_offsets, uint32_t *status);
#ifdef __cplusplus
}
#endif
#endif
