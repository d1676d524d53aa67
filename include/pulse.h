/*
 * pulse.h -- C ABI of the MI355X (gfx950) trainer->sampler weight-delta codec.
 *
 * Sender (trainer): cast FP32 master weights to the served BF16 view, compare
 * it bitwise with the previous served view, and ship either sparse patches of
 * (index, new absolute value) or an LZ4-block-encoded XOR mask.  Receiver
 * (sampler): scatter the patches, or decode the mask and XOR it in place,
 * rebuilding the new BF16 view bit for bit; optionally stack q/k/v or
 * gate/up and quantise to FP8-E4M3 per 128x128 block for an FP8 sampler.
 *
 * Sources cited below:
 *  [Jiang talk]    "Taking Reinforcement Learning Cross Datacenter -- Nan Jiang,
 *                  Modal", talk transcript (timecodes mm:ss).
 *  [PULSE summary] gist.science technical summary of arXiv 2602.03839 (PULSE),
 *                  section "1. PULSESync" (Processo / Ricostruzione / Compressione).
 *  [Teleport]      Turkish write-up of the humansand.ai "GPU weight teleportation"
 *                  post, sections "XOR masks", "Moving the pipeline onto GPUs".
 *  [Perplexity]    "Weight transfer for RL post-training in under 2 seconds",
 *                  sections "Potok zadan", "Kontrola uzycia pamieci GPU",
 *                  "Czysta separacja".
 *  The LZ4 byte format is the public LZ4 Block Format description; FP8 is OCP
 *  8-bit floating point E4M3 ("fn": bias 7, max 448, no Inf).
 *
 * Conventions (all entry points):
 *  - Pointers are DEVICE pointers unless marked (host).  Every call only
 *    enqueues work on `stream` (NULL = the null stream) and returns; results
 *    written to device memory are valid once the stream has reached them.
 *  - The caller owns every buffer.  The library never allocates device memory;
 *    calls that need scratch take a caller-provided workspace (the pages' cap on
 *    in-flight temporary GPU memory, [Perplexity] "Kontrola uzycia pamieci GPU").
 *  - Return value: PULSE_OK, or a negative PULSE_E* code for argument errors
 *    (nothing was enqueued) or a failed launch (PULSE_EHIP).
 *  - Data-dependent conditions are reported in a device status word: the
 *    PULSE_DS_* bits are OR-ed into *d_status; no call ever clears it, the
 *    caller zeroes it before the calls it wants to observe.
 *  - Dense buffers (weights, views, masks, LZ4 sources/destinations, FP8
 *    sources) must be 16-byte aligned (PULSE_EALIGN otherwise).
 *  - Calls that share a workspace must be ordered (same stream, or joined by
 *    events); concurrent calls on one workspace race.
 *  - One component per call, each testable in isolation ([Perplexity],
 *    "Czysta separacja").
 */
#ifndef PULSE_H
#define PULSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------- */
#define PULSE_OK 0
#define PULSE_EINVAL (-1)     /* NULL required pointer, bad mode/size/shape     */
#define PULSE_EALIGN (-2)     /* a dense buffer is not 16-byte aligned          */
#define PULSE_ERANGE (-3)     /* element count beyond int32 indices (2^31 - 1)   */
#define PULSE_EWORKSPACE (-4) /* workspace NULL or smaller than required        */
#define PULSE_EHIP (-5)       /* the kernel launch failed                       */

/* ---- device status bits (OR-ed into *d_status) ----------------------------- */
#define PULSE_DS_CAPACITY 0x1u /* more patch entries / payload bytes than the
                                  capacity; counts/totals stay exact, entries
                                  or whole blocks beyond the capacity are not
                                  written                                    */
#define PULSE_DS_BADINDEX 0x2u /* apply: entries with index >= n were skipped  */
#define PULSE_DS_CORRUPT 0x4u  /* lz4 decode: >= 1 malformed block; the dst
                                  range of such a block is left untouched    */
#define PULSE_DS_WORKSPACE 0x8u /* the workspace state was inconsistent (never
                                  initialised, shared between ops, or used by
                                  overlapping calls); this call's outputs are
                                  invalid, but the call still terminates;
                                  re-initialise the workspace               */
#define PULSE_DS_BADSEGMENT 0x10u /* a list call met a segment whose table entry
                                  breaks its preconditions (size, alignment,
                                  tile numbering, b_new presence); nothing
                                  was written for its tiles                 */

/* ---- workspaces ------------------------------------------------------------ */
#define PULSE_OP_CAST_DIFF 1  /* n = element count                               */
#define PULSE_OP_COMPACT 2    /* n = element count                               */
#define PULSE_OP_LZ4_ENCODE 3 /* n = source bytes, aux = block_bytes              */
#define PULSE_OP_LZ4_DECODE 4 /* n = number of blocks, aux = payload bytes         */
#define PULSE_OP_FP8_DELTA 5  /* n = max(code count, scale count)                 */
#define PULSE_OP_LOCO_GATE 6  /* n = element count                               */
#define PULSE_OP_PATCH_UNPACK 7 /* n = patch entries                            */
#define PULSE_OP_CAST_DIFF_SEGMENTS 8 /* n = tile count (pulse_segment_tiles)    */
#define PULSE_OP_CAST_DIFF_LZ4 9 /* n = element count, aux = block_bytes           */
#define PULSE_OP_APPLY_QUANT 10 /* n = element count of the view (segment index)   */

/* Bytes of workspace the op needs for the given size (0 if it needs none).
 * A workspace serves any number of calls of the op it was sized for, of any
 * size up to the one it was sized for; it must not be shared between
 * different ops (cast_diff and compact count as one op).  Its look-back
 * status words live at offsets that depend only on the workspace size, so a
 * call never reads another call's per-block data as status. */
size_t pulse_workspace_bytes(int op, int64_t n, int64_t aux);

/* Zero a workspace before its first use.  After that each call leaves it
 * ready for the next one (it carries a per-call epoch so the status words of
 * earlier calls are never mistaken for the current call's), so it is called
 * once per allocation, not per call. */
int pulse_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Human-readable name of a return code (static string). */
const char *pulse_status_string(int code);

/* Library version, "major.minor.patch" (static string). */
const char *pulse_version(void);

/* ---- a1 + a2 + a3: cast, diff, compaction ----------------------------------
 * The served view is the master weight cast to BF16 with round-to-nearest-
 * even ([Jiang talk] 10:49-10:56; a value only changes once an update crosses
 * half a BF16 ulp, 07:24-08:07); versions are compared bitwise and the patch
 * holds the changed positions and their new absolute BF16 bits ([PULSE
 * summary] "1. PULSESync", Processo/Ricostruzione; [Jiang talk] 12:12-12:44).
 *
 *   w_new      [n] float32 master weights (read).
 *   b_old      [n] previous BF16 view (read), or NULL: pure cast (then xor_mask,
 *              patch_idx, patch_val, d_count must be NULL).
 *   b_new      [n] cast result (written), or NULL.  May equal b_old (in-place
 *              update of the sender's view).
 *   xor_mask   [n] b_old ^ b_new (written), or NULL.
 *   patch_idx  [patch_cap] int32 positions of the changed elements in strictly
 *              ascending order (written), or NULL together with patch_val and
 *              d_count.
 *   patch_val  [patch_cap] new BF16 bits at those positions (written).
 *   patch_cap  capacity of patch_idx/patch_val (>= 0).
 *   d_count    (device int64) exact number of changed elements (written).
 *   d_status   (device uint32) PULSE_DS_CAPACITY when count > patch_cap; the
 *              first patch_cap entries are still written.  May be NULL when no
 *              patch is requested.
 *   n          element count; with a patch, n <= 2^31 - 1 (PULSE_ERANGE).
 *   ws         workspace of pulse_workspace_bytes(PULSE_OP_CAST_DIFF, n, 0)
 *              bytes when a patch is requested; ignored otherwise.
 * NaN inputs give a quiet NaN with the input's sign and top payload bits.
 */
int pulse_cast_diff(const float *w_new, const uint16_t *b_old, uint16_t *b_new,
                    uint16_t *xor_mask, int32_t *patch_idx, uint16_t *patch_val,
                    int64_t patch_cap, int64_t *d_count, uint32_t *d_status, int64_t n,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- a3 on two existing BF16 views ----------------------------------------
 * Same patch as pulse_cast_diff, with the new view given directly.
 *   b_old, b_new [n] BF16 views (read).  Other arguments as above. */
int pulse_compact(const uint16_t *b_old, const uint16_t *b_new, int32_t *patch_idx,
                  uint16_t *patch_val, int64_t patch_cap, int64_t *d_count,
                  uint32_t *d_status, int64_t n, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* ---- a1 + a2 + a3 + a5 in one pass ----------------------------------------
 * The sender's whole encode in one launch: exactly the results of
 *   pulse_cast_diff(w_new, b_old, b_new, NULL, patch_idx, patch_val, patch_cap,
 *                   d_count, d_status, n, ...)
 * followed by
 *   lz4_encode_blocks(b_old, b_new, 2 n, block_bytes, payload, payload_cap,
 *                     comp_sizes, comp_offsets, d_total, d_status, ...),
 * i.e. the served view cast from the masters ([Jiang talk] 10:49-10:56), the
 * patch of changed elements with their new absolute values ([PULSE summary]
 * "1. PULSESync") and the LZ4 blocks of the XOR mask old ^ new ([Teleport]
 * "XOR masks", "Moving the pipeline onto GPUs"), with the mask kept on chip and
 * each view read once.  Where the separate calls would run two passes over
 * the views, this runs one.
 *   w_new      [n] float32 masters (read), 16-byte aligned.
 *   b_old      [n] previous BF16 view (read), 16-byte aligned.
 *   b_new      [n] new BF16 view (written), 16-byte aligned, or NULL; it may
 *              be b_old itself (the view is updated in place).
 *   patch_idx, patch_val, d_count  the patch as for pulse_cast_diff, or all
 *              three NULL (mask blocks only).
 *   tile_first [ceil(n/16384) + 1] int64 (written) or NULL (NULL without a
 *              patch): the patch's tile index, as pulse_patch_tiles writes it;
 *              the pass knows every tile's place and writes it at no cost.
 *   block_bytes, payload .. d_total  as for lz4_encode_blocks, over the 2 n
 *              bytes of the mask.
 *   d_status   PULSE_DS_CAPACITY when the patch or the payload exceeds its
 *              capacity (counts and totals stay exact).
 *   ws         pulse_workspace_bytes(PULSE_OP_CAST_DIFF_LZ4, n, block_bytes).
 * n >= 1, and n <= 2^31 - 1 when a patch is asked for. */
int pulse_cast_diff_lz4(const float *w_new, const uint16_t *b_old, uint16_t *b_new,
                        int32_t *patch_idx, uint16_t *patch_val, int64_t patch_cap,
                        int64_t *d_count, int64_t *tile_first, int64_t n, int32_t block_bytes,
                        uint8_t *payload,
                        int64_t payload_cap, uint32_t *comp_sizes, uint64_t *comp_offsets,
                        uint64_t *d_total, uint32_t *d_status, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* ---- the same pass without a workspace argument ----------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pulse_cast_diff_lz4 with every argument but ws / ws_bytes, its results
 * identical.  Its scratch (look-back words) is a static array of
 * PULSE_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the
 * process ends; the call allocates nothing.  The array holds the workspace
 * of up to 262144 mask blocks, so every n <= 2^31 - 1 at every block size
 * fits; a call that needs more returns PULSE_ERANGE before enqueuing
 * anything.  Every call on a GPU shares that GPU's array: calls that overlap
 * on one GPU (concurrent streams, threads) race and must be ordered by the
 * caller.  The first call on a device also clears the array, with a fill
 * kernel on `stream` ahead of its own kernels.  PULSE_EHIP when the array's
 * address cannot be obtained. */
#define PULSE_NOALLOC_SCRATCH_BYTES (256 + 2 * 262144 * 8)
int pulse_cast_diff_lz4_noalloc(const float *w_new, const uint16_t *b_old, uint16_t *b_new,
                                int32_t *patch_idx, uint16_t *patch_val, int64_t patch_cap,
                                int64_t *d_count, int64_t *tile_first, int64_t n,
                                int32_t block_bytes, uint8_t *payload, int64_t payload_cap,
                                uint32_t *comp_sizes, uint64_t *comp_offsets, uint64_t *d_total,
                                uint32_t *d_status, hipStream_t stream);

/* ---- a4: patch scatter-apply ---------------------------------------------
 * Selective override: b[patch_idx[k]] = patch_val[k] for k < count, bit-level
 * writes with no floating-point addition ([Jiang talk] 11:08-11:30; [PULSE
 * summary] "1. PULSESync", Ricostruzione); applied in sequence the patches of
 * consecutive versions bring a lagging copy up to date (16:52-16:58).
 *   b          [n] BF16 view, updated in place; n <= 2^31 - 1 (PULSE_ERANGE).
 *   patch_idx, patch_val  the patch (indices unique, as produced above).
 *   d_count    (device) number of entries; count = min(*d_count, max_count).
 *   max_count  (host) bound used to size the launch, e.g. the patch capacity.
 *   d_status   PULSE_DS_BADINDEX when an index lies outside [0, n) (skipped).
 * The count is read on the device, so encode -> apply needs no host sync. */
int pulse_apply_patch(uint16_t *b, int64_t n, const int32_t *patch_idx,
                      const uint16_t *patch_val, const int64_t *d_count, int64_t max_count,
                      uint32_t *d_status, hipStream_t stream);

/* ---- a4 with the patch's tile index ---------------------------------------
 * The tile index of an ascending patch: tile_first[t] = the first entry whose
 * index is >= 16384 t, for t = 0 .. ntiles (ntiles = ceil(n / 16384);
 * tile_first[ntiles] = count).  A small companion of the patch (8 bytes per
 * 32 KiB of view) with which the receiver finds each tile's entries at once.
 *   patch_idx  [count] ascending positions (read); d_count as for apply,
 *              count = min(*d_count, max_count).
 *   tile_first [ntiles + 1] int64 (written). */
int pulse_patch_tiles(const int32_t *patch_idx, const int64_t *d_count, int64_t max_count,
                      int64_t n, int64_t *tile_first, hipStream_t stream);

/* The same result as pulse_apply_patch, for a patch with its tile index
 * (pulse_patch_tiles or pulse_cast_diff_lz4): every 16384-element tile of b is
 * updated by one workgroup; a tile holding 1024 or more entries is read
 * whole, patched on chip and written back whole (no partially written lines),
 * a sparser one takes the entries' 2-byte stores.
 *   b          [n] BF16 view, 16-byte aligned, updated in place.
 *   tile_first the patch's tile index (read); entries are read only in
 *              [0, max_count).
 *   d_status   PULSE_DS_BADINDEX for an entry outside its tile (an index
 *              outside [0, n), or a tile index that does not fit the patch):
 *              such entries are skipped and no element outside a tile's own
 *              range is written. */
int pulse_apply_patch_tiled(uint16_t *b, int64_t n, const int32_t *patch_idx,
                            const uint16_t *patch_val, const int64_t *tile_first, int64_t max_count,
                            uint32_t *d_status, hipStream_t stream);

/* ---- a2/a6: dense XOR apply ------------------------------------------------
 * dst ^= mask over nbytes bytes: the sampler XORs the same-size mask into its
 * old weights and obtains the new ones, whatever the dtype ([Teleport] "XOR
 * masks").  dst and mask 16-byte aligned; nbytes any value >= 0. */
int xor_mask_apply(void *dst, const void *mask, int64_t nbytes, hipStream_t stream);

/* ---- a5: LZ4 block encode of a mask ---------------------------------------
 * The mask (mostly zero) is cut into independent blocks of block_bytes bytes
 * (the last one short) and each block is LZ4-encoded with the canonical
 * "offset-1 run" parse: every maximal run of one byte value [s, e) with
 * i = s+1, j = min(e, n-5), j-i >= 4 and i <= n-12 becomes one sequence
 * (literals since the previous such run, then a match of offset 1 and length
 * j-i); the rest of the block is the final literal run.  LZ4 was chosen on the
 * pages because it codes long runs in few commands and RL masks are long zero
 * runs ([Teleport] "Moving the pipeline onto GPUs").  The output is standard
 * LZ4 block format; any LZ4 block decoder accepts it.
 *   src          [nbytes] bytes to encode (read).
 *   src_xor      [nbytes] or NULL; when given the encoded bytes are
 *                src[i] ^ src_xor[i] (the XOR mask of two views, never
 *                materialised).
 *   block_bytes  16384, 32768 or 65536.
 *   payload      [payload_cap] concatenated encoded blocks (written).
 *                nblocks * (block_bytes + block_bytes/255 + 16) always suffices.
 *   comp_sizes   [nblocks] uint32 encoded size per block (written).
 *   comp_offsets [nblocks] uint64 exclusive prefix sum of comp_sizes (written).
 *   d_total      (device uint64) total encoded bytes, exact (written).
 *   d_status     PULSE_DS_CAPACITY when the total exceeds payload_cap; blocks
 *                that do not fit entirely are not written.
 *   ws           pulse_workspace_bytes(PULSE_OP_LZ4_ENCODE, nbytes, block_bytes).
 * nblocks = ceil(nbytes / block_bytes). */
int lz4_encode_blocks(const void *src, const void *src_xor, int64_t nbytes,
                      int32_t block_bytes, uint8_t *payload, int64_t payload_cap,
                      uint32_t *comp_sizes, uint64_t *comp_offsets, uint64_t *d_total,
                      uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- a6: LZ4 block decode + in-place apply -------------------------------
 * Decodes any valid LZ4 block (not only the canonical parse) and either stores
 * the bytes (mode 0) or XORs them into dst in place (mode 1): the sampler gets
 * exactly the new weights ([Teleport] "XOR masks"; the decoded mask is applied
 * in place in HBM, "Moving the pipeline onto GPUs").  Each block is validated
 * in full before any byte of its dst range is written; a malformed block
 * (length past its input, offset 0 or beyond the bytes produced, output past
 * its size, input not ending right after a literal run with the output exactly
 * full, bytes outside [0, payload_bytes), or a start before the end of any
 * earlier block in the payload) leaves its dst range untouched and sets
 * PULSE_DS_CORRUPT.
 *   payload        [payload_bytes] encoded blocks (read).
 *   comp_offsets, comp_sizes  [nblocks] block table (read).
 *   block_bytes    decoded size of every block but the last (<= 65536).
 *   nbytes         total decoded bytes; nblocks == ceil(nbytes / block_bytes).
 *   dst            [nbytes], 16-byte aligned.
 *   ws             pulse_workspace_bytes(PULSE_OP_LZ4_DECODE, nblocks, payload_bytes). */
int lz4_decode_blocks(const uint8_t *payload, int64_t payload_bytes,
                      const uint64_t *comp_offsets, const uint32_t *comp_sizes,
                      int64_t nblocks, int32_t block_bytes, int64_t nbytes, void *dst,
                      int32_t mode, uint32_t *d_status, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/* The same decode in two calls, so that a caller can run the serial part (the
 * token-chain parse of every block, latency-bound) on one stream while other
 * work keeps HBM busy, and the apply (the dense XOR or store into dst) later.
 * lz4_decode_parse validates the block table and parses every block into ws;
 * lz4_decode_apply then rebuilds each block and applies it to dst, exactly as
 * lz4_decode_blocks does.  Both take the same payload, block table, sizes and
 * ws (arguments as above); apply must run after its parse has completed (same
 * stream, or an event), and a workspace holds one parse at a time: every parse
 * is followed by its apply before the next parse on that workspace.  Corrupt
 * blocks are found by the parse and reported (PULSE_DS_CORRUPT) by either
 * call; their dst range is left untouched. */
int lz4_decode_parse(const uint8_t *payload, int64_t payload_bytes,
                     const uint64_t *comp_offsets, const uint32_t *comp_sizes,
                     int64_t nblocks, int32_t block_bytes, int64_t nbytes,
                     uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream);
int lz4_decode_apply(const uint8_t *payload, int64_t payload_bytes,
                     const uint64_t *comp_offsets, const uint32_t *comp_sizes,
                     int64_t nblocks, int32_t block_bytes, int64_t nbytes, void *dst,
                     int32_t mode, uint32_t *d_status, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* ---- a7: projection fusion + FP8-E4M3 block quantisation -----------------
 * The sender rebuilds the full weight, fuses projections and quantises BF16
 * training weights for FP8 inference ([Perplexity] opening paragraph and
 * "Potok zadan").  The sources are stacked along rows (the output dimension of
 * an nn.Linear [out, in] weight), e.g. [q; k; v] or per expert [gate; up];
 * the stacked [R, cols] matrix is cut into 128x128 blocks; per block
 * amax = max |x|, s = amax / 448 (IEEE float32 division; s = 1 when amax == 0)
 * and code = E4M3(x / s) (IEEE division, round to nearest even, saturating at
 * 448).  Dequantisation is E4M3(code) * s.  The inputs must be finite
 * (trained weights are): for a block holding Inf or NaN its codes and scale
 * are unspecified (the call still completes).
 *   srcs        (host) array of nsrc (1..8) device pointers to BF16 [rows_i, cols],
 *               row-major, 16-byte aligned.
 *   src_rows    (host) rows of each source.
 *   cols        columns, a multiple of 8.
 *   batch       number of stacked matrices (e.g. experts); source i of entry e
 *               starts at srcs[i] + e * src_batch_stride[i] elements.
 *   src_batch_stride (host) per-source stride in elements; NULL if batch == 1.
 *   codes       [batch][R][cols] uint8 (written), R = sum of rows.
 *   scales      [batch][ceil(R/128)][ceil(cols/128)] float32 (written). */
int fp8_block_quant(const uint16_t *const *srcs, const int64_t *src_rows, int32_t nsrc,
                    int64_t cols, int64_t batch, const int64_t *src_batch_stride,
                    uint8_t *codes, float *scales, hipStream_t stream);

/* Several stacked groups quantised in one launch: exactly the results of one
 * fp8_block_quant call (batch 1) per group, with the blocks of all groups
 * sharing the GPU, so that small groups (a layer's [q;k;v] or o projection)
 * do not run as launches too small to fill it.
 *   groups     (host) array of ngroups (1..PULSE_QUANT_MAX_GROUPS) descriptors,
 *              read during the call only.
 *   per group: src[0..nsrc) device BF16 sources [rows[i], cols], row-major,
 *              16-byte aligned, nsrc in 1..4; cols a multiple of 8; codes
 *              [R][cols] (8-byte aligned) and scales [ceil(R/128)][ceil(cols/128)]
 *              written, R = sum of rows > 0.  Groups must not overlap in their
 *              outputs. */
#define PULSE_QUANT_MAX_GROUPS 8
typedef struct {
    const uint16_t *src[4];
    int64_t rows[4];
    int32_t nsrc;
    int32_t reserved; /* 0 */
    int64_t cols;
    uint8_t *codes;
    float *scales;
} pulse_quant_group;
int fp8_block_quant_groups(const pulse_quant_group *groups, int32_t ngroups, hipStream_t stream);

/* ---- a4 + a7: the receiver's pass, patch apply and FP8 quantisation -------
 * The receiver overrides the patch's positions in its BF16 view ([Jiang talk]
 * 11:08-11:30; [PULSE summary] "1. PULSESync", Ricostruzione) and serves the
 * new weights quantised to FP8 in 128x128 blocks ([Perplexity] opening
 * paragraph and "Potok zadan").  pulse_apply_quant gives exactly the results
 * of pulse_apply_patch on the view followed by one fp8_block_quant call per
 * quantised group, in one read of the view: each 128x128 block is read once,
 * patched on chip, its changed 16-byte pieces written back and its codes
 * computed from the patched values.
 *
 * A plan describes the view as groups.  A group stacks 1..4 sources along
 * rows; every source is a row-major [rows, cols] matrix inside the view at an
 * element offset.  A quantised group (quantise = 1) writes codes [R][cols]
 * (8-byte aligned) and scales [ceil(R/128)][ceil(cols/128)] as fp8_block_quant
 * does, R = sum of rows; a group with quantise = 0 is only patched (norms,
 * biases: describe a 1-D tensor as [1, len]).  cols is a multiple of 8, every
 * offset a multiple of 8, and the sources of all groups together tile the view
 * [0, n) with neither gap nor overlap (so every entry of the patch is applied
 * exactly once).  Groups must not overlap in their outputs. */
typedef struct {
    int64_t src_offset[4]; /* element offset of source i in the view          */
    int64_t rows[4];
    int32_t nsrc;          /* 1..4                                          */
    int32_t quantise;      /* 1: codes + scales, 0: patch only                */
    int64_t cols;
    uint8_t *codes;        /* device, quantise = 1                          */
    float *scales;         /* device, quantise = 1                          */
} pulse_aq_group;

/* Bytes of a plan for ngroups groups (0 when ngroups < 1). */
int64_t pulse_apply_quant_plan_bytes(int32_t ngroups);

/* Checks the groups against a view of n elements (n <= 2^31 - 1) and writes
 * the plan into plan (device, 16-byte aligned, plan_bytes >= the size above);
 * the copy is synchronous, so groups may be freed on return.  *nblocks (host)
 * receives the number of 128x128 blocks, to be passed to pulse_apply_quant.
 * PULSE_EINVAL for a bad group or sources that do not tile [0, n),
 * PULSE_EALIGN for a misaligned offset or output, PULSE_EWORKSPACE when
 * plan_bytes is too small, PULSE_EHIP when the copy fails. */
int pulse_apply_quant_plan(const pulse_aq_group *groups, int32_t ngroups, int64_t n, void *plan,
                           int64_t plan_bytes, int64_t *nblocks);

/* The receiver's pass over a view b [n] (16-byte aligned, updated in place).
 *   patch_idx, patch_val  the patch, indices strictly ascending (as the
 *              compaction writes them); count = min(*d_count, max_count),
 *              max_count >= 1 (the buffers hold at least one entry, which
 *              is read even when count is 0).
 *   plan, nblocks  from pulse_apply_quant_plan for this n; the codes and
 *              scales go where the plan's groups say.
 *   d_status   PULSE_DS_BADINDEX when an index lies outside [0, n) or does
 *              not ascend (the view is then unspecified, but nothing outside
 *              it and the outputs is written); PULSE_DS_WORKSPACE when the
 *              plan was made for another n or block count (nothing written).
 *   ws         pulse_workspace_bytes(PULSE_OP_APPLY_QUANT, n, 0): the patch's
 *              segment index (first entry at or past every 128th element) and
 *              the counters from which the pass's workgroups take their
 *              blocks, both rebuilt by every call (no initialisation needed;
 *              calls sharing a workspace must not overlap).
 * The inputs must be finite, as for fp8_block_quant. */
int pulse_apply_quant(uint16_t *b, int64_t n, const int32_t *patch_idx, const uint16_t *patch_val,
                      const int64_t *d_count, int64_t max_count, const void *plan, int64_t nblocks,
                      uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- next: deltas of the FP8 served view ----------------------------------
 * When the sampler serves FP8, the view it must rebuild bit for bit is the
 * quantised one, and its coarser cells change fewer values per step ([Jiang
 * talk] 13:06-14:40; [PULSE summary] "Potenziale Futuro").  Two versions of
 * fp8_block_quant's output are compared bitwise (codes as bytes, scales as
 * 32-bit patterns) and each changed position is sent with its new absolute
 * value, as for the BF16 view.
 *   codes_old, codes_new   [n_codes] E4M3 codes, 16-byte aligned (read).
 *   scales_old, scales_new [n_scales] float32 block scales, 16-byte aligned.
 *   n_codes, n_scales      1 .. 2^31 - 1.
 *   code_idx, code_val     [code_cap] ascending int32 positions and new codes
 *                          (written); *d_code_count = exact number of changes.
 *   scale_idx, scale_val   [scale_cap] the same for the scales.
 *   d_status               PULSE_DS_CAPACITY when either list exceeds its cap
 *                          (entries beyond the cap are not written).
 *   ws                     pulse_workspace_bytes(PULSE_OP_FP8_DELTA,
 *                          max(n_codes, n_scales), 0). */
int fp8_view_delta(const uint8_t *codes_old, const uint8_t *codes_new, int64_t n_codes,
                   const float *scales_old, const float *scales_new, int64_t n_scales,
                   int32_t *code_idx, uint8_t *code_val, int64_t code_cap, int64_t *d_code_count,
                   int32_t *scale_idx, float *scale_val, int64_t scale_cap, int64_t *d_scale_count,
                   uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* The receiver's side: codes[code_idx[k]] = code_val[k] for
 * k < min(*d_code_count, max_code_count), and the same for the scales; the
 * result is the new quantisation bit for bit.  Entries with an index outside
 * the buffer are skipped and set PULSE_DS_BADINDEX.  Indices must be unique
 * (a delta's are). */
int fp8_view_apply(uint8_t *codes, int64_t n_codes, float *scales, int64_t n_scales,
                   const int32_t *code_idx, const uint8_t *code_val, const int64_t *d_code_count,
                   int64_t max_code_count, const int32_t *scale_idx, const float *scale_val,
                   const int64_t *d_scale_count, int64_t max_scale_count, uint32_t *d_status,
                   hipStream_t stream);

/* ---- next: PULSELoCo visibility gate with FP32 error feedback -------------
 * Trainer-to-trainer sync ([PULSE summary] "2. PULSELoCo", Processo): each
 * worker's pseudo-gradient (its parameter update over H local steps) is added
 * to its error-feedback buffer, a = resid + delta (float32); the entry is sent
 * only if it would change the BF16 view of the shared checkpoint,
 * bf16(theta + a) != bf16(theta) (float32 add, round to nearest even), and
 * otherwise stays in the buffer for the next round.
 *   theta   [n] float32 shared checkpoint (read), 16-byte aligned.
 *   delta   [n] float32 pseudo-gradient (read), 16-byte aligned.
 *   resid   [n] float32 error-feedback buffer, 16-byte aligned: read, then
 *           rewritten with 0 where the entry was sent and a elsewhere.
 *   idx, val [cap] ascending int32 positions and the sent float32 values a.
 *   d_count  exact number of visible entries.  Visible entries beyond cap are
 *           not sent and stay in resid (PULSE_DS_CAPACITY): nothing is lost.
 *   ws      pulse_workspace_bytes(PULSE_OP_LOCO_GATE, n, 0). */
int pulse_loco_gate(const float *theta, const float *delta, float *resid, int64_t n,
                    int32_t *idx, float *val, int64_t cap, int64_t *d_count, uint32_t *d_status,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/* The receiving trainer sums the workers' sparse updates before its outer
 * step: acc[idx[k]] += val[k] (float32) for k < min(*d_count, max_count), in
 * stream order, one patch per call (indices unique within a patch, so the
 * result is deterministic).  Out-of-range indices set PULSE_DS_BADINDEX. */
int pulse_loco_accumulate(float *acc, int64_t n, const int32_t *idx, const float *val,
                          const int64_t *d_count, int64_t max_count, uint32_t *d_status,
                          hipStream_t stream);

/* ---- next: compression of the patch stream ---------------------------------
 * The sparse patches are compressed further with a generic lossless codec
 * ([PULSE summary] "1. PULSESync", Compressione).  Here the codec is this
 * library's LZ4 block format (lz4_encode_blocks / lz4_decode_blocks with
 * 65536-byte blocks), whose canonical parse only finds runs of one byte, so
 * the patch is first packed: each index becomes its gap to the previous one
 * (gap = idx[k] - idx[k-1] - 1, idx[-1] = -1) and every group of 65536
 * entries becomes six 64 KiB byte planes (gap bytes 0-3, value bytes 0-1,
 * little-endian); entries past the count in the last group are zero.  Each
 * plane is one LZ4 block; the high gap planes compress to almost nothing.
 *
 * Bytes of the packed form of `count` entries (whole groups). */
int64_t patch_packed_bytes(int64_t count);

/*   idx, val   [count] ascending int32 positions and BF16 values (read),
 *              16-byte aligned (a pulse_cast_diff / pulse_compact patch).
 *   count      entries, host value, 0 .. 2^31.
 *   packed     [patch_packed_bytes(count)] (written), 16-byte aligned. */
int patch_pack(const int32_t *idx, const uint16_t *val, int64_t count, uint8_t *packed,
               hipStream_t stream);

/* Inverse of patch_pack (after lz4_decode_blocks in store mode): idx[k] is the
 * running sum of gap + 1, less one, over the whole patch.
 *   packed     [patch_packed_bytes(count)] (read).
 *   idx, val   [count] (written), 16-byte aligned.
 *   d_status   PULSE_DS_CORRUPT when a gap or an index passes 2^31 - 1 (data
 *              that no pack produces); the indices are then unspecified.
 *   ws         pulse_workspace_bytes(PULSE_OP_PATCH_UNPACK, count, 0). */
int patch_unpack(const uint8_t *packed, int64_t count, int32_t *idx, uint16_t *val,
                 uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- next: one launch over a list of tensors --------------------------------
 * The tiling and address-mapping metadata is prepared on the CPU so that one
 * kernel launch covers the whole model ([Teleport] "Moving the pipeline onto
 * GPUs").  The result is exactly that of pulse_cast_diff (patch output, and
 * b_new when given) on each tensor in list order, with indices local to each
 * tensor: one entry stream in which tensor s holds
 * [seg_offsets[s], seg_offsets[s + 1]).
 *
 * One tensor of the list (device table of nseg entries, 40 bytes each). */
typedef struct pulse_segment {
    const float *w_new;    /* [n] float32 masters (read), 16-byte aligned        */
    const uint16_t *b_old; /* [n] previous BF16 view (read), 16-byte aligned     */
    uint16_t *b_new;       /* [n] new view (written), 16-byte aligned, or NULL
                              (all segments alike, see with_new)                */
    int64_t n;             /* elements, 1 .. 2^31 - 1                            */
    int64_t tile0;         /* first tile of the tensor: pulse_segment_tiles      */
} pulse_segment;

/* One view of the receiver (device table of nseg entries, 16 bytes each). */
typedef struct pulse_view {
    uint16_t *b; /* [n] BF16 view (read and written) */
    int64_t n;
} pulse_view;

/* Host helper that prepares the tiling metadata: returns the number of
 * 16384-element tiles of the list (or a negative PULSE_E* code), writes each
 * tensor's first tile to tile0[nseg] and the tensor of every tile to
 * tile_seg[tiles] (host arrays; either may be NULL).  n: host array. */
int64_t pulse_segment_tiles(const int64_t *n, int32_t nseg, int64_t *tile0, uint32_t *tile_seg);

/*   segs       device table [nseg].
 *   tile_seg   device array [ntiles]: the tensor of every tile.
 *   ntiles     the return value of pulse_segment_tiles.
 *   patch_idx, patch_val [patch_cap] the entry stream (written).
 *   seg_offsets [nseg + 1] int64 (written): first entry of each tensor, total.
 *   with_new   1 if every segment has b_new, 0 if none has.
 *   d_status   PULSE_DS_CAPACITY, PULSE_DS_BADSEGMENT, PULSE_DS_WORKSPACE.
 *   ws         pulse_workspace_bytes(PULSE_OP_CAST_DIFF_SEGMENTS, ntiles, 0). */
int pulse_cast_diff_segments(const pulse_segment *segs, int32_t nseg, const uint32_t *tile_seg,
                             int64_t ntiles, int32_t *patch_idx, uint16_t *patch_val, int64_t patch_cap,
                             int64_t *seg_offsets, uint32_t *d_status, void *ws, size_t ws_bytes,
                             int32_t with_new, hipStream_t stream);

/* The receiver's side of a list call: for every tensor s,
 * views[s].b[patch_idx[k]] = patch_val[k] for k in [seg_offsets[s],
 * seg_offsets[s + 1]), k < max_count; out-of-range indices set
 * PULSE_DS_BADINDEX.  views: device table [nseg]. */
int pulse_apply_patch_segments(const pulse_view *views, int32_t nseg, const int32_t *patch_idx,
                               const uint16_t *patch_val, const int64_t *seg_offsets, int64_t max_count,
                               uint32_t *d_status, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PULSE_H */
