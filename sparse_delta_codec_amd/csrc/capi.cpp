// capi.cpp -- the C ABI of include/pulse.h: argument checks, workspace sizing
// and dispatch to the kernel launchers.  No device memory is allocated here;
// nothing is enqueued when a check fails.
#include "../../include/pulse.h"

#include <hip/hip_runtime.h>

#include <cstdint>

extern "C" {
int pulse_launch_cast_diff(const float *, const uint16_t *, const uint16_t *, uint16_t *, uint16_t *,
                           int32_t *, uint16_t *, int64_t, int64_t *, uint32_t *, int64_t, void *,
                           hipStream_t);
size_t pulse_cast_diff_ws_bytes(int64_t n);
int pulse_launch_apply_patch(uint16_t *, int64_t, const int32_t *, const uint16_t *, const int64_t *,
                             int64_t, uint32_t *, hipStream_t);
int pulse_launch_xor_apply(void *, const void *, int64_t, hipStream_t);
size_t pulse_lz4_encode_ws_bytes(int64_t nbytes, int32_t block_bytes);
int pulse_launch_lz4_encode(const void *, const void *, int64_t, int32_t, uint8_t *, int64_t, uint32_t *,
                            uint64_t *, uint64_t *, uint32_t *, void *, hipStream_t);
size_t pulse_lz4_decode_ws_bytes(int64_t nblocks, int64_t payload_bytes);
int pulse_launch_lz4_decode(const uint8_t *, int64_t, const uint64_t *, const uint32_t *, int64_t, int32_t,
                            int64_t, void *, int32_t, uint32_t *, void *, size_t, hipStream_t);
int pulse_lz4_decode_ws_fits(size_t ws, int64_t nblocks, int64_t payload_bytes);
int pulse_launch_lz4_decode_parse(const uint8_t *, int64_t, const uint64_t *, const uint32_t *, int64_t, int32_t,
                                  int64_t, uint32_t *, void *, size_t, hipStream_t);
int pulse_launch_lz4_decode_apply(const uint8_t *, int64_t, const uint64_t *, const uint32_t *, int64_t, int32_t,
                                  int64_t, void *, int32_t, uint32_t *, void *, size_t, hipStream_t);
int pulse_launch_fp8_block_quant(const uint16_t *const *, const int64_t *, int32_t, int64_t, int64_t,
                                 const int64_t *, uint8_t *, float *, hipStream_t);
size_t pulse_delta_compact_ws_bytes(int64_t n);
int pulse_launch_fp8_delta(const uint8_t *, const uint8_t *, int64_t, const float *, const float *, int64_t,
                           int32_t *, uint8_t *, int64_t, int64_t *, int32_t *, float *, int64_t, int64_t *,
                           uint32_t *, void *, hipStream_t);
int pulse_launch_fp8_apply(uint8_t *, int64_t, float *, int64_t, const int32_t *, const uint8_t *,
                           const int64_t *, int64_t, const int32_t *, const float *, const int64_t *, int64_t,
                           uint32_t *, hipStream_t);
int pulse_launch_loco_gate(const float *, const float *, float *, int64_t, int32_t *, float *, int64_t, int64_t *,
                           uint32_t *, void *, hipStream_t);
int pulse_launch_loco_accumulate(float *, int64_t, const int32_t *, const float *, const int64_t *, int64_t,
                                 uint32_t *, hipStream_t);
size_t pulse_patch_unpack_ws_bytes(int64_t count);
int64_t pulse_patch_packed_bytes_impl(int64_t count);
int pulse_launch_patch_pack(const int32_t *, const uint16_t *, int64_t, uint8_t *, hipStream_t);
int pulse_launch_patch_unpack(const uint8_t *, int64_t, int32_t *, uint16_t *, uint32_t *, void *, hipStream_t);
int pulse_launch_cast_diff_segments(const void *, int32_t, const uint32_t *, int64_t, int32_t *, uint16_t *, int64_t,
                                    int64_t *, uint32_t *, void *, int, hipStream_t);
int pulse_launch_apply_patch_segments(const void *, int32_t, const int32_t *, const uint16_t *, const int64_t *,
                                      int64_t, uint32_t *, hipStream_t);
int pulse_launch_fill_zero(void *, size_t, hipStream_t);
int pulse_launch_fp8_block_quant_groups(const void *, int32_t, hipStream_t);
size_t pulse_cast_diff_lz4_ws_bytes(int64_t n, int32_t block_bytes);
int pulse_launch_cast_diff_lz4(const float *, const uint16_t *, uint16_t *, int32_t *, uint16_t *, int64_t,
                               int64_t *, int64_t, int32_t, uint8_t *, int64_t, uint32_t *, uint64_t *, uint64_t *,
                               uint32_t *, int64_t *, void *, hipStream_t);
int pulse_launch_apply_patch_tiled(uint16_t *, int64_t, const int32_t *, const uint16_t *, const int64_t *, int64_t,
                                   uint32_t *, hipStream_t);
int pulse_launch_patch_tiles(const int32_t *, const int64_t *, int64_t, int64_t, int64_t *, hipStream_t);
int pulse_launch_write_count(int64_t *, int64_t, hipStream_t);
size_t pulse_noalloc_scratch_bytes(void);
void *pulse_noalloc_scratch(hipStream_t);
int64_t pulse_apply_quant_plan_size(int32_t);
int pulse_build_apply_quant_plan(const void *, int32_t, int64_t, void *, int64_t, int64_t *);
int pulse_launch_apply_quant(uint16_t *, int64_t, const int32_t *, const uint16_t *, const int64_t *, int64_t,
                             const void *, int64_t, uint32_t *, void *, hipStream_t);
size_t pulse_apply_quant_ws_bytes(int64_t n);
}

namespace {

constexpr int64_t kMaxIndexed = 2147483647;    // int32 patch indices
constexpr int64_t kMaxPayload = (1ll << 39) - 2; // look-back value field

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char *pulse_version(void) { return "0.1.0"; }

const char *pulse_status_string(int code) {
    switch (code) {
    case PULSE_OK: return "PULSE_OK";
    case PULSE_EINVAL: return "PULSE_EINVAL: invalid argument";
    case PULSE_EALIGN: return "PULSE_EALIGN: buffer not 16-byte aligned";
    case PULSE_ERANGE: return "PULSE_ERANGE: size beyond the supported range";
    case PULSE_EWORKSPACE: return "PULSE_EWORKSPACE: workspace missing or too small";
    case PULSE_EHIP: return "PULSE_EHIP: kernel launch failed";
    default: return "unknown pulse status";
    }
}

size_t pulse_workspace_bytes(int op, int64_t n, int64_t aux) {
    if (n < 0) return 0;
    switch (op) {
    case PULSE_OP_CAST_DIFF:
    case PULSE_OP_COMPACT: return pulse_cast_diff_ws_bytes(n);
    case PULSE_OP_LZ4_ENCODE:
        if (aux <= 0) return 0;
        return pulse_lz4_encode_ws_bytes(n, (int32_t)aux);
    case PULSE_OP_LZ4_DECODE:
        if (aux < 0) return 0;
        return pulse_lz4_decode_ws_bytes(n, aux);
    case PULSE_OP_FP8_DELTA:
    case PULSE_OP_LOCO_GATE: return pulse_delta_compact_ws_bytes(n);
    case PULSE_OP_PATCH_UNPACK: return pulse_patch_unpack_ws_bytes(n);
    case PULSE_OP_CAST_DIFF_SEGMENTS: return sizeof(uint64_t) * 32 + (size_t)(n > 0 ? n : 1) * sizeof(uint64_t);
    case PULSE_OP_CAST_DIFF_LZ4:
        if (aux != 16384 && aux != 32768 && aux != 65536) return 0;
        return pulse_cast_diff_lz4_ws_bytes(n, (int32_t)aux);
    case PULSE_OP_APPLY_QUANT: return pulse_apply_quant_ws_bytes(n);
    default: return 0;
    }
}

int pulse_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!ws) return PULSE_EINVAL;
    if (ws_bytes == 0) return PULSE_OK;
    return pulse_launch_fill_zero(ws, ws_bytes, stream);
}

int pulse_cast_diff(const float *w_new, const uint16_t *b_old, uint16_t *b_new, uint16_t *xor_mask,
                    int32_t *patch_idx, uint16_t *patch_val, int64_t patch_cap, int64_t *d_count,
                    uint32_t *d_status, int64_t n, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!w_new || n < 0) return PULSE_EINVAL;
    const bool patch = patch_idx || patch_val || d_count;
    if (patch && !(patch_idx && patch_val && d_count && d_status)) return PULSE_EINVAL;
    if (!b_old && (xor_mask || patch)) return PULSE_EINVAL;
    if (!b_new && !xor_mask && !patch) return PULSE_EINVAL;  // nothing to produce
    if (patch_cap < 0) return PULSE_EINVAL;
    if (!aligned16(w_new) || (b_old && !aligned16(b_old)) || (b_new && !aligned16(b_new)) ||
        (xor_mask && !aligned16(xor_mask)))
        return PULSE_EALIGN;
    if (patch) {
        if (n > kMaxIndexed) return PULSE_ERANGE;
        if (!ws || ws_bytes < pulse_cast_diff_ws_bytes(n)) return PULSE_EWORKSPACE;
        if (n == 0) return pulse_launch_write_count(d_count, 0, stream);
    }
    if (n == 0) return PULSE_OK;
    return pulse_launch_cast_diff(w_new, nullptr, b_old, b_new, xor_mask, patch_idx, patch_val, patch_cap,
                                  d_count, d_status, n, ws, stream);
}

int pulse_compact(const uint16_t *b_old, const uint16_t *b_new, int32_t *patch_idx, uint16_t *patch_val,
                  int64_t patch_cap, int64_t *d_count, uint32_t *d_status, int64_t n, void *ws,
                  size_t ws_bytes, hipStream_t stream) {
    if (!b_old || !b_new || !patch_idx || !patch_val || !d_count || !d_status || n < 0 || patch_cap < 0)
        return PULSE_EINVAL;
    if (!aligned16(b_old) || !aligned16(b_new)) return PULSE_EALIGN;
    if (n > kMaxIndexed) return PULSE_ERANGE;
    if (!ws || ws_bytes < pulse_cast_diff_ws_bytes(n)) return PULSE_EWORKSPACE;
    if (n == 0) return pulse_launch_write_count(d_count, 0, stream);
    return pulse_launch_cast_diff(nullptr, b_new, b_old, nullptr, nullptr, patch_idx, patch_val, patch_cap,
                                  d_count, d_status, n, ws, stream);
}

}  // extern "C"

namespace {

// Argument checks shared by pulse_cast_diff_lz4 and its allocation-free form
// (everything but the workspace).
int check_cast_diff_lz4(const float *w_new, const uint16_t *b_old, uint16_t *b_new, int32_t *patch_idx,
                        uint16_t *patch_val, int64_t patch_cap, int64_t *d_count, int64_t *tile_first, int64_t n,
                        int32_t block_bytes, uint8_t *payload, int64_t payload_cap, uint32_t *comp_sizes,
                        uint64_t *comp_offsets, uint64_t *d_total, uint32_t *d_status) {
    if (!w_new || !b_old || !payload || !comp_sizes || !comp_offsets || !d_total || !d_status || n <= 0 ||
        payload_cap < 0 || patch_cap < 0)
        return PULSE_EINVAL;
    const bool patch = patch_idx || patch_val || d_count;
    if (patch && !(patch_idx && patch_val && d_count)) return PULSE_EINVAL;
    if (tile_first && !patch) return PULSE_EINVAL;
    if (block_bytes != 16384 && block_bytes != 32768 && block_bytes != 65536) return PULSE_EINVAL;
    if (!aligned16(w_new) || !aligned16(b_old) || (b_new && !aligned16(b_new))) return PULSE_EALIGN;
    if (patch && n > kMaxIndexed) return PULSE_ERANGE;
    const int64_t nb = (2 * n + block_bytes - 1) / block_bytes;
    if (nb > 0xFFFFFFFFll || 2 * n > kMaxPayload / 2) return PULSE_ERANGE;
    return PULSE_OK;
}

}  // namespace

extern "C" {

int pulse_cast_diff_lz4(const float *w_new, const uint16_t *b_old, uint16_t *b_new, int32_t *patch_idx,
                        uint16_t *patch_val, int64_t patch_cap, int64_t *d_count, int64_t *tile_first,
                        int64_t n, int32_t block_bytes,
                        uint8_t *payload, int64_t payload_cap, uint32_t *comp_sizes, uint64_t *comp_offsets,
                        uint64_t *d_total, uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream) {
    const int rc = check_cast_diff_lz4(w_new, b_old, b_new, patch_idx, patch_val, patch_cap, d_count, tile_first, n,
                                       block_bytes, payload, payload_cap, comp_sizes, comp_offsets, d_total,
                                       d_status);
    if (rc != PULSE_OK) return rc;
    if (!ws || ws_bytes < pulse_cast_diff_lz4_ws_bytes(n, block_bytes)) return PULSE_EWORKSPACE;
    return pulse_launch_cast_diff_lz4(w_new, b_old, b_new, patch_idx, patch_val, patch_cap, d_count, n,
                                      block_bytes, payload, payload_cap, comp_sizes, comp_offsets, d_total,
                                      d_status, tile_first, ws, stream);
}

int pulse_cast_diff_lz4_noalloc(const float *w_new, const uint16_t *b_old, uint16_t *b_new, int32_t *patch_idx,
                                uint16_t *patch_val, int64_t patch_cap, int64_t *d_count, int64_t *tile_first,
                                int64_t n, int32_t block_bytes, uint8_t *payload, int64_t payload_cap,
                                uint32_t *comp_sizes, uint64_t *comp_offsets, uint64_t *d_total, uint32_t *d_status,
                                hipStream_t stream) {
    const int rc = check_cast_diff_lz4(w_new, b_old, b_new, patch_idx, patch_val, patch_cap, d_count, tile_first, n,
                                       block_bytes, payload, payload_cap, comp_sizes, comp_offsets, d_total,
                                       d_status);
    if (rc != PULSE_OK) return rc;
    if (pulse_cast_diff_lz4_ws_bytes(n, block_bytes) > pulse_noalloc_scratch_bytes()) return PULSE_ERANGE;
    void *ws = pulse_noalloc_scratch(stream);
    if (!ws) return PULSE_EHIP;
    return pulse_launch_cast_diff_lz4(w_new, b_old, b_new, patch_idx, patch_val, patch_cap, d_count, n,
                                      block_bytes, payload, payload_cap, comp_sizes, comp_offsets, d_total,
                                      d_status, tile_first, ws, stream);
}

int pulse_patch_tiles(const int32_t *patch_idx, const int64_t *d_count, int64_t max_count, int64_t n,
                      int64_t *tile_first, hipStream_t stream) {
    if (!patch_idx || !d_count || !tile_first || max_count < 0 || n < 1) return PULSE_EINVAL;
    if (n > kMaxIndexed + 1) return PULSE_ERANGE;
    return pulse_launch_patch_tiles(patch_idx, d_count, max_count, n, tile_first, stream);
}

int pulse_apply_patch_tiled(uint16_t *b, int64_t n, const int32_t *patch_idx, const uint16_t *patch_val,
                            const int64_t *tile_first, int64_t max_count, uint32_t *d_status, hipStream_t stream) {
    if (!b || !patch_idx || !patch_val || !tile_first || !d_status || n < 1 || max_count < 0) return PULSE_EINVAL;
    if (!aligned16(b)) return PULSE_EALIGN;
    if (n > kMaxIndexed + 1) return PULSE_ERANGE;
    return pulse_launch_apply_patch_tiled(b, n, patch_idx, patch_val, tile_first, max_count, d_status, stream);
}

int pulse_apply_patch(uint16_t *b, int64_t n, const int32_t *patch_idx, const uint16_t *patch_val,
                      const int64_t *d_count, int64_t max_count, uint32_t *d_status, hipStream_t stream) {
    if (!b || !patch_idx || !patch_val || !d_count || !d_status || n < 0 || max_count < 0)
        return PULSE_EINVAL;
    if (n > kMaxIndexed) return PULSE_ERANGE;  // the stores address the view's 2 n bytes in 32 bits
    if (max_count == 0) return PULSE_OK;
    return pulse_launch_apply_patch(b, n, patch_idx, patch_val, d_count, max_count, d_status, stream);
}

int xor_mask_apply(void *dst, const void *mask, int64_t nbytes, hipStream_t stream) {
    if (!dst || !mask || nbytes < 0) return PULSE_EINVAL;
    if (!aligned16(dst) || !aligned16(mask)) return PULSE_EALIGN;
    if (nbytes == 0) return PULSE_OK;
    return pulse_launch_xor_apply(dst, mask, nbytes, stream);
}

int lz4_encode_blocks(const void *src, const void *src_xor, int64_t nbytes, int32_t block_bytes,
                      uint8_t *payload, int64_t payload_cap, uint32_t *comp_sizes, uint64_t *comp_offsets,
                      uint64_t *d_total, uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!src || !payload || !comp_sizes || !comp_offsets || !d_total || !d_status || nbytes <= 0 ||
        payload_cap < 0)
        return PULSE_EINVAL;
    if (block_bytes != 16384 && block_bytes != 32768 && block_bytes != 65536) return PULSE_EINVAL;
    if (!aligned16(src) || (src_xor && !aligned16(src_xor))) return PULSE_EALIGN;
    const int64_t nb = (nbytes + block_bytes - 1) / block_bytes;
    if (nb > 0xFFFFFFFFll || nbytes > kMaxPayload / 2) return PULSE_ERANGE;
    if (!ws || ws_bytes < pulse_lz4_encode_ws_bytes(nbytes, block_bytes)) return PULSE_EWORKSPACE;
    return pulse_launch_lz4_encode(src, src_xor, nbytes, block_bytes, payload, payload_cap, comp_sizes,
                                   comp_offsets, d_total, d_status, ws, stream);
}

namespace {
// argument checks shared by the decode calls (dst and mode only where given)
int check_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *comp_offsets,
                 const uint32_t *comp_sizes, int64_t nblocks, int32_t block_bytes, int64_t nbytes, const void *dst,
                 bool need_dst, int32_t mode, const uint32_t *d_status, const void *ws, size_t ws_bytes) {
    if (!payload || !comp_offsets || !comp_sizes || (need_dst && !dst) || !d_status || payload_bytes < 0 ||
        nbytes <= 0 || nblocks <= 0)
        return PULSE_EINVAL;
    if (mode != 0 && mode != 1) return PULSE_EINVAL;
    if (block_bytes <= 0 || block_bytes > 65536 || block_bytes % 16 != 0) return PULSE_EINVAL;
    if (nblocks != (nbytes + block_bytes - 1) / block_bytes) return PULSE_EINVAL;
    if (need_dst && !aligned16(dst)) return PULSE_EALIGN;
    if (payload_bytes > kMaxPayload || nblocks > 0x3FFFFFFFll) return PULSE_ERANGE;
    if (!ws || !pulse_lz4_decode_ws_fits(ws_bytes, nblocks, payload_bytes)) return PULSE_EWORKSPACE;
    return PULSE_OK;
}
}  // namespace

int lz4_decode_blocks(const uint8_t *payload, int64_t payload_bytes, const uint64_t *comp_offsets,
                      const uint32_t *comp_sizes, int64_t nblocks, int32_t block_bytes, int64_t nbytes,
                      void *dst, int32_t mode, uint32_t *d_status, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
    const int rc = check_decode(payload, payload_bytes, comp_offsets, comp_sizes, nblocks, block_bytes, nbytes, dst,
                                true, mode, d_status, ws, ws_bytes);
    if (rc != PULSE_OK) return rc;
    return pulse_launch_lz4_decode(payload, payload_bytes, comp_offsets, comp_sizes, nblocks, block_bytes, nbytes,
                                   dst, mode, d_status, ws, ws_bytes, stream);
}

int lz4_decode_parse(const uint8_t *payload, int64_t payload_bytes, const uint64_t *comp_offsets,
                     const uint32_t *comp_sizes, int64_t nblocks, int32_t block_bytes, int64_t nbytes,
                     uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream) {
    const int rc = check_decode(payload, payload_bytes, comp_offsets, comp_sizes, nblocks, block_bytes, nbytes,
                                nullptr, false, 0, d_status, ws, ws_bytes);
    if (rc != PULSE_OK) return rc;
    return pulse_launch_lz4_decode_parse(payload, payload_bytes, comp_offsets, comp_sizes, nblocks, block_bytes,
                                         nbytes, d_status, ws, ws_bytes, stream);
}

int lz4_decode_apply(const uint8_t *payload, int64_t payload_bytes, const uint64_t *comp_offsets,
                     const uint32_t *comp_sizes, int64_t nblocks, int32_t block_bytes, int64_t nbytes, void *dst,
                     int32_t mode, uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream) {
    const int rc = check_decode(payload, payload_bytes, comp_offsets, comp_sizes, nblocks, block_bytes, nbytes, dst,
                                true, mode, d_status, ws, ws_bytes);
    if (rc != PULSE_OK) return rc;
    return pulse_launch_lz4_decode_apply(payload, payload_bytes, comp_offsets, comp_sizes, nblocks, block_bytes,
                                         nbytes, dst, mode, d_status, ws, ws_bytes, stream);
}

int fp8_block_quant(const uint16_t *const *srcs, const int64_t *src_rows, int32_t nsrc, int64_t cols,
                    int64_t batch, const int64_t *src_batch_stride, uint8_t *codes, float *scales,
                    hipStream_t stream) {
    if (!srcs || !src_rows || !codes || !scales || nsrc < 1 || nsrc > 8 || cols <= 0 || batch < 1)
        return PULSE_EINVAL;
    if (cols % 8 != 0) return PULSE_EINVAL;
    if (batch > 1 && !src_batch_stride) return PULSE_EINVAL;
    int64_t R = 0;
    for (int i = 0; i < nsrc; ++i) {
        if (!srcs[i] || src_rows[i] < 0) return PULSE_EINVAL;
        if (!aligned16(srcs[i])) return PULSE_EALIGN;
        if (batch > 1 && (src_batch_stride[i] < 0 || src_batch_stride[i] % 8 != 0)) return PULSE_EALIGN;
        R += src_rows[i];
    }
    if (R == 0) return PULSE_EINVAL;
    if ((R + 127) / 128 > 65535 || batch > 65535 || (cols + 127) / 128 > 0x7FFFFFFF) return PULSE_ERANGE;
    if (reinterpret_cast<uintptr_t>(codes) % 8 != 0 || reinterpret_cast<uintptr_t>(scales) % 4 != 0)
        return PULSE_EALIGN;
    return pulse_launch_fp8_block_quant(srcs, src_rows, nsrc, cols, batch, src_batch_stride, codes, scales, stream);
}

int fp8_block_quant_groups(const pulse_quant_group *groups, int32_t ngroups, hipStream_t stream) {
    if (!groups || ngroups < 1 || ngroups > PULSE_QUANT_MAX_GROUPS) return PULSE_EINVAL;
    int64_t total = 0;
    for (int g = 0; g < ngroups; ++g) {
        const pulse_quant_group &q = groups[g];
        if (q.nsrc < 1 || q.nsrc > 4 || q.cols <= 0 || q.cols % 8 != 0 || !q.codes || !q.scales) return PULSE_EINVAL;
        int64_t R = 0;
        for (int i = 0; i < q.nsrc; ++i) {
            if (!q.src[i] || q.rows[i] < 0) return PULSE_EINVAL;
            if (!aligned16(q.src[i])) return PULSE_EALIGN;
            R += q.rows[i];
        }
        if (R == 0) return PULSE_EINVAL;
        if (reinterpret_cast<uintptr_t>(q.codes) % 8 != 0 || reinterpret_cast<uintptr_t>(q.scales) % 4 != 0)
            return PULSE_EALIGN;
        total += ((R + 127) / 128) * ((q.cols + 127) / 128);
        if (total > 0x7FFFFFFFll) return PULSE_ERANGE;
    }
    return pulse_launch_fp8_block_quant_groups(groups, ngroups, stream);
}

int fp8_view_delta(const uint8_t *codes_old, const uint8_t *codes_new, int64_t n_codes, const float *scales_old,
                   const float *scales_new, int64_t n_scales, int32_t *code_idx, uint8_t *code_val,
                   int64_t code_cap, int64_t *d_code_count, int32_t *scale_idx, float *scale_val,
                   int64_t scale_cap, int64_t *d_scale_count, uint32_t *d_status, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
    if (!codes_old || !codes_new || !scales_old || !scales_new || !code_idx || !code_val || !d_code_count ||
        !scale_idx || !scale_val || !d_scale_count || !d_status || n_codes < 1 || n_scales < 1 ||
        code_cap < 0 || scale_cap < 0)
        return PULSE_EINVAL;
    if (!aligned16(codes_old) || !aligned16(codes_new) || !aligned16(scales_old) || !aligned16(scales_new))
        return PULSE_EALIGN;
    if (n_codes > kMaxIndexed || n_scales > kMaxIndexed) return PULSE_ERANGE;
    const int64_t n = n_codes > n_scales ? n_codes : n_scales;
    if (!ws || ws_bytes < pulse_delta_compact_ws_bytes(n)) return PULSE_EWORKSPACE;
    return pulse_launch_fp8_delta(codes_old, codes_new, n_codes, scales_old, scales_new, n_scales, code_idx,
                                  code_val, code_cap, d_code_count, scale_idx, scale_val, scale_cap,
                                  d_scale_count, d_status, ws, stream);
}

int fp8_view_apply(uint8_t *codes, int64_t n_codes, float *scales, int64_t n_scales, const int32_t *code_idx,
                   const uint8_t *code_val, const int64_t *d_code_count, int64_t max_code_count,
                   const int32_t *scale_idx, const float *scale_val, const int64_t *d_scale_count,
                   int64_t max_scale_count, uint32_t *d_status, hipStream_t stream) {
    if (!codes || !scales || !code_idx || !code_val || !d_code_count || !scale_idx || !scale_val ||
        !d_scale_count || !d_status || n_codes < 0 || n_scales < 0 || max_code_count < 0 || max_scale_count < 0)
        return PULSE_EINVAL;
    if (n_codes > kMaxIndexed + 1 || n_scales > kMaxIndexed + 1) return PULSE_ERANGE;
    return pulse_launch_fp8_apply(codes, n_codes, scales, n_scales, code_idx, code_val, d_code_count,
                                  max_code_count, scale_idx, scale_val, d_scale_count, max_scale_count, d_status,
                                  stream);
}

int pulse_loco_gate(const float *theta, const float *delta, float *resid, int64_t n, int32_t *idx, float *val,
                    int64_t cap, int64_t *d_count, uint32_t *d_status, void *ws, size_t ws_bytes,
                    hipStream_t stream) {
    if (!theta || !delta || !resid || !idx || !val || !d_count || !d_status || n < 0 || cap < 0)
        return PULSE_EINVAL;
    if (!aligned16(theta) || !aligned16(delta) || !aligned16(resid)) return PULSE_EALIGN;
    if (n > kMaxIndexed) return PULSE_ERANGE;
    if (!ws || ws_bytes < pulse_delta_compact_ws_bytes(n)) return PULSE_EWORKSPACE;
    if (n == 0) return pulse_launch_write_count(d_count, 0, stream);
    return pulse_launch_loco_gate(theta, delta, resid, n, idx, val, cap, d_count, d_status, ws, stream);
}

int pulse_loco_accumulate(float *acc, int64_t n, const int32_t *idx, const float *val, const int64_t *d_count,
                          int64_t max_count, uint32_t *d_status, hipStream_t stream) {
    if (!acc || !idx || !val || !d_count || !d_status || n < 0 || max_count < 0) return PULSE_EINVAL;
    if (n > kMaxIndexed + 1) return PULSE_ERANGE;
    if (max_count == 0) return PULSE_OK;
    return pulse_launch_loco_accumulate(acc, n, idx, val, d_count, max_count, d_status, stream);
}

int64_t patch_packed_bytes(int64_t count) {
    if (count < 0) return 0;
    return pulse_patch_packed_bytes_impl(count);
}

int patch_pack(const int32_t *idx, const uint16_t *val, int64_t count, uint8_t *packed, hipStream_t stream) {
    if (!idx || !val || !packed || count < 0) return PULSE_EINVAL;
    if (!aligned16(idx) || !aligned16(val) || !aligned16(packed)) return PULSE_EALIGN;
    if (count > kMaxIndexed + 1) return PULSE_ERANGE;
    if (count == 0) return PULSE_OK;
    return pulse_launch_patch_pack(idx, val, count, packed, stream);
}

int patch_unpack(const uint8_t *packed, int64_t count, int32_t *idx, uint16_t *val, uint32_t *d_status, void *ws,
                 size_t ws_bytes, hipStream_t stream) {
    if (!packed || !idx || !val || !d_status || count < 0) return PULSE_EINVAL;
    if (!aligned16(idx) || !aligned16(val) || !aligned16(packed)) return PULSE_EALIGN;
    if (count > kMaxIndexed + 1) return PULSE_ERANGE;
    if (count == 0) return PULSE_OK;
    if (!ws || ws_bytes < pulse_patch_unpack_ws_bytes(count)) return PULSE_EWORKSPACE;
    return pulse_launch_patch_unpack(packed, count, idx, val, d_status, ws, stream);
}

static_assert(sizeof(pulse_segment) == 40, "pulse_segment is five 8-byte fields");
static_assert(sizeof(pulse_view) == 16, "pulse_view is two 8-byte fields");

int64_t pulse_segment_tiles(const int64_t *n, int32_t nseg, int64_t *tile0, uint32_t *tile_seg) {
    if (!n || nseg < 1) return PULSE_EINVAL;
    int64_t t = 0;
    for (int32_t s = 0; s < nseg; ++s) {
        if (n[s] < 1 || n[s] > kMaxIndexed) return PULSE_ERANGE;
        const int64_t k = (n[s] + 16383) / 16384;
        if (tile0) tile0[s] = t;
        if (tile_seg)
            for (int64_t j = 0; j < k; ++j) tile_seg[t + j] = (uint32_t)s;
        t += k;
    }
    if (t > 0xFFFFFFFFll) return PULSE_ERANGE;
    return t;
}

int pulse_cast_diff_segments(const pulse_segment *segs, int32_t nseg, const uint32_t *tile_seg, int64_t ntiles,
                             int32_t *patch_idx, uint16_t *patch_val, int64_t patch_cap, int64_t *seg_offsets,
                             uint32_t *d_status, void *ws, size_t ws_bytes, int32_t with_new, hipStream_t stream) {
    if (!segs || !tile_seg || !patch_idx || !patch_val || !seg_offsets || !d_status || nseg < 1 || ntiles < nseg ||
        patch_cap < 0 || (with_new != 0 && with_new != 1))
        return PULSE_EINVAL;
    if (ntiles > 0xFFFFFFFFll) return PULSE_ERANGE;
    if (!ws || ws_bytes < pulse_workspace_bytes(PULSE_OP_CAST_DIFF_SEGMENTS, ntiles, 0)) return PULSE_EWORKSPACE;
    return pulse_launch_cast_diff_segments(segs, nseg, tile_seg, ntiles, patch_idx, patch_val, patch_cap, seg_offsets,
                                           d_status, ws, with_new, stream);
}

int pulse_apply_patch_segments(const pulse_view *views, int32_t nseg, const int32_t *patch_idx,
                               const uint16_t *patch_val, const int64_t *seg_offsets, int64_t max_count,
                               uint32_t *d_status, hipStream_t stream) {
    if (!views || !patch_idx || !patch_val || !seg_offsets || !d_status || nseg < 1 || max_count < 0)
        return PULSE_EINVAL;
    if (max_count == 0) return PULSE_OK;
    return pulse_launch_apply_patch_segments(views, nseg, patch_idx, patch_val, seg_offsets, max_count, d_status,
                                             stream);
}

}  // extern "C"


extern "C" {

int64_t pulse_apply_quant_plan_bytes(int32_t ngroups) { return pulse_apply_quant_plan_size(ngroups); }

int pulse_apply_quant_plan(const pulse_aq_group *groups, int32_t ngroups, int64_t n, void *plan, int64_t plan_bytes,
                           int64_t *nblocks) {
    if (!groups || ngroups < 1 || !plan || !nblocks || n < 1) return PULSE_EINVAL;
    if (n > kMaxIndexed) return PULSE_ERANGE;
    if (!aligned16(plan)) return PULSE_EALIGN;
    const int r = pulse_build_apply_quant_plan(groups, ngroups, n, plan, plan_bytes, nblocks);
    switch (r) {
    case 0: return PULSE_OK;
    case -2: return PULSE_EALIGN;
    case -3: return PULSE_ERANGE;
    case -4: return PULSE_EWORKSPACE;
    case -5: return PULSE_EHIP;
    default: return PULSE_EINVAL;
    }
}

int pulse_apply_quant(uint16_t *b, int64_t n, const int32_t *patch_idx, const uint16_t *patch_val,
                      const int64_t *d_count, int64_t max_count, const void *plan, int64_t nblocks,
                      uint32_t *d_status, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!b || !patch_idx || !patch_val || !d_count || !plan || !d_status || n < 1 || max_count < 1 || nblocks < 1)
        return PULSE_EINVAL;
    if (!aligned16(b) || !aligned16(plan)) return PULSE_EALIGN;
    if (n > kMaxIndexed || max_count > kMaxIndexed || nblocks > kMaxIndexed) return PULSE_ERANGE;
    if (!ws || ws_bytes < pulse_workspace_bytes(PULSE_OP_APPLY_QUANT, n, 0)) return PULSE_EWORKSPACE;
    return pulse_launch_apply_quant(b, n, patch_idx, patch_val, d_count, max_count, plan, nblocks, d_status, ws,
                                    stream);
}

}  // extern "C"
