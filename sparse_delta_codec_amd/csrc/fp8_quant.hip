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

template <int MAXS>
__device__ __forceinline__ void quant_block(const QBlock &a, int64_t br, int64_t bc, int64_t e, uint32_t *s_red) {
    const int t = threadIdx.x;
    const int rg = t >> 4, seg = t & 15;
    const int64_t col = bc * 128 + seg * 8;
    const bool col_ok = col < a.cols;  // cols is a multiple of 8

    uint4 v[8];
    bool ok[8];
    uint32_t amax = 0;  // max |x| as BF16 magnitude bits (ordered like the values)
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
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
                amax = lo > amax ? lo : amax;
                amax = hi > amax ? hi : amax;
            }
        }
    }
    amax = wave_reduce_max(amax);
    if (lane_id() == 0) s_red[wave_id()] = amax;
    __syncthreads();
    amax = s_red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) amax = s_red[w] > amax ? s_red[w] : amax;

    const float amax_f = __uint_as_float(amax << 16);
    const float s = amax == 0 ? 1.0f : amax_f / 448.0f;  // IEEE division
    if (t == 0) a.scales[(e * ((a.R + 127) / 128) + br) * a.nbc + bc] = s;

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
        const int64_t r = br * 128 + rg + 16 * i;
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
        *reinterpret_cast<uint2 *>(a.codes + (e * a.R + r) * a.cols + col) = make_uint2(packed[0], packed[1]);
    }
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
