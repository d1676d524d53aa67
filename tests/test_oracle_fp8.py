"""Pins of the oracle's stacking + BF16 -> FP8-E4M3 128x128 block quantiser (row a7).

The pages only say the sender fuses projections and quantises BF16 training
weights for FP8 inference [Perplexity, "Potok zadan"; opening paragraph]; the
format (OCP E4M3 "fn"), block shape, scale rule and rounding are readings.
Pins: torch.float8_e4m3fn (a library conversion), a nearest-of-set search over
the E4M3 values, numpy's IEEE float32 division, closed forms for constant
blocks, the stacking invariant and the rounding error bound.
"""
import numpy as np
import torch

import oracle


def e4m3_values():
    """All 254 finite E4M3 codes and their values (binary64), from the format:
    bias 7, 3 mantissa bits, subnormals m * 2^-9, 0x7F / 0xFF are NaN."""
    codes, vals = [], []
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(-v if c & 0x80 else v)
    return np.array(codes), np.array(vals)


def nearest_of_set(x):
    """Nearest finite E4M3 (ties to even code), saturating beyond 448."""
    codes, vals = e4m3_values()
    pos = codes < 0x80
    pc, pv = codes[pos], vals[pos]
    order = np.argsort(pv)
    pc, pv = pc[order], pv[order]
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    j = np.clip(np.searchsorted(pv, a), 1, pv.size - 1)
    lo, hi = pv[j - 1], pv[j]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & ((pc[j] & 1) == 0))
    res = np.where(pick_hi, pc[j], pc[j - 1])
    sign = (x.view(np.uint32) >> 31).astype(np.int64) << 7
    return (res | sign).astype(np.uint8)


def oracle_codes(x):
    return np.array([oracle.e4m3_rne(float(v)) for v in x], np.uint8)


def probe_values():
    """All BF16 values below 464 in magnitude, every E4M3 midpoint and its float32
    neighbours, and a random float32 sample in range."""
    b = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b) & (np.abs(b) < 464)]
    _, vals = e4m3_values()
    pv = np.unique(np.abs(vals))
    mids = ((pv[:-1] + pv[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rng = np.random.default_rng(21)
    r = (rng.random(60000) * 928 - 464).astype(np.float32)
    tiny = (rng.random(20000) * 2.0 ** -5).astype(np.float32)
    allv = np.concatenate([b, mids, -mids, r, tiny, -tiny, np.float32([0.0, -0.0, 448.0, 463.9, 464.0])])
    return allv.astype(np.float32)


def test_e4m3_matches_torch_and_nearest_of_set():
    x = probe_values()
    ours = oracle_codes(x)
    below = np.abs(x) < 464
    ref_t = torch.from_numpy(x[below]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[below], ref_t)
    assert np.array_equal(ours, nearest_of_set(x))


def test_e4m3_special_values():
    assert oracle.e4m3_rne(448.0) == 0x7E
    assert oracle.e4m3_rne(463.9) == 0x7E
    assert oracle.e4m3_rne(464.0) == 0x7E          # saturating (no Inf in E4M3 "fn")
    assert oracle.e4m3_rne(1e6) == 0x7E and oracle.e4m3_rne(-1e6) == 0xFE
    assert oracle.e4m3_rne(2.0 ** -10) == 0x00     # tie between 0 and 2^-9 -> even
    assert oracle.e4m3_rne(1.5 * 2.0 ** -9) == 0x02
    assert oracle.e4m3_rne(-0.0) == 0x80
    assert oracle.e4m3_rne(2.0 ** -6) == 0x08      # smallest normal


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def as_f32(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


def test_block_quant_against_numpy_division_and_torch():
    """codes == e4m3(fl32(x / s)), s = fl32(amax / 448), recomputed with numpy's
    IEEE float32 division and torch's E4M3 conversion."""
    rng = np.random.default_rng(2)
    w = bf16(rng.standard_normal((256, 384)) * 0.02)
    w[0:128, 0:128] = bf16(rng.standard_normal((128, 128)) * 1e-38)  # subnormal-scale block
    w[128:256, 256:384] = 0                                          # zero block -> s = 1
    codes, scales = oracle.fp8_block_quant([w])
    xf = as_f32(w)
    for br in range(2):
        for bc in range(3):
            blk = xf[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            assert scales[0, br, bc] == s
            q = (blk / s).astype(np.float32)
            ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[0, br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128], ref)


def quant_by_numpy_and_torch(x_u16):
    """Block by block over a stacked [R, C] BF16 matrix: amax by numpy over the
    block's valid elements, s = fl32(amax / 448) (numpy float32 division),
    q = fl32(x / s) (numpy float32 division), codes by torch's E4M3 conversion
    (|q| stays below 464, where torch and the saturating rule agree)."""
    xf = as_f32(x_u16)
    R, C = xf.shape
    codes = np.empty((R, C), np.uint8)
    scales = np.empty(((R + 127) // 128, (C + 127) // 128), np.float32)
    for br in range(scales.shape[0]):
        for bc in range(scales.shape[1]):
            rs, cs = slice(br * 128, min(R, br * 128 + 128)), slice(bc * 128, min(C, bc * 128 + 128))
            blk = xf[rs, cs]
            amax = np.float32(np.abs(blk).max())
            s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            q = (blk / s).astype(np.float32)
            assert np.all(np.abs(q) < 464)
            codes[rs, cs] = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            scales[br, bc] = s
    return codes, scales


def ragged_source(rng, shape, seed_scale=0.02):
    """BF16 weights with blocks at very different scales: normal, subnormal,
    all zero and constant stretches, so edge blocks see every scale rule."""
    w = bf16(rng.standard_normal(shape) * seed_scale)
    r, c = shape
    if r > 3 and c > 3:
        w[: r // 3, : c // 3] = bf16(rng.standard_normal((r // 3, c // 3)) * 1e-39)
        w[r // 2:, c // 2:] = 0
        w[r - 1, :] = bf16([0.75])[0]
    return w


def test_block_quant_ragged_shapes_against_numpy_and_torch():
    """Edge blocks (rows or columns not a multiple of 128) use only their valid
    elements; each of them checked against numpy's division and torch's E4M3,
    block by block, for single sources and for a stack whose second source
    starts and ends inside a 128-row band."""
    rng = np.random.default_rng(12)
    for shapes in ([(200, 136)], [(7, 8)], [(130, 264), (5, 264)], [(1, 1)], [(129, 127)]):
        srcs = [ragged_source(rng, sh) for sh in shapes]
        codes, scales = oracle.fp8_block_quant(srcs)
        ref_c, ref_s = quant_by_numpy_and_torch(np.concatenate(srcs, 0))
        assert np.array_equal(codes[0], ref_c), shapes
        assert np.array_equal(scales[0].view(np.uint32), ref_s.view(np.uint32)), shapes


def test_block_quant_batch_strides_against_numpy_and_torch():
    """A batch of 3 experts laid [gate; up; down] one after another in one
    buffer: [gate; up] of expert e read at a stride of the whole expert (not
    the stacked sources' own size), with ragged rows and columns."""
    rng = np.random.default_rng(13)
    F, H = 72, 136  # gate/up [F, H], down [H, F]
    E = 3
    expert = 3 * F * H
    base = np.concatenate([ragged_source(rng, (F, H), 0.02 * (1 + e)).reshape(-1) for e in range(3 * E)])
    assert base.size == E * expert
    codes, scales = oracle.fp8_block_quant_strided(base, [0, F * H], [F, F], H, E, [expert, expert])
    downc, downs = oracle.fp8_block_quant_strided(base, [2 * F * H], [H], F, E, [expert])
    for e in range(E):
        g = base[e * expert: e * expert + F * H].reshape(F, H)
        u = base[e * expert + F * H: e * expert + 2 * F * H].reshape(F, H)
        d = base[e * expert + 2 * F * H: (e + 1) * expert].reshape(H, F)
        rc, rs = quant_by_numpy_and_torch(np.concatenate([g, u], 0))
        assert np.array_equal(codes[e], rc) and np.array_equal(scales[e].view(np.uint32), rs.view(np.uint32)), e
        rc, rs = quant_by_numpy_and_torch(d)
        assert np.array_equal(downc[e], rc) and np.array_equal(downs[e].view(np.uint32), rs.view(np.uint32)), e


def test_constant_block_closed_form():
    for c in (0.75, -3.0, 1e-3, 2.0 ** -130):
        w = np.full((128, 128), bf16([c])[0], np.uint16)
        codes, scales = oracle.fp8_block_quant([w])
        cf = float(as_f32(np.array([w[0, 0]]))[0])
        assert scales[0, 0, 0] == np.float32(np.float32(abs(cf)) / np.float32(448.0))
        assert np.all(codes == (0xFE if cf < 0 else 0x7E))


def test_stacking_equals_per_source_quantisation():
    """Stacking [q; k; v] (rows multiple of 128) along the output dimension and
    quantising equals quantising each source and stacking the results."""
    rng = np.random.default_rng(8)
    q = bf16(rng.standard_normal((256, 200)) * 0.02)
    k = bf16(rng.standard_normal((128, 200)) * 0.05)
    v = bf16(rng.standard_normal((384, 200)) * 0.01)
    codes, scales = oracle.fp8_block_quant([q, k, v])
    parts = [oracle.fp8_block_quant([s]) for s in (q, k, v)]
    assert np.array_equal(codes[0], np.concatenate([p[0][0] for p in parts], 0))
    assert np.array_equal(scales[0], np.concatenate([p[1][0] for p in parts], 0))
    # batch of experts: entry e is the quantisation of that expert alone
    g = bf16(rng.standard_normal((3, 128, 256)) * 0.02)
    u = bf16(rng.standard_normal((3, 128, 256)) * 0.02)
    cb, sb = oracle.fp8_block_quant([g, u], batch=3)
    for e in range(3):
        ce, se = oracle.fp8_block_quant([g[e], u[e]])
        assert np.array_equal(cb[e], ce[0]) and np.array_equal(sb[e], se[0])


def test_dequantisation_error_bound():
    """|x - e4m3(code) * s| <= s * (half the E4M3 spacing at |x/s|)."""
    rng = np.random.default_rng(6)
    w = bf16(rng.standard_normal((128, 256)) * 0.1)
    codes, scales = oracle.fp8_block_quant([w])
    cvals = dict(zip(*e4m3_values()))
    xf = as_f32(w).astype(np.float64)
    for bc in range(2):
        s = float(scales[0, 0, bc])
        blk = xf[:, bc * 128:(bc + 1) * 128]
        deq = np.vectorize(lambda c: cvals[int(c)])(codes[0][:, bc * 128:(bc + 1) * 128]) * s
        a = np.abs(blk / s)
        spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 3))
        assert np.all(np.abs(blk - deq) <= s * spacing / 2 * (1 + 1e-6))
