"""GPU parity of the next rows through the C ABI: FP8-view deltas and the
PULSELoCo gate, bit-exact against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_delta_codec_amd as pulse
    from tests.gpu_util import dev, host, zeros  # noqa: E402

SIZES = [1, 15, 16, 17, 1000, 16383, 16384, 16385, 3 * 16384 + 5, 100_007]
# the codes' tiles are 65536 bytes (four rounds of 16384): both sides of a tile, partial rounds
CODE_SIZES = SIZES + [65535, 65536, 65537, 3 * 65536 + 16389, 262_147]


def u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def gpu_fp8_delta(co, cn, so, sn, code_cap=None, scale_cap=None, ws=None):
    nc, ns = co.size, so.size
    code_cap = nc if code_cap is None else code_cap
    scale_cap = ns if scale_cap is None else scale_cap
    ci, cv = zeros(code_cap, torch.int32), zeros(code_cap, torch.uint8)
    si, sv = zeros(scale_cap, torch.int32), zeros(scale_cap, torch.float32)
    cc, sc, st = zeros(1, torch.int64), zeros(1, torch.int64), zeros(1, torch.int32)
    if ws is None:
        ws = pulse.workspace(pulse.PULSE_OP_FP8_DELTA, max(nc, ns))
    pulse.fp8_view_delta(dev(co), dev(cn), dev(so), dev(sn), ci, cv, cc, si, sv, sc, st, ws,
                         code_cap=code_cap, scale_cap=scale_cap)
    torch.cuda.synchronize()
    m, k = int(host(cc)[0]), int(host(sc)[0])
    return dict(code_idx=host(ci)[:min(m, code_cap)], code_val=host(cv)[:min(m, code_cap)], code_count=m,
                scale_idx=host(si)[:min(k, scale_cap)], scale_val=host(sv)[:min(k, scale_cap)], scale_count=k,
                status=int(host(st)[0]))


def same_delta(g, r):
    assert g["code_count"] == r["code_count"] and g["scale_count"] == r["scale_count"]
    assert np.array_equal(g["code_idx"], r["code_idx"]) and np.array_equal(g["code_val"], r["code_val"])
    assert np.array_equal(g["scale_idx"], r["scale_idx"])
    assert np.array_equal(u32(g["scale_val"]), u32(r["scale_val"]))
    assert g["status"] == r["status"]


@pytest.mark.parametrize("n", CODE_SIZES)
@pytest.mark.parametrize("p", [0.0, 0.01, 0.5, 1.0])
def test_fp8_view_delta_matches_oracle(n, p):
    rng = np.random.default_rng(n * 7 + int(p * 100))
    co = rng.integers(0, 256, n, dtype=np.uint8)
    cn = np.where(rng.random(n) < p, (co + rng.integers(1, 256, n)).astype(np.uint8), co)
    ns = max(1, n // 100 + (n % 3))
    so = (np.abs(rng.standard_normal(ns)) * 1e-3).astype(np.float32)
    sn = np.where(rng.random(ns) < p, np.nextafter(so, np.float32(1)), so).astype(np.float32)
    same_delta(gpu_fp8_delta(co, cn, so, sn), oracle.fp8_delta(co, cn, so, sn))


def test_fp8_view_delta_capacity_and_workspace_reuse():
    rng = np.random.default_rng(5)
    big = 5 * 16384 + 77
    ws = pulse.workspace(pulse.PULSE_OP_FP8_DELTA, big)
    for n, p, cap in [(big, 0.3, 1000), (2000, 0.5, None), (big, 0.02, None), (40000, 1.0, 5)]:
        co = rng.integers(0, 256, n, dtype=np.uint8)
        cn = np.where(rng.random(n) < p, (co ^ rng.integers(1, 256, n)).astype(np.uint8), co)
        so = rng.random(n // 1000 + 1).astype(np.float32)
        sn = so.copy()
        sn[::3] *= np.float32(2)
        g = gpu_fp8_delta(co, cn, so, sn, code_cap=cap, ws=ws)
        r = oracle.fp8_delta(co, cn, so, sn, code_cap=cap)
        same_delta(g, r)


def test_fp8_view_round_trip_on_quantised_weights():
    """Quantise two versions on the GPU, take the delta, apply it to the old
    quantisation on the GPU: the new quantisation comes back bit for bit, and
    the delta equals the oracle's."""
    w0, w1 = workload.c1_masters()
    b0 = oracle.cast_bf16(w0).reshape(4096, 1024)
    b1 = oracle.cast_bf16(w1).reshape(4096, 1024)
    nb = 32 * 8
    c0, s0 = zeros(b0.size, torch.uint8), zeros(nb, torch.float32)
    c1, s1 = zeros(b0.size, torch.uint8), zeros(nb, torch.float32)
    pulse.fp8_block_quant([dev(b0)], c0, s0)
    pulse.fp8_block_quant([dev(b1)], c1, s1)
    ci, cv = zeros(b0.size, torch.int32), zeros(b0.size, torch.uint8)
    si, sv = zeros(nb, torch.int32), zeros(nb, torch.float32)
    cc, sc, st = zeros(1, torch.int64), zeros(1, torch.int64), zeros(1, torch.int32)
    ws = pulse.workspace(pulse.PULSE_OP_FP8_DELTA, b0.size)
    pulse.fp8_view_delta(c0, c1, s0, s1, ci, cv, cc, si, sv, sc, st, ws)
    rc0, rs0 = oracle.fp8_block_quant([b0])
    rc1, rs1 = oracle.fp8_block_quant([b1])
    r = oracle.fp8_delta(rc0, rc1, rs0, rs1)
    codes, scales = c0.clone(), s0.clone()
    pulse.fp8_view_apply(codes, scales, ci, cv, cc, si, sv, sc, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    m = int(host(cc)[0])
    assert m == r["code_count"] and np.array_equal(host(ci)[:m], r["code_idx"])
    assert np.array_equal(host(cv)[:m], r["code_val"])
    assert np.array_equal(host(codes), host(c1)) and np.array_equal(host(codes), rc1.reshape(-1))
    assert np.array_equal(u32(host(scales)), u32(rs1).reshape(-1))


def test_fp8_view_apply_bad_index():
    codes, scales = zeros(100, torch.uint8), zeros(4, torch.float32)
    ci = dev(np.array([5, 100, 7], np.int32))
    cv = dev(np.array([1, 2, 3], np.uint8))
    si, sv = dev(np.array([3], np.int32)), dev(np.array([2.5], np.float32))
    cc, sc = dev(np.array([3], np.int64)), dev(np.array([1], np.int64))
    st = zeros(1, torch.int32)
    pulse.fp8_view_apply(codes, scales, ci, cv, cc, si, sv, sc, st)
    torch.cuda.synchronize()
    c = host(codes)
    assert int(host(st)[0]) == pulse.PULSE_DS_BADINDEX and c[5] == 1 and c[7] == 3 and host(scales)[3] == 2.5


# ---- PULSELoCo gate -----------------------------------------------------------------
def gate_inputs(n, scale, seed):
    rng = np.random.default_rng(seed)
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    theta[: n // 8] = (1 + rng.standard_normal(n // 8) * 0.01).astype(np.float32)
    delta = (rng.standard_normal(n) * scale).astype(np.float32)
    resid = (rng.standard_normal(n) * scale * (rng.random(n) < 0.5)).astype(np.float32)
    # subnormals, signed zeros and exact ties must survive on the device
    k = min(n, 8)
    resid[:k] = np.array([1e-40, -1e-41, -0.0, 0.0, 2.0 ** -8, -(2.0 ** -9), 3e-39, 0.0], np.float32)[:k]
    theta[:k] = np.array([1e-38, 0.0, -0.0, 1e-39, 1.0, 1.0, -2e-38, 5.0], np.float32)[:k]
    return theta, delta, resid


def gpu_gate(theta, delta, resid, cap=None, ws=None):
    n = theta.size
    cap = n if cap is None else cap
    idx, val = zeros(cap, torch.int32), zeros(cap, torch.float32)
    cnt, st = zeros(1, torch.int64), zeros(1, torch.int32)
    R = dev(resid)
    if ws is None:
        ws = pulse.workspace(pulse.PULSE_OP_LOCO_GATE, n)
    pulse.pulse_loco_gate(dev(theta), dev(delta), R, idx, val, cnt, st, ws, cap=cap)
    torch.cuda.synchronize()
    m = int(host(cnt)[0])
    return dict(idx=host(idx)[:min(m, cap)], val=host(val)[:min(m, cap)], count=m, resid=host(R),
                status=int(host(st)[0]))


def same_gate(g, r):
    assert g["count"] == r["count"] and g["status"] == r["status"]
    assert np.array_equal(g["idx"], r["idx"])
    assert np.array_equal(u32(g["val"]), u32(r["val"]))
    bad = np.flatnonzero(u32(g["resid"]) != u32(r["resid"]))
    assert bad.size == 0, bad[:5]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("scale", [3e-6, 1e-4, 1e-2])
def test_loco_gate_matches_oracle(n, scale):
    theta, delta, resid = gate_inputs(n, scale, n + int(scale * 1e6))
    same_gate(gpu_gate(theta, delta, resid), oracle.loco_gate(theta, delta, resid))


def test_loco_gate_capacity_keeps_unsent_entries():
    n = 3 * 16384 + 11
    theta, delta, resid = gate_inputs(n, 1e-2, 21)
    for cap in (0, 1, 700, 20000):
        same_gate(gpu_gate(theta, delta, resid, cap=cap), oracle.loco_gate(theta, delta, resid, cap=cap))


def test_loco_rounds_and_accumulate():
    """Eight rounds of one worker against a fixed checkpoint (the buffer carried
    from round to round on the device), each round's patch summed into an FP32
    accumulator: every round equals the oracle's."""
    n = 200_003
    rng = np.random.default_rng(31)
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    R, A = zeros(n, torch.float32), zeros(n, torch.float32)
    r_host, a_host = np.zeros(n, np.float32), np.zeros(n, np.float32)
    idx, val = zeros(n, torch.int32), zeros(n, torch.float32)
    cnt, st = zeros(1, torch.int64), zeros(1, torch.int32)
    ws = pulse.workspace(pulse.PULSE_OP_LOCO_GATE, n)
    T = dev(theta)
    for rnd in range(8):
        delta = (rng.standard_normal(n) * 3e-5).astype(np.float32)
        pulse.pulse_loco_gate(T, dev(delta), R, idx, val, cnt, st, ws)
        pulse.pulse_loco_accumulate(A, idx, val, cnt, st)
        torch.cuda.synchronize()
        ref = oracle.loco_gate(theta, delta, r_host)
        r_host = ref["resid"]
        a_host, _ = oracle.loco_accumulate(a_host, ref["idx"], ref["val"])
        m = int(host(cnt)[0])
        assert m == ref["count"], rnd
        assert np.array_equal(host(idx)[:m], ref["idx"]), rnd
        assert np.array_equal(u32(host(R)), u32(r_host)), rnd
        assert np.array_equal(u32(host(A)), u32(a_host)), rnd
    assert int(host(st)[0]) == 0


# ---- patch-stream compression -------------------------------------------------------
def random_patch(m, n, seed):
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(n, m, replace=False)).astype(np.int32)
    val = rng.integers(0, 1 << 16, m, dtype=np.uint16)
    return idx, val


PATCH_CASES = [(1, 1, 1), (3, 100, 2), (4, 10, 3), (1000, 2 ** 31 - 1, 4), (65535, 10 ** 6, 5),
               (65536, 65536, 6), (65537, 3 * 10 ** 6, 7), (200_003, 2_400_000, 8), (140_000, 2 ** 31 - 1, 9)]


@pytest.mark.parametrize("m,n,seed", PATCH_CASES)
def test_patch_pack_and_unpack_match_oracle(m, n, seed):
    idx, val = random_patch(m, n, seed)
    nb = pulse.patch_packed_bytes(m)
    P = zeros(nb, torch.uint8)
    pulse.patch_pack(dev(idx), dev(val), m, P)
    torch.cuda.synchronize()
    ref = oracle.patch_pack(idx, val)
    assert nb == ref.size and np.array_equal(host(P)[:nb], ref)
    I, V, st = zeros(m, torch.int32), zeros(m, torch.int16), zeros(1, torch.int32)
    ws = pulse.workspace(pulse.PULSE_OP_PATCH_UNPACK, m)
    pulse.patch_unpack(dev(ref), m, I, V, st, ws)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert np.array_equal(host(I)[:m], idx) and np.array_equal(host(V, np.uint16)[:m], val)


def test_patch_unpack_flags_index_overflow_and_reuses_workspace():
    ws = pulse.workspace(pulse.PULSE_OP_PATCH_UNPACK, 300_000)
    for it, (m, n, seed) in enumerate([(300_000, 10 ** 7, 1), (5, 50, 2), (70_000, 2 ** 31 - 1, 3)]):
        idx, val = random_patch(m, n, seed)
        p = oracle.patch_pack(idx, val)
        I, V, st = zeros(m, torch.int32), zeros(m, torch.int16), zeros(1, torch.int32)
        pulse.patch_unpack(dev(p), m, I, V, st, ws)
        torch.cuda.synchronize()
        assert int(host(st)[0]) == 0 and np.array_equal(host(I)[:m], idx), it
    p = oracle.patch_pack(np.array([2 ** 31 - 2, 2 ** 31 - 1], np.int32), np.array([1, 2], np.uint16))
    p[1] = 1  # second gap 1: index 2^31
    I, V, st = zeros(2, torch.int32), zeros(2, torch.int16), zeros(1, torch.int32)
    pulse.patch_unpack(dev(p), 2, I, V, st, ws)
    torch.cuda.synchronize()
    assert int(host(st)[0]) & pulse.PULSE_DS_CORRUPT


def test_compressed_patch_round_trip_through_the_lz4_kernels():
    """The sender's cast/diff/compact patch of the C1 step, packed and LZ4-encoded
    on the GPU, equals the oracle's payload byte for byte; decoded and unpacked
    on the GPU it is the patch again, and applying it rebuilds the new view."""
    w0, w1 = workload.c1_masters()
    b0 = oracle.cast_bf16(w0).reshape(-1)
    r = oracle.cast_diff(w1, b0, want_mask=False)
    m = r["count"]
    nb = pulse.patch_packed_bytes(m)
    P = zeros(nb, torch.uint8)
    pulse.patch_pack(dev(r["idx"]), dev(r["val"]), m, P)
    cap = pulse.lz4_payload_bound(nb)
    payload = zeros(cap, torch.uint8)
    nblk = nb // 65536
    sizes, offs = zeros(nblk, torch.int32), zeros(nblk, torch.int64)
    tot, st = zeros(1, torch.int64), zeros(1, torch.int32)
    pulse.lz4_encode_blocks(P, payload, sizes, offs, tot, st, pulse.workspace(pulse.PULSE_OP_LZ4_ENCODE, nb, 65536))
    torch.cuda.synchronize()
    packed_ref, enc = oracle.patch_compress(r["idx"], r["val"])
    t = int(host(tot)[0])
    assert int(host(st)[0]) == 0 and t == enc["total"] and np.array_equal(host(payload)[:t], enc["payload"])
    D = zeros(nb, torch.uint8)
    pulse.lz4_decode_blocks(payload, offs, sizes, D, st, pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nblk, cap),
                            mode=0, nbytes=nb, payload_bytes=cap)
    I, V = zeros(m, torch.int32), zeros(m, torch.int16)
    pulse.patch_unpack(D, m, I, V, st, pulse.workspace(pulse.PULSE_OP_PATCH_UNPACK, m))
    B = dev(b0)
    pulse.pulse_apply_patch(B, I, V, dev(np.array([m], np.int64)), st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert np.array_equal(host(I)[:m], r["idx"]) and np.array_equal(host(V, np.uint16)[:m], r["val"])
    assert np.array_equal(host(B, np.uint16), r["b_new"])


# ---- one launch over a list of tensors -------------------------------------------------
def tensor_list(sizes, seed):
    rng = np.random.default_rng(seed)
    ws, bs = [], []
    for n in sizes:
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        if n > 3:
            w0[: n // 4] = (1 + rng.standard_normal(n // 4) * 0.01).astype(np.float32)
        w1 = (w0 - np.float32(3e-6) * np.clip(rng.standard_normal(n), -3, 3).astype(np.float32)).astype(np.float32)
        ws.append(w1)
        bs.append(oracle.cast_bf16(w0))
    return ws, bs


def run_segments(ws, bs, with_new=True, cap=None):
    W = [dev(w) for w in ws]
    B = [dev(b) for b in bs]
    N = [zeros(b.size, torch.int16) for b in bs] if with_new else None
    table = pulse.SegmentTable(W, B, N)
    total = sum(w.size for w in ws)
    cap = total if cap is None else cap
    idx, val = zeros(cap, torch.int32), zeros(cap, torch.int16)
    offs, st = zeros(len(ws) + 1, torch.int64), zeros(1, torch.int32)
    ws_ = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_SEGMENTS, table.ntiles)
    pulse.pulse_cast_diff_segments(table, idx[:cap] if cap else idx[:1], val, offs, st, ws_)
    torch.cuda.synchronize()
    return table, W, B, N, idx, val, offs, st


@pytest.mark.parametrize("seed,sizes", [
    (1, [1, 15, 16384, 16385, 40000, 3 * 16384 + 7, 2]),
    (2, [5] * 40 + [70000]),
    (3, list(np.random.default_rng(9).integers(1, 50000, 300))),
])
def test_cast_diff_segments_match_oracle(seed, sizes):
    ws, bs = tensor_list(sizes, seed)
    ref = oracle.cast_diff_segments(ws, bs)
    table, W, B, N, idx, val, offs, st = run_segments(ws, bs)
    assert int(host(st)[0]) == 0
    assert np.array_equal(host(offs)[: len(ws) + 1], ref["seg_offsets"])
    m = ref["count"]
    assert np.array_equal(host(idx)[:m], ref["idx"]) and np.array_equal(host(val, np.uint16)[:m], ref["val"])
    for s in range(len(ws)):
        assert np.array_equal(host(N[s], np.uint16), ref["b_new"][s]), s
    # the receiver's side over separately allocated views
    R = [dev(b) for b in bs]
    pulse.pulse_apply_patch_segments(pulse.ViewTable(R), idx, val, offs, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    for s in range(len(ws)):
        assert np.array_equal(host(R[s], np.uint16), ref["b_new"][s]), s


def test_cast_diff_segments_without_new_view_and_capacity():
    ws, bs = tensor_list([20000, 33, 16384 * 2], 4)
    ref = oracle.cast_diff_segments(ws, bs, cap=100)
    table, W, B, N, idx, val, offs, st = run_segments(ws, bs, with_new=False, cap=100)
    assert int(host(st)[0]) == pulse.PULSE_DS_CAPACITY
    assert np.array_equal(host(offs)[:4], ref["seg_offsets"])
    assert np.array_equal(host(idx)[:100], ref["idx"]) and np.array_equal(host(val, np.uint16)[:100], ref["val"])


def test_cast_diff_segments_flags_a_broken_table_entry():
    ws, bs = tensor_list([3000, 3000], 5)
    W = [dev(w) for w in ws]
    B = [dev(b) for b in bs]
    table = pulse.SegmentTable(W, B)
    tab = table.segs.cpu()
    tab[1, 1] += 2  # b_old of tensor 1 no longer 16-byte aligned
    table.segs = tab.cuda()
    idx, val = zeros(6000, torch.int32), zeros(6000, torch.int16)
    offs, st = zeros(3, torch.int64), zeros(1, torch.int32)
    pulse.pulse_cast_diff_segments(table, idx, val, offs, st, pulse.workspace(pulse.PULSE_OP_CAST_DIFF_SEGMENTS, 2))
    torch.cuda.synchronize()
    ref = oracle.cast_diff_segments(ws[:1], bs[:1])
    assert int(host(st)[0]) & pulse.PULSE_DS_BADSEGMENT
    m = ref["count"]
    assert host(offs)[2] == m and np.array_equal(host(idx)[:m], ref["idx"])
