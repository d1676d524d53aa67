"""Pins of the oracle's FP8-view deltas and of the PULSELoCo gate.

FP8-view deltas: numpy's flatnonzero over the codes and over the scale bit
patterns (a library routine), the round trip apply(quant(old), delta) ==
quant(new) with the quantiser pinned in test_oracle_fp8, and the pages' claim
that coarser cells change fewer served values.

LoCo gate: torch's float32 add and BF16 cast (both library routines, the cast
pinned on all 2^32 patterns in test_oracle_cast), the exact conservation of the
accumulated update, closed forms for constant updates around 1.0 (the rounding
boundaries of the pages' worked example), and numpy's add.at for the
receiver's accumulation.
"""
import numpy as np
import torch

import oracle
import workload


def u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


# ---- FP8-view deltas -----------------------------------------------------------
def _quant_pair():
    w0, w1 = workload.c1_masters()
    b0 = oracle.cast_bf16(w0).reshape(4096, 1024)
    b1 = oracle.cast_bf16(w1).reshape(4096, 1024)
    c0, s0 = oracle.fp8_block_quant([b0])
    c1, s1 = oracle.fp8_block_quant([b1])
    return b0, b1, c0, s0, c1, s1


def test_fp8_delta_matches_flatnonzero():
    rng = np.random.default_rng(3)
    for n, p in [(0, 0.1), (1, 1.0), (1000, 0.0), (4097, 0.02), (70000, 0.5), (33, 1.0)]:
        co = rng.integers(0, 256, n, dtype=np.uint8)
        cn = np.where(rng.random(n) < p, rng.integers(0, 256, n, dtype=np.uint8), co)
        so = rng.standard_normal(n // 7 + 1).astype(np.float32)
        sn = np.where(rng.random(so.size) < p, so * np.float32(1.5), so).astype(np.float32)
        sn[0] = -0.0 if so[0] == 0 else sn[0]
        d = oracle.fp8_delta(co, cn, so, sn)
        ref = np.flatnonzero(co != cn)
        assert d["code_count"] == ref.size and np.array_equal(d["code_idx"], ref)
        assert np.array_equal(d["code_val"], cn[ref])
        sref = np.flatnonzero(u32(so) != u32(sn))
        assert d["scale_count"] == sref.size and np.array_equal(d["scale_idx"], sref)
        assert np.array_equal(u32(d["scale_val"]), u32(sn)[sref])
        assert d["status"] == 0


def test_fp8_delta_signed_zero_scale_is_a_change():
    d = oracle.fp8_delta(np.zeros(4, np.uint8), np.zeros(4, np.uint8),
                         np.array([0.0, 1.0], np.float32), np.array([-0.0, 1.0], np.float32))
    assert d["code_count"] == 0 and d["scale_count"] == 1 and list(d["scale_idx"]) == [0]


def test_fp8_delta_capacity():
    co = np.zeros(100, np.uint8)
    cn = co.copy()
    cn[[3, 10, 50, 99]] = 7
    d = oracle.fp8_delta(co, cn, np.ones(2, np.float32), np.ones(2, np.float32), code_cap=2)
    assert d["code_count"] == 4 and list(d["code_idx"]) == [3, 10] and d["status"] == oracle.CAPACITY


def test_fp8_delta_round_trip_rebuilds_new_quantisation():
    """apply(quant(B_old), delta) == quant(B_new), codes and scales bit for bit."""
    b0, b1, c0, s0, c1, s1 = _quant_pair()
    d = oracle.fp8_delta(c0, c1, s0, s1)
    c, s, st = oracle.fp8_apply_delta(c0, s0, d["code_idx"], d["code_val"], d["scale_idx"], d["scale_val"])
    assert st == 0
    assert np.array_equal(c, c1.reshape(-1)) and np.array_equal(u32(s), u32(s1).reshape(-1))


def test_fp8_view_changes_less_than_bf16_view():
    """Coarser cells change fewer served values: the E4M3 floor is 2^4 times the
    BF16 one (theta / 2^(m+1) with m = 3 against m = 7), so on the same step
    the FP8 codes change several times less often than the BF16 values."""
    b0, b1, c0, s0, c1, s1 = _quant_pair()
    f_bf16 = (b0 != b1).mean()
    f_fp8 = (c0 != c1).mean()
    assert 0.0 < f_fp8 < f_bf16 / 4


def test_fp8_apply_bad_index():
    c, s, st = oracle.fp8_apply_delta(np.zeros(8, np.uint8), np.ones(2, np.float32),
                                      np.array([1, 8], np.int32), np.array([5, 6], np.uint8),
                                      np.array([2], np.int32), np.array([3.0], np.float32))
    assert st == oracle.BADINDEX and c[1] == 5 and list(s) == [1.0, 1.0]


# ---- LoCo gate ------------------------------------------------------------------
def torch_gate(theta, delta, resid):
    th, de, r = (torch.from_numpy(np.ascontiguousarray(x, np.float32)) for x in (theta, delta, resid))
    a = r + de
    moved = th + a
    vis = moved.to(torch.bfloat16).view(torch.int16) != th.to(torch.bfloat16).view(torch.int16)
    new_r = torch.where(vis, torch.zeros_like(a), a)
    return vis.numpy(), a.numpy(), new_r.numpy()


def test_gate_matches_torch():
    rng = np.random.default_rng(11)
    for n, scale in [(0, 1e-3), (1, 1.0), (5000, 3e-6), (20000, 1e-4), (777, 1e-2)]:
        theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
        theta[: n // 10] = (1 + rng.standard_normal(n // 10) * 0.01).astype(np.float32)
        delta = (rng.standard_normal(n) * scale).astype(np.float32)
        resid = (rng.standard_normal(n) * scale * (rng.random(n) < 0.5)).astype(np.float32)
        d = oracle.loco_gate(theta, delta, resid)
        vis, a, new_r = torch_gate(theta, delta, resid)
        ref = np.flatnonzero(vis)
        assert d["count"] == ref.size and np.array_equal(d["idx"], ref)
        assert np.array_equal(u32(d["val"]), u32(a)[ref])
        assert np.array_equal(u32(d["resid"]), u32(new_r))


def test_gate_conserves_the_update():
    """Nothing is lost: the new buffer plus the sent entries equal, element by
    element and exactly, the old buffer plus the pseudo-gradient."""
    rng = np.random.default_rng(12)
    n = 50000
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    delta = (rng.standard_normal(n) * 2e-5).astype(np.float32)
    resid = (rng.standard_normal(n) * 2e-5).astype(np.float32)
    d = oracle.loco_gate(theta, delta, resid)
    dense = np.zeros(n, np.float32)
    dense[d["idx"]] = d["val"]
    a = resid + delta
    assert np.array_equal(u32(d["resid"] + dense), u32(a))
    sent = np.zeros(n, bool)
    sent[d["idx"]] = True
    assert np.all(d["resid"][sent] == 0)
    # every entry held back leaves the BF16 view of the checkpoint as it is
    kept = ~sent
    b_th = oracle.cast_bf16(theta)
    b_mv = oracle.cast_bf16((theta + d["resid"]).astype(np.float32))
    assert np.array_equal(b_th[kept], b_mv[kept])
    assert np.all(b_th[sent] != oracle.cast_bf16((theta + dense).astype(np.float32))[sent])


def _rounds(theta, step, rounds):
    th = np.full(1, theta, np.float32)
    r = np.zeros(1, np.float32)
    sent_at = []
    for k in range(1, rounds + 1):
        d = oracle.loco_gate(th, np.full(1, step, np.float32), r)
        r = d["resid"]
        if d["count"]:
            sent_at.append((k, float(d["val"][0])))
    return sent_at, float(r[0])


def test_gate_closed_form_near_one():
    """theta = 1: upward the view moves once the update exceeds 2^-8 (an exact
    2^-8 is a tie back to 1.0); downward the spacing halves, so 2^-9 is the
    boundary.  A constant update of 1e-3 is therefore sent every 4th round
    going up and every 2nd round going down, with the accumulated value."""
    up, r = _rounds(1.0, 1e-3, 12)
    assert [k for k, _ in up] == [4, 8, 12] and r == 0.0
    acc = np.float32(0)
    for _ in range(4):
        acc = np.float32(acc + np.float32(1e-3))
    assert all(v == float(acc) for _, v in up)
    down, _ = _rounds(1.0, -1e-3, 6)
    assert [k for k, _ in down] == [2, 4, 6]
    # an update at exactly half an ulp is a tie to even and never alone visible
    tie, r = _rounds(1.0, 2.0 ** -8, 1)
    assert tie == [] and r == 2.0 ** -8


def test_gate_zero_update_sends_nothing():
    n = 1000
    d = oracle.loco_gate(np.ones(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32))
    assert d["count"] == 0 and np.all(d["resid"] == 0)


def test_gate_capacity():
    n = 100
    d = oracle.loco_gate(np.zeros(n, np.float32), np.ones(n, np.float32), np.zeros(n, np.float32), cap=10)
    assert d["count"] == n and list(d["idx"]) == list(range(10)) and d["status"] == oracle.CAPACITY
    # what could not be sent stays in the buffer: nothing is lost
    assert np.all(d["resid"][:10] == 0) and np.all(d["resid"][10:] == 1.0)


def test_accumulate_matches_numpy():
    rng = np.random.default_rng(13)
    n = 10000
    acc = rng.standard_normal(n).astype(np.float32)
    idx = np.sort(rng.choice(n, 700, replace=False)).astype(np.int32)
    val = (rng.standard_normal(700) * 1e-3).astype(np.float32)
    ours, st = oracle.loco_accumulate(acc, idx, val)
    ref = acc.copy()
    np.add.at(ref, idx, val)
    assert st == 0 and np.array_equal(u32(ours), u32(ref))
    _, st = oracle.loco_accumulate(acc, np.array([n], np.int32), np.array([1.0], np.float32))
    assert st == oracle.BADINDEX


# ---- patch-stream compression ---------------------------------------------------------
def numpy_pack(idx, val, G=65536):
    """The packed form built with numpy: np.diff for the gaps, little-endian byte
    views for the planes."""
    m = idx.size
    groups = (m + G - 1) // G
    gaps = np.zeros(groups * G, np.uint32)
    vals = np.zeros(groups * G, np.uint16)
    gaps[:m] = (np.diff(idx.astype(np.int64), prepend=-1) - 1).astype(np.uint32)
    vals[:m] = val
    gb = gaps.view(np.uint8).reshape(groups, G, 4)
    vb = vals.view(np.uint8).reshape(groups, G, 2)
    planes = np.concatenate([gb.transpose(0, 2, 1), vb.transpose(0, 2, 1)], axis=1)  # [groups, 6, G]
    return planes.reshape(-1)


def random_patch(m, n, seed):
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(n, m, replace=False)).astype(np.int32)
    val = rng.integers(0, 1 << 16, m, dtype=np.uint16)
    return idx, val


def test_pack_matches_numpy_and_round_trips():
    for m, n, seed in [(0, 10, 1), (1, 1, 2), (5, 2 ** 31 - 1, 3), (65535, 10 ** 6, 4), (65536, 65536, 5),
                       (65537, 2 * 10 ** 6, 6), (200_000, 2 ** 31 - 1, 7), (150_000, 1_900_000, 8)]:
        idx, val = random_patch(m, n, seed)
        p = oracle.patch_pack(idx, val)
        assert np.array_equal(p, numpy_pack(idx, val)), (m, n)
        back = oracle.patch_unpack(p, m)
        assert back is not None and np.array_equal(back[0], idx) and np.array_equal(back[1], val)


def test_pack_closed_forms():
    """Consecutive indices from 0 with one value: every plane of the group is a
    constant 64 KiB block, whose canonical LZ4 encoding is 267 bytes (pinned in
    test_oracle_lz4), so a full group compresses to 6 * 267 bytes."""
    m = 65536
    idx = np.arange(m, dtype=np.int32)
    val = np.full(m, 0x3F80, np.uint16)
    packed, enc = oracle.patch_compress(idx, val)
    assert np.all(packed[: 4 * m] == 0) and np.all(packed[4 * m: 5 * m] == 0x80) and np.all(packed[5 * m:] == 0x3F)
    assert enc["total"] == 6 * 267


def test_unpack_rejects_index_overflow():
    p = oracle.patch_pack(np.array([2 ** 31 - 2], np.int32), np.array([1], np.uint16))
    assert oracle.patch_unpack(p, 1)[0][0] == 2 ** 31 - 2
    p[0:4 * 65536:65536] = 0xFF  # gap 2^32 - 1
    assert oracle.patch_unpack(p, 1) is None


def test_compressed_patch_round_trip_on_the_c1_step():
    """The whole path on the C1 step: cast/diff/compact, pack, LZ4 encode, LZ4
    decode, unpack gives the patch back, smaller than the raw 6 B per entry."""
    w0, w1 = workload.c1_masters()
    r = oracle.cast_diff(w1, oracle.cast_bf16(w0), want_mask=False)
    packed, enc = oracle.patch_compress(r["idx"], r["val"])
    dec, st = oracle.lz4_decode_blocks(enc["payload"], enc["offsets"], enc["sizes"],
                                       np.zeros(packed.size, np.uint8), mode=0)
    assert st == 0 and np.array_equal(dec, packed)
    back = oracle.patch_unpack(dec, r["count"])
    assert np.array_equal(back[0], r["idx"]) and np.array_equal(back[1], r["val"])
    assert enc["total"] < 6 * r["count"] * 0.6


# ---- one call over a list of tensors ----------------------------------------------------
def torch_cast(w):
    return torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def tensor_list(sizes, seed):
    rng = np.random.default_rng(seed)
    ws, bs = [], []
    for n in sizes:
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        w1 = (w0 - np.float32(3e-6) * np.clip(rng.standard_normal(n), -3, 3).astype(np.float32)).astype(np.float32)
        ws.append(w1)
        bs.append(torch_cast(w0))
    return ws, bs


def test_segments_match_per_tensor_brute_force():
    """The list call equals, tensor by tensor, torch's cast compared with the
    old view and numpy's flatnonzero, the entries concatenated in list order."""
    sizes = [1, 16383, 16384, 16385, 5, 40000, 2, 3 * 16384 + 7]
    ws, bs = tensor_list(sizes, 21)
    r = oracle.cast_diff_segments(ws, bs)
    pos = 0
    for s, (w, b) in enumerate(zip(ws, bs)):
        new = torch_cast(w)
        loc = np.flatnonzero(new != b)
        assert r["seg_offsets"][s] == pos
        assert np.array_equal(r["idx"][pos:pos + loc.size], loc)
        assert np.array_equal(r["val"][pos:pos + loc.size], new[loc])
        assert np.array_equal(r["b_new"][s], new)
        pos += loc.size
    assert r["seg_offsets"][-1] == pos == r["count"] and r["status"] == 0
    views, st = oracle.apply_patch_segments(bs, r["idx"], r["val"], r["seg_offsets"])
    assert st == 0 and all(np.array_equal(v, nb) for v, nb in zip(views, r["b_new"]))


def test_segments_capacity():
    ws, bs = tensor_list([1000, 2000], 22)
    full = oracle.cast_diff_segments(ws, bs)
    r = oracle.cast_diff_segments(ws, bs, cap=10)
    assert r["count"] == full["count"] and r["status"] == oracle.CAPACITY
    assert np.array_equal(r["idx"], full["idx"][:10]) and np.array_equal(r["seg_offsets"], full["seg_offsets"])
