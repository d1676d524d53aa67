"""CPU checks of the full-size parity checker (tests/fullsize.py): run piece by
piece on the host threads, it must accept exactly the outputs that the
oracle produces in one whole call, and reject each kind of mistake a GPU
output could carry (a wrong view element, a dropped, extra or shifted patch
entry, a wrong value, a wrong LZ4 size, offset or payload byte, a wrong FP8
code or scale).  The "GPU outputs" here are the oracle's own whole-call
results, copied and then damaged."""
import numpy as np
import pytest

import oracle
import workload
from tests import fullsize as fs


@pytest.fixture
def small_pieces(monkeypatch):
    # 4 mask blocks of 64 KiB per piece, so a few hundred thousand elements span many pieces
    monkeypatch.setattr(fs, "PIECE", 1 << 16)


def masters(n, seed):
    w0, w1 = workload.host_masters(n, seed)
    return w0, w1, oracle.cast_bf16(w0)


def test_patch_and_views_by_pieces(small_pieces):
    n = (1 << 16) * 5 + 12345
    w0, w1, bo = masters(n, 3)
    assert np.array_equal(fs.oracle_cast(w0), bo)
    whole = oracle.cast_diff(w1, bo, want_mask=False)
    ref = fs.OraclePatch(w1, bo)
    assert len(ref.ranges) == 6 and ref.count == whole["count"]
    assert np.array_equal(ref.b_new, whole["b_new"])
    ref.check(whole["count"], whole["idx"], whole["val"], "whole call")
    applied = ref.applied(bo)
    assert np.array_equal(applied, whole["b_new"])
    fs.check_equal(applied, whole["b_new"], "applied")
    c = whole["count"]
    idx, val = whole["idx"].copy(), whole["val"].copy()
    with pytest.raises(AssertionError):
        ref.check(c - 1, idx[:-1], val[:-1], "dropped last entry")
    with pytest.raises(AssertionError):
        k = c // 2
        ref.check(c, np.concatenate([idx[:k], idx[k + 1:], [n - 1]]).astype(np.int32),
                  np.concatenate([val[:k], val[k + 1:], [0]]).astype(np.uint16), "dropped entry, one added")
    bad = idx.copy()
    bad[c // 3] += 1
    with pytest.raises(AssertionError):
        ref.check(c, bad, val, "shifted index")
    badv = val.copy()
    badv[-1] ^= 1
    with pytest.raises(AssertionError):
        ref.check(c, idx, badv, "wrong value")
    view = whole["b_new"].copy()
    view[n - 1] ^= 0x8000
    with pytest.raises(AssertionError):
        fs.check_equal(view, ref.b_new, "view")


def test_lz4_by_pieces(small_pieces):
    n = (1 << 16) * 4 + 777  # a short last block
    w0, w1, bo = masters(n, 4)
    bn = oracle.cast_bf16(w1)
    enc = oracle.lz4_encode_blocks(bo, 65536, src_xor=bn)
    pay, sizes, offs = enc["payload"], enc["sizes"], enc["offsets"]
    assert fs.check_lz4(bo, bn, sizes, offs, enc["total"], pay, "whole call") == enc["total"]
    for damage in ("size", "offset", "byte", "total"):
        s2, o2, p2, t2 = sizes.copy(), offs.copy(), pay.copy(), enc["total"]
        if damage == "size":
            s2[3] += 1
        elif damage == "offset":
            o2[5] += 1
        elif damage == "byte":
            p2[p2.size // 2] ^= 0x40
        else:
            t2 += 1
        with pytest.raises(AssertionError):
            fs.check_lz4(bo, bn, s2, o2, t2, p2, damage)


def test_fp8_by_bands():
    rng = np.random.default_rng(9)
    a = oracle.cast_bf16(rng.standard_normal(300 * 136).astype(np.float32) * 0.02).reshape(300, 136)
    b = oracle.cast_bf16(rng.standard_normal(70 * 136).astype(np.float32) * 0.5).reshape(70, 136)
    view = np.concatenate([np.zeros(8, np.uint16), a.reshape(-1), b.reshape(-1)])
    codes, scales = oracle.fp8_block_quant([a, b])
    fs.check_fp8(view, [(8, 300), (8 + a.size, 70)], 136, codes.reshape(-1), scales.reshape(-1), "whole call")
    c2 = codes.reshape(-1).copy()
    c2[-1] ^= 1
    with pytest.raises(AssertionError):
        fs.check_fp8(view, [(8, 300), (8 + a.size, 70)], 136, c2, scales.reshape(-1), "code")
    s2 = scales.reshape(-1).copy()
    s2[1] = np.nextafter(s2[1], np.float32(1))
    with pytest.raises(AssertionError):
        fs.check_fp8(view, [(8, 300), (8 + a.size, 70)], 136, codes.reshape(-1), s2, "scale")
    with pytest.raises(AssertionError):
        fs.check_fp8(view, [(8, 300), (8 + a.size, 70)], 136, codes.reshape(-1), scales.reshape(-1), "more",
                     more=[(c2, scales.reshape(-1))])


def test_fp8_views_and_delta_by_pieces(small_pieces):
    rng = np.random.default_rng(10)
    rows, cols = 1024, 384
    old = oracle.cast_bf16(rng.standard_normal(rows * cols).astype(np.float32) * 0.02)
    new = old.copy()
    hit = rng.random(old.size) < 0.05
    new[hit] = oracle.cast_bf16(rng.standard_normal(int(hit.sum())).astype(np.float32) * 0.02)
    srcs = [(0, 640), (640 * cols, 384)]
    ref_o = oracle.fp8_block_quant([old.reshape(rows, cols)])
    ref_n = oracle.fp8_block_quant([new.reshape(rows, cols)])
    co, so = np.empty(rows * cols, np.uint8), np.empty(8 * 3, np.float32)
    cn, sn = np.empty_like(co), np.empty_like(so)
    fs.oracle_fp8(old, srcs, cols, co, so)
    fs.oracle_fp8(new, srcs, cols, cn, sn)
    assert np.array_equal(co, ref_o[0].reshape(-1)) and np.array_equal(sn, ref_n[1].reshape(-1))
    whole = oracle.fp8_delta(co, cn, so, sn)
    d = fs.OracleDelta(co, cn, so, sn)
    assert len(d.ranges) == 6 and d.count == whole["code_count"] > 0
    args = (whole["code_count"], whole["code_idx"], whole["code_val"], whole["scale_count"], whole["scale_idx"],
            whole["scale_val"])
    d.check(*args, "whole call")
    bad = list(args)
    bad[1] = bad[1].copy()
    bad[1][0] += 1
    with pytest.raises(AssertionError):
        d.check(*bad, "shifted code index")
    bad = list(args)
    bad[5] = bad[5].copy()
    bad[5][0] = np.float32(bad[5][0]) * np.float32(2)
    with pytest.raises(AssertionError):
        d.check(*bad, "scale value")
