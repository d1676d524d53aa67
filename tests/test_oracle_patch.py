"""Pins of the oracle's diff / compaction / apply / XOR (rows a2, a3, a4).

Pinned by numpy's own routines (flatnonzero, fancy indexing, bitwise_xor),
exhaustive enumeration of tiny inputs, and the invariants the pages state:
applying the patch rebuilds the new version bit for bit, XOR twice is the
identity, and a chain of patches never drifts from the direct cast.
"""
import itertools

import numpy as np

import oracle
import workload

VALS = np.array([0x0000, 0x8000, 0x3F80, 0x3F81], np.uint16)  # includes the +-0 flip


def test_compaction_matches_flatnonzero():
    rng = np.random.default_rng(3)
    for n in (0, 1, 2, 63, 64, 65, 4095, 4096, 4097, 3 * 4096 + 7, 100003):
        old = rng.integers(0, 1 << 16, n, dtype=np.uint16)
        new = old.copy()
        flip = rng.random(n) < 0.1
        new[flip] = rng.integers(0, 1 << 16, int(flip.sum()), dtype=np.uint16)
        idx, val, m, st = oracle.compact(old, new)
        ref = np.flatnonzero(old != new)
        assert m == ref.size and st == 0
        assert np.array_equal(idx, ref.astype(np.int32))
        assert np.array_equal(val, new[ref])


def test_compaction_exhaustive_tiny():
    """All n <= 4 with both views drawn from VALS: 4^(2n) cases per n."""
    for n in range(1, 5):
        for old_t in itertools.product(range(4), repeat=n):
            old = VALS[list(old_t)]
            for new_t in itertools.product(range(4), repeat=n):
                new = VALS[list(new_t)]
                idx, val, m, _ = oracle.compact(old, new)
                expect = [i for i in range(n) if old[i] != new[i]]
                assert list(idx) == expect and m == len(expect)
                assert list(val) == [int(new[i]) for i in expect]


def test_capacity_overflow_keeps_exact_count():
    old = np.zeros(1000, np.uint16)
    new = old.copy()
    new[::3] = 7
    idx, val, m, st = oracle.compact(old, new, cap=100)
    assert m == 334 and st == oracle.CAPACITY
    assert np.array_equal(idx, np.arange(0, 300, 3, dtype=np.int32))


def test_cast_diff_equals_cast_then_compact_on_c1():
    w0, w1 = workload.c1_masters()
    b0 = oracle.cast_bf16(w0)
    r = oracle.cast_diff(w1, b0)
    b1 = oracle.cast_bf16(w1)
    assert np.array_equal(r["b_new"], b1.reshape(-1))
    assert np.array_equal(r["mask"], np.bitwise_xor(b0, b1).reshape(-1))
    ref = np.flatnonzero(b0.reshape(-1) != b1.reshape(-1))
    assert r["count"] == ref.size == np.count_nonzero(r["mask"])
    assert np.array_equal(r["idx"], ref.astype(np.int32))
    # pure cast / mask only
    r2 = oracle.cast_diff(w1, None)
    assert np.array_equal(r2["b_new"], b1.reshape(-1)) and r2["mask"] is None


def test_apply_rebuilds_new_version():
    """Applying (index, absolute value) to the old view gives the new view bit for
    bit [PULSE summary, "1. PULSESync" -- Ricostruzione]."""
    w0, w1 = workload.c1_masters()
    b0, b1 = oracle.cast_bf16(w0).reshape(-1), oracle.cast_bf16(w1).reshape(-1)
    idx, val, m, _ = oracle.compact(b0, b1)
    got, st = oracle.apply_patch(b0, idx, val)
    assert st == 0 and np.array_equal(got, b1)
    # same result as numpy fancy-index assignment
    ref = b0.copy()
    ref[idx] = val
    assert np.array_equal(got, ref)


def test_apply_skips_bad_indices():
    b = np.arange(10, dtype=np.uint16)
    got, st = oracle.apply_patch(b, np.array([-1, 1, 3, 10], np.int32),
                                 np.array([300, 100, 400, 200], np.uint16))
    assert st == oracle.BADINDEX
    assert list(got) == [0, 100, 2, 400, 4, 5, 6, 7, 8, 9]


def test_apply_in_any_entry_order():
    """The definition b[idx[k]] = val[k] does not depend on the entries' order
    when the indices are unique: a patch in random order equals numpy's fancy
    assignment, and out-of-range entries met in any order are skipped."""
    rng = np.random.default_rng(17)
    b = rng.integers(0, 1 << 16, 5000, dtype=np.uint16)
    idx = rng.permutation(5000)[:1700].astype(np.int32)
    assert np.any(np.diff(idx) < 0)
    val = rng.integers(0, 1 << 16, idx.size, dtype=np.uint16)
    got, st = oracle.apply_patch(b, idx, val)
    ref = b.copy()
    ref[idx] = val
    assert st == 0 and np.array_equal(got, ref)
    b10 = np.arange(10, dtype=np.uint16)
    got, st = oracle.apply_patch(b10, np.array([1, 10, -1, 3], np.int32), np.array([100, 200, 300, 400], np.uint16))
    assert st == oracle.BADINDEX
    assert list(got) == [0, 100, 2, 400, 4, 5, 6, 7, 8, 9]


def test_patch_chain_has_no_drift():
    """B_t = apply(B_{t-1}, P_t) equals the direct cast of W_t at every step
    [Jiang talk 11:08-11:30: replacement bits, no additive drift; 16:52-16:58:
    a lagging engine applies the missing transitions]."""
    ws = workload.host_masters(200_003, seed=11, steps=20)
    b = oracle.cast_bf16(ws[0])
    for t in range(1, 21):
        r = oracle.cast_diff(ws[t], b)
        b, st = oracle.apply_patch(b, r["idx"], r["val"])
        assert st == 0
        assert np.array_equal(b, oracle.cast_bf16(ws[t]))


def test_xor_mask_invariants():
    """mask = old ^ new has the weights' size; XOR into old gives new; XOR twice
    is the identity [Teleport, "XOR masks"]."""
    rng = np.random.default_rng(5)
    old = rng.integers(0, 1 << 16, 100_001, dtype=np.uint16)
    new = old.copy()
    new[rng.random(old.size) < 0.05] ^= 0x0101
    m = np.bitwise_xor(old, new)
    assert np.array_equal(oracle.xor_apply(old, m), new)
    assert np.array_equal(oracle.xor_apply(oracle.xor_apply(old, m), m), old)
    assert np.count_nonzero(m) == np.count_nonzero(old != new)
