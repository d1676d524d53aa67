"""Pins of the oracle's FP32 -> BF16 round-to-nearest-even cast (row a1).

Each pin is independent of oracle.c: values printed on the pages, torch's CPU
cast (a library routine), and a nearest-of-set search over all BF16 values in
binary64.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workload


def f2u(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


def bf16_value(h):
    return float(np.array([h << 16], np.uint32).view(np.float32)[0])


# ---- values the pages print -------------------------------------------------
def _golden(name):
    vals = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                vals[line[0]] = (float(line[1]), float(line[2]))
    return vals


def test_pages_worked_values_near_one():
    """The pages' worked example for a weight near 1 (tests/golden, with its
    citation): the oracle's cast has that spacing and boundary, an update of the
    printed size leaves the served value unchanged, and one just past the printed
    boundary changes it."""
    g = _golden("bf16_worked_values_near_one.txt")
    one = oracle.bf16_rne(f2u(1.0))
    assert one == 0x3F80
    # spacing: the value right above 1 the cast can produce
    up = next(h for h in range(0x3F81, 0x3F90) if oracle.bf16_rne(f2u(bf16_value(h))) == h)
    spacing = bf16_value(up) - 1.0
    val, tol = g["bf16_spacing_near_one"]
    assert abs(spacing - val) <= tol
    # boundary: the smallest upward step that changes the served value
    lo, hi = 0.0, spacing
    for _ in range(60):
        mid = (lo + hi) / 2
        if oracle.bf16_rne(f2u(np.float32(1.0 + mid))) == one:
            lo = mid
        else:
            hi = mid
    boundary = hi
    val, tol = g["rounding_boundary_near_one"]
    assert abs(boundary - val) <= tol
    val, _ = g["boundary_over_theta"]
    assert abs(boundary - val * 1.0) <= 2.0 ** -23
    step, _ = g["typical_adam_step"]
    assert oracle.bf16_rne(f2u(np.float32(1.0) + np.float32(step))) == one
    assert oracle.bf16_rne(f2u(np.float32(1.0) - np.float32(step))) == one
    ratio, _ = g["min_boundary_over_step"]
    assert boundary / step > ratio
    # exact ties around the boundary go to even
    assert oracle.bf16_rne(f2u(1.0 + 2.0 ** -8)) == 0x3F80
    assert oracle.bf16_rne(f2u(1.0 + 2.0 ** -8 + 2.0 ** -23)) == 0x3F81
    assert oracle.bf16_rne(f2u(1.0 + 3 * 2.0 ** -8)) == 0x3F82


def test_push_vs_floor_threshold():
    """A change is visible only once the update crosses half a BF16 ulp, which
    lies in (|w|/512, |w|/256] [PULSE summary, "Osservazione Centrale"]."""
    rng = np.random.default_rng(1)
    # random normal BF16 values theta > 0 (exponent 100..150)
    hs = rng.integers(100 << 7, 150 << 7, size=2000).astype(np.uint32)
    for h in hs:
        theta = bf16_value(int(h))
        below = np.float32(theta + theta / 512 * 0.999)
        above = np.float32(theta + theta / 256 * 1.01)
        assert oracle.bf16_rne(f2u(below)) == h
        assert oracle.bf16_rne(f2u(above)) != h


# ---- library routine: torch's CPU cast ------------------------------------------
EDGE_LO = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)


def edge_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32)
    return ((hi[:, None] << 16) | EDGE_LO[None, :]).reshape(-1)


def torch_bf16(bits):
    f = torch.from_numpy(bits.view(np.float32).copy())
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_edge_set_matches_torch():
    """Every upper half x {0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF}: the
    rounding decision only depends on these classes of the lower half."""
    bits = edge_patterns()
    f = bits.view(np.float32)
    ours = oracle.cast_bf16(f)
    ref = torch_bf16(bits)
    fin = ~np.isnan(f)
    assert np.array_equal(ours[fin], ref[fin])
    # NaN: stays NaN with its sign (our reading; torch is not consistent here)
    nan_out = ours[~fin]
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all((nan_out & 0x7F) != 0)
    assert np.array_equal(nan_out >> 15, (bits[~fin] >> 31).astype(np.uint16))


def test_full_sweep_matches_torch():
    """All 2^32 patterns, chunked (NaNs excluded, see above)."""
    chunk = 1 << 26
    for c in range((1 << 32) // chunk):
        bits = np.arange(chunk, dtype=np.uint32) + np.uint32(c * chunk)
        f = bits.view(np.float32)
        ours = oracle.cast_bf16(f)
        ref = torch_bf16(bits)
        fin = ~np.isnan(f)
        bad = np.flatnonzero(ours[fin] != ref[fin])
        assert bad.size == 0, hex(int(bits[fin][bad[0]]))


# ---- textbook: nearest member of the BF16 set, binary64 --------------------------
def nearest_bf16_by_search(x):
    """Nearest finite BF16 to each finite float32 x (as binary64), ties to the even
    pattern; beyond the largest finite value + half an ulp -> infinity."""
    pos = np.arange(0x0000, 0x7F81, dtype=np.uint32)           # +0 .. +Inf
    vals = (pos << 16).view(np.float32).astype(np.float64)
    vals[-1] = 2.0 ** 128                                         # Inf sits where 2^128 would
    x64 = np.abs(x.astype(np.float64))
    j = np.searchsorted(vals, x64)                                # vals[j-1] < x <= vals[j]
    j = np.clip(j, 1, vals.size - 1)
    lo, hi = vals[j - 1], vals[j]
    dlo, dhi = x64 - lo, hi - x64
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((pos[j] & 1) == 0))
    res = np.where(pick_hi, pos[j], pos[j - 1])
    sign = (x.view(np.uint32) >> 31).astype(np.uint32)
    return (res | (sign << 15)).astype(np.uint16)


def test_edge_set_matches_nearest_of_set():
    bits = edge_patterns()
    f = bits.view(np.float32)
    fin = np.isfinite(f)
    assert np.array_equal(oracle.cast_bf16(f)[fin], nearest_bf16_by_search(f[fin]))
    rng = np.random.default_rng(7)
    r = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    fr = r.view(np.float32)
    fin = np.isfinite(fr)
    assert np.array_equal(oracle.cast_bf16(fr)[fin], nearest_bf16_by_search(fr[fin]))


def test_signed_zero_subnormal_overflow():
    assert oracle.bf16_rne(0x80000000) == 0x8000                  # -0 keeps its sign
    assert oracle.bf16_rne(0x00008000) == 0x0000                  # subnormal tie -> even
    assert oracle.bf16_rne(0x00018000) == 0x0002
    assert oracle.bf16_rne(0x7F7FFFFF) == 0x7F80                  # overflow -> +Inf
    assert oracle.bf16_rne(0xFF800000) == 0xFF80                  # -Inf stays


# ---- the workloads' density (a property of the synthetic generator) -------------
def test_config1_density():
    """The c1 generator (w ~ N(0,0.02), lr 3e-6) changes ~8.06% of BF16 values,
    not the ~1% the pages measure on real checkpoints: sigma=0.02 weights have
    ulps ~1e-4 and below, far smaller than the theta~1 example.  Norm-like
    weights near 1 change ~0.05%, as the push-vs-floor argument predicts."""
    w0, w1 = workload.c1_masters()
    r = oracle.cast_diff(w1, oracle.cast_bf16(w0))
    assert r["count"] == 337906
    n0, n1 = workload.host_masters(1 << 20, 5, kind="norm")
    d = oracle.cast_diff(n1, oracle.cast_bf16(n0))["count"] / (1 << 20)
    assert 0.0002 < d < 0.001
