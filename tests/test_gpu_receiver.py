"""GPU parity of the receiver's pass (pulse_apply_quant): the view must equal the
oracle's patch apply, and every quantised group's codes and scales the oracle's
FP8 block quantisation of that group taken from the patched view, bit for bit.

The view holds tensors in an order unrelated to the groups (a stacked [q; k; v]
whose sources are apart, patched-only 1-D tensors between them), with rows and
columns that are and are not multiples of 128; the patch densities run from
none to all changed per tensor, with long unchanged runs; the count is capped
by max_count; the same plan and segment index serve a second, different patch.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise
    pulse = None

from tests.gpu_util import dev, host, u16, zeros  # noqa: E402

# (name, shape) in view order; every size is a multiple of 8
TENSORS = [("q", (200, 328)), ("norm", (1000,)), ("k", (72, 328)), ("v", (40, 328)), ("o", (256, 256)),
           ("bias", (8,)), ("down", (130, 1032)), ("one", (1, 8)), ("tail", (3, 1024))]
QUANT = [["q", "k", "v"], ["o"], ["down"], ["one"], ["tail"]]
PLAIN = ["norm", "bias"]


def bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def layout():
    offs, o = {}, 0
    for nm, sh in TENSORS:
        offs[nm] = o
        o += int(np.prod(sh))
    return offs, o


def make_patch(rng, b0, offs, density):
    """Ascending unique indices, density per tensor; new values drawn apart."""
    shapes = dict(TENSORS)
    idx = []
    for nm, d in density.items():
        size = int(np.prod(shapes[nm]))
        hit = np.nonzero(rng.random(size) < d)[0]
        idx.append(offs[nm] + hit)
    idx = np.sort(np.concatenate(idx)).astype(np.int32)
    val = bf16_bits(rng.standard_normal(idx.size) * rng.choice([0.02, 1.0, 40.0]))
    return idx, val


def reference(b0, idx, val, offs, count=None):
    shapes = dict(TENSORS)
    b1, st = oracle.apply_patch(b0, idx, val, count)
    out = []
    for g in QUANT:
        srcs = []
        for nm in g:
            sh = shapes[nm]
            sh2 = sh if len(sh) == 2 else (1, sh[0])
            srcs.append(b1[offs[nm]: offs[nm] + int(np.prod(sh))].reshape(sh2))
        out.append(oracle.fp8_block_quant(srcs))
    return b1, st, out


def make_plan(offs, n):
    shapes = dict(TENSORS)
    groups, outs = [], []
    for g in QUANT:
        cols = shapes[g[0]][-1]
        srcs = [(offs[nm], shapes[nm][0] if len(shapes[nm]) == 2 else 1) for nm in g]
        R = sum(r for _, r in srcs)
        codes = torch.full((R * cols,), 0xAB, dtype=torch.uint8, device="cuda")
        scales = torch.full((((R + 127) // 128) * ((cols + 127) // 128),), -3.0, dtype=torch.float32,
                            device="cuda")
        groups.append((srcs, cols, codes, scales))
        outs.append((codes, scales))
    for nm in PLAIN:
        groups.append(([(offs[nm], 1)], shapes[nm][0], None, None))
    return pulse.pulse_apply_quant_plan(groups, n), outs


def check(B, outs, ref):
    b1, _, qref = ref
    assert np.array_equal(u16(B), b1)
    for (codes, scales), (rc, rs) in zip(outs, qref):
        assert np.array_equal(host(scales).view(np.uint32), rs.reshape(-1).view(np.uint32))
        assert np.array_equal(host(codes), rc.reshape(-1))


def run(B, idx_t, val_t, count, plan, ws, max_count=None):
    cnt = torch.tensor([count], dtype=torch.int64, device="cuda")
    st = zeros(1, torch.int32)
    pulse.pulse_apply_quant(B, idx_t, val_t, cnt, plan, st, ws, max_count=max_count)
    torch.cuda.synchronize()
    return int(host(st)[0])


DENSITIES = {
    "sparse": {"q": 0.08, "norm": 0.08, "k": 0.08, "v": 0.08, "o": 0.08, "bias": 0.5, "down": 0.08, "tail": 0.08},
    "mixed": {"q": 1.0, "norm": 1.0, "v": 0.5, "o": 0.01, "bias": 1.0, "down": 0.002, "one": 1.0},
    "all": {nm: 1.0 for nm, _ in TENSORS},
    "ends": {"q": 0.0005, "tail": 0.01},   # long unchanged runs between few entries
}


@pytest.mark.parametrize("case", sorted(DENSITIES))
def test_receiver_pass_matches_apply_then_quant(case):
    rng = np.random.default_rng(len(case) * 7 + 1)
    offs, n = layout()
    b0 = bf16_bits(rng.standard_normal(n) * 0.05)
    idx, val = make_patch(rng, b0, offs, DENSITIES[case])
    print(f"receiver pass: case {case}, n {n}, entries {idx.size}", flush=True)
    plan, outs = make_plan(offs, n)
    ws = pulse.workspace(pulse.PULSE_OP_APPLY_QUANT, n)
    B = dev(b0)
    cap = max(idx.size, 1)
    idx_t, val_t = zeros(cap, torch.int32), zeros(cap, torch.int16)
    if idx.size:
        idx_t[: idx.size] = dev(idx)
        val_t[: idx.size] = dev(val)
    assert run(B, idx_t, val_t, idx.size, plan, ws) == 0
    check(B, outs, reference(b0, idx, val, offs))


def test_receiver_pass_empty_capped_and_reused():
    """No entries (the codes of the old view); then a patch whose count is
    capped by max_count; then another patch through the same plan and index."""
    rng = np.random.default_rng(5)
    offs, n = layout()
    b0 = bf16_bits(rng.standard_normal(n) * 0.05)
    plan, outs = make_plan(offs, n)
    ws = pulse.workspace(pulse.PULSE_OP_APPLY_QUANT, n)
    ws.fill_(0x5A)  # the index is rebuilt by every call
    B = dev(b0)
    idx_t, val_t = zeros(n, torch.int32), zeros(n, torch.int16)
    print("receiver pass: empty patch", flush=True)
    assert run(B, idx_t, val_t, 0, plan, ws) == 0
    check(B, outs, reference(b0, np.zeros(0, np.int32), np.zeros(0, np.uint16), offs))

    idx, val = make_patch(rng, b0, offs, DENSITIES["sparse"])
    idx_t[: idx.size] = dev(idx)
    val_t[: idx.size] = dev(val)
    cap = idx.size // 3
    print(f"receiver pass: {idx.size} entries capped at {cap}", flush=True)
    assert run(B, idx_t, val_t, idx.size, plan, ws, max_count=cap) == 0
    ref = reference(b0, idx, val, offs, count=cap)
    check(B, outs, ref)

    b1 = ref[0]
    idx2, val2 = make_patch(rng, b1, offs, DENSITIES["mixed"])
    idx_t[: idx2.size] = dev(idx2)
    val_t[: idx2.size] = dev(val2)
    print(f"receiver pass: second patch, {idx2.size} entries", flush=True)
    assert run(B, idx_t, val_t, idx2.size, plan, ws) == 0
    check(B, outs, reference(b1, idx2, val2, offs))


def test_receiver_pass_reports_bad_patches_and_plans():
    """An index past the view or out of order sets PULSE_DS_BADINDEX and writes
    nothing outside the view; a plan made for another view size sets
    PULSE_DS_WORKSPACE and writes nothing."""
    rng = np.random.default_rng(9)
    offs, n = layout()
    b0 = bf16_bits(rng.standard_normal(n) * 0.05)
    plan, outs = make_plan(offs, n)
    ws = pulse.workspace(pulse.PULSE_OP_APPLY_QUANT, n + 4096)
    guard = 4096
    Bg = dev(np.concatenate([b0, np.full(guard, 0x7777, np.uint16)]))
    idx = np.array([5, 900, 3000, n + 10, n + 2000], np.int32)
    val = np.full(idx.size, 0x3F80, np.uint16)
    print("receiver pass: index past the view", flush=True)
    st = run(Bg, dev(idx), dev(val), idx.size, plan, ws)
    assert st & pulse.PULSE_DS_BADINDEX
    got = u16(Bg)
    assert np.all(got[n:] == 0x7777)
    assert np.array_equal(got[:n], oracle.apply_patch(b0, idx[:3], val[:3])[0])

    B = dev(b0)
    idx = np.array([10, 400, 300, 5000], np.int32)
    print("receiver pass: indices out of order", flush=True)
    st = run(B, dev(idx), dev(np.full(4, 0x3F80, np.uint16)), 4, plan, ws)
    assert st & pulse.PULSE_DS_BADINDEX

    other, _ = make_plan(offs, n)
    other.n = n - 8  # the call's view size no longer matches the plan's
    B = dev(b0)
    print("receiver pass: plan for another view", flush=True)
    st = run(B, dev(np.array([1], np.int32)), dev(np.array([0x3F80], np.uint16)), 1, other, ws)
    assert st & pulse.PULSE_DS_WORKSPACE
    assert np.array_equal(u16(B), b0)
