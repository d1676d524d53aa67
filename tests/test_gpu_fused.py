"""GPU parity of the fused sender pass (pulse_cast_diff_lz4): every output must
equal the oracle's cast/diff/compaction followed by its canonical LZ4 block
encoding of old ^ new, bit for bit.

Sizes span several mask blocks and ragged tails (n counts BF16 elements; a
64 KiB block holds 32768 of them); densities run from none to all changed,
past the point where a wave's entries no longer fit its staging area; the
patch and the payload overflow their capacities; the new view is omitted or
written over the old one; the patch is omitted; one workspace serves calls of
different sizes.
"""
import numpy as np
import pytest
import torch

import oracle
import workload

pytestmark = pytest.mark.gpu

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise
    pulse = None

from tests.gpu_util import dev, host, u16, zeros  # noqa: E402


def masters(n, seed, density=None):
    w0, w1 = workload.host_masters(n, seed)
    if density is not None:
        rng = np.random.default_rng(seed + 99)
        w1 = w0.copy()
        hit = rng.random(n) < density
        w1[hit] = w0[hit] * np.float32(1.5) + np.float32(0.01)
    return w0, w1


def tile_index(idx, count, n):
    """The patch's tile index from its definition: first entry >= 16384 t."""
    starts = np.arange(0, (n + 16383) // 16384, dtype=np.int64) * 16384
    return np.append(np.searchsorted(idx[:count].astype(np.int64), starts, side="left"), count).astype(np.int64)


def fused(w1, b0, block_bytes=65536, cap=None, pcap=None, want_new=True, want_patch=True, in_place=False, ws=None):
    n = w1.size
    nb = (2 * n + block_bytes - 1) // block_bytes
    cap = n if cap is None else cap
    pcap = pulse.lz4_payload_bound(2 * n, block_bytes) if pcap is None else pcap
    W, B0 = dev(w1), dev(b0)
    bn = B0 if in_place else (zeros(n, torch.int16) if want_new else None)
    idx = zeros(cap, torch.int32)[:cap] if want_patch else None
    val = zeros(cap, torch.int16)[:cap] if want_patch else None
    cnt = zeros(1, torch.int64) if want_patch else None
    tf = torch.full((pulse.patch_tile_count(n),), -7, dtype=torch.int64, device="cuda") if want_patch else None
    payload = zeros(pcap, torch.uint8)[:pcap] if pcap else zeros(1, torch.uint8)[:0]
    sizes, offs = zeros(nb, torch.int32), zeros(nb, torch.int64)
    tot, st = zeros(1, torch.int64), zeros(1, torch.int32)
    if ws is None:
        ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_LZ4, n, block_bytes)
    pulse.pulse_cast_diff_lz4(W, B0, bn, idx, val, cnt, payload, sizes, offs, tot, st, ws, block_bytes=block_bytes,
                              tile_first=tf)
    torch.cuda.synchronize()
    t = int(host(tot)[0])
    out = dict(total=t, status=int(host(st)[0]), sizes=host(sizes, np.uint32)[:nb], offsets=host(offs, np.uint64)[:nb],
               payload=host(payload)[: min(t, pcap)])
    out["b_new"] = u16(bn)[:n] if bn is not None else None
    if want_patch:
        c = int(host(cnt)[0])
        k = min(c, cap)
        out.update(count=c, idx=host(idx)[:k], val=u16(val)[:k], tile_first=host(tf))
    return out


def check(got, w1, b0, block_bytes=65536, cap=None):
    ref = oracle.cast_diff(w1, b0)
    enc = oracle.lz4_encode_blocks(b0, block_bytes, src_xor=ref["b_new"])
    assert got["total"] == enc["total"]
    assert np.array_equal(got["sizes"], enc["sizes"]) and np.array_equal(got["offsets"], enc["offsets"])
    assert np.array_equal(got["payload"], enc["payload"][: got["payload"].size])
    if got["b_new"] is not None:
        assert np.array_equal(got["b_new"], ref["b_new"])
    if "count" in got:
        k = ref["count"] if cap is None else min(cap, ref["count"])
        assert got["count"] == ref["count"]
        assert np.array_equal(got["idx"], ref["idx"][:k]) and np.array_equal(got["val"], ref["val"][:k])
        assert np.array_equal(got["tile_first"], tile_index(ref["idx"], ref["count"], w1.size))
    return ref


SIZES = [1, 2, 7, 12, 13, 4097, 32767, 32768, 32769, 3 * 32768 + 5, 200_003, (1 << 20) + 11]


@pytest.mark.parametrize("n", SIZES)
def test_fused_matches_oracle_generator_step(n):
    w0, w1 = masters(n, seed=3 * n + 1)
    b0 = oracle.cast_bf16(w0)
    got = fused(w1, b0)
    check(got, w1, b0)
    assert got["status"] == 0


@pytest.mark.parametrize("density", [0.0, 0.003, 0.08, 0.12, 0.3, 1.0])
def test_fused_densities(density):
    """0.12 and above: some waves hold more changed elements than they can
    stage, and the block stores its patch directly."""
    n = 5 * 32768 + 333
    w0, w1 = masters(n, seed=int(density * 1000) + 5, density=density)
    b0 = oracle.cast_bf16(w0)
    got = fused(w1, b0)
    check(got, w1, b0)
    assert got["status"] == 0


@pytest.mark.parametrize("block_bytes", [16384, 32768])
def test_fused_other_block_sizes(block_bytes):
    n = 9 * block_bytes // 2 + 77
    for density in (None, 0.4):
        w0, w1 = masters(n, seed=block_bytes + (0 if density is None else 1), density=density)
        b0 = oracle.cast_bf16(w0)
        got = fused(w1, b0, block_bytes=block_bytes)
        check(got, w1, b0, block_bytes=block_bytes)


def test_fused_capacities():
    n = 7 * 32768 + 19
    w0, w1 = masters(n, seed=77)
    b0 = oracle.cast_bf16(w0)
    ref = oracle.cast_diff(w1, b0)
    cap = ref["count"] // 3
    got = fused(w1, b0, cap=cap)
    check(got, w1, b0, cap=cap)
    assert got["status"] == pulse.PULSE_DS_CAPACITY
    enc = oracle.lz4_encode_blocks(b0, 65536, src_xor=ref["b_new"])
    pcap = int(enc["offsets"][4]) + 3
    got = fused(w1, b0, pcap=pcap)
    assert got["status"] == pulse.PULSE_DS_CAPACITY and got["total"] == enc["total"]
    assert np.array_equal(got["payload"][: int(enc["offsets"][4])], enc["payload"][: int(enc["offsets"][4])])
    assert got["count"] == ref["count"] and np.array_equal(got["idx"], ref["idx"])


def test_fused_optional_outputs_and_in_place():
    n = 3 * 32768 + 1001
    w0, w1 = masters(n, seed=91)
    b0 = oracle.cast_bf16(w0)
    check(fused(w1, b0, want_new=False), w1, b0)
    check(fused(w1, b0, want_patch=False), w1, b0)
    check(fused(w1, b0, want_new=False, want_patch=False), w1, b0)
    got = fused(w1, b0, in_place=True)   # the view becomes the new one
    check(got, w1, b0)


def test_fused_chain_and_workspace_reuse():
    """One workspace, calls of different sizes, and a 6-step version chain in
    place: each step's mask blocks decode + XOR back onto the receiver's copy,
    and its patch applied to another copy, both give the cast of the step."""
    big = 6 * 32768 + 123
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_LZ4, big, 65536)
    rng = np.random.default_rng(8)
    for it, n in enumerate([big, 1000, 2 * 32768, big, 5, big]):
        w0, w1 = masters(n, seed=400 + it, density=float(rng.choice([0.0, 0.02, 0.5])) if it % 2 else None)
        b0 = oracle.cast_bf16(w0)
        check(fused(w1, b0, ws=ws), w1, b0)
    n = 100_003
    ws_host = workload.host_masters(n, seed=31, steps=6)
    send = dev(oracle.cast_bf16(ws_host[0]))
    recv_p, recv_x = send.clone(), send.clone()
    nb = (2 * n + 65535) // 65536
    cap = pulse.lz4_payload_bound(2 * n)
    payload = zeros(cap, torch.uint8)
    sizes, offs = zeros(nb, torch.int32), zeros(nb, torch.int64)
    tot, st, cnt = zeros(1, torch.int64), zeros(1, torch.int32), zeros(1, torch.int64)
    idx, val = zeros(n, torch.int32), zeros(n, torch.int16)
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_LZ4, n, 65536)
    dws = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nb, cap)
    for t in range(1, 6):
        pulse.pulse_cast_diff_lz4(dev(ws_host[t]), send, send, idx, val, cnt, payload, sizes, offs, tot, st, ws)
        pulse.pulse_apply_patch(recv_p, idx, val, cnt, st, max_count=n)
        pulse.lz4_decode_blocks(payload, offs, sizes, recv_x, st, dws, mode=1, payload_bytes=cap)
        torch.cuda.synchronize()
        want = oracle.cast_bf16(ws_host[t])
        assert np.array_equal(u16(send), want)
        assert np.array_equal(u16(recv_p), want) and np.array_equal(u16(recv_x), want)
    assert int(host(st)[0]) == 0


@pytest.mark.parametrize("density", [None, 0.004, 0.3])
def test_patch_tiles_and_tiled_apply(density):
    """The tile index written by pulse_patch_tiles equals the one the fused pass
    writes (and the definition); the tiled apply rebuilds the new view."""
    n = 9 * 16384 + 1234
    w0, w1 = masters(n, seed=600 + (0 if density is None else int(density * 1000)), density=density)
    b0 = oracle.cast_bf16(w0)
    got = fused(w1, b0)
    ref = check(got, w1, b0)
    m = ref["count"]
    I = dev(ref["idx"]) if m else zeros(1, torch.int32)
    V = dev(ref["val"]) if m else zeros(1, torch.int16)
    tf = torch.full((pulse.patch_tile_count(n),), -3, dtype=torch.int64, device="cuda")
    pulse.pulse_patch_tiles(I, dev(np.array([m], np.int64)), tf, n, max_count=max(m, 1))
    B, st = dev(b0), zeros(1, torch.int32)
    pulse.pulse_apply_patch_tiled(B, I, V, tf, st, max_count=max(m, 1))
    torch.cuda.synchronize()
    assert np.array_equal(host(tf), got["tile_first"])
    assert np.array_equal(u16(B), ref["b_new"]) and int(host(st)[0]) == 0
