"""GPU parity of every C-ABI entry point against the CPU oracle (bit-exact).

Sizes span several tiles / blocks plus ragged tails; the edge cases are the
empty input, single elements, tile boundaries, all-changed / none-changed
inputs, the RNE edge patterns, capacity overflow, bad indices, corrupt LZ4
blocks and streams that need the decoder's general path.
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
        raise  # on a GPU machine the HIP library must be there
    pulse = None

from tests.gpu_util import dev, host, u16, zeros  # noqa: E402
from tests import lz4_spec, lz4_system  # noqa: E402

TILE = 16384  # elements per compaction tile
SIZES = [1, 2, 63, 64, 65, 4095, 4097, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, (1 << 20) + 7]


def masters(n, seed, density=None):
    """(w_old, w_new) float32: generator step, or a forced changed fraction."""
    w0, w1 = workload.host_masters(n, seed)
    if density is not None:
        rng = np.random.default_rng(seed + 99)
        w1 = w0.copy()
        hit = rng.random(n) < density
        w1[hit] = w0[hit] * np.float32(1.5) + np.float32(0.01)
    return w0, w1


def gpu_cast_diff(w1, b0, cap=None, want_new=True, want_mask=True, ws=None):
    n = w1.size
    cap = n if cap is None else cap
    W, B0 = dev(w1), dev(b0)
    bn = zeros(n, torch.int16) if want_new else None
    mk = zeros(n, torch.int16) if want_mask else None
    idx, val = zeros(cap, torch.int32), zeros(cap, torch.int16)
    cnt, st = zeros(1, torch.int64), zeros(1, torch.int32)
    if ws is None:
        ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, n)
    pulse.pulse_cast_diff(W, B0, bn, mk, idx[:cap] if cap else idx[:0], val[:cap] if cap else val[:0], cnt, st, ws, n=n)
    torch.cuda.synchronize()
    c = int(host(cnt)[0])
    k = min(c, cap)
    return dict(b_new=None if bn is None else u16(bn)[:n], mask=None if mk is None else u16(mk)[:n],
                idx=host(idx)[:k], val=u16(val)[:k], count=c, status=int(host(st)[0]))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("density", [None, 0.0, 1.0, 0.5])
def test_cast_diff_matches_oracle(n, density):
    w0, w1 = masters(n, seed=n, density=density)
    b0 = oracle.cast_bf16(w0)
    ref = oracle.cast_diff(w1, b0)
    got = gpu_cast_diff(w1, b0)
    assert got["count"] == ref["count"] and got["status"] == 0
    assert np.array_equal(got["b_new"], ref["b_new"])
    assert np.array_equal(got["mask"], ref["mask"])
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["val"], ref["val"])


def test_cast_diff_config1():
    w0, w1 = workload.c1_masters()
    b0 = oracle.cast_bf16(w0).reshape(-1)
    ref = oracle.cast_diff(w1, b0)
    got = gpu_cast_diff(w1.reshape(-1), b0)
    assert got["count"] == ref["count"] == 337906
    for k in ("b_new", "mask", "idx", "val"):
        assert np.array_equal(got[k], ref[k]), k


def test_changes_at_tile_edges_and_alternating():
    n = 5 * TILE + 3
    b0 = np.zeros(n, np.uint16)
    w1 = np.zeros(n, np.float32)
    for i in (0, TILE - 1, TILE, 2 * TILE - 1, 4 * TILE, n - 1):
        w1[i] = 1.0
    w1[3 * TILE:4 * TILE:2] = -2.0                     # alternating inside one tile
    ref = oracle.cast_diff(w1, b0)
    got = gpu_cast_diff(w1, b0)
    assert got["count"] == ref["count"]
    assert np.array_equal(got["idx"], ref["idx"]) and np.array_equal(got["val"], ref["val"])


def test_signed_zero_flip_counts_as_change():
    n = 1000
    b0 = np.zeros(n, np.uint16)
    w1 = np.zeros(n, np.float32)
    w1[::7] = -0.0
    got = gpu_cast_diff(w1, b0)
    ref = oracle.cast_diff(w1, b0)
    assert got["count"] == ref["count"] == len(range(0, n, 7))
    assert np.all(got["val"] == 0x8000)


def test_rne_edge_patterns_and_variants():
    hi = np.arange(1 << 16, dtype=np.uint32)
    lo = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = ((hi[:, None] << 16) | lo[None, :]).reshape(-1)
    f = bits.view(np.float32)
    ref = oracle.cast_bf16(f)
    n = f.size
    # pure cast
    W = dev(f)
    bn = zeros(n, torch.int16)
    pulse.pulse_cast_diff(W, b_new=bn)
    torch.cuda.synchronize()
    assert np.array_equal(u16(bn), ref)
    # mask only (no patch), against an arbitrary old view
    b0 = np.random.default_rng(1).integers(0, 1 << 16, n, dtype=np.uint16)
    mk = zeros(n, torch.int16)
    pulse.pulse_cast_diff(W, b_old=dev(b0), xor_mask=mk)
    torch.cuda.synchronize()
    assert np.array_equal(u16(mk), b0 ^ ref)
    # in place: b_new is b_old
    B = dev(b0)
    mk2 = zeros(n, torch.int16)
    idx, val = zeros(n, torch.int32), zeros(n, torch.int16)
    cnt, st = zeros(1, torch.int64), zeros(1, torch.int32)
    pulse.pulse_cast_diff(W, B, B, mk2, idx, val, cnt, st, pulse.workspace(pulse.PULSE_OP_CAST_DIFF, n))
    torch.cuda.synchronize()
    r = oracle.cast_diff(f, b0)
    assert np.array_equal(u16(B), ref) and np.array_equal(u16(mk2), r["mask"])
    assert int(host(cnt)[0]) == r["count"] and np.array_equal(host(idx)[: r["count"]], r["idx"])


def test_full_rne_sweep():
    """All 2^32 FP32 patterns through the GPU cast, compared with the oracle."""
    chunk = 1 << 26
    bn = zeros(chunk, torch.int16)
    for c in range((1 << 32) // chunk):
        bits = np.arange(chunk, dtype=np.uint32) + np.uint32(c * chunk)
        W = dev(bits.view(np.float32))
        pulse.pulse_cast_diff(W, b_new=bn)
        got = u16(bn)
        ref = oracle.cast_bf16(bits.view(np.float32))
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, hex(int(bits[bad[0]]))


def test_capacity_overflow():
    n = 50_000
    w0, w1 = masters(n, seed=5, density=0.3)
    b0 = oracle.cast_bf16(w0)
    ref = oracle.cast_diff(w1, b0)
    cap = ref["count"] // 3
    got = gpu_cast_diff(w1, b0, cap=cap)
    assert got["count"] == ref["count"] and got["status"] == pulse.PULSE_DS_CAPACITY
    assert np.array_equal(got["idx"], ref["idx"][:cap]) and np.array_equal(got["val"], ref["val"][:cap])


def test_empty_input_writes_zero_count():
    cnt = torch.full((1,), 123, dtype=torch.int64, device="cuda")
    st = zeros(1, torch.int32)
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, 0)
    pulse.pulse_cast_diff(zeros(1, torch.float32), zeros(1, torch.int16), zeros(1, torch.int16), None,
                          zeros(1, torch.int32), zeros(1, torch.int16), cnt, st, ws, n=0)
    torch.cuda.synchronize()
    assert int(host(cnt)[0]) == 0


def test_workspace_reuse_across_calls_and_sizes():
    """One workspace, many calls of varying sizes: per-call epochs keep status
    words of earlier calls from being read as this call's."""
    big = 40 * TILE + 11
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, big)
    rng = np.random.default_rng(3)
    for it, n in enumerate([big, 5, 3 * TILE, big, 1, 17 * TILE + 1, big, TILE]):
        w0, w1 = masters(n, seed=100 + it, density=float(rng.random()))
        b0 = oracle.cast_bf16(w0)
        ref = oracle.cast_diff(w1, b0)
        got = gpu_cast_diff(w1, b0, ws=ws)
        assert got["count"] == ref["count"]
        assert np.array_equal(got["idx"], ref["idx"]) and np.array_equal(got["val"], ref["val"])


def test_compact_matches_oracle():
    rng = np.random.default_rng(11)
    for n in SIZES + [0]:
        b0 = rng.integers(0, 1 << 16, n, dtype=np.uint16)
        b1 = b0.copy()
        hit = rng.random(n) < 0.2
        b1[hit] = rng.integers(0, 1 << 16, int(hit.sum()), dtype=np.uint16)
        b1[::97] ^= 0x8000  # sign flips
        idx_r, val_r, m, st_r = oracle.compact(b0, b1)
        idx, val = zeros(n, torch.int32), zeros(n, torch.int16)  # at least one element: a valid pointer
        cnt, st = zeros(1, torch.int64), zeros(1, torch.int32)
        pulse.pulse_compact(dev(b0) if n else zeros(1, torch.int16), dev(b1) if n else zeros(1, torch.int16),
                            idx, val, cnt, st, pulse.workspace(pulse.PULSE_OP_COMPACT, n), n=n)
        torch.cuda.synchronize()
        assert int(host(cnt)[0]) == m
        assert np.array_equal(host(idx)[:m], idx_r) and np.array_equal(u16(val)[:m], val_r)


def test_apply_patch_matches_oracle_and_rebuilds():
    for n in SIZES:
        w0, w1 = masters(n, seed=2 * n + 1)
        b0 = oracle.cast_bf16(w0)
        r = oracle.cast_diff(w1, b0)
        B = dev(b0)
        cnt, st = dev(np.array([r["count"]], np.int64)), zeros(1, torch.int32)
        idx = dev(r["idx"]) if r["count"] else zeros(1, torch.int32)
        val = dev(r["val"]) if r["count"] else zeros(1, torch.int16)
        pulse.pulse_apply_patch(B, idx, val, cnt, st, max_count=max(r["count"], 1))
        torch.cuda.synchronize()
        assert np.array_equal(u16(B), r["b_new"]) and int(host(st)[0]) == 0


def test_apply_bad_index_and_count_bound():
    b = np.arange(100, dtype=np.uint16)
    idx = np.array([-5, 1, 3, 7, 100], np.int32)
    val = np.array([11, 12, 13, 14, 15], np.uint16)
    for count, want in ((4, pulse.PULSE_DS_BADINDEX), (3, pulse.PULSE_DS_BADINDEX), (5, pulse.PULSE_DS_BADINDEX)):
        B = dev(b)
        st = zeros(1, torch.int32)
        pulse.pulse_apply_patch(B, dev(idx), dev(val), dev(np.array([count], np.int64)), st, max_count=5)
        torch.cuda.synchronize()
        ref, rst = oracle.apply_patch(b, idx, val, count=count)
        assert np.array_equal(u16(B), ref) and int(host(st)[0]) == rst == want
    # in-range entries only: no status
    B, st = dev(b), zeros(1, torch.int32)
    pulse.pulse_apply_patch(B, dev(idx[1:]), dev(val[1:]), dev(np.array([3], np.int64)), st, max_count=4)
    torch.cuda.synchronize()
    ref, rst = oracle.apply_patch(b, idx[1:], val[1:], count=3)
    assert np.array_equal(u16(B), ref) and int(host(st)[0]) == rst == 0
    # indices just past the view inside a larger buffer: skipped, the rest of
    # the buffer untouched
    G = dev(np.concatenate([b, np.full(64, 0x7777, np.uint16)]))
    bad = np.array([2, 99, 100, 101, 163], np.int32)
    st = zeros(1, torch.int32)
    pulse.pulse_apply_patch(G[:100], dev(bad), dev(val), dev(np.array([5], np.int64)), st, max_count=5)
    torch.cuda.synchronize()
    ref, rst = oracle.apply_patch(b, bad, val)
    got = u16(G)
    assert np.array_equal(got[:100], ref) and np.all(got[100:] == 0x7777) and int(host(st)[0]) == rst
    # device count above max_count: only max_count entries are applied
    B = dev(b)
    pulse.pulse_apply_patch(B, dev(idx[1:]), dev(val[1:]), dev(np.array([4], np.int64)), zeros(1, torch.int32),
                            max_count=1)
    torch.cuda.synchronize()
    ref, _ = oracle.apply_patch(b, idx[1:], val[1:], count=1)
    assert np.array_equal(u16(B), ref)


@pytest.mark.parametrize("density", [1.0, 0.5, 0.08, 0.004])
def test_apply_every_line_offset(density):
    """The view may start anywhere in a 64-byte line (any 2-byte offset): the
    lines cut by either end of it, and lines whose entries straddle chunk and
    wave boundaries, against the oracle.  The entries always include the first
    and the last element."""
    rng = np.random.default_rng(int(density * 1000) + 7)
    backing = rng.integers(0, 1 << 16, 70_000, dtype=np.uint16)
    Back = dev(backing)
    for off in list(range(0, 33)) + [47, 63]:
        n = 66_000 - 37 * off
        pos = np.flatnonzero(rng.random(n) < density)
        pos = np.union1d(pos, [0, n - 1]).astype(np.int32)
        val = rng.integers(0, 1 << 16, pos.size, dtype=np.uint16)
        B = Back.clone()
        st = zeros(1, torch.int32)
        pad = np.zeros(13, np.int32)   # capacity above the count
        pulse.pulse_apply_patch(B[off:off + n], dev(np.concatenate([pos, pad])),
                                dev(np.concatenate([val, pad.astype(np.uint16)])),
                                dev(np.array([pos.size], np.int64)), st, max_count=pos.size + 13)
        torch.cuda.synchronize()
        ref = backing.copy()
        ref[off:off + n], rst = oracle.apply_patch(backing[off:off + n], pos, val)
        got = u16(B)
        assert np.array_equal(got, ref), (off, np.flatnonzero(got != ref)[:8])
        assert int(host(st)[0]) == rst == 0


def test_apply_many_waves_large_patch():
    """A patch long enough for every wave of the launch to take several chunks
    (entries 2^22 over 2^23 + 11 elements), and a sparse one whose chunks own
    more lines than one LDS pass holds."""
    rng = np.random.default_rng(12)
    n = (1 << 23) + 11
    b = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    for density in (0.5, 0.0015):
        pos = np.flatnonzero(rng.random(n) < density).astype(np.int32)
        val = rng.integers(0, 1 << 16, pos.size, dtype=np.uint16)
        B, st = dev(b), zeros(1, torch.int32)
        pulse.pulse_apply_patch(B, dev(pos), dev(val), dev(np.array([pos.size], np.int64)), st, max_count=pos.size)
        torch.cuda.synchronize()
        ref, rst = oracle.apply_patch(b, pos, val)
        assert np.array_equal(u16(B), ref) and int(host(st)[0]) == rst == 0


@pytest.mark.parametrize("density", [1.0, 0.3, 0.07, 0.05, 0.01, 0.0])
def test_apply_tiled_matches_oracle(density):
    """The tiled apply against the oracle, with tiles above and below the dense
    threshold in one patch, a ragged last tile, and the tile index built on the
    device; the same with out-of-range entries at both ends (reported, skipped)."""
    rng = np.random.default_rng(int(density * 100) + 3)
    n = 13 * 16384 + 4321
    b = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    d = np.full(n, density)
    d[5 * 16384: 7 * 16384] = 0.9       # two dense tiles in any patch
    d[9 * 16384: 10 * 16384] = 0.001     # a sparse one
    pos = np.flatnonzero(rng.random(n) < d).astype(np.int32)
    for extra in (False, True):
        p = np.concatenate([np.array([-9, -1], np.int32), pos, np.array([n, n + 77], np.int32)]) if extra else pos
        val = rng.integers(0, 1 << 16, p.size, dtype=np.uint16)
        m = p.size
        I, V = (dev(p), dev(val)) if m else (zeros(1, torch.int32), zeros(1, torch.int16))
        tf = zeros(pulse.patch_tile_count(n), torch.int64)
        cnt = dev(np.array([m], np.int64))
        pulse.pulse_patch_tiles(I, cnt, tf, n, max_count=max(m, 1))
        B, st = dev(b), zeros(1, torch.int32)
        pulse.pulse_apply_patch_tiled(B, I, V, tf, st, max_count=max(m, 1))
        torch.cuda.synchronize()
        ref, rst = oracle.apply_patch(b, p, val)
        assert np.array_equal(u16(B), ref), np.flatnonzero(u16(B) != ref)[:8]
        assert int(host(st)[0]) == rst == (pulse.PULSE_DS_BADINDEX if extra else 0)


def test_patch_chain_20_steps_no_drift():
    """Encode -> apply on the device each step, no host sync between them; the
    receiver stays bit-identical to the direct cast of every version."""
    n = 300_007
    ws_host = workload.host_masters(n, seed=21, steps=20)
    b_send = dev(oracle.cast_bf16(ws_host[0]))
    b_recv = b_send.clone()
    idx, val = zeros(n, torch.int32), zeros(n, torch.int16)
    cnt, st = zeros(1, torch.int64), zeros(1, torch.int32)
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, n)
    for t in range(1, 21):
        pulse.pulse_cast_diff(dev(ws_host[t]), b_send, b_send, None, idx, val, cnt, st, ws)
        pulse.pulse_apply_patch(b_recv, idx, val, cnt, st, max_count=n)
        torch.cuda.synchronize()
        assert np.array_equal(u16(b_recv), oracle.cast_bf16(ws_host[t]))
    assert int(host(st)[0]) == 0


@pytest.mark.parametrize("nbytes", [1, 15, 16, 17, 4096, 1000003])
def test_xor_mask_apply(nbytes):
    rng = np.random.default_rng(nbytes)
    d = rng.integers(0, 256, nbytes, dtype=np.uint8)
    m = rng.integers(0, 256, nbytes, dtype=np.uint8)
    D = dev(d)
    pulse.xor_mask_apply(D, dev(m))
    torch.cuda.synchronize()
    assert np.array_equal(host(D), oracle.xor_apply(d, m))


# ---- LZ4 ---------------------------------------------------------------------------
def mask_bytes(nbytes, density, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros(nbytes, np.uint8)
    hit = rng.random(nbytes) < density
    m[hit] = rng.integers(1, 256, int(hit.sum()), dtype=np.uint8)
    return m


def gpu_encode(src, block_bytes=65536, src_xor=None, cap=None):
    nbytes = src.size
    nb = (nbytes + block_bytes - 1) // block_bytes
    cap = pulse.lz4_payload_bound(nbytes, block_bytes) if cap is None else cap
    payload = zeros(cap, torch.uint8)
    sizes, offs = zeros(nb, torch.int32), zeros(nb, torch.int64)
    tot, st = zeros(1, torch.int64), zeros(1, torch.int32)
    ws = pulse.workspace(pulse.PULSE_OP_LZ4_ENCODE, nbytes, block_bytes)
    pulse.lz4_encode_blocks(dev(src), payload[:cap] if cap else payload[:0], sizes, offs, tot, st, ws,
                            src_xor=None if src_xor is None else dev(src_xor), block_bytes=block_bytes)
    torch.cuda.synchronize()
    t = int(host(tot)[0])
    return dict(payload=host(payload)[:min(t, cap)], sizes=host(sizes, np.uint32)[:nb],
                offsets=host(offs, np.uint64)[:nb], total=t, status=int(host(st)[0]))


def runs_block(rng, nruns, size=65536):
    """`size` bytes holding `nruns` runs of exactly five zeros, evenly spread
    between non-zero literals with no two equal neighbours (each run is one
    sequence of the canonical parse), then literals to the end."""
    gap = (size - 64) // nruns - 5
    r = rng.integers(1, 254, size, dtype=np.int64)
    lit = (np.cumsum(r) % 255 + 1).astype(np.uint8)  # 1 .. 255, neighbours differ
    out = lit.copy()
    for k in range(nruns):
        s0 = k * (gap + 5) + gap
        out[s0:s0 + 5] = 0
    return out


@pytest.mark.parametrize("block_bytes,counts", [
    (65536, [1, 2, 3, 17, 250, 1000, 1796, 1797, 1798, 1799]),
    (32768, [1, 3, 100, 1000, 1796, 1797, 1798, 1799]),
    (16384, [1, 3, 50, 300, 600, 900]),
])
def test_lz4_encode_large_blocks_around_the_table_size(block_bytes, counts):
    """Blocks whose encoding is larger than the encoder's 14 KiB window, with
    1 to 1,799 sequences: up to 1,797 (the sequence table's size less one)
    they are written by output piece, from 1,798 on in window passes; every
    block size class, a ragged last block, payload offsets at many
    alignments.  The payload equals the oracle's byte for byte."""
    rng = np.random.default_rng(41 + block_bytes)
    blocks = [runs_block(rng, n, block_bytes) for n in counts]
    blocks.append(runs_block(rng, 20 if block_bytes < 65536 else 300, block_bytes - 1000))
    m = np.concatenate(blocks)
    ref = oracle.lz4_encode_blocks(m, block_bytes)
    assert ref["status"] == 0 and int(ref["sizes"].min()) > 14336
    assert len({int(o) % 16 for o in ref["offsets"]}) > 3
    got = gpu_encode(m, block_bytes)
    assert got["status"] == 0 and got["total"] == ref["total"]
    assert np.array_equal(got["sizes"], ref["sizes"]) and np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["payload"], ref["payload"][:ref["total"]])
    dst = rng.integers(0, 256, m.size, dtype=np.uint8)
    d, st = gpu_decode(ref["payload"], ref["offsets"], ref["sizes"], dst, 1, block_bytes=block_bytes)
    assert st == 0 and np.array_equal(d, dst ^ m)


@pytest.mark.parametrize("nbytes", [1, 12, 13, 100, 65536, 65537, 3 * 65536 + 1234, 1 << 22])
@pytest.mark.parametrize("density", [0.0, 0.01, 0.08, 0.5, 1.0])
def test_lz4_encode_matches_oracle(nbytes, density):
    m = mask_bytes(nbytes, density, seed=nbytes + int(density * 1000))
    got = gpu_encode(m)
    ref = oracle.lz4_encode_blocks(m, 65536)
    assert got["total"] == ref["total"] and got["status"] == 0
    assert np.array_equal(got["sizes"], ref["sizes"]) and np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["payload"], ref["payload"])


@pytest.mark.parametrize("block_bytes", [16384, 32768])
def test_lz4_encode_other_block_sizes(block_bytes):
    m = mask_bytes(5 * block_bytes + 77, 0.05, seed=block_bytes)
    got = gpu_encode(m, block_bytes)
    ref = oracle.lz4_encode_blocks(m, block_bytes)
    assert np.array_equal(got["payload"], ref["payload"]) and np.array_equal(got["sizes"], ref["sizes"])


def test_lz4_encode_runs_and_patterns():
    """Long runs of non-zero values, runs crossing thread chunks and blocks, and
    the closed-form blocks (all zero, no runs)."""
    parts = [np.zeros(70000, np.uint8), np.full(1000, 7, np.uint8), (np.arange(65536) & 0xFF).astype(np.uint8),
             np.full(300, 9, np.uint8), np.zeros(255, np.uint8), np.array([1, 2, 2, 2, 2, 2, 3], np.uint8),
             np.full(65536 * 2 + 5, 0xAB, np.uint8)]
    m = np.concatenate(parts)
    got = gpu_encode(m)
    ref = oracle.lz4_encode_blocks(m, 65536)
    assert np.array_equal(got["payload"], ref["payload"]) and np.array_equal(got["sizes"], ref["sizes"])
    z = gpu_encode(np.zeros(65536, np.uint8))
    assert z["total"] == 267
    r = gpu_encode((np.arange(65536) & 0xFF).astype(np.uint8))
    assert r["total"] == 65794


def test_lz4_encode_xor_of_two_views_and_capacity():
    rng = np.random.default_rng(17)
    a = rng.integers(0, 1 << 16, 200_003, dtype=np.uint16)
    b = a.copy()
    hit = rng.random(a.size) < 0.08
    b[hit] ^= rng.integers(1, 1 << 16, int(hit.sum()), dtype=np.uint16)
    ref = oracle.lz4_encode_blocks(a, 65536, src_xor=b)
    got = gpu_encode(a.view(np.uint8), src_xor=b.view(np.uint8))
    assert np.array_equal(got["payload"], ref["payload"])
    cap = int(ref["offsets"][3]) + 5
    got = gpu_encode(a.view(np.uint8), src_xor=b.view(np.uint8), cap=cap)
    assert got["status"] == pulse.PULSE_DS_CAPACITY and got["total"] == ref["total"]
    assert np.array_equal(got["payload"][: int(ref["offsets"][3])], ref["payload"][: int(ref["offsets"][3])])


def gpu_decode(payload, offsets, sizes, dst, mode, block_bytes=65536, payload_bytes=None):
    nbytes = dst.size
    nb = (nbytes + block_bytes - 1) // block_bytes
    P = dev(payload) if payload.size else zeros(1, torch.uint8)
    D = dev(dst)
    st = zeros(1, torch.int32)
    pb = payload.size if payload_bytes is None else payload_bytes
    ws = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nb, pb)
    pulse.lz4_decode_blocks(P, dev(offsets.astype(np.uint64)), dev(sizes.astype(np.uint32)), D, st, ws, mode=mode,
                            block_bytes=block_bytes, nbytes=nbytes, payload_bytes=pb)
    torch.cuda.synchronize()
    return host(D), int(host(st)[0])


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("density", [0.0, 0.00005, 0.0005, 0.002, 0.01, 0.08, 1.0])
def test_lz4_decode_canonical_payloads(mode, density):
    nbytes = 7 * 65536 + 999
    m = mask_bytes(nbytes, density, seed=int(density * 100) + mode)
    enc = oracle.lz4_encode_blocks(m, 65536)
    dst = np.random.default_rng(5).integers(0, 256, nbytes, dtype=np.uint8)
    got, st = gpu_decode(enc["payload"], enc["offsets"], enc["sizes"], dst, mode)
    ref, rst = oracle.lz4_decode_blocks(enc["payload"], enc["offsets"], enc["sizes"], dst, mode=mode)
    assert st == rst == 0 and np.array_equal(got, ref)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_long_zero_runs_at_window_edges(mode):
    """Canonical sequences of l non-zero-ended literal runs (l = 1 .. 12)
    followed by zero runs whose match lengths need k bytes of 255 and a final
    byte: every k from 0 to one past what fits in a 16-byte window after the
    literals, and final bytes 0, 1 and 254 -- both sides of the decoder's
    one-window path and its byte-by-byte path."""
    rng = np.random.default_rng(77 + mode)
    parts = []
    for ll in range(1, 13):
        for k in range(0, 14 - ll):
            for f in (0, 1, 254):
                L = 19 + 255 * k + f  # match length: 15 in the token, then k bytes 255 and f
                lit = rng.integers(1, 256, ll - 1, dtype=np.uint8)
                parts += [lit, np.zeros(L + 1, np.uint8)]  # the run's first zero is the last literal
    parts.append(rng.integers(1, 256, 40, dtype=np.uint8))
    m = np.concatenate(parts)
    enc = oracle.lz4_encode_blocks(m, 65536)
    dst = np.random.default_rng(6).integers(0, 256, m.size, dtype=np.uint8)
    got, st = gpu_decode(enc["payload"], enc["offsets"], enc["sizes"], dst, mode)
    ref, rst = oracle.lz4_decode_blocks(enc["payload"], enc["offsets"], enc["sizes"], dst, mode=mode)
    assert st == rst == 0 and np.array_equal(got, ref)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shift", [0, 1, 2, 3, 7, 13])
def test_lz4_decode_dense_short_sequences(mode, shift):
    """Canonical blocks made of the shortest sequences (literal runs of 1 .. 13
    bytes, zero runs of 5 .. 22 bytes, so 4 .. 17-byte sequences, a few with
    one match-length byte and a few with a literal run too long for the
    decoder's fast step), shifted by `shift` leading bytes: the parse takes
    several such sequences per step at every offset of its ring, and its
    per-step window limit and ring refills fall between and inside them."""
    rng = np.random.default_rng(1000 + 10 * shift + mode)
    parts = [rng.integers(1, 256, shift, dtype=np.uint8)]
    total = shift
    while total < 5 * 65536 + 4321:
        ll = int(rng.choice([1, 1, 1, 2, 2, 3, 4, 5, 8, 12, 13]))
        run = int(rng.choice([5, 5, 5, 6, 7, 9, 12, 19, 20, 22]))
        lit = rng.integers(1, 256, ll - 1, dtype=np.uint8)
        parts += [lit, np.zeros(run + 1, np.uint8)]  # the run's first zero is the last literal
        total += ll + run
    m = np.concatenate(parts)[: 5 * 65536 + 4321]
    enc = oracle.lz4_encode_blocks(m, 65536)
    assert enc["sizes"].max() > 20000  # dense blocks: thousands of sequences each
    dst = np.random.default_rng(9 + shift).integers(0, 256, m.size, dtype=np.uint8)
    got, st = gpu_decode(enc["payload"], enc["offsets"], enc["sizes"], dst, mode)
    ref, rst = oracle.lz4_decode_blocks(enc["payload"], enc["offsets"], enc["sizes"], dst, mode=mode)
    assert st == rst == 0 and np.array_equal(got, ref)
    assert np.array_equal(ref, m if mode == 0 else dst ^ m)


def random_payload(rng, nblocks, last, block_bytes=65536, **kw):
    comps, plains = [], []
    for b in range(nblocks):
        size = last if b == nblocks - 1 else block_bytes
        c, p = lz4_spec.random_block(rng, size, **kw)
        comps.append(c)
        plains.append(p)
    sizes = np.array([len(c) for c in comps], np.uint32)
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
    return np.frombuffer(b"".join(comps), np.uint8).copy(), offs, sizes, np.frombuffer(b"".join(plains), np.uint8)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_general_streams(mode):
    """Streams the canonical encoder never writes: long literal runs, matches
    reaching into earlier sequences (general path), overlapping copies."""
    rng = np.random.default_rng(31 + mode)
    payload, offs, sizes, plain = random_payload(rng, 6, 12345)
    dst = rng.integers(0, 256, plain.size, dtype=np.uint8)
    got, st = gpu_decode(payload, offs, sizes, dst, mode)
    ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
    assert st == rst == 0 and np.array_equal(got, ref)
    assert np.array_equal(ref, plain if mode == 0 else dst ^ plain)
    # offset-1 matches only, mixing blocks for both decode paths
    rng = np.random.default_rng(77)
    payload, offs, sizes, plain = random_payload(rng, 5, 999, max_off=1)
    dst2 = rng.integers(0, 256, plain.size, dtype=np.uint8)
    got, st = gpu_decode(payload, offs, sizes, dst2, mode)
    ref, _ = oracle.lz4_decode_blocks(payload, offs, sizes, dst2, mode=mode)
    assert st == 0 and np.array_equal(got, ref)


def test_lz4_decode_corrupt_blocks_leave_dst():
    data = mask_bytes(4 * 65536, 0.05, seed=8)
    enc = oracle.lz4_encode_blocks(data, 65536)
    dst = np.full(data.size, 0x5A, np.uint8)
    cases = []
    p = enc["payload"].copy()
    p[int(enc["offsets"][1])] ^= 0xFF
    cases.append((p, enc["offsets"], enc["sizes"]))                       # broken token
    s = enc["sizes"].copy()
    s[2] -= 1
    cases.append((enc["payload"], enc["offsets"], s))                      # truncated block
    o = enc["offsets"].copy()
    o[3] = o[2] + 1
    cases.append((enc["payload"], o, enc["sizes"]))                        # overlaps an earlier block
    s = enc["sizes"].copy()
    s[3] += 100000
    cases.append((enc["payload"], enc["offsets"], s))                      # outside the payload
    for payload, offs, sizes in cases:
        for mode in (0, 1):
            got, st = gpu_decode(payload, offs, sizes, dst, mode)
            ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
            assert rst == pulse.PULSE_DS_CORRUPT and st == rst
            assert np.array_equal(got, ref)


def ext_len(n):
    """LZ4 length bytes after a nibble of 15 for a length n >= 15 (else 0)."""
    return 0 if n < 15 else (n - 15) // 255 + 1


def literal_mix(block_bytes, nlit, tail, seed):
    """Blocks alternating between incompressible bytes (no two equal
    neighbours, so no run qualifies: each is one literal run) and a
    compressible block (random bytes, then zeros) whose encoding is chosen so
    that a literal block and a compressible one together take an odd number of
    payload bytes: the literal blocks then start at every alignment mod 16.
    The last block is `tail` bytes of incompressible data."""
    rng = np.random.default_rng(seed)

    def lit(v):
        return (np.cumsum(rng.integers(1, 256, v, dtype=np.int64)) % 256).astype(np.uint8)  # neighbours differ

    lit_size = 1 + ext_len(block_bytes) + block_bytes
    for p in range(20, 60):
        cmp = np.zeros(block_bytes, np.uint8)
        cmp[:p] = rng.integers(1, 256, p, dtype=np.uint8)
        if (lit_size + int(oracle.lz4_encode_blocks(cmp, block_bytes)["total"])) % 2 == 1:
            break
    out = []
    for _ in range(nlit):
        out += [lit(block_bytes), cmp]
    out.append(lit(tail))
    return np.concatenate(out)


@pytest.mark.parametrize("block_bytes", [65536, 16384])
def test_lz4_literal_only_blocks(block_bytes):
    """Incompressible blocks (one literal run each: token, length bytes up to
    a 258-byte header for 64 KiB, then the bytes) at every payload alignment
    and with ragged tails on both sides of every length-byte boundary: the
    encoder's payload equals the oracle's byte for byte, and both decode modes
    equal the oracle's."""
    for tail in (15, 16, 31, 269, 270, 271, 524, 525, 4097, block_bytes):
        m = literal_mix(block_bytes, 16, tail, seed=tail)
        ref = oracle.lz4_encode_blocks(m, block_bytes)
        lit_blocks = [b for b in range(0, ref["sizes"].size, 2)]
        lens = [min(block_bytes, m.size - b * block_bytes) for b in lit_blocks]
        assert all(int(ref["sizes"][b]) == 1 + ext_len(n) + n for b, n in zip(lit_blocks, lens))
        shifts = {(int(ref["offsets"][b]) + 1 + ext_len(n)) % 16 for b, n in zip(lit_blocks, lens)}
        assert len(shifts) == 16
        got = gpu_encode(m, block_bytes)
        assert got["status"] == 0 and got["total"] == ref["total"]
        assert np.array_equal(got["sizes"], ref["sizes"]) and np.array_equal(got["offsets"], ref["offsets"])
        assert np.array_equal(got["payload"], ref["payload"][:ref["total"]])
        dst = np.random.default_rng(tail + 1).integers(0, 256, m.size, dtype=np.uint8)
        for mode in (0, 1):
            d, st = gpu_decode(ref["payload"], ref["offsets"], ref["sizes"], dst, mode, block_bytes=block_bytes)
            r, rst = oracle.lz4_decode_blocks(ref["payload"], ref["offsets"], ref["sizes"], dst,
                                              block_bytes=block_bytes, mode=mode)
            assert st == rst == 0 and np.array_equal(d, r)
            assert np.array_equal(r, m if mode == 0 else dst ^ m)


def length_bytes(n):
    return [255] * ((n - 15) // 255) + [(n - 15) % 255]


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_literal_shaped_blocks_of_other_forms(mode):
    """Blocks with the first token (0xF0) and the size of a single literal run
    of their full length that are something else: (a) a valid block of two
    sequences (25515 literals, a 4-byte match at offset 1, 40017 literals),
    whose length bytes disagree with a single run, decodes like the oracle;
    (b) a single run with one length byte changed is corrupt and leaves its
    dst range as it was; the blocks around them decode as usual."""
    rng = np.random.default_rng(900 + mode)
    l1, l2 = 25515, 40017
    a1, a2 = rng.integers(1, 256, l1, dtype=np.uint8), rng.integers(1, 256, l2, dtype=np.uint8)
    two = np.concatenate([np.array([0xF0] + length_bytes(l1), np.uint8), a1, np.array([1, 0, 0xF0] + length_bytes(l2), np.uint8), a2])
    assert two.size == 65536 + 1 + ext_len(65536)
    plain_two = np.concatenate([a1, np.full(4, a1[-1], np.uint8), a2])
    lit = rng.integers(1, 256, 65536, dtype=np.uint8)
    one = np.concatenate([np.array([0xF0] + length_bytes(65536), np.uint8), lit])
    for k, (blk, valid) in enumerate([(two, True), (one, False), (one, False)]):
        bad = blk.copy()
        if not valid:
            bad[1 + (100 if k == 1 else ext_len(65536) - 1)] ^= 1   # a middle 255, then the last length byte
        comps = [oracle.lz4_encode_blocks(mask_bytes(65536, 0.05, seed=k), 65536)["payload"], bad,
                 oracle.lz4_encode_blocks(mask_bytes(65536, 1.0, seed=k), 65536)["payload"]]
        sizes = np.array([c.size for c in comps], np.uint32)
        offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
        payload = np.concatenate(comps)
        dst = np.full(3 * 65536, 0x5A, np.uint8)
        got, st = gpu_decode(payload, offs, sizes, dst, mode)
        ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
        assert st == rst == (0 if valid else pulse.PULSE_DS_CORRUPT)
        assert np.array_equal(got, ref)
        if valid:
            assert np.array_equal(ref[65536:131072], plain_two if mode == 0 else dst[65536:131072] ^ plain_two)
        else:
            assert np.all(ref[65536:131072] == 0x5A)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_length_chains_across_the_ring(mode):
    """Length chains longer than the parse's 256-byte ring of compressed
    bytes, at many ring phases: all-zero blocks (a 257-byte match-length
    chain), p literals then zeros (p = 1 .. 40: a chain of about 255 bytes
    after each offset position), and 65040 .. 65530 literals then zeros (a
    literal-length chain of 256 or 257 bytes).  The encoder's payload equals
    the oracle's, and both decode modes equal the oracle's."""
    rng = np.random.default_rng(40 + mode)
    blocks = [np.zeros(65536, np.uint8)]
    for p in range(1, 41):
        b = np.zeros(65536, np.uint8)
        b[:p] = rng.integers(1, 256, p, dtype=np.uint8)
        blocks.append(b)
    for L in (65040, 65041, 65100, 65295, 65296, 65300, 65530):
        b = np.zeros(65536, np.uint8)
        b[:L] = rng.integers(1, 256, L, dtype=np.uint8)
        blocks.append(b)
    blocks.append(np.zeros(65536 - 7, np.uint8))
    m = np.concatenate(blocks)
    enc = oracle.lz4_encode_blocks(m, 65536)
    got = gpu_encode(m)
    assert got["status"] == 0 and got["total"] == enc["total"]
    assert np.array_equal(got["payload"], enc["payload"][:enc["total"]])
    dst = rng.integers(0, 256, m.size, dtype=np.uint8)
    d, st = gpu_decode(enc["payload"], enc["offsets"], enc["sizes"], dst, mode)
    r, rst = oracle.lz4_decode_blocks(enc["payload"], enc["offsets"], enc["sizes"], dst, mode=mode)
    assert st == rst == 0 and np.array_equal(d, r)
    assert np.array_equal(r, m if mode == 0 else dst ^ m)


def canonical_seq(lit, ml):
    """One canonical sequence: one literal byte, offset 1, a match of ml >= 4
    (the literal repeated): its bytes and the bytes it decodes to."""
    mc = min(ml - 4, 15)
    ext = length_bytes(ml - 4) if ml - 4 >= 15 else []
    return [0x10 | mc, lit, 1, 0] + ext, [lit] * (ml + 1)


def canonical_block(rng, nseq, ml, lf):
    """nseq canonical sequences (match length ml each, non-zero literals), then
    a final run of lf >= 5 literals."""
    comp, plain = [], []
    for lit in rng.integers(1, 256, nseq):
        c, p = canonical_seq(int(lit), ml)
        comp += c
        plain += p
    tail = [int(x) for x in rng.integers(1, 256, lf)]
    comp += [min(lf, 15) << 4] + (length_bytes(lf) if lf >= 15 else []) + tail
    plain += tail
    return np.array(comp, np.uint8), np.array(plain, np.uint8)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_checkpoint_intervals(mode):
    """The decode's checkpoint interval is chosen per block from its
    compressed size S (1 sequence up to S = 768, doubling at 768, 1536, 3072
    and 6144 bytes, 16 above).  Blocks of the densest canonical sequences (4
    bytes each) at sizes on both sides of every threshold, after a 64 KiB
    block of 13,106 such sequences (820 segments: K2's threads take several
    each) and a staged block of 5-byte sequences: both modes equal the
    oracle's decode and the plain bytes."""
    rng = np.random.default_rng(60 + mode)
    a = canonical_block(rng, 13106, 4, 6)                      # 64 KiB out, S = 52,431
    b = canonical_block(rng, 1074, 60, 65536 - 1074 * 61)      # 64 KiB out, S = 5,37x
    assert a[1].size == 65536 and b[1].size == 65536 and a[0].size == 52431 and b[0].size < 6144
    for target in (6, 200, 767, 768, 769, 1535, 1536, 1537, 3071, 3072, 3073, 6143, 6144, 6145, 13001):
        lf = 5 + (target - 1 - 5) % 4                          # S = 4 k + 1 + lf
        k = (target - 1 - lf) // 4
        c, p = canonical_block(rng, k, 4, lf)
        assert c.size == target
        comps, plains = [a[0], b[0], c], [a[1], b[1], p]
        sizes = np.array([x.size for x in comps], np.uint32)
        offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
        payload = np.concatenate(comps)
        plain = np.concatenate(plains)
        dst = rng.integers(0, 256, plain.size, dtype=np.uint8)
        got, st = gpu_decode(payload, offs, sizes, dst, mode)
        ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
        assert st == rst == 0, target
        assert np.array_equal(ref, plain if mode == 0 else dst ^ plain), target
        assert np.array_equal(got, ref), target


def literal_run_block(rng, nseq, total, ml):
    """A canonical block of nseq sequences, each a run of non-zero literals and
    an offset-1 match of ml, then a final literal run, decoding to `total`
    bytes: its bytes and its plain bytes."""
    ll = (total - 16) // nseq - ml
    assert ll >= 1 and ml >= 4
    comp, plain = [], []
    for _ in range(nseq):
        lits = [int(x) for x in rng.integers(1, 256, ll)]
        mc = min(ml - 4, 15)
        comp += [(min(ll, 15) << 4) | mc] + (length_bytes(ll) if ll >= 15 else []) + lits + [1, 0]
        comp += length_bytes(ml - 4) if ml - 4 >= 15 else []
        plain += lits + [lits[-1]] * ml
    lf = total - len(plain)
    tail = [int(x) for x in rng.integers(1, 256, lf)]
    comp += [min(lf, 15) << 4] + (length_bytes(lf) if lf >= 15 else []) + tail
    plain += tail
    return np.array(comp, np.uint8), np.array(plain, np.uint8)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_large_blocks_of_few_sequences(mode):
    """Blocks over 6 KiB compressed hold 16-sequence checkpoints; those that
    compress to more than half their length (long literal runs) also keep one
    per sequence for their first 128, and are rebuilt one sequence per thread
    when they have no more.  Blocks of 2 to 300 sequences of both kinds --
    64 KiB blocks from global memory, a short last block from the LDS stage --
    after a dense block: both modes equal the oracle's decode and the plain
    bytes."""
    rng = np.random.default_rng(70 + mode)
    dense = canonical_block(rng, 13106, 4, 6)
    for nseq in (2, 16, 17, 127, 128, 129, 300):
        lit_heavy = literal_run_block(rng, nseq, 65536, 8)          # S > 32 KiB
        match_heavy = literal_run_block(rng, nseq, 65536, (65536 - 16) // nseq - max(48, 7000 // nseq + 1))
        last = literal_run_block(rng, nseq, 13000, 8)               # S in (6 KiB, 14 KiB]: staged
        assert lit_heavy[0].size > 32768 and 6144 < match_heavy[0].size < 32768, nseq
        assert 6500 < last[0].size <= 14336 and last[0].size > 6144, nseq
        blocks = [lit_heavy, dense, match_heavy, last]
        comps, plains = [x[0] for x in blocks], [x[1] for x in blocks]
        sizes = np.array([x.size for x in comps], np.uint32)
        offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
        payload = np.concatenate(comps)
        plain = np.concatenate(plains)
        dst = rng.integers(0, 256, plain.size, dtype=np.uint8)
        got, st = gpu_decode(payload, offs, sizes, dst, mode)
        ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
        assert st == rst == 0, nseq
        assert np.array_equal(ref, plain if mode == 0 else dst ^ plain), nseq
        assert np.array_equal(got, ref), nseq


def sequence_block(rng, seqs, total):
    """A canonical block of the sequences (literal count, match length) given,
    each with non-zero literals and an offset-1 match, then a final literal
    run that brings the plain bytes to `total`: its bytes and plain bytes."""
    comp, plain = [], []
    for ll, ml in seqs:
        lits = [int(x) for x in rng.integers(1, 256, ll)]
        comp += [(min(ll, 15) << 4) | min(ml - 4, 15)] + (length_bytes(ll) if ll >= 15 else []) + lits + [1, 0]
        comp += length_bytes(ml - 4) if ml - 4 >= 15 else []
        plain += lits + [lits[-1]] * ml
    lf = total - len(plain)
    assert lf >= 5
    tail = [int(x) for x in rng.integers(1, 256, lf)]
    comp += [min(lf, 15) << 4] + (length_bytes(lf) if lf >= 15 else []) + tail
    plain += tail
    return np.array(comp, np.uint8), np.array(plain, np.uint8)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_literal_runs_past_the_ring_walk(mode):
    """The parse hands a block with a literal run longer than 2055 bytes (a
    length chain of nine bytes or more) to its walk from global memory, which
    also writes the per-sequence checkpoints of a large literal-heavy block.
    Runs of 2055 to 3000 bytes, first, in the middle and last; blocks of more
    and of fewer than 128 sequences, over and under 32 KiB compressed; a short
    last block from the LDS stage, one with fewer than 6 KiB compressed: both
    modes equal the oracle's decode and the plain bytes."""
    rng = np.random.default_rng(95 + mode)
    B = 65536
    blocks = [
        sequence_block(rng, [(2056, 4)] + [(200, 4)] * 150, B),           # 152 sequences, S > 64 KiB
        sequence_block(rng, [(1, 4)] * 100 + [(2100, 4)] + [(1, 300)] * 100, B),
        sequence_block(rng, [(2055, 4)] + [(1, 500)] * 100, B),          # the ring walk keeps it
        sequence_block(rng, [(1, 4)] * 3 + [(2240 + 7 * k, 4) for k in range(12)], B),
        sequence_block(rng, [(3000, 8)] * 10, B),                         # 11 sequences, S > 32 KiB
        sequence_block(rng, [(1, 8)] * 40 + [(2056, 4)] + [(1, 1000)] * 60, B),  # S < 6 KiB, a long last run
        canonical_block(rng, 13106, 4, 6),
    ]
    assert blocks[0][0].size > B and blocks[4][0].size > 32768 and blocks[5][0].size < 6144
    for last in ([(2500, 8)] * 4, [(2200, 4)] + [(1, 4)] * 50):
        tot = sum(a * 1 + b for a, b in last) + 6
        blk = sequence_block(rng, last, tot)
        comps = [x[0] for x in blocks] + [blk[0]]
        plains = [x[1] for x in blocks] + [blk[1]]
        assert all(p.size == B for p in plains[:-1])
        sizes = np.array([x.size for x in comps], np.uint32)
        offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
        payload = np.concatenate(comps)
        plain = np.concatenate(plains)
        dst = rng.integers(0, 256, plain.size, dtype=np.uint8)
        got, st = gpu_decode(payload, offs, sizes, dst, mode)
        ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
        assert st == rst == 0, last[0]
        assert np.array_equal(ref, plain if mode == 0 else dst ^ plain), last[0]
        assert np.array_equal(got, ref), last[0]


def raw_block(rng, seqs, total=None, final=None):
    """LZ4 block bytes from (literal count, match offset, match length)
    triples, any offsets; then a final literal run of `final` bytes, or of the
    bytes that bring the plain length to `total`."""
    comp, n = [], 0
    for ll, off, ml in seqs:
        comp += [(min(ll, 15) << 4) | min(ml - 4, 15)] + (length_bytes(ll) if ll >= 15 else [])
        comp += [int(x) for x in rng.integers(1, 256, ll)] + [off & 255, off >> 8]
        comp += length_bytes(ml - 4) if ml - 4 >= 15 else []
        n += ll + ml
    lf = total - n if final is None else final
    comp += [min(lf, 15) << 4] + (length_bytes(lf) if lf >= 15 else []) + [int(x) for x in rng.integers(1, 256, lf)]
    return np.array(comp, np.uint8)


@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_long_blocks_of_other_forms(mode):
    """Blocks that start with a literal run longer than 2055 bytes (so the
    parse lists them for its wave-per-block walk from global memory), then go
    on in forms other than the canonical one: valid ones (a match of offset
    2, a match right after a match, a long run of offset 1 matches) decode like
    the oracle through the serial kernel or the fast path; corrupt ones (an
    offset of 0 or past the output, a literal run or a match past the block,
    a length chain that runs off the block, a block that decodes short) are
    reported and leave their dst range as it was, while the blocks around
    them decode as usual."""
    rng = np.random.default_rng(300 + mode)
    B = 65536
    L = 2100
    valid = [
        raw_block(rng, [(L, 1, 4)] * 6, B),                                # canonical
        raw_block(rng, [(L, 1, 4), (300, 2, 9), (L, 1, 4)], B),            # offset 2
        raw_block(rng, [(L, 1, 4), (0, 1, 7), (L, 1, 20)], B),             # a match right after a match
        raw_block(rng, [(L, 1, 40000)], B),                                # a long offset-1 run
        raw_block(rng, [(3000 + 17 * k, 1, 4 + k) for k in range(12)], B),
    ]
    bad = [
        raw_block(rng, [(L, 1, 4), (20, 0, 4)], B),                        # offset 0
        raw_block(rng, [(L, 1, 4), (20, 4000, 4)], B),                     # offset past the output
        raw_block(rng, [(L, 1, 4)], None, 3000)[:L + 3000],                # final run past the block
        raw_block(rng, [(L, 1, 70000)], None, 5),                          # match past the block length
        np.concatenate([raw_block(rng, [(L, 1, 4)], None, 5)[:-6], np.array([0x0F, 1, 0] + [255] * 40, np.uint8)]),
        raw_block(rng, [(L, 1, 4)] * 3, B - 100),                          # decodes 100 bytes short
    ]
    for blocks, want in ((valid, 0), (valid[:2] + bad[:1] + valid[2:4] + bad[1:] + valid[4:], pulse.PULSE_DS_CORRUPT)):
        sizes = np.array([x.size for x in blocks], np.uint32)
        offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
        payload = np.concatenate(blocks)
        dst = rng.integers(0, 256, B * len(blocks), dtype=np.uint8)
        got, st = gpu_decode(payload, offs, sizes, dst, mode)
        ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
        assert st == rst == want
        assert np.array_equal(got, ref)
        if want:  # each corrupt block's range is untouched, each valid one changed
            for k, blk in enumerate(blocks):
                same = np.array_equal(got[k * B:(k + 1) * B], dst[k * B:(k + 1) * B])
                assert same == any(blk is x for x in bad), k


def test_lz4_decode_more_long_blocks_than_walk_waves():
    """More blocks for the parse's wave-per-block walk than that kernel has
    waves (2,048 workgroups of four): 8,450 incompressible 16 KiB blocks (each
    one literal run), with a compressible block every 97th and a ragged last
    block, so that waves take several list entries in turn.  The encoding
    equals the oracle's byte for byte, and both decode modes equal the
    oracle's decode."""
    rng = np.random.default_rng(77)
    B = 16384
    nblk = 8450
    m = (np.cumsum(rng.integers(1, 256, nblk * B - 777, dtype=np.int64)) % 256).astype(np.uint8)  # neighbours differ
    for k in range(0, nblk - 1, 97):
        m[k * B + 40:(k + 1) * B] = 0  # a compressible block now and then
    ref = oracle.lz4_encode_blocks(m, B)
    assert ref["status"] == 0
    dense = int(np.sum(4 * ref["sizes"].astype(np.int64) > 3 * B))
    assert dense > 4 * 2048
    got = gpu_encode(m, B)
    assert got["status"] == 0 and got["total"] == ref["total"]
    assert np.array_equal(got["sizes"], ref["sizes"]) and np.array_equal(got["payload"], ref["payload"][:ref["total"]])
    dst = rng.integers(0, 256, m.size, dtype=np.uint8)
    for mode in (0, 1):
        d, st = gpu_decode(ref["payload"], ref["offsets"], ref["sizes"], dst, mode, block_bytes=B)
        r, rst = oracle.lz4_decode_blocks(ref["payload"], ref["offsets"], ref["sizes"], dst, block_bytes=B, mode=mode)
        assert st == rst == 0
        assert np.array_equal(d, r)
        assert np.array_equal(r, m if mode == 0 else dst ^ m)


@pytest.mark.skipif(not lz4_system.available(), reason="liblz4 is not installed")
@pytest.mark.parametrize("mode", [0, 1])
def test_lz4_decode_library_blocks(mode):
    """Blocks written by the system's LZ4 library (its own parse: matches at
    any offset, so most go to the serial kernel; random bytes become one
    literal run, walked a wave per block): both decode modes give back the
    bytes the library compressed, like the oracle's decode."""
    rng = np.random.default_rng(500 + mode)
    cases = [mask_bytes(5 * 65536 + 321, d, seed=int(d * 1e4) + mode) for d in (0.0, 0.0005, 0.01, 0.08, 0.5)]
    cases.append(np.repeat(rng.integers(0, 256, 9000, dtype=np.uint8), rng.integers(1, 60, 9000))[:3 * 65536])
    cases.append((np.cumsum(rng.integers(1, 256, 2 * 65536 + 77, dtype=np.int64)) % 256).astype(np.uint8))
    for k, data in enumerate(cases):
        payload, offs, sizes = lz4_system.compress_blocks(data, 65536, 1 + 7 * (k % 2))
        dst = rng.integers(0, 256, data.size, dtype=np.uint8)
        got, st = gpu_decode(payload, offs, sizes, dst, mode)
        ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
        assert st == rst == 0, k
        assert np.array_equal(ref, data if mode == 0 else dst ^ data), k
        assert np.array_equal(got, ref), k


def test_lz4_decode_in_two_calls_on_two_streams():
    """parse on one stream, apply on another after an event, several payloads in
    a row on one workspace (canonical, general and corrupt blocks, and blocks
    of long literal runs that the parse walks a wave per block): the same
    bytes and status as the one-call decode and the oracle, every time."""
    rng = np.random.default_rng(91)
    cases = []
    m = mask_bytes(5 * 65536 + 4321, 0.08, seed=12)
    enc = oracle.lz4_encode_blocks(m, 65536)
    cases.append((enc["payload"], enc["offsets"], enc["sizes"], m.size))
    payload, offs, sizes, plain = random_payload(rng, 4, 7777)
    cases.append((payload, offs, sizes, plain.size))
    bad = enc["payload"].copy()
    bad[int(enc["offsets"][2])] ^= 0xFF
    cases.append((bad, enc["offsets"], enc["sizes"], m.size))
    cases.append((enc["payload"], enc["offsets"], enc["sizes"], m.size))
    # blocks of long literal runs, walked a wave per block: valid, corrupt, valid
    longb = [raw_block(rng, [(2100, 1, 4)] * 6, 65536), raw_block(rng, [(2100, 1, 4), (20, 0, 4)], 65536),
             raw_block(rng, [(2100, 1, 40000)], 65536)]
    lsz = np.array([x.size for x in longb], np.uint32)
    cases.append((np.concatenate(longb), np.concatenate([[0], np.cumsum(lsz)[:-1]]).astype(np.uint64), lsz,
                  3 * 65536))
    nbmax = max(len(c[1]) for c in cases)
    pbmax = max(c[0].size for c in cases)
    ws = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nbmax, pbmax)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for k, (payload, offs, sizes, nbytes) in enumerate(cases):
        for mode in (0, 1):
            dst = rng.integers(0, 256, nbytes, dtype=np.uint8)
            P, O, S, D = dev(payload), dev(offs.astype(np.uint64)), dev(sizes.astype(np.uint32)), dev(dst)
            st = zeros(1, torch.int32)
            side.wait_stream(main)
            with torch.cuda.stream(side):
                pulse.lz4_decode_parse(P, O, S, nbytes, st, ws, stream=side)
                done = torch.cuda.Event()
                done.record(side)
            main.wait_event(done)
            pulse.lz4_decode_apply(P, O, S, D, st, ws, mode=mode)
            torch.cuda.synchronize()
            ref, rst = oracle.lz4_decode_blocks(payload, offs, sizes, dst, mode=mode)
            one, ost = gpu_decode(payload, offs, sizes, dst, mode)
            assert int(host(st)[0]) == rst == ost, (k, mode)
            assert np.array_equal(host(D), ref) and np.array_equal(one, ref), (k, mode)


def test_lz4_round_trip_restores_new_view():
    """Sender: mask of two BF16 views -> encode; receiver: decode + XOR into the
    old view gives the new view bit for bit; XOR twice is the identity."""
    w0, w1 = workload.c1_masters()
    b0, b1 = oracle.cast_bf16(w0).reshape(-1), oracle.cast_bf16(w1).reshape(-1)
    enc = gpu_encode(b0.view(np.uint8), src_xor=b1.view(np.uint8))
    got, st = gpu_decode(enc["payload"], enc["offsets"], enc["sizes"], b0.view(np.uint8), 1)
    assert st == 0 and np.array_equal(got.view(np.uint16), b1)
    back, st = gpu_decode(enc["payload"], enc["offsets"], enc["sizes"], got, 1)
    assert np.array_equal(back.view(np.uint16), b0)


# ---- FP8 -----------------------------------------------------------------------------
def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gpu_quant(srcs, batch=1):
    cols = srcs[0].shape[-1]
    R = sum(s.shape[-2] for s in srcs)
    codes = zeros(batch * R * cols, torch.uint8)
    scales = zeros(batch * ((R + 127) // 128) * ((cols + 127) // 128), torch.float32)
    pulse.fp8_block_quant([dev(s) for s in srcs], codes, scales, batch=batch)
    torch.cuda.synchronize()
    return (host(codes)[: batch * R * cols].reshape(batch, R, cols),
            host(scales).reshape(batch, (R + 127) // 128, (cols + 127) // 128))


@pytest.mark.parametrize("shape_list", [[(128, 128)], [(256, 384), (128, 384), (384, 384)],
                                        [(200, 136)], [(7, 8)], [(130, 264), (5, 264)]])
def test_fp8_quant_matches_oracle(shape_list):
    rng = np.random.default_rng(len(shape_list) * 7 + shape_list[0][0])
    srcs = [bf16_bits(rng.standard_normal(s) * rng.choice([0.02, 1.0, 100.0])) for s in shape_list]
    codes, scales = gpu_quant(srcs)
    rc, rs = oracle.fp8_block_quant(srcs)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes, rc)


def test_fp8_quant_special_blocks_and_batch():
    rng = np.random.default_rng(4)
    w = bf16_bits(rng.standard_normal((384, 256)) * 0.02)
    w[0:128, 0:128] = bf16_bits(rng.standard_normal((128, 128)) * 1e-38)   # subnormal scale
    w[128:256, 128:256] = 0                                                # amax 0 -> s = 1
    w[256:384, 0:128] = bf16_bits(np.full((128, 128), -2.0 ** -130))      # constant subnormal
    w[256:384, 128:256] = bf16_bits(rng.standard_normal((128, 128)) * 3e4)
    codes, scales = gpu_quant([w])
    rc, rs = oracle.fp8_block_quant([w])
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32)) and np.array_equal(codes, rc)
    g = bf16_bits(rng.standard_normal((3, 256, 128)) * 0.02)
    u = bf16_bits(rng.standard_normal((3, 128, 128)) * 0.05)
    codes, scales = gpu_quant([g, u], batch=3)
    rc, rs = oracle.fp8_block_quant([g, u], batch=3)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32)) and np.array_equal(codes, rc)


def test_fp8_groups_in_one_launch_match_per_group_oracle():
    """Eight stacked groups of different shapes (1 to 4 sources, rows and
    columns that are and are not multiples of 128, a lone block) in one launch:
    every group's codes and scales equal the oracle's quantisation of that
    group alone; then a second call with one group."""
    rng = np.random.default_rng(44)
    shapes = [[(128, 256), (32, 256), (32, 256)],      # [q; k; v]-like
              [(256, 256)],                             # o-like
              [(200, 136), (72, 136)],                  # [gate; up]-like, ragged
              [(128, 1024)],                            # down-like
              [(1, 8)],                                 # one partial block
              [(130, 64), (2, 64), (5, 64), (7, 64)],   # four sources
              [(384, 128)],
              [(64, 520)]]
    groups, refs, outs = [], [], []
    for g, sh in enumerate(shapes):
        srcs = [bf16_bits(rng.standard_normal(s) * rng.choice([0.02, 1.0, 300.0])) for s in sh]
        R, cols = sum(s[0] for s in sh), sh[0][1]
        codes = zeros(R * cols, torch.uint8)
        scales = zeros(((R + 127) // 128) * ((cols + 127) // 128), torch.float32)
        groups.append(([dev(x) for x in srcs], codes, scales))
        refs.append(oracle.fp8_block_quant(srcs))
        outs.append((R, cols))
    pulse.fp8_block_quant_groups(groups)
    torch.cuda.synchronize()
    for (srcs, codes, scales), (rc, rs), (R, cols) in zip(groups, refs, outs):
        nsc = ((R + 127) // 128) * ((cols + 127) // 128)
        assert np.array_equal(host(scales)[:nsc].view(np.uint32), rs.reshape(-1).view(np.uint32))
        assert np.array_equal(host(codes)[:R * cols], rc.reshape(-1))
    srcs, codes, scales = groups[3]
    codes.zero_()
    pulse.fp8_block_quant_groups([groups[3]])
    torch.cuda.synchronize()
    assert np.array_equal(host(codes)[:128 * 1024], refs[3][0].reshape(-1))


def test_fp8_all_bf16_values_through_one_scale():
    """Every finite BF16 value quantised against a range of scales (one 128x128
    block holds 16384 values; 4 blocks cover all 65536 patterns)."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite((pats.astype(np.uint32) << 16).view(np.float32))
    pats = np.where(fin, pats, np.uint16(0))
    w = pats.reshape(512, 128)
    codes, scales = gpu_quant([w])
    rc, rs = oracle.fp8_block_quant([w])
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32)) and np.array_equal(codes, rc)


def test_fp8_every_magnitude_under_many_scales():
    """Every BF16 magnitude up to amax, with random signs, under 70 block maxima
    (edge values and random patterns from the smallest subnormal to the largest
    finite value): per maximum two 128x128 blocks hold magnitudes 0..32767
    clipped to amax, so each block's scale is amax / 448 and every quotient
    x / s in [0, 448] occurs."""
    rng = np.random.default_rng(91)
    edge = [0x0001, 0x0002, 0x007F, 0x0080, 0x0081, 0x00FF, 0x3F80, 0x43E0, 0x43E1,
            0x7F7F, 0x7F00, 0x1000, 0x2000, 0x5E80, 0x5F00, 0x5F7F]
    amaxes = np.array(edge + list(rng.integers(1, 0x7F80, 54)), np.uint32)
    n = amaxes.size
    w = np.zeros((128, 256 * n), np.uint16)
    for j, am in enumerate(amaxes):
        mags = np.minimum(np.arange(32768, dtype=np.uint32), am)
        signs = rng.integers(0, 2, 32768, dtype=np.uint32) << 15
        for b in range(2):
            w[:, 256 * j + 128 * b: 256 * j + 128 * (b + 1)] = \
                (mags[16384 * b: 16384 * (b + 1)] | signs[16384 * b: 16384 * (b + 1)]).reshape(128, 128)
    codes, scales = gpu_quant([w])
    rc, rs = oracle.fp8_block_quant([w])
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    bad = np.argwhere(codes != rc)
    assert bad.size == 0, (bad[:4], amaxes[bad[0][2] // 256] if bad.size else None)


def test_lz4_workspace_reuse_across_sizes():
    """Encode and decode workspaces reused by many calls of different sizes: the
    status words of one call never meet another call's per-block data."""
    big = 9 * 65536 + 4321
    enc_ws = pulse.workspace(pulse.PULSE_OP_LZ4_ENCODE, big, 65536)
    cap = pulse.lz4_payload_bound(big)
    dec_ws = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, (big + 65535) // 65536, cap)
    payload = zeros(cap, torch.uint8)
    nbm = (big + 65535) // 65536
    sizes, offs = zeros(nbm, torch.int32), zeros(nbm, torch.int64)
    tot, st = zeros(1, torch.int64), zeros(1, torch.int32)
    rng = np.random.default_rng(44)
    for it, nbytes in enumerate([big, 70000, 3 * 65536, big, 100, big, 2 * 65536 + 1, big, 65536, big]):
        m = mask_bytes(nbytes, float(rng.choice([0.0, 0.02, 0.08, 0.6])), seed=200 + it)
        pulse.lz4_encode_blocks(dev(m), payload, sizes, offs, tot, st, enc_ws)
        dst = rng.integers(0, 256, nbytes, dtype=np.uint8)
        D = dev(dst)
        pulse.lz4_decode_blocks(payload, offs, sizes, D, st, dec_ws, mode=1, nbytes=nbytes, payload_bytes=cap)
        torch.cuda.synchronize()
        ref = oracle.lz4_encode_blocks(m, 65536)
        t = int(host(tot)[0])
        assert int(host(st)[0]) == 0, it
        assert t == ref["total"] and np.array_equal(host(payload)[:t], ref["payload"]), it
        assert np.array_equal(host(D), dst ^ m), it
