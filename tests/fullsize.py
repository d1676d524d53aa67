"""Host side of the full-size parity tests: every output the GPU writes is
compared, element by element, with the oracle run on host copies of the same
inputs.

The oracle is called once per independent piece of the work -- a range of
whole LZ4 blocks of the mask, one 128-row band of FP8 blocks, one tensor --
and each call is single-threaded; the pieces are spread over a pool of host
threads (ctypes releases the GIL for the duration of a call).  Splitting at
piece boundaries changes nothing in what is computed: every element's
result depends only on its own inputs (cast, diff, apply), on its own LZ4
block (encode) or on its own 128x128 block (FP8), and patch indices local to
a piece are shifted by the piece's start.

GPU buffers reach the host through pinned staging buffers kept per slot and
reused.  No codec arithmetic is done here: expected values come from the
oracle only, and this module only moves data and compares it.
"""
import concurrent.futures
import os

import numpy as np
import torch

import oracle

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
PIECE = 1 << 24  # elements per oracle call: 512 mask blocks of 64 KiB (32768 BF16 each)
BLOCK = 65536

_pool = concurrent.futures.ThreadPoolExecutor(THREADS)
_pinned = {}


def pmap(fn, items):
    """fn over items on the host threads, results in order (exceptions re-raised)."""
    return list(_pool.map(fn, items))


def to_host(t, slot, dtype=None):
    """numpy view of a copy of the GPU tensor `t`, made in the pinned buffer of
    `slot` (grown when too small); valid until the slot is used again."""
    nbytes = t.numel() * t.element_size()
    buf = _pinned.get(slot)
    if buf is None or buf.numel() < nbytes:
        _pinned.pop(slot, None)
        buf = torch.empty(max(nbytes, 16), dtype=torch.uint8, pin_memory=True)
        _pinned[slot] = buf
    if nbytes:
        buf[:nbytes].copy_(t.reshape(-1).view(torch.uint8))
    a = buf[:nbytes].numpy()
    if dtype is None:
        dtype = {torch.int16: np.uint16, torch.bfloat16: np.uint16, torch.int32: np.int32,
                 torch.int64: np.int64, torch.float32: np.float32, torch.uint8: np.uint8}[t.dtype]
    return a.view(dtype)


def release():
    """Free the pinned staging buffers."""
    _pinned.clear()
    torch._C._host_emptyCache()


def pieces(m, piece=None):
    piece = PIECE if piece is None else piece
    return [(a, min(m, a + piece)) for a in range(0, m, piece)]


def same(a, b):
    return a.shape == b.shape and np.array_equal(a, b)


# ---------------------------------------------------------------------------
def oracle_cast(w_h, out=None):
    """The oracle's BF16 view of float32 masters, piece by piece on the pool
    (into `out` when given)."""
    out = np.empty(w_h.size, np.uint16) if out is None else out

    def one(r):
        a, b = r
        out[a:b] = oracle.cast_bf16(w_h[a:b])
    pmap(one, pieces(w_h.size))
    return out


def check_equal(got_h, ref_h, what):
    """Element-wise equality of two host arrays, compared piece by piece on the pool."""
    assert got_h.size == ref_h.size, (what, got_h.size, ref_h.size)

    def one(r):
        a, b = r
        return None if np.array_equal(got_h[a:b], ref_h[a:b]) else a
    bad = [a for a in pmap(one, pieces(got_h.size, 1 << 26)) if a is not None]
    if bad:
        a = bad[0]
        d = np.flatnonzero(got_h[a:a + (1 << 26)] != ref_h[a:a + (1 << 26)])
        raise AssertionError(f"{what}: {len(bad)} pieces differ, first at element {a + int(d[0])}")


class OraclePatch:
    """The oracle's cast + diff + compaction of one call's input, by pieces:
    b_new, and per piece the ascending local indices and values."""

    def __init__(self, w_h, bo_h):
        self.n = w_h.size
        self.ranges = pieces(self.n)
        self.b_new = np.empty(self.n, np.uint16)

        def one(r):
            a, b = r
            res = oracle.cast_diff(w_h[a:b], bo_h[a:b], want_mask=False)
            assert res["status"] == 0
            self.b_new[a:b] = res["b_new"]
            return res["idx"].copy(), res["val"].copy()
        out = pmap(one, self.ranges)
        self.idx = [o[0] for o in out]
        self.val = [o[1] for o in out]
        self.counts = np.array([i.size for i in self.idx], np.int64)
        self.starts = np.concatenate([[0], np.cumsum(self.counts)])
        self.count = int(self.starts[-1])

    def check(self, count, idx_h, val_h, what):
        """The GPU's count and entries [0, count) against the oracle's."""
        assert count == self.count, (what, count, self.count)

        def one(p):
            a = self.ranges[p][0]
            c0, c1 = int(self.starts[p]), int(self.starts[p + 1])
            ok = same(idx_h[c0:c1], self.idx[p] + np.int32(a)) and same(val_h[c0:c1], self.val[p])
            return None if ok else p
        bad = [p for p in pmap(one, range(len(self.ranges))) if p is not None]
        assert not bad, f"{what}: patch entries differ in pieces {bad[:5]} (of {len(self.ranges)})"

    def applied(self, bo_h, out=None):
        """The oracle's apply of this patch to the old view (piece by piece)."""
        out = np.empty(self.n, np.uint16) if out is None else out

        def one(p):
            a, b = self.ranges[p]
            res, st = oracle.apply_patch(bo_h[a:b], self.idx[p], self.val[p])
            assert st == 0
            out[a:b] = res
        pmap(one, range(len(self.ranges)))
        return out


def check_lz4(old_h, new_h, sizes_h, offs_h, total, payload_h, what, block_bytes=BLOCK):
    """Every block of the GPU's LZ4 encoding of old ^ new against the oracle's
    canonical encoding: sizes, the offsets as the exclusive scan of the
    oracle's sizes, the total, and every payload byte.  old_h, new_h: uint16
    views whose byte ranges the blocks cut."""
    nbytes = 2 * old_h.size
    nb = (nbytes + block_bytes - 1) // block_bytes
    assert sizes_h.size >= nb and offs_h.size >= nb
    per = PIECE * 2 // block_bytes  # blocks per piece

    def one(k):
        b0 = k * per
        b1 = min(nb, b0 + per)
        lo, hi = b0 * block_bytes // 2, min(old_h.size, b1 * block_bytes // 2)
        enc = oracle.lz4_encode_blocks(old_h[lo:hi], block_bytes, src_xor=new_h[lo:hi])
        assert enc["status"] == 0
        ok_sizes = same(sizes_h[b0:b1].astype(np.uint32), enc["sizes"])
        start = int(offs_h[b0])
        ok_bytes = same(payload_h[start:start + enc["total"]], enc["payload"])
        return enc["sizes"], ok_sizes, ok_bytes
    out = pmap(one, range((nb + per - 1) // per))
    bad = [k for k, o in enumerate(out) if not (o[1] and o[2])]
    assert not bad, f"{what}: LZ4 blocks differ in pieces {bad[:5]}"
    ref_sizes = np.concatenate([o[0] for o in out]).astype(np.uint64)
    ref_offs = np.concatenate([[0], np.cumsum(ref_sizes[:-1])]).astype(np.uint64)
    assert same(offs_h[:nb].astype(np.uint64), ref_offs), f"{what}: block offsets"
    assert total == int(ref_sizes.sum()), (what, total, int(ref_sizes.sum()))
    return total


def check_fp8(view_h, sources, cols, codes_h, scales_h, what, bands_per_task=4, more=()):
    """The GPU's codes [R, cols] and scales [ceil(R/128), ceil(cols/128)] of the
    stack of `sources` (element offsets into view_h and row counts, stacked
    along rows) against the oracle's quantisation of every 128-row band of the
    stack.  `more`: further (codes, scales) pairs of the same stack, compared
    with the same oracle result."""
    R = sum(r for _, r in sources)
    nbr, nbc = (R + 127) // 128, (cols + 127) // 128
    outs = []
    for c, sc in [(codes_h, scales_h)] + list(more):
        assert c.size == R * cols and sc.size == nbr * nbc, what
        outs.append((c.reshape(R, cols), sc.reshape(nbr, nbc)))
    row_src = []
    r = 0
    for off, rows in sources:
        row_src.append((r, r + rows, off))
        r += rows

    def band(r0, r1):
        parts = []
        for s0, s1, off in row_src:
            a, b = max(r0, s0), min(r1, s1)
            if a < b:
                parts.append(view_h[off + (a - s0) * cols: off + (b - s0) * cols].reshape(b - a, cols))
        return parts[0] if len(parts) == 1 else np.concatenate(parts, 0)

    def one(k):
        bad = []
        for br in range(k * bands_per_task, min(nbr, (k + 1) * bands_per_task)):
            r0, r1 = br * 128, min(R, br * 128 + 128)
            rc, rs = oracle.fp8_block_quant([band(r0, r1)])
            for c, sc in outs:
                if not (same(c[r0:r1], rc[0]) and same(sc[br].view(np.uint32), rs[0, 0].view(np.uint32))):
                    bad.append(br)
                    break
        return bad
    bad = [b for lst in pmap(one, range((nbr + bands_per_task - 1) // bands_per_task)) for b in lst]
    assert not bad, f"{what}: FP8 bands differ: {bad[:5]} (of {nbr})"


def oracle_fp8(view_h, sources, cols, codes_out, scales_out, bands_per_task=4):
    """The oracle's codes [R, cols] and scales of the stack of `sources`
    (element offsets into view_h, row counts), written into the host arrays
    codes_out (R * cols) and scales_out, one 128-row band per oracle call."""
    R = sum(r for _, r in sources)
    nbr, nbc = (R + 127) // 128, (cols + 127) // 128
    codes_out = codes_out.reshape(R, cols)
    scales_out = scales_out.reshape(nbr, nbc)
    row_src, r = [], 0
    for off, rows in sources:
        row_src.append((r, r + rows, off))
        r += rows

    def one(k):
        for br in range(k * bands_per_task, min(nbr, (k + 1) * bands_per_task)):
            r0, r1 = br * 128, min(R, br * 128 + 128)
            parts = []
            for s0, s1, off in row_src:
                a, b = max(r0, s0), min(r1, s1)
                if a < b:
                    parts.append(view_h[off + (a - s0) * cols: off + (b - s0) * cols].reshape(b - a, cols))
            band = parts[0] if len(parts) == 1 else np.concatenate(parts, 0)
            rc, rs = oracle.fp8_block_quant([band])
            codes_out[r0:r1] = rc[0]
            scales_out[br] = rs[0, 0]
    pmap(one, range((nbr + bands_per_task - 1) // bands_per_task))


class OracleDelta:
    """The oracle's FP8-view delta of two quantised views (codes compared as
    bytes, scales as 32-bit patterns), by pieces of the codes."""

    def __init__(self, co, cn, so, sn):
        self.ranges = pieces(co.size)
        e = np.zeros(0, np.float32)

        def one(r):
            a, b = r
            d = oracle.fp8_delta(co[a:b], cn[a:b], e, e)
            assert d["status"] == 0
            return d["code_idx"].copy(), d["code_val"].copy()
        out = pmap(one, self.ranges)
        self.idx = [o[0] for o in out]
        self.val = [o[1] for o in out]
        self.starts = np.concatenate([[0], np.cumsum([i.size for i in self.idx])]).astype(np.int64)
        self.count = int(self.starts[-1])
        z = np.zeros(0, np.uint8)
        d = oracle.fp8_delta(z, z, so, sn)
        assert d["status"] == 0
        self.scale_idx, self.scale_val, self.scale_count = d["scale_idx"], d["scale_val"], d["scale_count"]

    def check(self, count, idx_h, val_h, scount, sidx_h, sval_h, what):
        assert count == self.count, (what, count, self.count)
        assert scount == self.scale_count, (what, scount, self.scale_count)

        def one(p):
            a = self.ranges[p][0]
            c0, c1 = int(self.starts[p]), int(self.starts[p + 1])
            ok = same(idx_h[c0:c1], self.idx[p] + np.int32(a)) and same(val_h[c0:c1], self.val[p])
            return None if ok else p
        bad = [p for p in pmap(one, range(len(self.ranges))) if p is not None]
        assert not bad, f"{what}: code entries differ in pieces {bad[:5]}"
        assert same(sidx_h, self.scale_idx) and same(sval_h.view(np.uint32), self.scale_val.view(np.uint32)), \
            f"{what}: scale entries"
