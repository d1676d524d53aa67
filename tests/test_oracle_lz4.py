"""Pins of the oracle's LZ4 block encode / decode (rows a5, a6).

The canonical parse and the decoder's validation rules are readings (the pages
only name LZ4 and its reason: long zero runs in RL masks [Teleport, "Moving the
pipeline onto GPUs"]); the byte format is the public LZ4 block format.  Pins:
closed-form blocks, an independent spec decoder (tests/lz4_spec.py), brute force
on tiny inputs, random spec-valid streams with known output, corrupt streams.
"""
import itertools

import numpy as np
import pytest

import oracle
from tests import lz4_spec


# ---- closed forms -----------------------------------------------------------------
def test_all_zero_block_is_267_bytes():
    enc = oracle.lz4_encode_block(bytes(65536))
    # token 0x1F, literal 0x00, offset 01 00, 257 length bytes (65511 = 256*255 + 231),
    # then the final token 0x50 and five zero literals
    expect = bytes([0x1F, 0x00, 0x01, 0x00]) + bytes([255] * 256) + bytes([231]) + bytes([0x50]) + bytes(5)
    assert enc == expect and len(enc) == 267


def test_runless_block_is_65794_bytes():
    data = bytes(i & 0xFF for i in range(65536))   # no two equal neighbours
    enc = oracle.lz4_encode_block(data)
    expect = bytes([0xF0]) + bytes([255] * 256) + bytes([241]) + data  # 65521 = 256*255 + 241
    assert enc == expect and len(enc) == 65794


@pytest.mark.parametrize("n", range(0, 13))
def test_short_blocks_are_all_literal(n):
    data = bytes(n)  # even a zero run cannot be matched below 13 bytes
    assert oracle.lz4_encode_block(data) == bytes([n << 4]) + data


def test_thirteen_zero_bytes_use_one_match():
    # i = 1, j = min(13, 8) = 8, L = 7 >= 4, i <= 1: one sequence, then 5 literals
    assert oracle.lz4_encode_block(bytes(13)) == bytes([0x13, 0x00, 0x01, 0x00, 0x50]) + bytes(5)


# ---- brute force and round trips -------------------------------------------------
def test_bruteforce_binary_strings_up_to_16():
    """Every byte string of length <= 16 over {0x00, 0x01}: the oracle equals the
    canonical parse written out with itertools, and the spec decoder inverts it."""
    for n in range(0, 17):
        for t in itertools.product(b"\x00\x01", repeat=n):
            data = bytes(t)
            enc = oracle.lz4_encode_block(data)
            assert enc == lz4_spec.canonical_encode_bruteforce(data), data
            assert lz4_spec.decode(enc, n) == data


def test_canonical_structure_on_masks():
    """Every match is offset 1 and >= 4 long, the last 5 bytes are literals, the
    last match starts >= 12 bytes before the end, and decoding gives the input."""
    rng = np.random.default_rng(9)
    for n in (13, 100, 4096, 65536):
        for d in (0.0, 0.01, 0.08, 0.5, 1.0):
            m = np.zeros(n, np.uint8)
            hit = rng.random(n) < d
            m[hit] = rng.integers(1, 256, int(hit.sum()), dtype=np.uint8)
            data = m.tobytes()
            enc = oracle.lz4_encode_block(data)
            assert lz4_spec.decode(enc, n) == data
            pos = 0
            seqs = lz4_spec.sequences(enc)
            for ll, off, ml in seqs[:-1]:
                pos += ll
                assert off == 1 and ml >= 4 and pos <= n - 12
                pos += ml
            assert seqs[-1][0] >= 5 or n < 13
            if n <= 600:
                assert enc == lz4_spec.canonical_encode_bruteforce(data)


def test_multi_block_layout_and_round_trip():
    rng = np.random.default_rng(4)
    nbytes = 3 * 65536 + 1234
    m = np.zeros(nbytes, np.uint8)
    hit = rng.random(nbytes) < 0.04
    m[hit] = rng.integers(1, 256, int(hit.sum()), dtype=np.uint8)
    r = oracle.lz4_encode_blocks(m, 65536)
    assert r["status"] == 0 and r["sizes"].size == 4
    assert r["offsets"][0] == 0 and np.all(r["offsets"][1:] == np.cumsum(r["sizes"])[:-1])
    assert r["total"] == int(r["sizes"].sum()) == r["payload"].size
    for b in range(4):
        blk = m[b * 65536:(b + 1) * 65536].tobytes()
        o, s = int(r["offsets"][b]), int(r["sizes"][b])
        assert r["payload"][o:o + s].tobytes() == oracle.lz4_encode_block(blk)
        assert lz4_spec.decode(r["payload"][o:o + s].tobytes(), len(blk)) == blk
    # XOR of two sources == encoding of their XOR
    a = rng.integers(0, 256, nbytes, dtype=np.uint8)
    r2 = oracle.lz4_encode_blocks(a, 65536, src_xor=a ^ m)
    assert r2["total"] == r["total"] and np.array_equal(r2["payload"], r["payload"])
    d, st = oracle.lz4_decode_blocks(r["payload"], r["offsets"], r["sizes"], np.zeros(nbytes, np.uint8))
    assert st == 0 and np.array_equal(d, m)
    x, st = oracle.lz4_decode_blocks(r["payload"], r["offsets"], r["sizes"], a, mode=1)
    assert st == 0 and np.array_equal(x, a ^ m)


def test_encode_capacity():
    m = np.zeros(4 * 65536, np.uint8)
    m[::7] = 3
    full = oracle.lz4_encode_blocks(m, 65536)
    cap = int(full["offsets"][2]) + 10          # blocks 0, 1 fit; 2, 3 do not
    r = oracle.lz4_encode_blocks(m, 65536, cap=cap)
    assert r["status"] == oracle.CAPACITY and r["total"] == full["total"]
    assert np.array_equal(r["payload"][: int(full["offsets"][2])], full["payload"][: int(full["offsets"][2])])


# ---- decoder on streams it did not produce ----------------------------------------
def test_random_spec_valid_streams():
    rng = np.random.default_rng(12)
    for trial in range(300):
        out_size = int(rng.choice([1, 5, 17, 300, 4096, 65536, int(rng.integers(1, 65537))]))
        comp, plain = lz4_spec.random_block(rng, out_size)
        assert lz4_spec.decode(comp, out_size) == plain
        assert oracle.lz4_decode_block(comp, out_size) == plain, trial


def test_corrupt_streams_are_rejected_and_leave_dst():
    rng = np.random.default_rng(13)
    comp, plain = lz4_spec.random_block(rng, 5000)
    bad = [
        comp[:-1],                                   # truncated
        comp + b"\x00",                              # trailing garbage
        bytes([0x0F]) + comp,                        # match before any output
        bytes([0x10, 0x41, 0x00, 0x00]) + comp[1:],  # offset 0
        bytes([0x10, 0x41, 0x05, 0x00]),             # offset beyond produced bytes
        b"",                                         # no token
    ]
    for c in bad:
        assert oracle.lz4_decode_block(c, 5000) is None
    assert oracle.lz4_decode_block(comp, 4999) is None   # overflow
    assert oracle.lz4_decode_block(comp, 5001) is None   # short
    # multi-block: a corrupt middle block leaves its dst range untouched
    data = np.zeros(3 * 65536, np.uint8)
    data[::11] = 9
    r = oracle.lz4_encode_blocks(data, 65536)
    payload = r["payload"].copy()
    payload[int(r["offsets"][1])] ^= 0xFF                # break block 1's first token
    dst = np.full(data.size, 0x5A, np.uint8)
    got, st = oracle.lz4_decode_blocks(payload, r["offsets"], r["sizes"], dst)
    assert st == oracle.CORRUPT
    assert np.array_equal(got[:65536], data[:65536])
    assert np.all(got[65536:131072] == 0x5A)
    assert np.array_equal(got[131072:], data[131072:])
    # a block starting before the end of an earlier one
    offs = r["offsets"].copy()
    offs[2] = offs[1] + 1
    got, st = oracle.lz4_decode_blocks(r["payload"], offs, r["sizes"], dst)
    assert st == oracle.CORRUPT and np.array_equal(got[:131072], data[:131072]) and np.all(got[131072:] == 0x5A)
    # block lying outside the payload
    sizes = r["sizes"].copy()
    sizes[2] += 1000
    got, st = oracle.lz4_decode_blocks(r["payload"], r["offsets"], sizes, dst)
    assert st == oracle.CORRUPT and np.all(got[131072:] == 0x5A)
