"""The oracle's LZ4 blocks against the system's LZ4 library (liblz4, the
reference implementation of the public block format), both ways:

* every block the oracle's encoder writes is decoded by the library to the
  bytes it encodes (so the canonical offset-1 parse is valid LZ4, length
  bytes, end-of-block rules and all);
* every block the library's compressor writes (matches at any offset, its
  own parse) is decoded by the oracle, in store and XOR mode, to the bytes
  the library compressed.

Inputs: XOR-mask-like bytes from empty to dense, runs of one value, bytes
with no equal neighbours, a packed patch's planes, and ragged lengths.  The
tests are skipped where the library is not installed.
"""
import numpy as np
import pytest

import oracle
from tests import lz4_system

pytestmark = pytest.mark.skipif(not lz4_system.available(), reason="liblz4 is not installed")

B = 65536


def mask_bytes(nbytes, density, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros(nbytes, np.uint8)
    hit = rng.random(nbytes) < density
    m[hit] = rng.integers(1, 256, int(hit.sum()), dtype=np.uint8)
    return m


def inputs():
    rng = np.random.default_rng(2024)
    out = {}
    for d in (0.0, 0.0001, 0.002, 0.01, 0.08, 0.3, 1.0):
        out[f"mask {d}"] = mask_bytes(3 * B + 1234, d, seed=int(d * 1e4) + 1)
    out["runs"] = np.repeat(rng.integers(0, 256, 4000, dtype=np.uint8), rng.integers(1, 90, 4000))[:2 * B + 17]
    out["no equal neighbours"] = (np.cumsum(rng.integers(1, 256, B + 99, dtype=np.int64)) % 256).astype(np.uint8)
    # a packed patch: gaps of a sparse index set and BF16 values, as byte planes
    idx = np.sort(rng.choice(8 * B, B, replace=False)).astype(np.int32)
    val = (rng.standard_normal(B).astype(np.float32) * 0.02).view(np.uint32) >> 16
    packed = np.asarray(oracle.patch_pack(idx, val.astype(np.uint16))).view(np.uint8)
    out["packed patch"] = packed
    for n in (1, 5, 12, 13, 14, 100, B - 1, B + 1):
        out[f"zeros {n}"] = np.zeros(n, np.uint8)
    return out


@pytest.mark.parametrize("name", sorted(inputs()))
def test_library_decodes_oracle_blocks(name):
    data = inputs()[name]
    enc = oracle.lz4_encode_blocks(data, B)
    assert enc["status"] == 0
    raw = data.tobytes()
    for k in range(enc["sizes"].size):
        o, s = int(enc["offsets"][k]), int(enc["sizes"][k])
        plain = raw[k * B:(k + 1) * B]
        got = lz4_system.decompress_block(enc["payload"][o:o + s].tobytes(), len(plain))
        assert got == plain, (name, k)


@pytest.mark.parametrize("accel", [1, 8])
@pytest.mark.parametrize("name", sorted(inputs()))
def test_oracle_decodes_library_blocks(name, accel):
    data = inputs()[name]
    payload, offsets, sizes = lz4_system.compress_blocks(data, B, accel)
    dst = np.random.default_rng(len(data)).integers(0, 256, data.size, dtype=np.uint8)
    for mode in (0, 1):
        out, st = oracle.lz4_decode_blocks(payload, offsets, sizes, dst, mode=mode)
        assert st == 0, (name, mode)
        assert np.array_equal(out, data if mode == 0 else dst ^ data), (name, mode)


def test_library_and_oracle_reject_a_truncated_block():
    data = mask_bytes(B, 0.05, seed=3)
    payload, offsets, sizes = lz4_system.compress_blocks(data, B)
    cut = payload[: int(sizes[0]) - 3]
    assert lz4_system.decompress_block(cut.tobytes(), B) is None
    dst = np.full(B, 0x33, np.uint8)
    out, st = oracle.lz4_decode_blocks(cut, np.array([0], np.uint64), np.array([cut.size], np.uint32), dst, mode=0)
    assert st == oracle.CORRUPT
    assert np.array_equal(out, dst)
