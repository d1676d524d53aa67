"""Test-side LZ4 helpers written from the public "LZ4 Block Format Description".

Independent of the oracle and of the HIP library: a plain sequential decoder,
a generator of random spec-valid blocks with their known decoded bytes, and a
brute-force implementation of the canonical "offset-1 run" parse used to pin
the encoders on tiny inputs.
"""
import itertools

import numpy as np


class Malformed(Exception):
    pass


def decode(comp: bytes, out_size: int) -> bytes:
    """Decode one block; raise Malformed unless it ends right after a literal run
    with exactly out_size bytes produced."""
    src = memoryview(bytes(comp))
    out = bytearray()
    p = 0
    while True:
        if p >= len(src):
            raise Malformed("missing token")
        token = src[p]
        p += 1
        lit = token >> 4
        if lit == 15:
            while True:
                if p >= len(src):
                    raise Malformed("literal length runs off the end")
                b = src[p]
                p += 1
                lit += b
                if b != 255:
                    break
        if p + lit > len(src) or len(out) + lit > out_size:
            raise Malformed("literals overflow")
        out += src[p:p + lit]
        p += lit
        if p == len(src):
            if len(out) != out_size:
                raise Malformed("short output")
            return bytes(out)
        if p + 2 > len(src):
            raise Malformed("truncated offset")
        off = src[p] | (src[p + 1] << 8)
        p += 2
        if off == 0 or off > len(out):
            raise Malformed("bad offset")
        ml = (token & 15) + 4
        if (token & 15) == 15:
            while True:
                if p >= len(src):
                    raise Malformed("match length runs off the end")
                b = src[p]
                p += 1
                ml += b
                if b != 255:
                    break
        if len(out) + ml > out_size:
            raise Malformed("match overflow")
        start = len(out) - off
        for k in range(ml):
            out.append(out[start + k])


def sequences(comp: bytes):
    """List of (literal_length, offset, match_length) of a well-formed block;
    the last entry has offset None."""
    src = bytes(comp)
    p, res = 0, []
    while True:
        token = src[p]
        p += 1
        lit = token >> 4
        if lit == 15:
            while True:
                b = src[p]
                p += 1
                lit += b
                if b != 255:
                    break
        p += lit
        if p == len(src):
            res.append((lit, None, 0))
            return res
        off = src[p] | (src[p + 1] << 8)
        p += 2
        ml = (token & 15) + 4
        if (token & 15) == 15:
            while True:
                b = src[p]
                p += 1
                ml += b
                if b != 255:
                    break
        res.append((lit, off, ml))


def _length_bytes(v):
    out = bytearray()
    v -= 15
    while v >= 255:
        out.append(255)
        v -= 255
    out.append(v)
    return bytes(out)


def emit(seqs, literal_bytes):
    """Serialise [(literals: bytes, offset|None, match_len)] into a block."""
    out = bytearray()
    for lits, off, ml in seqs:
        ll = len(lits)
        tok = (min(ll, 15) << 4) | (0 if off is None else min(ml - 4, 15))
        out.append(tok)
        if ll >= 15:
            out += _length_bytes(ll)
        out += lits
        if off is not None:
            out += bytes([off & 255, off >> 8])
            if ml - 4 >= 15:
                out += _length_bytes(ml - 4)
    return bytes(out)


def random_block(rng, out_size, max_lit=600, max_match=600, max_off=65535):
    """A random spec-valid block that decodes to out_size bytes.  Returns
    (compressed, decoded).  Literal and match lengths cross the 15 / 270 / 525
    continuation thresholds; offsets range over 1..min(position, max_off) so
    overlapping copies occur."""
    out = bytearray()
    seqs = []
    while True:
        remaining = out_size - len(out)
        ll = int(rng.integers(0, min(max_lit, remaining) + 1))
        if len(out) == 0 and ll == 0:
            ll = min(1, remaining)
        lits = bytes(rng.integers(0, 256, ll, dtype=np.uint8)) if rng.random() < 0.7 else bytes(ll)
        out += lits
        remaining = out_size - len(out)
        if remaining < 4 or len(out) == 0 or rng.random() < 0.02:
            # finish: remaining bytes as final literals
            tail = bytes(rng.integers(0, 256, remaining, dtype=np.uint8))
            seqs.append((lits + tail, None, 0))
            out += tail
            return emit(seqs, None), bytes(out)
        ml = int(rng.integers(4, min(max_match, remaining) + 1))
        off = int(rng.integers(1, min(len(out), max_off) + 1))
        if rng.random() < 0.3:
            off = int(rng.integers(1, min(len(out), 8) + 1))  # short, overlapping
        start = len(out) - off
        for k in range(ml):
            out.append(out[start + k])
        seqs.append((lits, off, ml))


def canonical_encode_bruteforce(data: bytes) -> bytes:
    """The canonical parse, written out directly from its definition with
    itertools.groupby (only meant for small inputs)."""
    n = len(data)
    seqs = []
    a = 0
    pos = 0
    for _, grp in itertools.groupby(data):
        length = len(list(grp))
        s, e = pos, pos + length
        pos = e
        i, j = s + 1, min(e, n - 5)
        if j - i >= 4 and i <= n - 12:
            seqs.append((data[a:i], 1, j - i))
            a = j
    seqs.append((data[a:], None, 0))
    return emit(seqs, None)
