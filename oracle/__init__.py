"""CPU oracle of the trainer->sampler weight-delta codec (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does, and shares no code with it.  The arithmetic lives in
``oracle.c`` (plain C, built by ``oracle/_build.py``); this module only moves
numpy arrays in and out.  Parity status per function: see the header of
``oracle.c``.
"""
import ctypes
import os

import numpy as np

from . import _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

CAPACITY = 1
BADINDEX = 2
CORRUPT = 4

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("SDC_ORACLE_LIB", _build.LIB)  # the sanitizer test loads its own build
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_bf16_rne.argtypes = [ctypes.c_uint32]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_cast_bf16.argtypes = [_P, _P, _I64]
        L.oracle_cast_diff.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I64]
        L.oracle_compact.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _I64]
        L.oracle_apply_patch.argtypes = [_P, _I64, _P, _P, _I64, _P]
        L.oracle_xor_apply.argtypes = [_P, _P, _I64]
        L.oracle_lz4_encode_block.argtypes = [_P, _I64, _P]
        L.oracle_lz4_encode_block.restype = _I64
        L.oracle_lz4_encode_blocks.argtypes = [_P, _P, _I64, _I32, _P, _I64, _P, _P, _P, _P]
        L.oracle_lz4_decode_block.argtypes = [_P, _I64, _P, _I64]
        L.oracle_lz4_decode_block.restype = ctypes.c_int
        L.oracle_lz4_decode_blocks.argtypes = [_P, _I64, _P, _P, _I64, _I32, _I64, _P, _I32, _P]
        L.oracle_e4m3_rne.argtypes = [ctypes.c_float]
        L.oracle_e4m3_rne.restype = ctypes.c_uint8
        L.oracle_fp8_block_quant.argtypes = [_P, _P, _I32, _I64, _I64, _P, _P, _P]
        L.oracle_fp8_delta.argtypes = [_P, _P, _I64, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I64, _P, _P]
        L.oracle_fp8_apply_delta.argtypes = [_P, _I64, _P, _I64, _P, _P, _I64, _P, _P, _I64, _P]
        L.oracle_loco_gate.argtypes = [_P, _P, _P, _I64, _P, _P, _I64, _P, _P]
        L.oracle_loco_accumulate.argtypes = [_P, _I64, _P, _P, _I64, _P]
        L.oracle_patch_packed_bytes.argtypes = [_I64]
        L.oracle_patch_packed_bytes.restype = _I64
        L.oracle_patch_pack.argtypes = [_P, _P, _I64, _P]
        L.oracle_patch_unpack.argtypes = [_P, _I64, _P, _P]
        L.oracle_patch_unpack.restype = ctypes.c_int
        L.oracle_cast_diff_segments.argtypes = [_P, _P, _P, _P, _I32, _P, _P, _I64, _P, _P]
        L.oracle_apply_patch_segments.argtypes = [_P, _P, _I32, _P, _P, _P, _P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def bf16_rne(bits: int) -> int:
    return int(lib().oracle_bf16_rne(ctypes.c_uint32(bits)))


def cast_bf16(w):
    w = _c(w, np.float32)
    out = np.empty(w.shape, np.uint16)
    lib().oracle_cast_bf16(_ptr(w), _ptr(out), w.size)
    return out


def cast_diff(w_new, b_old=None, cap=None, want_new=True, want_mask=True, want_patch=True):
    """Returns dict(b_new, mask, idx, val, count, status) for the requested outputs."""
    w_new = _c(w_new, np.float32).reshape(-1)
    n = w_new.size
    b_old = None if b_old is None else _c(b_old, np.uint16).reshape(-1)
    cap = n if cap is None else int(cap)
    b_new = np.empty(n, np.uint16) if want_new else None
    mask = np.empty(n, np.uint16) if (want_mask and b_old is not None) else None
    idx = np.empty(max(cap, 1), np.int32) if (want_patch and b_old is not None) else None
    val = np.empty(max(cap, 1), np.uint16) if (want_patch and b_old is not None) else None
    count = np.zeros(1, np.int64)
    status = np.zeros(1, np.uint32)
    lib().oracle_cast_diff(_ptr(w_new), _ptr(b_old), _ptr(b_new), _ptr(mask), _ptr(idx), _ptr(val),
                           cap, _ptr(count), _ptr(status), n)
    m = int(count[0])
    if idx is not None:
        idx, val = idx[:min(m, cap)], val[:min(m, cap)]
    return dict(b_new=b_new, mask=mask, idx=idx, val=val,
                count=m if b_old is not None else None, status=int(status[0]))


def compact(b_old, b_new, cap=None):
    b_old = _c(b_old, np.uint16).reshape(-1)
    b_new = _c(b_new, np.uint16).reshape(-1)
    n = b_old.size
    cap = n if cap is None else int(cap)
    idx = np.empty(max(cap, 1), np.int32)
    val = np.empty(max(cap, 1), np.uint16)
    count = np.zeros(1, np.int64)
    status = np.zeros(1, np.uint32)
    lib().oracle_compact(_ptr(b_old), _ptr(b_new), _ptr(idx), _ptr(val), cap, _ptr(count), _ptr(status), n)
    m = int(count[0])
    return idx[:min(m, cap)], val[:min(m, cap)], m, int(status[0])


def apply_patch(b, idx, val, count=None):
    """Applies in place to a copy; returns (new array, status)."""
    b = _c(b, np.uint16).reshape(-1).copy()
    idx = _c(idx, np.int32)
    val = _c(val, np.uint16)
    count = idx.size if count is None else int(count)
    status = np.zeros(1, np.uint32)
    lib().oracle_apply_patch(_ptr(b), b.size, _ptr(idx), _ptr(val), count, _ptr(status))
    return b, int(status[0])


def xor_apply(dst, mask):
    d = np.ascontiguousarray(dst).copy()
    m = np.ascontiguousarray(mask)
    assert d.nbytes == m.nbytes
    lib().oracle_xor_apply(_ptr(d), _ptr(m), d.nbytes)
    return d


def lz4_encode_block(src) -> bytes:
    s = np.frombuffer(bytes(src), np.uint8) if not isinstance(src, np.ndarray) else _c(src, np.uint8)
    n = s.size
    out = np.empty(n + n // 255 + 64, np.uint8)
    sz = lib().oracle_lz4_encode_block(_ptr(s) if n else None, n, _ptr(out))
    return out[:sz].tobytes()


def lz4_encode_blocks(src, block_bytes=65536, src_xor=None, cap=None):
    """src, src_xor: any contiguous arrays (viewed as bytes).
    Returns dict(payload, sizes, offsets, total, status)."""
    s = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    x = None if src_xor is None else np.ascontiguousarray(src_xor).view(np.uint8).reshape(-1)
    nbytes = s.size
    nb = (nbytes + block_bytes - 1) // block_bytes
    worst = nb * (block_bytes + block_bytes // 255 + 16)
    cap = worst if cap is None else int(cap)
    payload = np.empty(max(cap, 1), np.uint8)
    sizes = np.zeros(max(nb, 1), np.uint32)
    offsets = np.zeros(max(nb, 1), np.uint64)
    total = np.zeros(1, np.uint64)
    status = np.zeros(1, np.uint32)
    lib().oracle_lz4_encode_blocks(_ptr(s), _ptr(x), nbytes, block_bytes, _ptr(payload), cap,
                                   _ptr(sizes), _ptr(offsets), _ptr(total), _ptr(status))
    t = int(total[0])
    return dict(payload=payload[:min(t, cap)], sizes=sizes[:nb], offsets=offsets[:nb], total=t,
                status=int(status[0]))


def lz4_decode_block(comp, out_size):
    c = np.frombuffer(bytes(comp), np.uint8)
    out = np.zeros(max(out_size, 1), np.uint8)
    rc = lib().oracle_lz4_decode_block(_ptr(c) if c.size else None, c.size, _ptr(out), out_size)
    return (out[:out_size].tobytes() if rc == 0 else None)


def lz4_decode_blocks(payload, offsets, sizes, dst, block_bytes=65536, mode=0, payload_bytes=None):
    """Decodes into a copy of dst (any dtype, viewed as bytes).  Returns (new dst, status)."""
    p = _c(payload, np.uint8).reshape(-1)
    offs = _c(offsets, np.uint64)
    szs = _c(sizes, np.uint32)
    d = np.ascontiguousarray(dst).copy()
    db = d.view(np.uint8).reshape(-1)
    status = np.zeros(1, np.uint32)
    pb = p.size if payload_bytes is None else int(payload_bytes)
    lib().oracle_lz4_decode_blocks(_ptr(p), pb, _ptr(offs), _ptr(szs), offs.size, block_bytes,
                                   db.size, _ptr(db), mode, _ptr(status))
    return d, int(status[0])


def e4m3_rne(q: float) -> int:
    return int(lib().oracle_e4m3_rne(ctypes.c_float(q)))


def fp8_block_quant(srcs, batch=1):
    """srcs: list of uint16 arrays shaped [batch, rows_i, cols] (or [rows_i, cols] when batch == 1).
    Returns (codes [batch, R, cols] uint8, scales [batch, ceil(R/128), ceil(cols/128)] float32)."""
    arrs = [_c(s, np.uint16) for s in srcs]
    if batch == 1:
        arrs = [a.reshape((1,) + a.shape[-2:]) for a in arrs]
    cols = arrs[0].shape[-1]
    rows = np.array([a.shape[1] for a in arrs], np.int64)
    strides = np.array([a.shape[1] * cols for a in arrs], np.int64)
    R = int(rows.sum())
    codes = np.empty((batch, R, cols), np.uint8)
    scales = np.empty((batch, (R + 127) // 128, (cols + 127) // 128), np.float32)
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    lib().oracle_fp8_block_quant(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(rows), len(arrs), cols,
                                 batch, _ptr(strides), _ptr(codes), _ptr(scales))
    return codes, scales


def fp8_block_quant_strided(base, src_offsets, src_rows, cols, batch, batch_strides):
    """Sources inside one flat uint16 buffer: source i of batch entry e is the
    row-major [src_rows[i], cols] matrix that starts at element
    src_offsets[i] + e * batch_strides[i] of `base` (the experts of an MoE
    layer laid gate, up, down after one another).  Returns (codes, scales) as
    fp8_block_quant does."""
    base = _c(base, np.uint16).reshape(-1)
    rows = np.array(src_rows, np.int64)
    strides = np.array(batch_strides, np.int64)
    for o, r, st in zip(src_offsets, rows, strides):
        assert 0 <= o and o + (batch - 1) * st + r * cols <= base.size
    R = int(rows.sum())
    codes = np.empty((batch, R, cols), np.uint8)
    scales = np.empty((batch, (R + 127) // 128, (cols + 127) // 128), np.float32)
    ptrs = (ctypes.c_void_p * len(rows))(*[base.ctypes.data + 2 * int(o) for o in src_offsets])
    lib().oracle_fp8_block_quant(ctypes.cast(ptrs, ctypes.c_void_p), _ptr(rows), len(rows), cols,
                                 batch, _ptr(strides), _ptr(codes), _ptr(scales))
    return codes, scales


def fp8_delta(codes_old, codes_new, scales_old, scales_new, code_cap=None, scale_cap=None):
    """Returns dict(code_idx, code_val, code_count, scale_idx, scale_val, scale_count, status)."""
    co = _c(codes_old, np.uint8).reshape(-1)
    cn = _c(codes_new, np.uint8).reshape(-1)
    so = _c(scales_old, np.float32).reshape(-1)
    sn = _c(scales_new, np.float32).reshape(-1)
    assert co.size == cn.size and so.size == sn.size
    code_cap = co.size if code_cap is None else int(code_cap)
    scale_cap = so.size if scale_cap is None else int(scale_cap)
    ci, cv = np.empty(max(code_cap, 1), np.int32), np.empty(max(code_cap, 1), np.uint8)
    si, sv = np.empty(max(scale_cap, 1), np.int32), np.empty(max(scale_cap, 1), np.float32)
    cc, sc = np.zeros(1, np.int64), np.zeros(1, np.int64)
    status = np.zeros(1, np.uint32)
    lib().oracle_fp8_delta(_ptr(co), _ptr(cn), co.size, _ptr(so), _ptr(sn), so.size, _ptr(ci), _ptr(cv),
                           code_cap, _ptr(cc), _ptr(si), _ptr(sv), scale_cap, _ptr(sc), _ptr(status))
    m, k = int(cc[0]), int(sc[0])
    return dict(code_idx=ci[:min(m, code_cap)], code_val=cv[:min(m, code_cap)], code_count=m,
                scale_idx=si[:min(k, scale_cap)], scale_val=sv[:min(k, scale_cap)], scale_count=k,
                status=int(status[0]))


def fp8_apply_delta(codes, scales, code_idx, code_val, scale_idx, scale_val):
    """Applies to copies; returns (codes, scales, status)."""
    c = _c(codes, np.uint8).reshape(-1).copy()
    s = _c(scales, np.float32).reshape(-1).copy()
    ci, cv = _c(code_idx, np.int32), _c(code_val, np.uint8)
    si, sv = _c(scale_idx, np.int32), _c(scale_val, np.float32)
    status = np.zeros(1, np.uint32)
    lib().oracle_fp8_apply_delta(_ptr(c), c.size, _ptr(s), s.size, _ptr(ci), _ptr(cv), ci.size,
                                 _ptr(si), _ptr(sv), si.size, _ptr(status))
    return c, s, int(status[0])


def loco_gate(theta, delta, resid, cap=None):
    """Returns dict(idx, val, count, resid (new array), status)."""
    th = _c(theta, np.float32).reshape(-1)
    de = _c(delta, np.float32).reshape(-1)
    r = _c(resid, np.float32).reshape(-1).copy()
    n = th.size
    assert de.size == n and r.size == n
    cap = n if cap is None else int(cap)
    idx, val = np.empty(max(cap, 1), np.int32), np.empty(max(cap, 1), np.float32)
    count, status = np.zeros(1, np.int64), np.zeros(1, np.uint32)
    lib().oracle_loco_gate(_ptr(th), _ptr(de), _ptr(r), n, _ptr(idx), _ptr(val), cap, _ptr(count), _ptr(status))
    m = int(count[0])
    return dict(idx=idx[:min(m, cap)], val=val[:min(m, cap)], count=m, resid=r, status=int(status[0]))


def loco_accumulate(acc, idx, val):
    """acc[idx[k]] += val[k] on a copy; returns (acc, status)."""
    a = _c(acc, np.float32).reshape(-1).copy()
    i, v = _c(idx, np.int32), _c(val, np.float32)
    status = np.zeros(1, np.uint32)
    lib().oracle_loco_accumulate(_ptr(a), a.size, _ptr(i), _ptr(v), i.size, _ptr(status))
    return a, int(status[0])


PACK_GROUP = 65536


def patch_pack(idx, val):
    """Gap + byte-plane form of an ascending patch (uint8 array, whole groups)."""
    i, v = _c(idx, np.int32), _c(val, np.uint16)
    assert i.size == v.size
    out = np.empty(max(int(lib().oracle_patch_packed_bytes(i.size)), 1), np.uint8)
    lib().oracle_patch_pack(_ptr(i), _ptr(v), i.size, _ptr(out))
    return out[: int(lib().oracle_patch_packed_bytes(i.size))]


def patch_unpack(packed, count):
    """Returns (idx, val), or None when the packed data overflows int32 indices."""
    p = _c(packed, np.uint8)
    idx, val = np.empty(max(count, 1), np.int32), np.empty(max(count, 1), np.uint16)
    rc = lib().oracle_patch_unpack(_ptr(p), count, _ptr(idx), _ptr(val))
    return None if rc else (idx[:count], val[:count])


def patch_compress(idx, val, block_bytes=65536):
    """The whole sender side: pack, then the canonical LZ4 block encoding."""
    packed = patch_pack(idx, val)
    return packed, lz4_encode_blocks(packed, block_bytes)


def _ptrs(arrs):
    return (ctypes.c_void_p * max(len(arrs), 1))(*[a.ctypes.data for a in arrs])


def cast_diff_segments(ws_new, bs_old, cap=None):
    """Lists of float32 masters and BF16 old views, one per tensor.  Returns
    dict(b_new (list), idx, val, seg_offsets, count, status)."""
    ws_new = [_c(w, np.float32).reshape(-1) for w in ws_new]
    bs_old = [_c(b, np.uint16).reshape(-1) for b in bs_old]
    ns = np.array([w.size for w in ws_new], np.int64)
    total = int(ns.sum())
    cap = total if cap is None else int(cap)
    b_new = [np.empty(w.size, np.uint16) for w in ws_new]
    idx, val = np.empty(max(cap, 1), np.int32), np.empty(max(cap, 1), np.uint16)
    offs = np.zeros(len(ws_new) + 1, np.int64)
    status = np.zeros(1, np.uint32)
    pw, po, pn = _ptrs(ws_new), _ptrs(bs_old), _ptrs(b_new)
    lib().oracle_cast_diff_segments(ctypes.cast(pw, ctypes.c_void_p), ctypes.cast(po, ctypes.c_void_p),
                                    ctypes.cast(pn, ctypes.c_void_p), _ptr(ns), len(ws_new), _ptr(idx),
                                    _ptr(val), cap, _ptr(offs), _ptr(status))
    m = int(offs[-1])
    return dict(b_new=b_new, idx=idx[:min(m, cap)], val=val[:min(m, cap)], seg_offsets=offs, count=m,
                status=int(status[0]))


def apply_patch_segments(views, idx, val, seg_offsets):
    """Applies to copies of the views; returns (views, status)."""
    vs = [_c(v, np.uint16).reshape(-1).copy() for v in views]
    ns = np.array([v.size for v in vs], np.int64)
    i, v = _c(idx, np.int32), _c(val, np.uint16)
    offs = _c(seg_offsets, np.int64)
    status = np.zeros(1, np.uint32)
    pv = _ptrs(vs)
    lib().oracle_apply_patch_segments(ctypes.cast(pv, ctypes.c_void_p), _ptr(ns), len(vs), _ptr(i), _ptr(v),
                                      _ptr(offs), _ptr(status))
    return vs, int(status[0])

