"""Python binding of libpulse.so, the MI355X weight-delta codec (include/pulse.h).

Argument marshalling only: every function takes torch tensors that already live
on the GPU, passes their data pointers, sizes and torch's current HIP stream to
the C entry point of the same name, and raises if that entry point returns an
error.  Every step of the codec runs in the library's HIP kernels.  There is no
fallback: if the library is not built, importing this package fails.
"""
import ctypes
import os

import torch

__all__ = [
    "PULSE_DS_CAPACITY", "PULSE_DS_BADINDEX", "PULSE_DS_CORRUPT", "PULSE_DS_WORKSPACE",
    "PULSE_OP_CAST_DIFF", "PULSE_OP_COMPACT", "PULSE_OP_LZ4_ENCODE", "PULSE_OP_LZ4_DECODE",
    "pulse_version", "pulse_workspace_bytes", "pulse_workspace_init", "workspace",
    "pulse_cast_diff", "pulse_compact", "pulse_apply_patch", "xor_mask_apply",
    "lz4_encode_blocks", "lz4_decode_blocks", "fp8_block_quant", "lz4_payload_bound", "lib_path",
    "PULSE_OP_FP8_DELTA", "PULSE_OP_LOCO_GATE", "fp8_view_delta", "fp8_view_apply",
    "pulse_loco_gate", "pulse_loco_accumulate",
    "PULSE_OP_PATCH_UNPACK", "patch_packed_bytes", "patch_pack", "patch_unpack",
    "PULSE_OP_CAST_DIFF_SEGMENTS", "PULSE_DS_BADSEGMENT", "PULSE_OP_CAST_DIFF_LZ4", "pulse_cast_diff_lz4", "fp8_block_quant_groups", "PULSE_QUANT_MAX_GROUPS", "pulse_patch_tiles", "PULSE_OP_APPLY_QUANT", "ApplyQuantPlan", "pulse_apply_quant_plan", "pulse_apply_quant",
    "pulse_apply_patch_tiled", "patch_tile_count", "pulse_segment_tiles", "SegmentTable", "ViewTable",
    "pulse_cast_diff_segments", "pulse_apply_patch_segments", "lz4_decode_parse", "lz4_decode_apply",
    "pulse_cast_diff_lz4_noalloc", "PULSE_NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("SDC_PULSE_LIB") or os.path.join(_HERE, "libpulse.so")  # (a sanitizer build in tests)
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python sparse_delta_codec_amd/_build.py) first")
_lib = ctypes.CDLL(_LIB_PATH)

PULSE_DS_CAPACITY = 0x1
PULSE_DS_BADINDEX = 0x2
PULSE_DS_CORRUPT = 0x4
PULSE_DS_WORKSPACE = 0x8
PULSE_OP_CAST_DIFF = 1
PULSE_OP_COMPACT = 2
PULSE_OP_LZ4_ENCODE = 3
PULSE_OP_LZ4_DECODE = 4
PULSE_OP_FP8_DELTA = 5
PULSE_OP_LOCO_GATE = 6
PULSE_OP_PATCH_UNPACK = 7
PULSE_OP_CAST_DIFF_SEGMENTS = 8
PULSE_OP_CAST_DIFF_LZ4 = 9
PULSE_OP_APPLY_QUANT = 10
PULSE_DS_BADSEGMENT = 0x10
PULSE_NOALLOC_SCRATCH_BYTES = 256 + 2 * 262144 * 8

_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_lib.pulse_version.restype = ctypes.c_char_p
_lib.pulse_status_string.restype = ctypes.c_char_p
_lib.pulse_status_string.argtypes = [ctypes.c_int]
_lib.pulse_workspace_bytes.restype = _SZ
_lib.pulse_workspace_bytes.argtypes = [ctypes.c_int, _I64, _I64]
_lib.pulse_workspace_init.argtypes = [_P, _SZ, _P]
_lib.pulse_cast_diff.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I64, _P, _SZ, _P]
_lib.pulse_compact.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _I64, _P, _SZ, _P]
_lib.pulse_apply_patch.argtypes = [_P, _I64, _P, _P, _P, _I64, _P, _P]
_lib.xor_mask_apply.argtypes = [_P, _P, _I64, _P]
_lib.lz4_encode_blocks.argtypes = [_P, _P, _I64, _I32, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]
_lib.lz4_decode_blocks.argtypes = [_P, _I64, _P, _P, _I64, _I32, _I64, _P, _I32, _P, _P, _SZ, _P]
_lib.lz4_decode_parse.argtypes = [_P, _I64, _P, _P, _I64, _I32, _I64, _P, _P, _SZ, _P]
_lib.lz4_decode_apply.argtypes = [_P, _I64, _P, _P, _I64, _I32, _I64, _P, _I32, _P, _P, _SZ, _P]
_lib.fp8_block_quant.argtypes = [_P, _P, _I32, _I64, _I64, _P, _P, _P, _P]
_lib.fp8_view_delta.argtypes = [_P, _P, _I64, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]
_lib.fp8_view_apply.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _I64, _P, _P, _P, _I64, _P, _P]
_lib.pulse_loco_gate.argtypes = [_P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _SZ, _P]
_lib.pulse_loco_accumulate.argtypes = [_P, _I64, _P, _P, _P, _I64, _P, _P]
_lib.patch_packed_bytes.argtypes = [_I64]
_lib.patch_packed_bytes.restype = _I64
_lib.patch_pack.argtypes = [_P, _P, _I64, _P, _P]
_lib.patch_unpack.argtypes = [_P, _I64, _P, _P, _P, _P, _SZ, _P]
_lib.pulse_segment_tiles.argtypes = [_P, _I32, _P, _P]
_lib.pulse_segment_tiles.restype = _I64
_lib.pulse_cast_diff_segments.argtypes = [_P, _I32, _P, _I64, _P, _P, _I64, _P, _P, _P, _SZ, _I32, _P]
_lib.pulse_apply_patch_segments.argtypes = [_P, _I32, _P, _P, _P, _I64, _P, _P]
_lib.fp8_block_quant_groups.argtypes = [_P, _I32, _P]
_lib.pulse_cast_diff_lz4.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I32, _P, _I64, _P, _P, _P, _P, _P, _SZ,
                                     _P]
_lib.pulse_cast_diff_lz4_noalloc.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I32, _P, _I64, _P, _P, _P,
                                             _P, _P]
_lib.pulse_patch_tiles.argtypes = [_P, _P, _I64, _I64, _P, _P]
_lib.pulse_apply_patch_tiled.argtypes = [_P, _I64, _P, _P, _P, _I64, _P, _P]
_lib.pulse_apply_quant_plan_bytes.argtypes = [_I32]
_lib.pulse_apply_quant_plan_bytes.restype = _I64
_lib.pulse_apply_quant_plan.argtypes = [_P, _I32, _I64, _P, _I64, _P]
_lib.pulse_apply_quant.argtypes = [_P, _I64, _P, _P, _P, _I64, _P, _I64, _P, _P, _SZ, _P]
for _f in ("pulse_cast_diff_segments", "pulse_apply_patch_segments", "patch_pack", "patch_unpack",
           "pulse_workspace_init", "pulse_cast_diff", "pulse_compact", "pulse_apply_patch",
           "xor_mask_apply", "lz4_encode_blocks", "lz4_decode_blocks", "fp8_block_quant",
           "fp8_view_delta", "fp8_view_apply", "pulse_loco_gate", "pulse_loco_accumulate",
           "lz4_decode_parse", "lz4_decode_apply", "pulse_cast_diff_lz4", "fp8_block_quant_groups",
           "pulse_patch_tiles", "pulse_apply_patch_tiled", "pulse_apply_quant_plan", "pulse_apply_quant",
           "pulse_cast_diff_lz4_noalloc"):
    getattr(_lib, _f).restype = ctypes.c_int


def lib_path() -> str:
    return _LIB_PATH


def pulse_version() -> str:
    return _lib.pulse_version().decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: {_lib.pulse_status_string(rc).decode()} ({rc})")


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _need(t, nbytes, name):
    """Host-side size check: the kernels trust the sizes they are given."""
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_U16 = (torch.uint16, torch.int16, torch.bfloat16)


def pulse_workspace_bytes(op: int, n: int, aux: int = 0) -> int:
    return int(_lib.pulse_workspace_bytes(op, n, aux))


def pulse_workspace_init(ws: torch.Tensor, stream=None):
    _check(_lib.pulse_workspace_init(_dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "pulse_workspace_init")


def workspace(op: int, n: int, aux: int = 0, device="cuda") -> torch.Tensor:
    """A zeroed workspace of the size the op needs (allocation is the caller's)."""
    nbytes = max(pulse_workspace_bytes(op, n, aux), 256)
    return torch.zeros((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def _ws(ws):
    if ws is None:
        return None, 0
    return _dev(ws, "ws"), ws.numel() * ws.element_size()


def pulse_cast_diff(w_new, b_old=None, b_new=None, xor_mask=None, patch_idx=None, patch_val=None,
                    d_count=None, d_status=None, ws=None, n=None, stream=None):
    n = w_new.numel() if n is None else n
    cap = 0 if patch_idx is None else patch_idx.numel()
    _need(w_new, 4 * n, "w_new")
    for t, nm in ((b_old, "b_old"), (b_new, "b_new"), (xor_mask, "xor_mask")):
        _need(t, 2 * n, nm)
    _need(patch_val, 2 * cap, "patch_val")
    wsp, wsb = _ws(ws)
    _check(_lib.pulse_cast_diff(
        _dev(w_new, "w_new", torch.float32), _dev(b_old, "b_old", _U16), _dev(b_new, "b_new", _U16),
        _dev(xor_mask, "xor_mask", _U16), _dev(patch_idx, "patch_idx", torch.int32),
        _dev(patch_val, "patch_val", _U16), cap, _dev(d_count, "d_count", torch.int64),
        _dev(d_status, "d_status", torch.int32), n, wsp, wsb, _stream(stream)), "pulse_cast_diff")


def pulse_compact(b_old, b_new, patch_idx, patch_val, d_count, d_status, ws, n=None, stream=None):
    n = b_old.numel() if n is None else n
    _need(b_old, 2 * n, "b_old")
    _need(b_new, 2 * n, "b_new")
    _need(patch_val, 2 * patch_idx.numel(), "patch_val")
    wsp, wsb = _ws(ws)
    _check(_lib.pulse_compact(
        _dev(b_old, "b_old", _U16), _dev(b_new, "b_new", _U16), _dev(patch_idx, "patch_idx", torch.int32),
        _dev(patch_val, "patch_val", _U16), patch_idx.numel(), _dev(d_count, "d_count", torch.int64),
        _dev(d_status, "d_status", torch.int32), n, wsp, wsb, _stream(stream)), "pulse_compact")


def pulse_apply_patch(b, patch_idx, patch_val, d_count, d_status, max_count=None, n=None, stream=None):
    n = b.numel() if n is None else n
    max_count = patch_idx.numel() if max_count is None else max_count
    _need(b, 2 * n, "b")
    _need(patch_idx, 4 * max_count, "patch_idx")
    _need(patch_val, 2 * max_count, "patch_val")
    _check(_lib.pulse_apply_patch(
        _dev(b, "b", _U16), n, _dev(patch_idx, "patch_idx", torch.int32), _dev(patch_val, "patch_val", _U16),
        _dev(d_count, "d_count", torch.int64), max_count, _dev(d_status, "d_status", torch.int32),
        _stream(stream)), "pulse_apply_patch")


def xor_mask_apply(dst, mask, nbytes=None, stream=None):
    nbytes = dst.numel() * dst.element_size() if nbytes is None else nbytes
    _need(dst, nbytes, "dst")
    _need(mask, nbytes, "mask")
    _check(_lib.xor_mask_apply(_dev(dst, "dst"), _dev(mask, "mask"), nbytes, _stream(stream)), "xor_mask_apply")


def lz4_payload_bound(nbytes: int, block_bytes: int = 65536) -> int:
    nb = (nbytes + block_bytes - 1) // block_bytes
    return nb * (block_bytes + block_bytes // 255 + 16)


def lz4_encode_blocks(src, payload, comp_sizes, comp_offsets, d_total, d_status, ws, src_xor=None,
                      block_bytes=65536, nbytes=None, stream=None):
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    nb = (nbytes + block_bytes - 1) // block_bytes
    _need(src, nbytes, "src")
    _need(src_xor, nbytes, "src_xor")
    _need(comp_sizes, 4 * nb, "comp_sizes")
    _need(comp_offsets, 8 * nb, "comp_offsets")
    wsp, wsb = _ws(ws)
    _check(_lib.lz4_encode_blocks(
        _dev(src, "src"), _dev(src_xor, "src_xor"), nbytes, block_bytes, _dev(payload, "payload", torch.uint8),
        payload.numel(), _dev(comp_sizes, "comp_sizes", torch.int32), _dev(comp_offsets, "comp_offsets", torch.int64),
        _dev(d_total, "d_total", torch.int64), _dev(d_status, "d_status", torch.int32), wsp, wsb,
        _stream(stream)), "lz4_encode_blocks")


PATCH_TILE = 16384


def patch_tile_count(n: int) -> int:
    """Entries of a patch's tile index over n elements (ceil(n / 16384) + 1)."""
    return (n + PATCH_TILE - 1) // PATCH_TILE + 1


def pulse_patch_tiles(patch_idx, d_count, tile_first, n, max_count=None, stream=None):
    max_count = patch_idx.numel() if max_count is None else max_count
    _need(patch_idx, 4 * max_count, "patch_idx")
    _need(tile_first, 8 * patch_tile_count(n), "tile_first")
    _check(_lib.pulse_patch_tiles(_dev(patch_idx, "patch_idx", torch.int32), _dev(d_count, "d_count", torch.int64),
                                  max_count, n, _dev(tile_first, "tile_first", torch.int64), _stream(stream)),
           "pulse_patch_tiles")


def pulse_apply_patch_tiled(b, patch_idx, patch_val, tile_first, d_status, max_count=None, n=None, stream=None):
    n = b.numel() if n is None else n
    max_count = patch_idx.numel() if max_count is None else max_count
    _need(b, 2 * n, "b")
    _need(patch_idx, 4 * max_count, "patch_idx")
    _need(patch_val, 2 * max_count, "patch_val")
    _need(tile_first, 8 * patch_tile_count(n), "tile_first")
    _check(_lib.pulse_apply_patch_tiled(
        _dev(b, "b", _U16), n, _dev(patch_idx, "patch_idx", torch.int32), _dev(patch_val, "patch_val", _U16),
        _dev(tile_first, "tile_first", torch.int64), max_count, _dev(d_status, "d_status", torch.int32),
        _stream(stream)), "pulse_apply_patch_tiled")


def pulse_cast_diff_lz4(w_new, b_old, b_new, patch_idx, patch_val, d_count, payload, comp_sizes, comp_offsets,
                        d_total, d_status, ws, block_bytes=65536, n=None, tile_first=None, stream=None):
    """cast + diff + patch + LZ4 blocks of the XOR mask in one pass (patch_idx,
    patch_val and d_count all None: mask blocks only); tile_first, when given,
    receives the patch's tile index."""
    n = w_new.numel() if n is None else n
    _need(tile_first, 8 * patch_tile_count(n), "tile_first")
    nb = (2 * n + block_bytes - 1) // block_bytes
    cap = 0 if patch_idx is None else patch_idx.numel()
    _need(w_new, 4 * n, "w_new")
    _need(b_old, 2 * n, "b_old")
    _need(b_new, 2 * n, "b_new")
    _need(patch_val, 2 * cap, "patch_val")
    _need(comp_sizes, 4 * nb, "comp_sizes")
    _need(comp_offsets, 8 * nb, "comp_offsets")
    wsp, wsb = _ws(ws)
    _check(_lib.pulse_cast_diff_lz4(
        _dev(w_new, "w_new", torch.float32), _dev(b_old, "b_old", _U16), _dev(b_new, "b_new", _U16),
        _dev(patch_idx, "patch_idx", torch.int32), _dev(patch_val, "patch_val", _U16), cap,
        _dev(d_count, "d_count", torch.int64), _dev(tile_first, "tile_first", torch.int64), n, block_bytes,
        _dev(payload, "payload", torch.uint8), payload.numel(),
        _dev(comp_sizes, "comp_sizes", torch.int32), _dev(comp_offsets, "comp_offsets", torch.int64),
        _dev(d_total, "d_total", torch.int64), _dev(d_status, "d_status", torch.int32), wsp, wsb,
        _stream(stream)), "pulse_cast_diff_lz4")


def pulse_cast_diff_lz4_noalloc(w_new, b_old, b_new, patch_idx, patch_val, d_count, payload, comp_sizes,
                                comp_offsets, d_total, d_status, block_bytes=65536, n=None, tile_first=None,
                                stream=None):
    """pulse_cast_diff_lz4 with the library's static per-GPU scratch instead of
    a workspace: the call allocates nothing (calls overlapping on one GPU race)."""
    n = w_new.numel() if n is None else n
    _need(tile_first, 8 * patch_tile_count(n), "tile_first")
    nb = (2 * n + block_bytes - 1) // block_bytes
    cap = 0 if patch_idx is None else patch_idx.numel()
    _need(w_new, 4 * n, "w_new")
    _need(b_old, 2 * n, "b_old")
    _need(b_new, 2 * n, "b_new")
    _need(patch_val, 2 * cap, "patch_val")
    _need(comp_sizes, 4 * nb, "comp_sizes")
    _need(comp_offsets, 8 * nb, "comp_offsets")
    _check(_lib.pulse_cast_diff_lz4_noalloc(
        _dev(w_new, "w_new", torch.float32), _dev(b_old, "b_old", _U16), _dev(b_new, "b_new", _U16),
        _dev(patch_idx, "patch_idx", torch.int32), _dev(patch_val, "patch_val", _U16), cap,
        _dev(d_count, "d_count", torch.int64), _dev(tile_first, "tile_first", torch.int64), n, block_bytes,
        _dev(payload, "payload", torch.uint8), payload.numel(),
        _dev(comp_sizes, "comp_sizes", torch.int32), _dev(comp_offsets, "comp_offsets", torch.int64),
        _dev(d_total, "d_total", torch.int64), _dev(d_status, "d_status", torch.int32),
        _stream(stream)), "pulse_cast_diff_lz4_noalloc")


def _decode_table(payload, comp_offsets, comp_sizes, nbytes, payload_bytes, block_bytes):
    payload_bytes = payload.numel() if payload_bytes is None else payload_bytes
    nb = (nbytes + block_bytes - 1) // block_bytes
    _need(payload, payload_bytes, "payload")
    _need(comp_sizes, 4 * nb, "comp_sizes")
    _need(comp_offsets, 8 * nb, "comp_offsets")
    return (_dev(payload, "payload", torch.uint8), payload_bytes, _dev(comp_offsets, "comp_offsets", torch.int64),
            _dev(comp_sizes, "comp_sizes", torch.int32), nb, block_bytes, nbytes)


def lz4_decode_blocks(payload, comp_offsets, comp_sizes, dst, d_status, ws, mode=1, block_bytes=65536,
                      nbytes=None, payload_bytes=None, stream=None):
    nbytes = dst.numel() * dst.element_size() if nbytes is None else nbytes
    _need(dst, nbytes, "dst")
    tab = _decode_table(payload, comp_offsets, comp_sizes, nbytes, payload_bytes, block_bytes)
    wsp, wsb = _ws(ws)
    _check(_lib.lz4_decode_blocks(*tab, _dev(dst, "dst"), mode, _dev(d_status, "d_status", torch.int32), wsp, wsb,
                                  _stream(stream)), "lz4_decode_blocks")


def lz4_decode_parse(payload, comp_offsets, comp_sizes, nbytes, d_status, ws, block_bytes=65536,
                     payload_bytes=None, stream=None):
    """First half of lz4_decode_blocks: parse every block into ws (no dst)."""
    tab = _decode_table(payload, comp_offsets, comp_sizes, nbytes, payload_bytes, block_bytes)
    wsp, wsb = _ws(ws)
    _check(_lib.lz4_decode_parse(*tab, _dev(d_status, "d_status", torch.int32), wsp, wsb, _stream(stream)),
           "lz4_decode_parse")


def lz4_decode_apply(payload, comp_offsets, comp_sizes, dst, d_status, ws, mode=1, block_bytes=65536,
                     nbytes=None, payload_bytes=None, stream=None):
    """Second half: apply what the last lz4_decode_parse on ws found to dst."""
    nbytes = dst.numel() * dst.element_size() if nbytes is None else nbytes
    _need(dst, nbytes, "dst")
    tab = _decode_table(payload, comp_offsets, comp_sizes, nbytes, payload_bytes, block_bytes)
    wsp, wsb = _ws(ws)
    _check(_lib.lz4_decode_apply(*tab, _dev(dst, "dst"), mode, _dev(d_status, "d_status", torch.int32), wsp, wsb,
                                 _stream(stream)), "lz4_decode_apply")


def _batch_src(t, name):
    """A [batch, rows, cols] source whose rows are contiguous; the batch stride
    (elements) may be anything, e.g. one expert's gate inside [gate, up, down]
    triples.  Returns (data pointer, batch stride)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in _U16:
        raise ValueError(f"{name} has dtype {t.dtype}, expected 16-bit")
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2] or t.stride(0) < t.shape[1] * t.shape[2]:
        raise ValueError(f"{name} must be [batch, rows, cols] with contiguous rows")
    return t.data_ptr(), t.stride(0)


def fp8_block_quant(srcs, codes, scales, batch=1, stream=None):
    """srcs: list of BF16/uint16 GPU tensors [rows_i, cols] (contiguous), or, when
    batch > 1, [batch, rows_i, cols] views with contiguous rows and any batch stride."""
    cols = srcs[0].shape[-1]
    R = sum(int(t.shape[-2]) for t in srcs)
    for i, t in enumerate(srcs):
        if t.shape[-1] != cols or (batch > 1 and (t.dim() != 3 or t.shape[0] != batch)):
            raise ValueError(f"srcs[{i}] has shape {tuple(t.shape)}")
    _need(codes, batch * R * cols, "codes")
    _need(scales, 4 * batch * ((R + 127) // 128) * ((cols + 127) // 128), "scales")
    if batch > 1:
        ps = [_batch_src(s, f"srcs[{i}]") for i, s in enumerate(srcs)]
        ptrs = (ctypes.c_void_p * len(srcs))(*[p for p, _ in ps])
        strides = (ctypes.c_int64 * len(srcs))(*[st for _, st in ps])
    else:
        ptrs = (ctypes.c_void_p * len(srcs))(*[_dev(s, f"srcs[{i}]", _U16) for i, s in enumerate(srcs)])
        strides = None
    rows = (ctypes.c_int64 * len(srcs))(*[s.shape[-2] for s in srcs])
    _check(_lib.fp8_block_quant(
        ctypes.cast(ptrs, ctypes.c_void_p), ctypes.cast(rows, ctypes.c_void_p), len(srcs), cols, batch,
        None if strides is None else ctypes.cast(strides, ctypes.c_void_p),
        _dev(codes, "codes", torch.uint8), _dev(scales, "scales", torch.float32), _stream(stream)),
        "fp8_block_quant")


PULSE_QUANT_MAX_GROUPS = 8


class _QuantGroup(ctypes.Structure):
    """The layout of pulse_quant_group."""
    _fields_ = [("src", ctypes.c_void_p * 4), ("rows", ctypes.c_int64 * 4), ("nsrc", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


def fp8_block_quant_groups(groups, stream=None):
    """groups: list (1..8) of (srcs, codes, scales), srcs a list (1..4) of
    contiguous BF16/uint16 GPU tensors [rows_i, cols]: one launch for all."""
    if not 1 <= len(groups) <= PULSE_QUANT_MAX_GROUPS:
        raise ValueError(f"{len(groups)} groups (1..{PULSE_QUANT_MAX_GROUPS} per call)")
    arr = (_QuantGroup * len(groups))()
    for g, (srcs, codes, scales) in enumerate(groups):
        if not 1 <= len(srcs) <= 4:
            raise ValueError(f"group {g}: {len(srcs)} sources (1..4)")
        cols = srcs[0].shape[-1]
        R = 0
        for i, t in enumerate(srcs):
            if t.dim() != 2 or t.shape[-1] != cols:
                raise ValueError(f"group {g} source {i} has shape {tuple(t.shape)}")
            arr[g].src[i] = _dev(t, f"groups[{g}].srcs[{i}]", _U16)
            arr[g].rows[i] = int(t.shape[0])
            R += int(t.shape[0])
        _need(codes, R * cols, f"groups[{g}].codes")
        _need(scales, 4 * ((R + 127) // 128) * ((cols + 127) // 128), f"groups[{g}].scales")
        arr[g].nsrc = len(srcs)
        arr[g].cols = cols
        arr[g].codes = _dev(codes, f"groups[{g}].codes", torch.uint8)
        arr[g].scales = _dev(scales, f"groups[{g}].scales", torch.float32)
    _check(_lib.fp8_block_quant_groups(ctypes.cast(arr, ctypes.c_void_p), len(groups), _stream(stream)),
           "fp8_block_quant_groups")


class _AQGroup(ctypes.Structure):
    """The layout of pulse_aq_group."""
    _fields_ = [("src_offset", ctypes.c_int64 * 4), ("rows", ctypes.c_int64 * 4), ("nsrc", ctypes.c_int32),
                ("quantise", ctypes.c_int32), ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class ApplyQuantPlan:
    """A view's groups for pulse_apply_quant, resident on the device.  Holds
    the output tensors it points into, so they live as long as the plan."""

    def __init__(self, tensor, nblocks, n, outputs):
        self.tensor, self.nblocks, self.n, self._outputs = tensor, nblocks, n, outputs


def pulse_apply_quant_plan(groups, n, device="cuda"):
    """groups: list of (sources, cols, codes, scales); sources a list (1..4) of
    (element offset, rows) of row-major [rows, cols] matrices inside the view
    of n elements, stacked in that order; codes [R * cols] uint8 and scales
    [ceil(R/128) * ceil(cols/128)] float32 GPU tensors, or both None for a
    group that is only patched.  The sources of all groups must tile [0, n)."""
    arr = (_AQGroup * len(groups))()
    outs = []
    for g, (srcs, cols, codes, scales) in enumerate(groups):
        if not 1 <= len(srcs) <= 4:
            raise ValueError(f"group {g}: {len(srcs)} sources (1..4)")
        R = 0
        for i, (off, rows) in enumerate(srcs):
            arr[g].src_offset[i] = int(off)
            arr[g].rows[i] = int(rows)
            R += int(rows)
        arr[g].nsrc = len(srcs)
        arr[g].cols = int(cols)
        if (codes is None) != (scales is None):
            raise ValueError(f"group {g}: codes and scales go together")
        if codes is not None:
            _need(codes, R * cols, f"groups[{g}].codes")
            _need(scales, 4 * ((R + 127) // 128) * ((cols + 127) // 128), f"groups[{g}].scales")
            arr[g].quantise = 1
            arr[g].codes = _dev(codes, f"groups[{g}].codes", torch.uint8)
            arr[g].scales = _dev(scales, f"groups[{g}].scales", torch.float32)
            outs += [codes, scales]
    nbytes = int(_lib.pulse_apply_quant_plan_bytes(len(groups)))
    plan = torch.empty((max(nbytes, 16) + 15) // 16 * 16, dtype=torch.uint8, device=device)
    nblocks = ctypes.c_int64(0)
    _check(_lib.pulse_apply_quant_plan(ctypes.cast(arr, ctypes.c_void_p), len(groups), n, _dev(plan, "plan"),
                                       plan.numel(), ctypes.byref(nblocks)), "pulse_apply_quant_plan")
    return ApplyQuantPlan(plan, int(nblocks.value), n, outs)


def pulse_apply_quant(b, patch_idx, patch_val, d_count, plan, d_status, ws, max_count=None, stream=None):
    """The receiver's pass: the patch applied to the view b and the plan's
    groups quantised to FP8 from the patched values, in one read of b."""
    n = plan.n
    max_count = patch_idx.numel() if max_count is None else max_count
    _need(b, 2 * n, "b")
    _need(patch_idx, 4 * max_count, "patch_idx")
    _need(patch_val, 2 * max_count, "patch_val")
    wsp, wsb = _ws(ws)
    _check(_lib.pulse_apply_quant(
        _dev(b, "b", _U16), n, _dev(patch_idx, "patch_idx", torch.int32), _dev(patch_val, "patch_val", _U16),
        _dev(d_count, "d_count", torch.int64), max_count, _dev(plan.tensor, "plan"), plan.nblocks,
        _dev(d_status, "d_status", torch.int32), wsp, wsb, _stream(stream)), "pulse_apply_quant")


def fp8_view_delta(codes_old, codes_new, scales_old, scales_new, code_idx, code_val, d_code_count,
                   scale_idx, scale_val, d_scale_count, d_status, ws, code_cap=None, scale_cap=None,
                   stream=None):
    """Changed E4M3 codes and block scales between two quantisations (flat views)."""
    nc, ns = codes_old.numel(), scales_old.numel()
    code_cap = code_idx.numel() if code_cap is None else code_cap
    scale_cap = scale_idx.numel() if scale_cap is None else scale_cap
    _need(codes_new, nc, "codes_new")
    _need(scales_new, 4 * ns, "scales_new")
    _need(code_idx, 4 * code_cap, "code_idx")
    _need(code_val, code_cap, "code_val")
    _need(scale_idx, 4 * scale_cap, "scale_idx")
    _need(scale_val, 4 * scale_cap, "scale_val")
    wsp, wsb = _ws(ws)
    _check(_lib.fp8_view_delta(
        _dev(codes_old, "codes_old", torch.uint8), _dev(codes_new, "codes_new", torch.uint8), nc,
        _dev(scales_old, "scales_old", torch.float32), _dev(scales_new, "scales_new", torch.float32), ns,
        _dev(code_idx, "code_idx", torch.int32), _dev(code_val, "code_val", torch.uint8), code_cap,
        _dev(d_code_count, "d_code_count", torch.int64), _dev(scale_idx, "scale_idx", torch.int32),
        _dev(scale_val, "scale_val", torch.float32), scale_cap,
        _dev(d_scale_count, "d_scale_count", torch.int64), _dev(d_status, "d_status", torch.int32),
        wsp, wsb, _stream(stream)), "fp8_view_delta")


def fp8_view_apply(codes, scales, code_idx, code_val, d_code_count, scale_idx, scale_val, d_scale_count,
                   d_status, max_code_count=None, max_scale_count=None, stream=None):
    mc = code_idx.numel() if max_code_count is None else max_code_count
    ms = scale_idx.numel() if max_scale_count is None else max_scale_count
    _need(code_idx, 4 * mc, "code_idx")
    _need(code_val, mc, "code_val")
    _need(scale_idx, 4 * ms, "scale_idx")
    _need(scale_val, 4 * ms, "scale_val")
    _check(_lib.fp8_view_apply(
        _dev(codes, "codes", torch.uint8), codes.numel(), _dev(scales, "scales", torch.float32), scales.numel(),
        _dev(code_idx, "code_idx", torch.int32), _dev(code_val, "code_val", torch.uint8),
        _dev(d_code_count, "d_code_count", torch.int64), mc, _dev(scale_idx, "scale_idx", torch.int32),
        _dev(scale_val, "scale_val", torch.float32), _dev(d_scale_count, "d_scale_count", torch.int64), ms,
        _dev(d_status, "d_status", torch.int32), _stream(stream)), "fp8_view_apply")


def pulse_loco_gate(theta, delta, resid, idx, val, d_count, d_status, ws, n=None, cap=None, stream=None):
    """Visible entries of resid + delta against the BF16 view of theta; resid rewritten in place."""
    n = theta.numel() if n is None else n
    cap = idx.numel() if cap is None else cap
    for t, nm in ((theta, "theta"), (delta, "delta"), (resid, "resid")):
        _need(t, 4 * n, nm)
    _need(idx, 4 * cap, "idx")
    _need(val, 4 * cap, "val")
    wsp, wsb = _ws(ws)
    _check(_lib.pulse_loco_gate(
        _dev(theta, "theta", torch.float32), _dev(delta, "delta", torch.float32),
        _dev(resid, "resid", torch.float32), n, _dev(idx, "idx", torch.int32), _dev(val, "val", torch.float32),
        cap, _dev(d_count, "d_count", torch.int64), _dev(d_status, "d_status", torch.int32),
        wsp, wsb, _stream(stream)), "pulse_loco_gate")


def pulse_loco_accumulate(acc, idx, val, d_count, d_status, max_count=None, stream=None):
    max_count = idx.numel() if max_count is None else max_count
    _need(idx, 4 * max_count, "idx")
    _need(val, 4 * max_count, "val")
    _check(_lib.pulse_loco_accumulate(
        _dev(acc, "acc", torch.float32), acc.numel(), _dev(idx, "idx", torch.int32),
        _dev(val, "val", torch.float32), _dev(d_count, "d_count", torch.int64), max_count,
        _dev(d_status, "d_status", torch.int32), _stream(stream)), "pulse_loco_accumulate")


def patch_packed_bytes(count: int) -> int:
    return int(_lib.patch_packed_bytes(count))


def patch_pack(idx, val, count, packed, stream=None):
    """Gap + byte-plane form of the first `count` entries of a patch."""
    _need(idx, 4 * count, "idx")
    _need(val, 2 * count, "val")
    _need(packed, patch_packed_bytes(count), "packed")
    _check(_lib.patch_pack(_dev(idx, "idx", torch.int32), _dev(val, "val", _U16), count,
                           _dev(packed, "packed", torch.uint8), _stream(stream)), "patch_pack")


def patch_unpack(packed, count, idx, val, d_status, ws, stream=None):
    _need(packed, patch_packed_bytes(count), "packed")
    _need(idx, 4 * count, "idx")
    _need(val, 2 * count, "val")
    wsp, wsb = _ws(ws)
    _check(_lib.patch_unpack(_dev(packed, "packed", torch.uint8), count, _dev(idx, "idx", torch.int32),
                             _dev(val, "val", _U16), _dev(d_status, "d_status", torch.int32), wsp, wsb,
                             _stream(stream)), "patch_unpack")


def pulse_segment_tiles(ns):
    """Host tiling metadata of a list of tensor sizes: (ntiles, tile0, tile_seg) as numpy arrays."""
    import numpy as np

    n = np.ascontiguousarray(ns, dtype=np.int64)
    t = int(_lib.pulse_segment_tiles(n.ctypes.data, n.size, None, None))
    if t < 0:
        raise RuntimeError(f"pulse_segment_tiles: {_lib.pulse_status_string(t).decode()} ({t})")
    tile0 = np.empty(n.size, np.int64)
    tile_seg = np.empty(max(t, 1), np.uint32)
    _lib.pulse_segment_tiles(n.ctypes.data, n.size, tile0.ctypes.data, tile_seg.ctypes.data)
    return t, tile0, tile_seg[:t]


class SegmentTable:
    """The device tables of a list call (pulse_segment[nseg] and the tile map),
    prepared once on the host for a list of tensors and reused every step.
    w_new: float32 GPU tensors; b_old, b_new: BF16/uint16 GPU tensors (b_new may be None)."""

    def __init__(self, w_new, b_old, b_new=None, device="cuda"):
        import numpy as np

        if len(w_new) != len(b_old) or (b_new is not None and len(b_new) != len(w_new)) or not w_new:
            raise ValueError("w_new, b_old (and b_new) must be lists of the same, non-zero length")
        ns = [t.numel() for t in w_new]
        for i, (w, b) in enumerate(zip(w_new, b_old)):
            _dev(w, f"w_new[{i}]", torch.float32)
            _dev(b, f"b_old[{i}]", _U16)
            _need(b, 2 * ns[i], f"b_old[{i}]")
            if b_new is not None:
                _dev(b_new[i], f"b_new[{i}]", _U16)
                _need(b_new[i], 2 * ns[i], f"b_new[{i}]")
        self.ntiles, tile0, tile_seg = pulse_segment_tiles(ns)
        tab = np.zeros((len(ns), 5), np.int64)
        for i in range(len(ns)):
            tab[i] = [w_new[i].data_ptr(), b_old[i].data_ptr(), 0 if b_new is None else b_new[i].data_ptr(),
                      ns[i], tile0[i]]
        self.nseg = len(ns)
        self.with_new = b_new is not None
        self.segs = torch.from_numpy(tab).to(device)
        self.tile_seg = torch.from_numpy(tile_seg.view(np.int32)).to(device)
        self._keep = (list(w_new), list(b_old), None if b_new is None else list(b_new))


class ViewTable:
    """Device table pulse_view[nseg] of the receiver's BF16 views (GPU tensors)."""

    def __init__(self, views, device="cuda"):
        import numpy as np

        tab = np.zeros((len(views), 2), np.int64)
        for i, v in enumerate(views):
            _dev(v, f"views[{i}]", _U16)
            tab[i] = [v.data_ptr(), v.numel()]
        self.nseg = len(views)
        self.views = torch.from_numpy(tab).to(device)
        self._keep = list(views)


def pulse_cast_diff_segments(table, patch_idx, patch_val, seg_offsets, d_status, ws, stream=None):
    cap = patch_idx.numel()
    _need(patch_val, 2 * cap, "patch_val")
    _need(seg_offsets, 8 * (table.nseg + 1), "seg_offsets")
    wsp, wsb = _ws(ws)
    _check(_lib.pulse_cast_diff_segments(
        table.segs.data_ptr(), table.nseg, table.tile_seg.data_ptr(), table.ntiles,
        _dev(patch_idx, "patch_idx", torch.int32), _dev(patch_val, "patch_val", _U16), cap,
        _dev(seg_offsets, "seg_offsets", torch.int64), _dev(d_status, "d_status", torch.int32), wsp, wsb,
        1 if table.with_new else 0, _stream(stream)), "pulse_cast_diff_segments")


def pulse_apply_patch_segments(views, patch_idx, patch_val, seg_offsets, d_status, max_count=None, stream=None):
    max_count = patch_idx.numel() if max_count is None else max_count
    _need(patch_idx, 4 * max_count, "patch_idx")
    _need(patch_val, 2 * max_count, "patch_val")
    _need(seg_offsets, 8 * (views.nseg + 1), "seg_offsets")
    _check(_lib.pulse_apply_patch_segments(
        views.views.data_ptr(), views.nseg, _dev(patch_idx, "patch_idx", torch.int32),
        _dev(patch_val, "patch_val", _U16), _dev(seg_offsets, "seg_offsets", torch.int64), max_count,
        _dev(d_status, "d_status", torch.int32), _stream(stream)), "pulse_apply_patch_segments")

