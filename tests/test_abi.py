"""CPU checks of the C ABI: the library loads, exports every entry point that
include/pulse.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pulse.h")
LIB = os.environ.get("SDC_PULSE_LIB") or os.path.join(ROOT, "sparse_delta_codec_amd", "libpulse.so")

EINVAL, EALIGN, ERANGE, EWORKSPACE = -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    L.pulse_status_string.restype = ctypes.c_char_p
    L.pulse_version.restype = ctypes.c_char_p
    L.pulse_workspace_bytes.restype = ctypes.c_size_t
    L.pulse_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    return L


def test_header_declares_the_codec_calls():
    fns = declared_functions()
    for name in ("pulse_cast_diff", "pulse_compact", "pulse_apply_patch", "xor_mask_apply",
                 "lz4_encode_blocks", "lz4_decode_blocks", "lz4_decode_parse", "lz4_decode_apply",
                 "fp8_block_quant", "fp8_block_quant_groups", "pulse_cast_diff_lz4", "pulse_patch_tiles",
                 "pulse_apply_patch_tiled", "pulse_apply_quant_plan_bytes", "pulse_apply_quant_plan",
                 "pulse_apply_quant", "pulse_workspace_bytes",
                 "pulse_workspace_init", "pulse_status_string", "pulse_version"):
        assert name in fns, name


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.pulse_status_string(0) == b"PULSE_OK"
    assert b"aligned" in lib.pulse_status_string(EALIGN)
    assert lib.pulse_version().count(b".") == 2


def test_workspace_sizes(lib):
    ws = lib.pulse_workspace_bytes
    assert ws(1, 16384, 0) == 256 + 8 and ws(1, 16385, 0) == 256 + 16
    assert ws(3, 65536 * 3 + 1, 65536) == 256 + 4 * 8
    assert ws(4, 10, 1 << 20) > (1 << 20) // 32
    # decode workspaces grow with both arguments and always fit their own call
    prev = 0
    for nb, pb in [(1, 10), (100, 10 ** 6), (60000, 1_400_000_000), (500000, 7 * 10 ** 9)]:
        cur = ws(4, nb, pb)
        assert cur > prev
        prev = cur
    assert ws(99, 10, 0) == 0
    # fused sender pass: header + two status words per mask block
    assert ws(9, 32768 * 3 + 1, 65536) == 256 + 2 * 4 * 8
    assert ws(9, 1000, 1000) == 0
    # receiver's pass: one int32 segment start per 128 elements plus the closing one (rounded to
    # 256 bytes), then 8 block counters 128 bytes apart
    assert ws(10, 128 * 5, 0) == 256 + 1024 and ws(10, 128 * 63, 0) == 256 + 1024
    assert ws(10, 128 * 64, 0) == 512 + 1024


V = ctypes.c_void_p
I64 = ctypes.c_int64


def test_argument_errors_return_before_any_launch(lib):
    al = V(0x10000)      # aligned fake pointers, never dereferenced on these paths
    mis = V(0x10002)
    cd = lib.pulse_cast_diff
    cd.argtypes = [V, V, V, V, V, V, I64, V, V, I64, V, ctypes.c_size_t, V]
    assert cd(None, None, al, None, None, None, 0, None, None, 10, None, 0, None) == EINVAL
    assert cd(al, None, None, None, None, None, 0, None, None, 10, None, 0, None) == EINVAL   # no output
    assert cd(al, None, None, al, None, None, 0, None, None, 10, None, 0, None) == EINVAL     # mask needs old
    assert cd(mis, None, al, None, None, None, 0, None, None, 10, None, 0, None) == EALIGN
    assert cd(al, al, al, None, al, al, 10, al, al, 1 << 31, al, 1 << 40, None) == ERANGE
    assert cd(al, al, al, None, al, al, 10, al, al, 100000, al, 64, None) == EWORKSPACE
    assert cd(al, al, al, None, al, None, 10, al, al, 100, al, 1 << 20, None) == EINVAL      # partial patch
    enc = lib.lz4_encode_blocks
    enc.argtypes = [V, V, I64, ctypes.c_int32, V, I64, V, V, V, V, V, ctypes.c_size_t, V]
    assert enc(al, None, 1000, 1000, al, 10, al, al, al, al, al, 1 << 20, None) == EINVAL    # block size
    assert enc(mis, None, 1000, 65536, al, 10, al, al, al, al, al, 1 << 20, None) == EALIGN
    assert enc(al, None, 1000, 65536, al, 10, al, al, al, al, al, 8, None) == EWORKSPACE
    dec = lib.lz4_decode_blocks
    dec.argtypes = [V, I64, V, V, I64, ctypes.c_int32, I64, V, ctypes.c_int32, V, V, ctypes.c_size_t, V]
    assert dec(al, 10, al, al, 2, 65536, 70000, al, 2, al, al, 1 << 20, None) == EINVAL     # mode
    assert dec(al, 10, al, al, 3, 65536, 70000, al, 1, al, al, 1 << 20, None) == EINVAL     # nblocks
    assert dec(al, 10, al, al, 2, 65536, 70000, mis, 1, al, al, 1 << 20, None) == EALIGN
    assert dec(al, 10, al, al, 2, 65536, 70000, al, 1, al, al, 16, None) == EWORKSPACE
    par = lib.lz4_decode_parse
    par.argtypes = [V, I64, V, V, I64, ctypes.c_int32, I64, V, V, ctypes.c_size_t, V]
    assert par(al, 10, al, al, 3, 65536, 70000, al, al, 1 << 20, None) == EINVAL          # nblocks
    assert par(al, 10, None, al, 2, 65536, 70000, al, al, 1 << 20, None) == EINVAL        # no offsets
    assert par(al, 10, al, al, 2, 65536, 70000, al, al, 16, None) == EWORKSPACE
    import sparse_delta_codec_amd as pk  # the binding's layout of pulse_quant_group
    fq = lib.fp8_block_quant_groups
    fq.argtypes = [V, ctypes.c_int32, V]
    grp = (pk._QuantGroup * 2)()
    for g in grp:
        g.src[0], g.rows[0], g.nsrc, g.cols, g.codes, g.scales = 0x10000, 128, 1, 128, 0x20000, 0x30000
    gp = ctypes.cast(grp, V)
    assert fq(gp, 0, None) == EINVAL and fq(gp, 9, None) == EINVAL and fq(None, 1, None) == EINVAL
    grp[1].cols = 100
    assert fq(gp, 2, None) == EINVAL                                              # cols % 8
    grp[1].cols, grp[1].nsrc = 128, 5
    assert fq(gp, 2, None) == EINVAL                                              # nsrc
    grp[1].nsrc, grp[1].src[0] = 1, 0x10002
    assert fq(gp, 2, None) == EALIGN                                              # source alignment
    grp[1].src[0], grp[1].rows[0] = 0x10000, 0
    assert fq(gp, 2, None) == EINVAL                                              # no rows
    fz = lib.pulse_cast_diff_lz4
    fz.argtypes = [V, V, V, V, V, I64, V, V, I64, ctypes.c_int32, V, I64, V, V, V, V, V, ctypes.c_size_t, V]
    fargs = [al, al, al, al, al, 10, al, al, 1000, 65536, al, 100, al, al, al, al, al, 1 << 20, None]
    assert fz(None, *fargs[1:]) == EINVAL                                         # no masters
    assert fz(*fargs[:8], 0, *fargs[9:]) == EINVAL                                # n = 0
    assert fz(*fargs[:9], 4096, *fargs[10:]) == EINVAL                            # block size
    assert fz(*fargs[:4], None, *fargs[5:]) == EINVAL                             # partial patch
    assert fz(*fargs[:3], None, None, 10, None, al, *fargs[8:]) == EINVAL         # tile index without patch
    assert fz(*fargs[:2], mis, *fargs[3:]) == EALIGN                              # b_new
    assert fz(*fargs[:8], 1 << 31, *fargs[9:]) == ERANGE                          # int32 indices
    assert fz(*fargs[:17], 16, None) == EWORKSPACE
    pt = lib.pulse_patch_tiles
    pt.argtypes = [V, V, I64, I64, V, V]
    assert pt(None, al, 10, 100, al, None) == EINVAL and pt(al, al, 10, 0, al, None) == EINVAL
    assert pt(al, al, 10, (1 << 31) + 1, al, None) == ERANGE
    at = lib.pulse_apply_patch_tiled
    at.argtypes = [V, I64, V, V, V, I64, V, V]
    assert at(mis, 100, al, al, al, 10, al, None) == EALIGN and at(al, 100, al, al, None, 10, al, None) == EINVAL
    app = lib.lz4_decode_apply
    app.argtypes = dec.argtypes
    assert app(al, 10, al, al, 2, 65536, 70000, al, 2, al, al, 1 << 20, None) == EINVAL     # mode
    assert app(al, 10, al, al, 2, 65536, 70000, None, 1, al, al, 1 << 20, None) == EINVAL   # no dst
    assert app(al, 10, al, al, 2, 65536, 70000, mis, 1, al, al, 1 << 20, None) == EALIGN
    assert app(al, 10, al, al, 2, 65536, 70000, al, 1, al, al, 16, None) == EWORKSPACE
    q = lib.fp8_block_quant
    q.argtypes = [V, V, ctypes.c_int32, I64, I64, V, V, V, V]
    ptrs = (V * 1)(0x10000)
    rows = (I64 * 1)(128)
    assert q(ctypes.cast(ptrs, V), ctypes.cast(rows, V), 1, 100, 1, None, al, al, None) == EINVAL  # cols % 8
    assert q(ctypes.cast(ptrs, V), ctypes.cast(rows, V), 9, 128, 1, None, al, al, None) == EINVAL  # nsrc
    mptrs = (V * 1)(0x10002)
    assert q(ctypes.cast(mptrs, V), ctypes.cast(rows, V), 1, 128, 1, None, al, al, None) == EALIGN
    ap = lib.pulse_apply_patch
    ap.argtypes = [V, I64, V, V, V, I64, V, V]
    assert ap(al, 10, None, al, al, 5, al, None) == EINVAL
    assert ap(al, 1 << 31, al, al, al, 5, al, None) == ERANGE
    x = lib.xor_mask_apply
    x.argtypes = [V, V, I64, V]
    assert x(mis, al, 100, None) == EALIGN and x(al, al, -1, None) == EINVAL


def test_next_rows_argument_errors(lib):
    al = V(0x10000)
    mis = V(0x10002)
    SZ = ctypes.c_size_t
    d = lib.fp8_view_delta
    d.argtypes = [V, V, I64, V, V, I64, V, V, I64, V, V, V, I64, V, V, V, SZ, V]
    args = [al, al, 1000, al, al, 10, al, al, 1000, al, al, al, 10, al, al, al, 1 << 20, None]
    assert d(*args[:2], 0, *args[3:]) == EINVAL                                  # empty codes
    assert d(None, *args[1:]) == EINVAL
    assert d(mis, *args[1:]) == EALIGN
    assert d(*args[:2], 1 << 31, *args[3:]) == ERANGE
    assert d(*args[:16], 8, None) == EWORKSPACE
    ap = lib.fp8_view_apply
    ap.argtypes = [V, I64, V, I64, V, V, V, I64, V, V, V, I64, V, V]
    assert ap(al, 10, al, 1, al, al, al, -1, al, al, al, 1, al, None) == EINVAL
    g = lib.pulse_loco_gate
    g.argtypes = [V, V, V, I64, V, V, I64, V, V, V, SZ, V]
    assert g(al, al, None, 100, al, al, 10, al, al, al, 1 << 20, None) == EINVAL        # resid required
    assert g(al, mis, al, 100, al, al, 10, al, al, al, 1 << 20, None) == EALIGN
    assert g(al, al, al, 1 << 31, al, al, 10, al, al, al, 1 << 40, None) == ERANGE
    assert g(al, al, al, 100000, al, al, 10, al, al, al, 64, None) == EWORKSPACE
    acc = lib.pulse_loco_accumulate
    acc.argtypes = [V, I64, V, V, V, I64, V, V]
    assert acc(al, 10, None, al, al, 5, al, None) == EINVAL
    ws = lib.pulse_workspace_bytes
    assert ws(5, 16384, 0) == 256 + 8 and ws(6, 16385, 0) == 256 + 16


def test_patch_pack_argument_errors(lib):
    al = V(0x10000)
    mis = V(0x10008)
    pb = lib.patch_packed_bytes
    pb.argtypes = [I64]
    pb.restype = I64
    assert pb(0) == 0 and pb(1) == 6 * 65536 and pb(65536) == 6 * 65536 and pb(65537) == 12 * 65536
    pk = lib.patch_pack
    pk.argtypes = [V, V, I64, V, V]
    assert pk(None, al, 10, al, None) == EINVAL
    assert pk(al, mis, 10, al, None) == EALIGN
    assert pk(al, al, (1 << 31) + 1, al, None) == ERANGE
    up = lib.patch_unpack
    up.argtypes = [V, I64, V, V, V, V, ctypes.c_size_t, V]
    assert up(al, 10, al, al, None, al, 1 << 20, None) == EINVAL
    assert up(al, 100000, al, al, al, al, 8, None) == EWORKSPACE
    ws = lib.pulse_workspace_bytes
    assert ws(7, 65536, 0) == 256 + 8 and ws(7, 65537, 0) == 256 + 16


def test_segment_tiles_and_list_call_errors(lib):
    st = lib.pulse_segment_tiles
    st.argtypes = [V, ctypes.c_int32, V, V]
    st.restype = I64
    n = (I64 * 4)(1, 16384, 16385, 40000)
    tile0 = (I64 * 4)()
    tseg = (ctypes.c_uint32 * 8)()
    assert st(ctypes.cast(n, V), 4, ctypes.cast(tile0, V), ctypes.cast(tseg, V)) == 1 + 1 + 2 + 3
    assert list(tile0) == [0, 1, 2, 4] and list(tseg)[:7] == [0, 1, 2, 2, 3, 3, 3]
    bad = (I64 * 2)(10, 0)
    assert st(ctypes.cast(bad, V), 2, None, None) == ERANGE
    cd = lib.pulse_cast_diff_segments
    al = V(0x10000)
    cd.argtypes = [V, ctypes.c_int32, V, I64, V, V, I64, V, V, V, ctypes.c_size_t, ctypes.c_int32, V]
    assert cd(al, 2, al, 1, al, al, 10, al, al, al, 1 << 20, 0, None) == EINVAL      # fewer tiles than tensors
    assert cd(al, 2, al, 5, al, al, 10, al, al, al, 16, 0, None) == EWORKSPACE
    assert cd(al, 2, al, 5, al, al, 10, al, al, al, 1 << 20, 2, None) == EINVAL      # with_new 0/1
    ap = lib.pulse_apply_patch_segments
    ap.argtypes = [V, ctypes.c_int32, V, V, V, I64, V, V]
    assert ap(al, 0, al, al, al, 10, al, None) == EINVAL


def test_receiver_pass_plan_and_argument_errors(lib):
    """pulse_apply_quant_plan checks every group and that the sources tile the
    view before it copies anything; pulse_apply_quant checks its arguments."""
    import sparse_delta_codec_amd as pk  # the binding's layout of pulse_aq_group
    al = V(0x10000)
    mis = V(0x10002)
    pb = lib.pulse_apply_quant_plan_bytes
    pb.argtypes, pb.restype = [ctypes.c_int32], I64
    assert pb(0) == 0 and pb(1) > 0 and pb(9) > pb(8) + ctypes.sizeof(pk._AQGroup)
    assert ctypes.sizeof(pk._AQGroup) == 4 * 8 + 4 * 8 + 4 + 4 + 8 + 8 + 8
    mk = lib.pulse_apply_quant_plan
    mk.argtypes = [V, ctypes.c_int32, I64, V, I64, V]
    nb = I64(0)

    def plan(groups, n, plan_bytes=1 << 20, ptr=al):
        arr = (pk._AQGroup * len(groups))()
        for g, (srcs, cols, quant) in enumerate(groups):
            for i, (off, rows) in enumerate(srcs):
                arr[g].src_offset[i], arr[g].rows[i] = off, rows
            arr[g].nsrc, arr[g].cols, arr[g].quantise = len(srcs), cols, quant
            arr[g].codes, arr[g].scales = (0x20000, 0x30000) if quant else (None, None)
        return mk(ctypes.cast(arr, V), len(groups), n, ptr, plan_bytes, ctypes.byref(nb))

    qkv = ([(0, 4), (512, 2), (768, 2)], 128, 1)    # 1024 elements in three sources
    mid = ([(1024, 1)], 16, 0)
    assert plan([qkv], 1040) == EINVAL                                  # [1024, 1040) not covered (gap)
    assert plan([qkv, mid], 1032) == EINVAL                             # past the view
    assert plan([qkv, mid, ([(1032, 1)], 8, 0)], 1040) == EINVAL        # overlap
    assert plan([([(0, 4), (520, 2), (776, 2)], 128, 1), ([(1032, 1)], 16, 0)], 1048) == EINVAL  # gap in a stack
    assert plan([([(0, 1)], 8, 0), ([(12, 1)], 8, 0)], 20) == EALIGN   # offset % 8
    assert plan([([(0, 1)], 1036, 0), ([(1036, 1)], 4, 0)], 1040) == EINVAL    # cols % 8
    assert plan([([(0, 1)], 1028, 0), ([(1028, 1)], 12, 0)], 1040) == EINVAL   # cols % 8
    assert plan([([(0, 1)], 1024, 0), ([(1024, 1)], 16, 0)], 1040, ptr=mis) == EALIGN
    assert plan([([(0, 1)], 4, 0)], 4) == EINVAL                         # cols 4
    assert plan([qkv, mid], 1040, plan_bytes=16) == EWORKSPACE
    assert plan([qkv, mid], 1 << 31) == ERANGE
    assert plan([([(0, 0)], 8, 0)], 8) == EINVAL                        # no rows
    assert mk(None, 1, 8, al, 1 << 20, ctypes.byref(nb)) == EINVAL
    arr = (pk._AQGroup * 1)()
    arr[0].src_offset[0], arr[0].rows[0], arr[0].nsrc, arr[0].cols, arr[0].quantise = 0, 1, 1, 8, 1
    assert mk(ctypes.cast(arr, V), 1, 8, al, 1 << 20, ctypes.byref(nb)) == EINVAL   # quantised, no outputs
    arr[0].codes, arr[0].scales = 0x20004, 0x30000
    assert mk(ctypes.cast(arr, V), 1, 8, al, 1 << 20, ctypes.byref(nb)) == EALIGN   # codes 8-byte aligned
    arr[0].quantise = 2
    assert mk(ctypes.cast(arr, V), 1, 8, al, 1 << 20, ctypes.byref(nb)) == EINVAL
    arr[0].quantise, arr[0].nsrc = 0, 5
    assert mk(ctypes.cast(arr, V), 1, 8, al, 1 << 20, ctypes.byref(nb)) == EINVAL   # five sources
    aq = lib.pulse_apply_quant
    aq.argtypes = [V, I64, V, V, V, I64, V, I64, V, V, ctypes.c_size_t, V]
    args = [al, 1000, al, al, al, 10, al, 3, al, al, 1 << 20, None]
    assert aq(None, *args[1:]) == EINVAL
    assert aq(*args[:6], None, *args[7:]) == EINVAL                    # no plan
    assert aq(*args[:7], 0, *args[8:]) == EINVAL                       # no blocks
    assert aq(*args[:5], 0, *args[6:]) == EINVAL                       # empty patch buffers
    assert aq(mis, *args[1:]) == EALIGN and aq(*args[:6], mis, *args[7:]) == EALIGN
    assert aq(al, 1 << 31, *args[2:]) == ERANGE
    assert aq(*args[:10], 16, None) == EWORKSPACE and aq(*args[:9], None, 1 << 20, None) == EWORKSPACE


def test_noalloc_entry_rejects_oversize_calls_before_any_launch(lib):
    """The allocation-free fused pass: sizes past its static scratch return
    PULSE_ERANGE before anything is enqueued; the header states the scratch
    size the library holds."""
    import sparse_delta_codec_amd as pk
    text = open(HEADER).read()
    m = re.search(r"#define PULSE_NOALLOC_SCRATCH_BYTES \((.*)\)", text)
    assert m and eval(m.group(1)) == pk.PULSE_NOALLOC_SCRATCH_BYTES == 256 + 2 * 262144 * 8
    f = lib.pulse_cast_diff_lz4_noalloc
    f.argtypes = [V, V, V, V, V, I64, V, V, I64, ctypes.c_int32, V, I64, V, V, V, V, V]
    al, mis = V(0x10000), V(0x10002)
    # 2^34 elements without a patch: 524288 blocks of 64 KiB, twice the scratch's 262144
    assert f(al, al, al, None, None, 0, None, None, 1 << 34, 65536, al, 10, al, al, al, al, None) == ERANGE
    # 2^32 + 1 elements at 32 KiB blocks: one block past the scratch
    assert f(al, al, al, None, None, 0, None, None, (1 << 32) + 1, 32768, al, 10, al, al, al, al, None) == ERANGE
    assert f(al, al, al, al, al, 10, al, None, 1 << 31, 65536, al, 10, al, al, al, al, None) == ERANGE  # int32 idx
    assert f(mis, al, al, None, None, 0, None, None, 1000, 65536, al, 10, al, al, al, al, None) == EALIGN
    assert f(al, al, al, None, None, 0, None, None, 1000, 1000, al, 10, al, al, al, al, None) == EINVAL
    assert f(al, al, al, al, None, 10, al, None, 1000, 65536, al, 10, al, al, al, al, None) == EINVAL  # partial
