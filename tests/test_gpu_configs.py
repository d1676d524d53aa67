"""Full-size parity of the configured workloads on the GPU (C2-C5).

At these sizes the oracle cannot redo the whole job, so each test checks
  * properties that hold at any size, over every element: the patched old view
    equals the new cast bit for bit, decode(encode(mask)) XOR old == new, the
    20-step chain equals the direct cast of the last masters;
  * sampled outputs against the oracle, element by element: cast+diff+compact
    on windows of the weights, LZ4 blocks byte for byte, FP8 codes and scales of
    whole experts and of 128-row bands of the stacked q/k/v.
C2 makes the calls bench.py times, with its chunking; the other configurations
use the single-purpose calls.  Every input comes from
workload/ (seeded); only host copies of the sampled windows go to the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from bench import build_plan

pytestmark = pytest.mark.gpu

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise  # on a GPU machine the HIP library must be there
    pulse = None

WIN = 65536
BLOCK = 65536


def say(msg):
    print(f"[cfg] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _fresh_memory():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def h16(t):
    return t.cpu().numpy().view(np.uint16)


def views_equal(a, b, chunk=1 << 30):
    for s in range(0, a.numel(), chunk):
        if not torch.equal(a[s:s + chunk], b[s:s + chunk]):
            return False
    return True


def check_patch_window(w, b_old, idx, val, count, o, win=WIN):
    """Oracle cast+diff+compact of the window [o, o+win) of one call's input
    against the GPU patch entries that fall in it."""
    win = min(win, w.numel() - o)
    ref = oracle.cast_diff(w[o:o + win].cpu().numpy(), h16(b_old[o:o + win]), want_mask=False)
    ii = idx[:count]
    bounds = torch.tensor([o, o + win], dtype=torch.int32, device=ii.device)
    lo, hi = (int(x) for x in torch.searchsorted(ii, bounds).cpu())
    assert hi - lo == ref["count"], (o, hi - lo, ref["count"])
    assert np.array_equal(ii[lo:hi].cpu().numpy() - o, ref["idx"])
    assert np.array_equal(h16(val[lo:hi]), ref["val"])
    return ref["count"]


def new_ws(op, n, aux=0):
    return pulse.workspace(op, n, aux, "cuda")


# ---------------------------------------------------------------------------
def test_c2_qwen32b_encode_and_apply_full_size():
    """C2: the whole Qwen2.5-32B-shaped set, one step, with bench.py's calls per
    chunk: the fused sender pass (pulse_cast_diff_lz4: new view, patch, LZ4
    blocks of the mask) and the receiver's pass (pulse_apply_quant over the
    chunk's FP8 groups and patched-only tensors).  Every element: the patched
    old view equals the new view.  Sampled against the oracle: windows of the
    patch, the first LZ4 block of every chunk, and 128-row bands of the FP8
    codes and scales of two groups per chunk."""
    from bench import quant_groups, receiver_plan
    dev = torch.device("cuda")
    rng = np.random.default_rng(22)
    specs = workload.qwen25_32b_specs()
    n = workload.total_numel(specs)
    chunks, offs = build_plan(specs)
    max_chunk = max(e - s for s, e, _ in chunks)
    W = torch.empty(n, dtype=torch.float32, device=dev)
    b = torch.empty(n, dtype=torch.int16, device=dev)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    for ti, s in enumerate(specs):
        w = W[offs[ti]: offs[ti] + s.numel]
        workload.fill_init(w, 2, ti, s.kind)
        pulse.pulse_cast_diff(w, b_new=b[offs[ti]: offs[ti] + s.numel])
        workload.apply_step(w, 2, ti, 1, tmp=tmp)
    del tmp, w
    torch.cuda.synchronize()
    say(f"C2 generated: {n} params")
    cap = int(max_chunk * 0.125)
    stage = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    val = torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    nbmax = (2 * max_chunk + BLOCK - 1) // BLOCK
    pcap = int(2 * max_chunk * 0.35)
    payload = torch.empty(pcap, dtype=torch.uint8, device=dev)
    csizes = torch.empty(nbmax, dtype=torch.int32, device=dev)
    coffs = torch.empty(nbmax, dtype=torch.int64, device=dev)
    ctotal = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_fz = new_ws(pulse.PULSE_OP_CAST_DIFF_LZ4, max_chunk, BLOCK)
    ws_aq = new_ws(pulse.PULSE_OP_APPLY_QUANT, max_chunk)
    codes = torch.empty(max_chunk, dtype=torch.uint8, device=dev)
    scales = torch.empty(max_chunk // 16384 + 4096, dtype=torch.float32, device=dev)
    total = checked = bands = 0
    for ci, ch in enumerate(chunks):
        s0, e0, tids = ch
        m = e0 - s0
        pulse.pulse_cast_diff_lz4(W[s0:e0], b[s0:e0], stage[:m], idx, val, cnt, payload, csizes, coffs, ctotal, st,
                                  ws_fz)
        count = int(cnt.item())
        assert int(st.item()) == 0 and 0 < count <= cap
        for o in [0, m - WIN] + [int(x) for x in rng.integers(0, m - WIN, 2)]:
            checked += check_patch_window(W[s0:e0], b[s0:e0], idx, val, count, o)
        # the first mask block, byte for byte
        old0, new0 = h16(b[s0:s0 + BLOCK // 2]), h16(stage[:BLOCK // 2])
        enc = oracle.lz4_encode_blocks(old0, BLOCK, src_xor=new0)
        sz = int(csizes[0].item())
        assert int(coffs[0].item()) == 0 and sz == enc["total"]
        assert np.array_equal(payload[:sz].cpu().numpy(), enc["payload"])
        # the receiver's pass
        plan = [(g, sum(specs[i].shape[0] for i in g), specs[g[0]].shape[1]) for g in quant_groups(specs, tids)]
        aq = receiver_plan(pulse, specs, offs, ch, plan, codes, scales, dev)
        pulse.pulse_apply_quant(b[s0:e0], idx, val, cnt, aq, st, ws_aq, max_count=count)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert views_equal(b[s0:e0], stage[:m]), f"chunk {ci}: patched old view != new view"
        # two groups, one 128-row band each, against the oracle's quantisation
        co = so = 0
        picks = set(int(x) for x in rng.integers(0, len(plan), 2))
        for gi, (g, rows, cols) in enumerate(plan):
            nbc = (cols + 127) // 128
            if gi in picks:
                br = int(rng.integers(0, (rows + 127) // 128))
                r0, r1 = br * 128, min(rows, br * 128 + 128)
                stack = torch.cat([b[offs[i]: offs[i] + specs[i].numel].view(specs[i].shape) for i in g])
                band = h16(stack[r0:r1].contiguous().view(-1)).reshape(r1 - r0, cols)
                rc, rs = oracle.fp8_block_quant([band])
                assert np.array_equal(codes[co + r0 * cols: co + r1 * cols].cpu().numpy(), rc.reshape(-1)), (ci, gi, br)
                got_s = scales[so + br * nbc: so + (br + 1) * nbc].cpu().numpy().view(np.uint32)
                assert np.array_equal(got_s, rs.reshape(-1).view(np.uint32)), (ci, gi, br)
                bands += 1
                del stack
            co += rows * cols
            so += ((rows + 127) // 128) * nbc
        del aq
        total += count
    say(f"C2: {total} changed ({total / n:.4%}); {checked} patch entries, {len(chunks)} LZ4 blocks and "
        f"{bands} FP8 bands checked against the oracle")
    assert 0.07 < total / n < 0.09


def test_c3_llama8b_twenty_step_chain_full_size():
    """C3: the Llama-3-8B-shaped set over 20 chained steps; after every step the
    receiver's view (patched cumulatively) equals the direct cast of the current
    masters, checked everywhere by the library's cast and on windows by the oracle."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(33)
    specs = workload.llama3_8b_specs()
    n = workload.total_numel(specs)
    chunks, offs = build_plan(specs)
    max_chunk = max(e - s for s, e, _ in chunks)
    W = torch.empty(n, dtype=torch.float32, device=dev)
    prev = torch.empty(n, dtype=torch.int16, device=dev)
    for ti, s in enumerate(specs):
        w = W[offs[ti]: offs[ti] + s.numel]
        workload.fill_init(w, 3, ti, s.kind)
        pulse.pulse_cast_diff(w, b_new=prev[offs[ti]: offs[ti] + s.numel])
    recv = prev.clone()
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    cap = int(max_chunk * 0.125)
    stage = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    val = torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = new_ws(pulse.PULSE_OP_CAST_DIFF, max_chunk)
    for step in range(1, 21):
        for ti, s in enumerate(specs):
            workload.apply_step(W[offs[ti]: offs[ti] + s.numel], 3, ti, step, tmp=tmp)
        changed = 0
        for ci, (s0, e0, _) in enumerate(chunks):
            m = e0 - s0
            pulse.pulse_cast_diff(W[s0:e0], prev[s0:e0], stage[:m], None, idx, val, cnt, st, ws)
            count = int(cnt.item())
            assert int(st.item()) == 0 and count <= cap
            if ci == step % len(chunks):
                o = int(rng.integers(0, m - WIN))
                check_patch_window(W[s0:e0], prev[s0:e0], idx, val, count, o)
            pulse.pulse_apply_patch(recv[s0:e0], idx, val, cnt, st, max_count=max(count, 1))
            prev[s0:e0].copy_(stage[:m])
            changed += count
        assert int(st.item()) == 0
        # everywhere: receiver == direct cast of the step's masters (the sender's new view)
        assert views_equal(recv, prev), f"step {step}: chained view drifted"
        # windows: the direct cast by the oracle
        for o in rng.integers(0, n - WIN, 4):
            o = int(o)
            assert np.array_equal(h16(recv[o:o + WIN]), oracle.cast_bf16(W[o:o + WIN].cpu().numpy())), (step, o)
        say(f"C3 step {step}: {changed} changed ({changed / n:.4%})")


def test_c4_xor_mask_lz4_round_trip_full_size():
    """C4: the first 16e9 elements of the C2 set; the XOR mask of old and new
    views LZ4-encoded in 64 KiB blocks (one call), decoded and XORed into the
    old view in place, which must then equal the new view.  Sampled blocks (and
    the short last block) must match the oracle's encoding byte for byte."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(44)
    specs = workload.qwen25_32b_specs()
    n = workload.C4_NUMEL
    old = torch.empty(n, dtype=torch.int16, device=dev)
    new = torch.empty(n, dtype=torch.int16, device=dev)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    tmp2 = torch.empty_like(tmp)
    o = 0
    for ti, s in enumerate(specs):
        if o >= n:
            break
        k = min(s.numel, n - o)
        w = tmp[: s.numel]
        workload.fill_init(w, 2, ti, s.kind)
        pulse.pulse_cast_diff(w[:k], b_new=old[o:o + k])
        workload.apply_step(w, 2, ti, 1, tmp=tmp2)
        pulse.pulse_cast_diff(w[:k], b_new=new[o:o + k])
        o += k
    del tmp, tmp2
    nbytes = 2 * n
    nb = (nbytes + BLOCK - 1) // BLOCK
    assert nb == 488282
    payload = torch.empty(int(nbytes * 0.35), dtype=torch.uint8, device=dev)
    sizes = torch.empty(nb, dtype=torch.int32, device=dev)
    offsets = torch.empty(nb, dtype=torch.int64, device=dev)
    total = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = new_ws(pulse.PULSE_OP_LZ4_ENCODE, nbytes, BLOCK)
    pulse.lz4_encode_blocks(old, payload, sizes, offsets, total, st, ws, src_xor=new)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    tot = int(total.item())
    szs = sizes.cpu().numpy().view(np.uint32)
    offs = offsets.cpu().numpy().view(np.uint64)
    assert tot == int(szs.sum(dtype=np.uint64))
    assert np.array_equal(offs[1:], np.cumsum(szs[:-1], dtype=np.uint64)) and offs[0] == 0
    say(f"C4: mask {nbytes} B -> {tot} B ({tot / nbytes:.2%}) in {nb} blocks")
    old_u8 = old.view(torch.uint8)
    new_u8 = new.view(torch.uint8)
    for blk in list(rng.integers(0, nb - 1, 24)) + [0, nb - 1]:
        blk = int(blk)
        lo, hi = blk * BLOCK, min(nbytes, (blk + 1) * BLOCK)
        ref = oracle.lz4_encode_blocks(old_u8[lo:hi].cpu().numpy(), BLOCK, src_xor=new_u8[lo:hi].cpu().numpy())
        got = payload[int(offs[blk]): int(offs[blk]) + int(szs[blk])].cpu().numpy()
        assert int(szs[blk]) == ref["total"] and np.array_equal(got, ref["payload"]), blk
    assert int(szs[-1]) == oracle.lz4_encode_blocks(
        old_u8[(nb - 1) * BLOCK:].cpu().numpy(), BLOCK, src_xor=new_u8[(nb - 1) * BLOCK:].cpu().numpy())["total"]
    # decode + XOR into the old view (in place): it becomes the new view
    dws = new_ws(pulse.PULSE_OP_LZ4_DECODE, nb, tot)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    pulse.lz4_decode_blocks(payload, offsets, sizes, old, st, dws, mode=1, payload_bytes=tot)
    ev[1].record()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert views_equal(old, new), "decode + XOR did not rebuild the new view"
    ms = ev[0].elapsed_time(ev[1])
    say(f"C4: decode+XOR {ms:.1f} ms, {nbytes / ms / 1e6:.1f} GB/s of mask")


def test_c5_kimi_layer_apply_and_fp8_full_size():
    """C5: the Kimi-K2-shaped MoE layer share; per tensor cast+diff+compact and
    patch apply (the patched view equals the new cast), then [gate; up] per
    expert, down, and [q; k; v] quantised to E4M3 with 128x128 FP32 scales.
    Sampled experts and 128-row bands of q/k/v match the oracle bit for bit."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(55)
    specs = workload.kimi_k2_layer_specs()
    n = workload.total_numel(specs)
    offs = np.concatenate([[0], np.cumsum([s.numel for s in specs])]).astype(np.int64)
    b = torch.empty(n, dtype=torch.int16, device=dev)
    maxn = max(s.numel for s in specs)
    w = torch.empty(maxn, dtype=torch.float32, device=dev)
    tmp = torch.empty(maxn, dtype=torch.float32, device=dev)
    stage = torch.empty(maxn, dtype=torch.int16, device=dev)
    cap = maxn // 4
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    val = torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = new_ws(pulse.PULSE_OP_CAST_DIFF, maxn)
    sample_t = {0, 2, 3 * 191 + 1, 3 * 383 + 2, len(specs) - 3, len(specs) - 1}
    for ti, s in enumerate(specs):
        k = s.numel
        bt = b[int(offs[ti]): int(offs[ti]) + k]
        wt = w[:k]
        workload.fill_init(wt, 5, ti, s.kind)
        pulse.pulse_cast_diff(wt, b_new=bt)
        workload.apply_step(wt, 5, ti, 1, tmp=tmp)
        pulse.pulse_cast_diff(wt, bt, stage[:k], None, idx, val, cnt, st, ws)
        if ti in sample_t:
            check_patch_window(wt, bt, idx, val, int(cnt.item()), int(rng.integers(0, k - WIN)))
        pulse.pulse_apply_patch(bt, idx, val, cnt, st)
        if ti in sample_t or ti % 97 == 0:
            assert torch.equal(bt, stage[:k]), f"tensor {s.name}: patched view != new cast"
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    say(f"C5: {n} params patched")

    E, H, F = 384, 7168, 2048
    tstride = 3 * F * H  # one expert's gate, up, down

    def expert_view(which, rows, cols):
        base = b[int(offs[which]):]
        return torch.as_strided(base, (E, rows, cols), (tstride, cols, 1))

    # [gate; up] per expert, one launch for all experts
    gate, up = expert_view(0, F, H), expert_view(1, F, H)
    R = 2 * F
    codes = torch.empty(E * R * H, dtype=torch.uint8, device=dev)
    scales = torch.empty(E * (R // 128) * (H // 128), dtype=torch.float32, device=dev)
    pulse.fp8_block_quant([gate, up], codes, scales, batch=E)
    torch.cuda.synchronize()
    for e in (0, int(rng.integers(1, E - 1)), E - 1):
        g = h16(gate[e].contiguous()).reshape(F, H)
        u = h16(up[e].contiguous()).reshape(F, H)
        rc, rs = oracle.fp8_block_quant([g, u])
        assert np.array_equal(codes[e * R * H:(e + 1) * R * H].cpu().numpy(), rc.reshape(-1)), e
        nsc = (R // 128) * (H // 128)
        assert np.array_equal(scales[e * nsc:(e + 1) * nsc].cpu().numpy(), rs.reshape(-1)), e
    # down per expert
    down = expert_view(2, H, F)
    pulse.fp8_block_quant([down], codes, scales, batch=E)
    torch.cuda.synchronize()
    for e in (0, E - 1):
        d = h16(down[e].contiguous()).reshape(H, F)
        rc, rs = oracle.fp8_block_quant([d])
        assert np.array_equal(codes[e * H * F:(e + 1) * H * F].cpu().numpy(), rc.reshape(-1)), e
        nsc = (H // 128) * (F // 128)
        assert np.array_equal(scales[e * nsc:(e + 1) * nsc].cpu().numpy(), rs.reshape(-1)), e
    # [q; k; v]
    qi = len(specs) - 3
    qkv = [b[int(offs[qi + j]): int(offs[qi + j + 1])].view(8192, H) for j in range(3)]
    RQ = 3 * 8192
    pulse.fp8_block_quant(qkv, codes, scales)
    torch.cuda.synchronize()
    ncb = H // 128
    for r0 in (0, 8192 + 128 * int(rng.integers(0, 64)), RQ - 128):
        src = qkv[r0 // 8192][(r0 % 8192):(r0 % 8192) + 128]
        rc, rs = oracle.fp8_block_quant([h16(src.contiguous()).reshape(128, H)])
        assert np.array_equal(codes[r0 * H:(r0 + 128) * H].cpu().numpy(), rc.reshape(-1)), r0
        assert np.array_equal(scales[(r0 // 128) * ncb:(r0 // 128 + 1) * ncb].cpu().numpy(), rs.reshape(-1)), r0
    say("C5: FP8 experts and q/k/v bands match the oracle")
