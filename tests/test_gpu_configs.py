"""Full-size parity of the configured workloads on the GPU (C2-C5), every
element against the oracle.

Each test generates its workload on the GPU (workload/, seeded), runs the
library's calls on it, copies the inputs and every output to the host and
compares them, element by element, with the oracle run on those host copies
(tests/fullsize.py spreads the oracle's single-threaded calls over the host
threads, piece by independent piece).  The oracle computes its own old views
from the host masters, so no GPU result feeds an expected value:

  C2  Qwen2.5-32B-shaped set, one step, with bench.py's calls per chunk (the
      fused sender pass, then the receiver's pass): the old view, the new
      view, the count and every patch entry, every LZ4 block (sizes, offsets,
      total, payload bytes), the receiver's patched view, every FP8 code and
      scale of every stacked group.  Six tests of three chunks each.
  C3  (tests/test_gpu_config_c3.py) the 20-step chain.
  C4  the first 16e9 elements of the C2 set: both views, every block of the
      LZ4-encoded mask, and the view rebuilt by decode + XOR in place.
  C5  Kimi-K2-shaped MoE layer share: per tensor the old view, new view,
      patch and patched view; every FP8 code and scale of [gate; up] and down
      for all 384 experts and of [q; k; v].
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from bench import build_plan, quant_groups, receiver_plan
from tests import fullsize as fs

pytestmark = pytest.mark.gpu

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise  # on a GPU machine the HIP library must be there
    pulse = None

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


def new_ws(op, n, aux=0):
    return pulse.workspace(op, n, aux, "cuda")


def check_view_gpu(t, ref_h, slot, what, step=1 << 28):
    """A GPU view against a host array, in slices through one pinned slot."""
    for a in range(0, t.numel(), step):
        b = min(t.numel(), a + step)
        fs.check_equal(fs.to_host(t[a:b], slot), ref_h[a:b], f"{what} [{a}:{b})")


# ---------------------------------------------------------------------------
C2_PARTS = 6


@pytest.mark.parametrize("part", range(C2_PARTS))
def test_c2_qwen32b_every_element(part):
    """C2, chunks 3 part .. 3 part + 2 of bench.py's 18: the fused sender pass
    (pulse_cast_diff_lz4) and the receiver's pass (pulse_apply_quant), every
    output against the oracle's cast, cast + diff + compaction, canonical LZ4
    of old ^ new, apply, and per-group FP8 quantisation of the patched view."""
    dev = torch.device("cuda")
    specs = workload.qwen25_32b_specs()
    chunks, offs = build_plan(specs)
    per = (len(chunks) + C2_PARTS - 1) // C2_PARTS
    sel = list(range(part * per, min(len(chunks), (part + 1) * per)))
    max_chunk = max(chunks[ci][1] - chunks[ci][0] for ci in sel)
    W = torch.empty(max_chunk, dtype=torch.float32, device=dev)
    bo = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    stage = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    tmp = torch.empty(max(specs[i].numel for ci in sel for i in chunks[ci][2]), dtype=torch.float32, device=dev)
    cap = int(max_chunk * 0.125)
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
    for ci in sel:
        s0, e0, tids = chunks[ci]
        m = e0 - s0
        Wc, boc = W[:m], bo[:m]
        # the old view: the library's cast of the initial masters (as in bench.py)
        for ti in tids:
            a, b = offs[ti] - s0, offs[ti] - s0 + specs[ti].numel
            workload.fill_init(Wc[a:b], 2, ti, specs[ti].kind)
            pulse.pulse_cast_diff(Wc[a:b], b_new=boc[a:b])
        ref_old = fs.oracle_cast(fs.to_host(Wc, "w"))
        fs.check_equal(fs.to_host(boc, "v"), ref_old, f"C2 chunk {ci}: old view")
        for ti in tids:
            a, b = offs[ti] - s0, offs[ti] - s0 + specs[ti].numel
            workload.apply_step(Wc[a:b], 2, ti, 1, tmp=tmp)
        w1_h = fs.to_host(Wc, "w")
        # the sender: bench.py's fused pass
        pulse.pulse_cast_diff_lz4(Wc, boc, stage[:m], idx, val, cnt, payload, csizes, coffs, ctotal, st, ws_fz)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        count, total = int(cnt.item()), int(ctotal.item())
        assert 0 < count <= cap
        ref = fs.OraclePatch(w1_h, ref_old)
        fs.check_equal(fs.to_host(stage[:m], "v"), ref.b_new, f"C2 chunk {ci}: new view")
        ref.check(count, fs.to_host(idx[:count], "idx"), fs.to_host(val[:count], "val"), f"C2 chunk {ci}")
        nb = (2 * m + BLOCK - 1) // BLOCK
        fs.check_lz4(ref_old, ref.b_new, fs.to_host(csizes[:nb], "sz", np.uint32),
                     fs.to_host(coffs[:nb], "of", np.uint64), total, fs.to_host(payload[:total], "pl"),
                     f"C2 chunk {ci}")
        # the receiver: bench.py's pass over the old view, in place
        plan = [(g, sum(specs[i].shape[0] for i in g), specs[g[0]].shape[1]) for g in quant_groups(specs, tids)]
        aq = receiver_plan(pulse, specs, offs, chunks[ci], plan, codes, scales, dev)
        pulse.pulse_apply_quant(boc, idx, val, cnt, aq, st, ws_aq, max_count=count)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        recv = ref.applied(ref_old)
        fs.check_equal(fs.to_host(boc, "v"), recv, f"C2 chunk {ci}: receiver view")
        nq = sum(r * c for _, r, c in plan)
        ns = sum(((r + 127) // 128) * ((c + 127) // 128) for _, r, c in plan)
        codes_h = fs.to_host(codes[:nq], "codes")
        scales_h = fs.to_host(scales[:ns], "scales")
        co = so = 0
        for (g, rows, cols) in plan:
            nsc = ((rows + 127) // 128) * ((cols + 127) // 128)
            fs.check_fp8(recv, [(offs[i] - s0, specs[i].shape[0]) for i in g], cols, codes_h[co:co + rows * cols],
                         scales_h[so:so + nsc], f"C2 chunk {ci} group {specs[g[0]].name}")
            co += rows * cols
            so += nsc
        del aq
        say(f"C2 chunk {ci}: {m} params, {count} changed ({count / m:.4%}), {total} LZ4 bytes, "
            f"{len(plan)} FP8 groups: every element equals the oracle")
    fs.release()


# ---------------------------------------------------------------------------
def test_c4_xor_mask_lz4_every_element():
    """C4: the first 16e9 elements of the C2 set; the XOR mask of the old and
    new views LZ4-encoded in 64 KiB blocks (one call), decoded and XORed into
    the old view in place.  Both views, every block of the encoding and the
    rebuilt view against the oracle (its casts of the host masters, its
    canonical encoding of their XOR)."""
    dev = torch.device("cuda")
    specs = workload.qwen25_32b_specs()
    n = workload.C4_NUMEL
    old = torch.empty(n, dtype=torch.int16, device=dev)
    new = torch.empty(n, dtype=torch.int16, device=dev)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    tmp2 = torch.empty_like(tmp)
    ref_old = np.empty(n, np.uint16)
    ref_new = np.empty(n, np.uint16)
    o = 0
    for ti, s in enumerate(specs):
        if o >= n:
            break
        k = min(s.numel, n - o)
        w = tmp[: s.numel]
        workload.fill_init(w, 2, ti, s.kind)
        pulse.pulse_cast_diff(w[:k], b_new=old[o:o + k])
        fs.oracle_cast(fs.to_host(w[:k], "w"), out=ref_old[o:o + k])
        workload.apply_step(w, 2, ti, 1, tmp=tmp2)
        pulse.pulse_cast_diff(w[:k], b_new=new[o:o + k])
        fs.oracle_cast(fs.to_host(w[:k], "w"), out=ref_new[o:o + k])
        o += k
    del tmp, tmp2
    check_view_gpu(old, ref_old, "v", "C4 old view")
    check_view_gpu(new, ref_new, "v", "C4 new view")
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
    fs.check_lz4(ref_old, ref_new, fs.to_host(sizes, "sz", np.uint32), fs.to_host(offsets, "of", np.uint64), tot,
                 fs.to_host(payload[:tot], "pl"), "C4")
    say(f"C4: mask {nbytes} B -> {tot} B ({tot / nbytes:.2%}) in {nb} blocks, every block equals the oracle's")
    dws = new_ws(pulse.PULSE_OP_LZ4_DECODE, nb, tot)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    pulse.lz4_decode_blocks(payload, offsets, sizes, old, st, dws, mode=1, payload_bytes=tot)
    ev[1].record()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    check_view_gpu(old, ref_new, "v", "C4 view rebuilt by decode + XOR")
    ms = ev[0].elapsed_time(ev[1])
    say(f"C4: decode+XOR {ms:.1f} ms, {nbytes / ms / 1e6:.1f} GB/s of mask; rebuilt view equals the oracle's new view")
    fs.release()


# ---------------------------------------------------------------------------
def test_c5_kimi_layer_every_element():
    """C5: the Kimi-K2-shaped MoE layer share.  Per tensor cast + diff +
    compaction and patch apply (old view, new view, patch and patched view
    against the oracle), then [gate; up] and down of all 384 experts (one
    launch each, expert stride) and [q; k; v] quantised to E4M3 with 128x128
    FP32 scales: every code and scale against the oracle's quantisation of
    its own patched view."""
    dev = torch.device("cuda")
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
    view = np.empty(n, np.uint16)  # the oracle's patched view

    def pinned(t):
        h = torch.empty(t.numel(), dtype=t.dtype, pin_memory=True)
        h.copy_(t.reshape(-1))
        return h

    def job(ti, o, hw0, hw1, hbo, hnew, hidx, hval, hrecv, count):
        u16 = lambda h: h.numpy().view(np.uint16)  # noqa: E731
        bo = oracle.cast_bf16(hw0.numpy())
        r = oracle.cast_diff(hw1.numpy(), bo, want_mask=False)
        ok = (np.array_equal(u16(hbo), bo) and np.array_equal(u16(hnew), r["b_new"]) and r["count"] == count
              and np.array_equal(hidx.numpy(), r["idx"]) and np.array_equal(u16(hval), r["val"]))
        res, st_ = oracle.apply_patch(bo, r["idx"], r["val"])
        ok = ok and st_ == 0 and np.array_equal(u16(hrecv), res)
        view[o:o + res.size] = res
        return None if ok else ti

    futures = []
    changed = 0
    for ti, s in enumerate(specs):
        k = s.numel
        o = int(offs[ti])
        bt, wt = b[o:o + k], w[:k]
        workload.fill_init(wt, 5, ti, s.kind)
        pulse.pulse_cast_diff(wt, b_new=bt)
        hw0, hbo = pinned(wt), pinned(bt)
        workload.apply_step(wt, 5, ti, 1, tmp=tmp)
        pulse.pulse_cast_diff(wt, bt, stage[:k], None, idx, val, cnt, st, ws)
        torch.cuda.synchronize()
        count = int(cnt.item())
        assert count <= cap
        hw1, hnew = pinned(wt), pinned(stage[:k])
        hidx, hval = pinned(idx[:count]), pinned(val[:count])
        pulse.pulse_apply_patch(bt, idx, val, cnt, st)
        hrecv = pinned(bt)
        changed += count
        futures.append(fs._pool.submit(job, ti, o, hw0, hw1, hbo, hnew, hidx, hval, hrecv, count))
        if len(futures) >= 3 * fs.THREADS:  # bounded host memory in flight
            bad = futures.pop(0).result()
            assert bad is None, f"C5 tensor {specs[bad].name} differs from the oracle"
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for f in futures:
        bad = f.result()
        assert bad is None, f"C5 tensor {specs[bad].name} differs from the oracle"
    say(f"C5: {n} params, {changed} changed ({changed / n:.4%}); every tensor's views and patch equal the oracle")

    E, H, F = 384, 7168, 2048
    tstride = 3 * F * H  # one expert's gate, up, down

    def expert_view(which, rows, cols):
        return torch.as_strided(b[int(offs[which]):], (E, rows, cols), (tstride, cols, 1))

    R = 2 * F
    codes = torch.empty(E * R * H, dtype=torch.uint8, device=dev)
    scales = torch.empty(E * (R // 128) * (H // 128), dtype=torch.float32, device=dev)
    pulse.fp8_block_quant([expert_view(0, F, H), expert_view(1, F, H)], codes, scales, batch=E)
    torch.cuda.synchronize()
    ch, sh = fs.to_host(codes, "codes"), fs.to_host(scales, "scales")
    nsc = (R // 128) * (H // 128)
    for e in range(E):
        fs.check_fp8(view, [(int(offs[3 * e]), F), (int(offs[3 * e + 1]), F)], H, ch[e * R * H:(e + 1) * R * H],
                     sh[e * nsc:(e + 1) * nsc], f"C5 expert {e} [gate; up]", bands_per_task=2)
    pulse.fp8_block_quant([expert_view(2, H, F)], codes, scales, batch=E)
    torch.cuda.synchronize()
    ch, sh = fs.to_host(codes[:E * H * F], "codes"), fs.to_host(scales[:E * (H // 128) * (F // 128)], "scales")
    nsc = (H // 128) * (F // 128)
    for e in range(E):
        fs.check_fp8(view, [(int(offs[3 * e + 2]), H)], F, ch[e * H * F:(e + 1) * H * F], sh[e * nsc:(e + 1) * nsc],
                     f"C5 expert {e} down", bands_per_task=4)
    qi = len(specs) - 3
    qkv = [b[int(offs[qi + j]): int(offs[qi + j + 1])].view(8192, H) for j in range(3)]
    RQ = 3 * 8192
    pulse.fp8_block_quant(qkv, codes, scales)
    torch.cuda.synchronize()
    fs.check_fp8(view, [(int(offs[qi + j]), 8192) for j in range(3)], H, fs.to_host(codes[:RQ * H], "codes"),
                 fs.to_host(scales[:(RQ // 128) * (H // 128)], "scales"), "C5 [q; k; v]")
    say("C5: every FP8 code and scale of [gate; up], down and [q; k; v] equals the oracle's")
    fs.release()


# ---------------------------------------------------------------------------
F1_ORACLE_CHUNKS = (1, 17)  # a four-layer decoder chunk and the final norm + lm_head


def test_f1_fp8_view_delta_full_size():
    """Next row f1 on the C2 set, bench.py's FP8-view leg: per chunk the old
    and new views are quantised (the chunk's groups laid end to end) and
    fp8_view_delta / fp8_view_apply run over the codes and scales.  Every
    chunk: the old quantisation with the delta applied equals the new one,
    every code and scale.  Chunks 1 and 17: the delta's count and every entry,
    codes and scales, against the oracle's delta of its own quantisation of
    its own casts of the host masters."""
    dev = torch.device("cuda")
    specs = workload.qwen25_32b_specs()
    chunks, offs = build_plan(specs)
    max_chunk = max(e - s for s, e, _ in chunks)
    plans = [[(g, sum(specs[i].shape[0] for i in g), specs[g[0]].shape[1]) for g in quant_groups(specs, tids)]
             for _, _, tids in chunks]
    max_q = max(sum(r * c for _, r, c in p) for p in plans)
    max_s = max(sum(((r + 127) // 128) * ((c + 127) // 128) for _, r, c in p) for p in plans)
    W = torch.empty(max_chunk, dtype=torch.float32, device=dev)
    old = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    new = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    co = torch.empty(max_q, dtype=torch.uint8, device=dev)
    cn = torch.empty(max_q, dtype=torch.uint8, device=dev)
    so = torch.empty(max_s, dtype=torch.float32, device=dev)
    sn = torch.empty(max_s, dtype=torch.float32, device=dev)
    ccap = max_q // 10
    ci_, cv_ = torch.empty(ccap, dtype=torch.int32, device=dev), torch.empty(ccap, dtype=torch.uint8, device=dev)
    si_, sv_ = torch.empty(max_s, dtype=torch.int32, device=dev), torch.empty(max_s, dtype=torch.float32, device=dev)
    cc, sc = torch.zeros(1, dtype=torch.int64, device=dev), torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = new_ws(pulse.PULSE_OP_FP8_DELTA, max_q)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    total_codes = total_changed = 0
    for ci, (s0, e0, tids) in enumerate(chunks):
        m = e0 - s0
        with_oracle = ci in F1_ORACLE_CHUNKS
        host = {}
        for which, view in (("old", old), ("new", new)):
            for ti in tids:
                a, b = offs[ti] - s0, offs[ti] - s0 + specs[ti].numel
                if which == "old":
                    workload.fill_init(W[a:b], 2, ti, specs[ti].kind)
                else:
                    workload.apply_step(W[a:b], 2, ti, 1, tmp=tmp)
                pulse.pulse_cast_diff(W[a:b], b_new=view[a:b])
            if with_oracle:
                host[which] = fs.oracle_cast(fs.to_host(W[:m], "w"))
        qo = so_o = 0
        groups = []
        for (g, rows, cols) in plans[ci]:
            nq, ns = rows * cols, ((rows + 127) // 128) * ((cols + 127) // 128)
            for view, c, s_ in ((old, co, so), (new, cn, sn)):
                pulse.fp8_block_quant([view[offs[i] - s0: offs[i] - s0 + specs[i].numel].view(specs[i].shape)
                                       for i in g], c[qo:qo + nq], s_[so_o:so_o + ns])
            groups.append(([(offs[i] - s0, specs[i].shape[0]) for i in g], cols, qo, nq, so_o, ns))
            qo, so_o = qo + nq, so_o + ns
        pulse.fp8_view_delta(co[:qo], cn[:qo], so[:so_o], sn[:so_o], ci_, cv_, cc, si_, sv_, sc, st, ws)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        count, scount = int(cc.item()), int(sc.item())
        assert count <= ccap
        if with_oracle:
            ref_q = {}
            for which in ("old", "new"):
                c_h, s_h = np.empty(qo, np.uint8), np.empty(so_o, np.float32)
                for srcs, cols, q0, nq, s0_, ns in groups:
                    fs.oracle_fp8(host[which], srcs, cols, c_h[q0:q0 + nq], s_h[s0_:s0_ + ns])
                ref_q[which] = (c_h, s_h)
            fs.check_equal(fs.to_host(co[:qo], "codes"), ref_q["old"][0], f"f1 chunk {ci}: old codes")
            fs.check_equal(fs.to_host(cn[:qo], "codes"), ref_q["new"][0], f"f1 chunk {ci}: new codes")
            ref = fs.OracleDelta(ref_q["old"][0], ref_q["new"][0], ref_q["old"][1], ref_q["new"][1])
            ref.check(count, fs.to_host(ci_[:count], "idx"), fs.to_host(cv_[:count], "val"), scount,
                      fs.to_host(si_[:scount], "sidx"), fs.to_host(sv_[:scount], "sval"), f"f1 chunk {ci}")
        pulse.fp8_view_apply(co[:qo], so[:so_o], ci_, cv_, cc, si_, sv_, sc, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(co[:qo], cn[:qo]), f"f1 chunk {ci}: apply(quant(old), delta) != quant(new) (codes)"
        assert torch.equal(so[:so_o].view(torch.int32), sn[:so_o].view(torch.int32)), f"f1 chunk {ci}: scales"
        total_codes += qo
        total_changed += count
        if with_oracle:
            say(f"f1 chunk {ci}: {qo} codes, {count} changed, {scount} scales changed: every entry equals the oracle")
    say(f"f1: {total_codes} codes, {total_changed} changed ({total_changed / total_codes:.3%}); "
        "apply(quant(old), delta) == quant(new) on every chunk")
    fs.release()
