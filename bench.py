"""Throughput of the trainer->sampler weight-delta codec on one MI355X.

One step = one pass of the whole hot path over a Qwen2.5-32B-shaped weight set
(32,763,876,352 parameters; FP32 masters, old BF16 view and the receiver's BF16
view resident in HBM before timing starts), processed in 18 chunks of whole
tensors (embed | 16 x four decoder layers | final norm + lm_head):

  sender    pulse_cast_diff_lz4  one pass: FP32 -> BF16 RNE cast, bitwise diff
                              against the old view, (int32 index, BF16 value)
                              patch, and the LZ4 blocks (64 KiB) of the XOR mask
                              old ^ new, the mask never leaving the chip
                              (--separate-encode: pulse_cast_diff, then
                              lz4_encode_blocks over old and new)
  receiver  lz4_decode_parse  the serial token-chain parse of every block, on a
                              second stream, beside the next one (--schedule)
  receiver  pulse_apply_quant one pass per 128x128 block: the patch applied to the
                              receiver's view (v0 -> v1) and the stacked [q;k;v],
                              o, [gate;up], down, embed, lm_head groups
                              quantised to E4M3 + FP32 scales from the patched
                              values; norms and biases only patched
                              (--receiver separate: pulse_apply_patch, then
                              fp8_block_quant_groups, up to 8 groups a launch;
                              --apply-tiled, --quant-per-group select their
                              variants)
  receiver  lz4_decode_apply  rebuild + XOR in place into the receiver's view
                              (--schedule serial: one lz4_decode_blocks call on
                              the main stream, no second stream)

The mask is symmetric, so the XOR step takes the receiver from v1 back to v0:
every step does identical work on identical data with no untimed restore.  The
sender writes its new view into a per-chunk staging buffer instead of over the
old view for the same reason (the same bytes move either way).

Prints one JSON line.  value = 2 * params / step time (BF16 weights processed
per second), the HBM fraction of the whole step is reported beside it, and the
roofline object covers the kernel that takes most of the step.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weights processed GB/s (encode+apply) and % of MI355X HBM peak, 1 GPU"
SCHEDULES = {
    "ahead": "parse of chunk c on a second stream beside the encode of chunk c + 1; the receiver's pass and "
             "the decode apply of chunk c on the main stream after it",
    "side": "parse on a second stream beside the receiver's pass of the same chunk, apply on the main stream",
    "behind": "main stream: receiver's pass of chunk c, encode of chunk c + 1, decode apply of chunk c; the parse "
              "of chunk c + 1 on a second stream beside that decode apply",
    "pipeline": "encode and parse of chunk c on a second stream while the main stream receives and decodes "
                "chunk c - 1",
    "serial": "one lz4_decode_blocks call per chunk, main stream",
}
PEAK_HBM = 8.0e12
BLOCK = 65536
PATCH_CAP_FRAC = 0.125   # patch capacity per chunk (measured density ~8.06%)
PAYLOAD_CAP_FRAC = 0.35  # LZ4 payload capacity per chunk, fraction of mask bytes


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--layers", type=int, default=64, help="decoder layers (64 = the full Qwen2.5-32B shape)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--separate-encode", action="store_true",
                   help="sender as two calls (pulse_cast_diff, then lz4_encode_blocks) instead of the fused pass")
    p.add_argument("--apply-tiled", action="store_true",
                   help="patch apply with pulse_apply_patch_tiled and the tile index the sender writes (faster "
                        "alone, slower beside the decode parse) instead of pulse_apply_patch")
    p.add_argument("--quant-per-group", action="store_true",
                   help="one fp8_block_quant launch per stacked group instead of grouped launches")
    p.add_argument("--receiver", choices=["fused", "separate"], default="fused",
                   help="fused: pulse_apply_quant (patch apply + FP8 quantisation in one read of the view); "
                        "separate: pulse_apply_patch, then fp8_block_quant_groups")
    p.add_argument("--schedule", choices=["ahead", "side", "behind", "pipeline", "serial"], default="side",
                   help="ahead: the decode parse of chunk c on a second stream beside the encode of chunk c + 1; "
                        "side: beside the receiver's pass of chunk c; "
                        "behind: beside the decode apply of chunk c - 1, which the main stream runs after the "
                        "encode of chunk c; "
                        "pipeline: encode and parse of chunk c on the second stream while the main stream "
                        "receives chunk c - 1; serial: one lz4_decode_blocks call per chunk, one stream")
    p.add_argument("--cpu-sample-frac", type=float, default=1.0,
                   help="fraction of the oracle's sample (decoder layer 0) it times")
    p.add_argument("--next", default="loco,patch,list,fp8", help="next-row legs measured after the timed steps, comma "
                   "separated: loco (PULSELoCo gate), patch (patch-stream compression), list (one launch over the "
                   "tensor list), fp8 (FP8-view deltas), none")
    p.add_argument("--probe-gib", type=float, default=4.0,
                   help="GiB per stream of the achievable-bandwidth probes (0: skip them)")
    p.add_argument("--encode-apply-reps", type=int, default=3,
                   help="timed passes of the patch path alone (pulse_cast_diff + pulse_apply_patch; 0: skip)")
    p.add_argument("--lr-sweep", default="2.5e-7,3e-8",
                   help="learning rates at which the step is measured again (comma separated; empty: skip)")
    p.add_argument("--configs", default="c1,c3,c4,c5",
                   help="other configurations measured after the main one (c1,c3,c4,c5 or none)")
    return p.parse_args()


# ---------------------------------------------------------------------------
def build_plan(specs, layers_per_chunk=4):
    """Chunks of whole tensors in tensor order: embed, groups of decoder layers,
    the tail (final norm + lm_head).  Returns [(start, end, [tensor indices])]."""
    offs, o = [], 0
    for s in specs:
        offs.append(o)
        o += s.numel
    chunks, cur, cur_layer_count, cur_layer = [], [], 0, None
    for i, s in enumerate(specs):
        if s.name == "embed":
            chunks.append([i])
            continue
        if s.name[0] == "l" and s.name[1].isdigit():
            layer = int(s.name[1:].split(".")[0])
            if layer != cur_layer:
                if cur_layer is not None and cur_layer_count == layers_per_chunk:
                    chunks.append(cur)
                    cur, cur_layer_count = [], 0
                cur_layer = layer
                cur_layer_count += 1
            cur.append(i)
        else:
            if cur and cur_layer is not None:
                chunks.append(cur)
                cur, cur_layer = [], None
            cur.append(i)
    if cur:
        chunks.append(cur)
    out = []
    for ch in chunks:
        start = offs[ch[0]]
        end = offs[ch[-1]] + specs[ch[-1]].numel
        out.append((start, end, ch))
    return out, offs


def quant_groups(specs, tensor_ids):
    """FP8 groups of a chunk: lists of tensor indices stacked along rows."""
    names = {specs[i].name: i for i in tensor_ids}
    groups = []
    for i in tensor_ids:
        nm = specs[i].name
        if len(specs[i].shape) != 2:
            continue
        if nm.endswith(".q"):
            p = nm[:-1]
            groups.append([i, names[p + "k"], names[p + "v"]])
        elif nm.endswith(".gate"):
            groups.append([i, names[nm[:-4] + "up"]])
        elif nm.endswith(".k") or nm.endswith(".v") or nm.endswith(".up"):
            continue
        else:
            groups.append([i])
    return groups


def grouped_quant_plan(pulse, specs, offs, plan, b_recv, codes, scales):
    """A chunk's FP8 groups as batches for fp8_block_quant_groups, each group
    with its own codes and scales (views into the shared buffers)."""
    lst, co, so = [], 0, 0
    for (g, rows, cols) in plan:
        srcs = [b_recv[offs[i]: offs[i] + specs[i].numel].view(specs[i].shape) for i in g]
        nsc = ((rows + 127) // 128) * ((cols + 127) // 128)
        lst.append((srcs, codes[co: co + rows * cols], scales[so: so + nsc]))
        co += rows * cols
        so += nsc
    m = pulse.PULSE_QUANT_MAX_GROUPS
    return [lst[k: k + m] for k in range(0, len(lst), m)]


def receiver_plan(pulse, specs, offs, chunk, plan, codes, scales, dev):
    """The receiver's pass over a chunk: its FP8 groups (codes and scales laid
    out as in grouped_quant_plan) and its other tensors, patched only."""
    s0, e0, tids = chunk
    groups, co, so, seen = [], 0, 0, set()
    for (g, rows, cols) in plan:
        nsc = ((rows + 127) // 128) * ((cols + 127) // 128)
        groups.append(([(offs[i] - s0, specs[i].shape[0]) for i in g], cols, codes[co: co + rows * cols],
                       scales[so: so + nsc]))
        co += rows * cols
        so += nsc
        seen.update(g)
    for i in tids:
        if i not in seen:
            sh = specs[i].shape
            rows, cols = (sh[0], sh[1]) if len(sh) == 2 else (1, specs[i].numel)
            groups.append(([(offs[i] - s0, rows)], cols, None, None))
    return pulse.pulse_apply_quant_plan(groups, e0 - s0, device=dev)


def views_equal(a, b, chunk=1 << 30):
    """Bitwise equality of two large device tensors, chunked to bound temporaries."""
    for s in range(0, a.numel(), chunk):
        if not bool((a[s:s + chunk] == b[s:s + chunk]).all()):
            return False
    return True


def independent_check(pulse, specs, offs, chunks, W, b_old, b_recv, stage, idx, val, cnt, codes, scales, status,
                      send_receive, decode):
    """The last chunk (final norm + lm_head) once more, checked against values
    computed on the host without the library: windows of the sender's new view
    and of the receiver's patched view against torch's CPU cast of the
    masters, the patch entries in those windows against numpy's flatnonzero
    of the two casts, and the FP8 codes and scales of the lm_head's first
    128-row band against numpy's float32 division and torch's E4M3
    conversion; after the decode + XOR the receiver's view is the old view."""
    import numpy as np
    import torch

    ci = len(chunks) - 1
    s0, e0, tids = chunks[ci]
    m = e0 - s0
    send_receive(ci)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit(f"check: device status {int(status.item())}")
    count = int(cnt[ci].item())
    ii = idx[:count]
    for o in (0, m // 2, m - 65536):
        w = W[s0 + o: s0 + o + 65536].cpu()
        ref = w.to(torch.bfloat16).view(torch.int16)
        old = b_old[s0 + o: s0 + o + 65536].cpu()
        if not (torch.equal(stage[o:o + 65536].cpu(), ref) and torch.equal(b_recv[s0 + o: s0 + o + 65536].cpu(), ref)):
            raise SystemExit(f"check: new or patched view differs from torch's cast at chunk offset {o}")
        pos = np.flatnonzero((ref != old).numpy()) + o
        lo, hi = (int(x) for x in torch.searchsorted(ii, torch.tensor([o, o + 65536], dtype=torch.int32,
                                                                       device=ii.device)).cpu())
        if not (np.array_equal(ii[lo:hi].cpu().numpy(), pos) and
                torch.equal(val[lo:hi].cpu(), ref[torch.from_numpy(pos - o)])):
            raise SystemExit(f"check: patch entries differ from numpy's flatnonzero at chunk offset {o}")
    head = [i for i in tids if specs[i].name == "lm_head"][0]
    cols = specs[head].shape[1]
    x = W[offs[head]: offs[head] + 128 * cols].cpu().to(torch.bfloat16).to(torch.float32).numpy().reshape(128, cols)
    for bc in range(0, (cols + 127) // 128):
        blk = x[:, bc * 128:(bc + 1) * 128]
        amax = np.float32(np.abs(blk).max())
        sc = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
        q = np.ascontiguousarray((blk / sc).astype(np.float32))
        ref_c = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got_c = codes[:128 * cols].view(128, cols)[:, bc * 128:(bc + 1) * 128].cpu().numpy()
        if not (np.array_equal(got_c, ref_c) and np.float32(scales[bc].item()) == sc):
            raise SystemExit(f"check: FP8 codes or scale of lm_head block (0, {bc}) differ from numpy + torch")
    decode(ci)
    torch.cuda.synchronize()
    if int(status.item()) != 0 or not views_equal(b_recv[s0:e0], b_old[s0:e0]):
        raise SystemExit("check: the decode + XOR did not return the receiver's view to the old view")


def log(msg):
    """Progress on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def run_env(torch):
    """The software and the device the numbers were taken on: HIP and torch
    versions, device name, architecture, compute units and memory.  (No
    helper program is started: a child of a process that holds the GPU must
    not replace itself with another program.)"""
    props = torch.cuda.get_device_properties(0)
    return {"hip": getattr(torch.version, "hip", None), "torch": torch.__version__, "device": props.name,
            "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "hbm_GiB": round(props.total_memory / 2 ** 30, 1)}


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): it measures one device's share of the "
              "path; sharded, each GPU would encode and receive its own shard's patch and LZ4 blocks", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_delta_codec_amd as pulse
    import workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.time()

    specs = workload.qwen25_32b_specs(args.layers)
    n = workload.total_numel(specs)
    chunks, offs = build_plan(specs)
    max_chunk = max(e - s for s, e, _ in chunks)
    max_tensor = max(s.numel for s in specs)

    # ---- resident inputs: FP32 masters (after the step), old view, receiver view
    W = torch.empty(n, dtype=torch.float32, device=dev)
    b_old = torch.empty(n, dtype=torch.int16, device=dev)
    tmp = torch.empty(max_tensor, dtype=torch.float32, device=dev)
    for ti, s in enumerate(specs):
        w = W[offs[ti]: offs[ti] + s.numel]
        workload.fill_init(w, 2, ti, s.kind)
        # the old served view is the library's own cast of the initial masters
        pulse.pulse_cast_diff(w, b_new=b_old[offs[ti]: offs[ti] + s.numel])
        workload.apply_step(w, 2, ti, 1, tmp=tmp)
    del tmp, w  # w is a view of W
    b_recv = b_old.clone()
    torch.cuda.synchronize()

    # ---- per-chunk scratch (reused by every chunk)
    cap = int(max_chunk * PATCH_CAP_FRAC)
    stage = torch.empty(max_chunk, dtype=torch.int16, device=dev)
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    val = torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    pcap = int(2 * max_chunk * PAYLOAD_CAP_FRAC)
    payload = torch.empty(pcap, dtype=torch.uint8, device=dev)
    nbmax = (2 * max_chunk + BLOCK - 1) // BLOCK
    csizes = torch.empty(nbmax, dtype=torch.int32, device=dev)
    coffs = torch.empty(nbmax, dtype=torch.int64, device=dev)
    ctotal = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    ws_cd = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, max_chunk, 0, dev)
    ws_en = pulse.workspace(pulse.PULSE_OP_LZ4_ENCODE, 2 * max_chunk, BLOCK, dev)
    ws_fz = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_LZ4, max_chunk, BLOCK, dev)
    tiles = torch.zeros(pulse.patch_tile_count(max_chunk), dtype=torch.int64, device=dev)  # the patch's tile index
    ws_de = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nbmax, pcap, dev)
    qplans = []
    max_codes = max_scales = 0
    for (s0, e0, tids) in chunks:
        plan = []
        for g in quant_groups(specs, tids):
            cols = specs[g[0]].shape[1]
            rows = sum(specs[i].shape[0] for i in g)
            plan.append((g, rows, cols))
            max_codes = max(max_codes, rows * cols)
            max_scales = max(max_scales, ((rows + 127) // 128) * ((cols + 127) // 128))
        qplans.append(plan)
    # every group of a chunk writes its own codes and scales (the grouped
    # launch quantises them together)
    max_chunk_codes = max(sum(r * c for _, r, c in plan) for plan in qplans)
    max_chunk_scales = max(sum(((r + 127) // 128) * ((c + 127) // 128) for _, r, c in plan) for plan in qplans)
    codes = torch.empty(max(max_codes, max_chunk_codes), dtype=torch.uint8, device=dev)
    scales = torch.empty(max(max_scales, max_chunk_scales), dtype=torch.float32, device=dev)
    n_quant = sum(rows * cols for plan in qplans for (_, rows, cols) in plan)
    # per chunk: lists of at most 8 (srcs, codes, scales) for fp8_block_quant_groups
    gplans = [grouped_quant_plan(pulse, specs, offs, plan, b_recv, codes, scales) for plan in qplans]
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    log(f"setup done in {t_setup:.1f} s: {n} params in {len(chunks)} chunks")

    fused = not args.separate_encode
    recv_fused = args.receiver == "fused"
    sched = args.schedule
    if sched in ("ahead", "pipeline") and not fused:
        raise SystemExit(f"--schedule {sched} goes with the fused encode")
    if args.apply_tiled and recv_fused:
        raise SystemExit("--apply-tiled goes with --receiver separate")
    if args.quant_per_group and recv_fused:
        raise SystemExit("--quant-per-group goes with --receiver separate")
    recv_stages = ["receiver"] if recv_fused else ["apply_patch", "fp8_quant"]
    stages = (["encode"] if fused else ["cast_diff", "lz4_encode"]) + recv_stages + ["lz4_decode"]
    ev = {k: [] for k in stages}

    if recv_fused:
        ws_aq = pulse.workspace(pulse.PULSE_OP_APPLY_QUANT, max_chunk, 0, dev)
        aq_plans = [receiver_plan(pulse, specs, offs, ch, plan, codes, scales, dev)
                    for ch, plan in zip(chunks, qplans)]
    # buffer sets: what a chunk's sender output and parse live in until the
    # receiver is done with them (two when a chunk's encode overlaps another's)
    bufs = [(idx, val, payload, csizes, coffs, ws_de, tiles)]
    if sched in ("ahead", "behind", "pipeline"):
        bufs.append((torch.empty_like(idx), torch.empty_like(val), torch.empty_like(payload),
                     torch.empty_like(csizes), torch.empty_like(coffs),
                     pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nbmax, pcap, dev), torch.zeros_like(tiles)))

    main_stream = torch.cuda.current_stream()
    side_stream = torch.cuda.Stream()  # default priority, like every stream here
    parse_ev = {"lz4_decode": []}      # parse events (side stream), added to the decode stage

    def rec(record, name, fn, store=None):
        # events on the stream the kernels run on (the current one)
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            (ev if store is None else store)[name].append((a, b))
        else:
            fn()

    def encode(record, ci, B):
        s0, e0, _ = chunks[ci]
        m = e0 - s0
        I, V, P, CS, CO, _, T = B
        if fused:
            rec(record, "encode", lambda: pulse.pulse_cast_diff_lz4(
                W[s0:e0], b_old[s0:e0], stage[:m], I, V, cnt[ci:ci + 1], P, CS, CO, ctotal[ci:ci + 1], status,
                ws_fz, tile_first=T if args.apply_tiled else None, stream=torch.cuda.current_stream()))
        else:
            rec(record, "cast_diff", lambda: pulse.pulse_cast_diff(W[s0:e0], b_old[s0:e0], stage[:m], None, I, V,
                                                                   cnt[ci:ci + 1], status, ws_cd))
            rec(record, "lz4_encode", lambda: pulse.lz4_encode_blocks(b_old[s0:e0], P, CS, CO, ctotal[ci:ci + 1],
                                                                      status, ws_en, src_xor=stage[:m]))

    def receive(record, ci, B):
        """The patch apply (v0 -> v1) and the FP8 quantisation of v1."""
        s0, e0, _ = chunks[ci]
        m = e0 - s0
        I, V, T = B[0], B[1], B[6]
        if recv_fused:
            rec(record, "receiver", lambda: pulse.pulse_apply_quant(b_recv[s0:e0], I, V, cnt[ci:ci + 1],
                                                                    aq_plans[ci], status, ws_aq))
            return

        def apply():
            if not args.apply_tiled:
                pulse.pulse_apply_patch(b_recv[s0:e0], I, V, cnt[ci:ci + 1], status)
                return
            if not fused:  # the receiver builds the tile index itself
                pulse.pulse_patch_tiles(I, cnt[ci:ci + 1], T, m)
            pulse.pulse_apply_patch_tiled(b_recv[s0:e0], I, V, T, status)

        def quant():
            if args.quant_per_group:
                for (g, rows, cols) in qplans[ci]:
                    srcs = [b_recv[offs[i]: offs[i] + specs[i].numel].view(specs[i].shape) for i in g]
                    pulse.fp8_block_quant(srcs, codes, scales)
            else:
                for batch in gplans[ci]:
                    pulse.fp8_block_quant_groups(batch)

        rec(record, "apply_patch", apply)
        rec(record, "fp8_quant", quant)  # reads the receiver's view before the XOR rewrites it

    def parse_chunk(record, ci, B):
        """The decode's token-chain parse, on the side stream."""
        s0, e0, _ = chunks[ci]
        _, _, P, CS, CO, WD, _ = B
        with torch.cuda.stream(side_stream):
            rec(record, "lz4_decode", lambda: pulse.lz4_decode_parse(P, CO, CS, 2 * (e0 - s0), status, WD,
                                                                     stream=side_stream), store=parse_ev)
            parsed = torch.cuda.Event()
            parsed.record(side_stream)
        return parsed

    def decode_apply(record, ci, B):
        s0, e0, _ = chunks[ci]
        _, _, P, CS, CO, WD, _ = B
        rec(record, "lz4_decode", lambda: pulse.lz4_decode_apply(P, CO, CS, b_recv[s0:e0], status, WD, mode=1))

    def after(stream):
        e = torch.cuda.Event()
        e.record(stream)
        return e

    last_decode = [None, None]  # pipeline: the decode apply that last used each buffer set
    seq = [0]                   # pipeline: chunks run so far (the sets alternate across steps)

    def run_step(record):
        N = len(chunks)
        if sched == "serial":
            for ci in range(N):
                s0, e0, _ = chunks[ci]
                encode(record, ci, bufs[0])
                receive(record, ci, bufs[0])
                rec(record, "lz4_decode", lambda: pulse.lz4_decode_blocks(payload, coffs, csizes, b_recv[s0:e0],
                                                                          status, ws_de, mode=1))
        elif sched == "side":
            # the parse of chunk c beside its apply and quant
            for ci in range(N):
                encode(record, ci, bufs[0])
                side_stream.wait_stream(main_stream)
                parsed = parse_chunk(record, ci, bufs[0])
                receive(record, ci, bufs[0])
                main_stream.wait_event(parsed)
                decode_apply(record, ci, bufs[0])
        elif sched == "behind":
            # the main stream runs receive(c), encode(c + 1), decode_apply(c):
            # the parse of chunk c + 1 (after its encode) runs beside the
            # decode apply of chunk c, whose kernel leaves most of each CU's
            # LDS and registers free, and no longer beside a receiver's pass.
            # Buffer sets alternate: chunk c + 1's encode writes the set that
            # chunk c - 1's decode apply (earlier on the main stream) used.
            encode(record, 0, bufs[0])
            side_stream.wait_stream(main_stream)
            parsed = parse_chunk(record, 0, bufs[0])
            for ci in range(N):
                B = bufs[ci % 2]
                receive(record, ci, B)
                nxt = None
                if ci + 1 < N:
                    Bn = bufs[(ci + 1) % 2]
                    encode(record, ci + 1, Bn)
                    side_stream.wait_stream(main_stream)
                    nxt = parse_chunk(record, ci + 1, Bn)
                main_stream.wait_event(parsed)
                decode_apply(record, ci, B)
                parsed = nxt
        elif sched == "ahead":
            # the parse of chunk c starts with the encode of chunk c + 1 (the
            # event before that encode also follows chunk c - 1's decode, the
            # last user of the buffer set chunk c + 1 writes), then the main
            # stream receives chunk c and decodes it once the parse is done
            encode(record, 0, bufs[0])
            for ci in range(N):
                B = bufs[ci % 2]
                side_stream.wait_event(after(main_stream))
                parsed = parse_chunk(record, ci, B)
                if ci + 1 < N:
                    encode(record, ci + 1, bufs[(ci + 1) % 2])
                receive(record, ci, B)
                main_stream.wait_event(parsed)
                decode_apply(record, ci, B)
        else:  # pipeline: encode and parse of chunk c on the side stream while the main stream receives chunk c - 1
            for ci in range(N):
                p = seq[0] % 2
                seq[0] += 1
                B = bufs[p]
                with torch.cuda.stream(side_stream):
                    if last_decode[p] is not None:
                        side_stream.wait_event(last_decode[p])
                    encode(record, ci, B)
                    encoded = after(side_stream)
                parsed = parse_chunk(record, ci, B)
                main_stream.wait_event(encoded)
                receive(record, ci, B)
                main_stream.wait_event(parsed)
                decode_apply(record, ci, B)
                last_decode[p] = after(main_stream)

    # ---- warm-up, with the end-to-end check after the first step
    for w in range(max(args.warmup, 1)):
        run_step(False)
        torch.cuda.synchronize()
        if w == 0:
            st = int(status.item())
            if st != 0:
                raise SystemExit(f"device status {st} after the first step (capacity or corrupt payload)")
            if not views_equal(b_recv, b_old):
                raise SystemExit("receiver view did not return to v0 after patch apply + XOR decode")
    independent_check(pulse, specs, offs, chunks, W, b_old, b_recv, stage, idx, val, cnt, codes, scales, status,
                      lambda ci: (encode(False, ci, bufs[0]), receive(False, ci, bufs[0])),
                      lambda ci: (side_stream.wait_stream(main_stream), main_stream.wait_event(
                          parse_chunk(False, ci, bufs[0])), decode_apply(False, ci, bufs[0])) if sched != "serial"
                      else pulse.lz4_decode_blocks(payload, coffs, csizes, b_recv[chunks[ci][0]:chunks[ci][1]], status,
                                                   ws_de, mode=1))
    log(f"warm-up done ({max(args.warmup, 1)} steps, end-to-end check passed)")
    counts = cnt.cpu().numpy()
    totals = ctotal.cpu().numpy()
    changed = int(counts.sum())
    comp_bytes = int(totals.sum())
    d = changed / n
    c = comp_bytes / n  # compressed bytes per element

    # ---- timed steps
    for k in ev:
        ev[k].clear()
    parse_ev["lz4_decode"].clear()
    torch.cuda.synchronize()
    # step boundaries as events on the main stream (the side stream joins it
    # within every step), for the per-step median and minimum
    step_marks = [torch.cuda.Event(enable_timing=True)]
    t0 = time.perf_counter()
    step_marks[0].record(main_stream)
    for _ in range(args.steps):
        run_step(True)
        step_marks.append(torch.cuda.Event(enable_timing=True))
        step_marks[-1].record(main_stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    step_each = [a.elapsed_time(b) for a, b in zip(step_marks[:-1], step_marks[1:])]
    if int(status.item()) != 0:
        raise SystemExit(f"device status {int(status.item())} during the timed steps")
    if not views_equal(b_recv, b_old):
        raise SystemExit("receiver view drifted during the timed steps")

    log(f"timed {args.steps} steps in {t_total:.2f} s")
    ms_step = 1e3 * t_total / args.steps
    stage_ms = {k: sum(a.elapsed_time(b) for a, b in ev[k]) / args.steps for k in stages}
    launches = {k: len(ev[k]) // args.steps for k in stages}
    # the decode stage is its apply (main stream); the parse runs on the side
    # stream beside apply_patch and fp8_quant and is reported beside it
    parse_ms = sum(a.elapsed_time(b) for a, b in parse_ev["lz4_decode"]) / args.steps
    # algorithmic bytes per step (what the method must move)
    alg = {
        "encode": n * (8 + 6 * d + c),          # read w (4) + old (2), write new (2) + patch (6 d) + payload (c)
        "cast_diff": n * (8 + 6 * d),           # read w (4) + old (2), write new (2) + patch (6 d)
        "receiver": n * 8 * d + n_quant * 3 + 4 * n_quant / 16384,  # apply_patch + fp8_quant
        "apply_patch": n * 8 * d,               # read patch (6 d), write 2 B per changed element
        "fp8_quant": n_quant * 3 + 4 * n_quant / 16384,  # read 2, write 1 + scales
        "lz4_encode": n * (4 + c),              # read old + new (4), write payload (c)
        "lz4_decode": n * (4 + c),              # read payload (c), read + write dst (4)
    }
    alg = {k: alg[k] for k in stages}
    alg_total = sum(alg.values())
    st_out = {}
    for k in stages:
        secs = stage_ms[k] / 1e3
        st_out[k] = {"ms": round(stage_ms[k], 3), "launches": launches[k], "alg_GB": round(alg[k] / 1e9, 3),
                     "GBps": round(alg[k] / secs / 1e9, 1), "frac_hbm": round(alg[k] / secs / PEAK_HBM, 4)}
    dom = max(stages, key=lambda k: stage_ms[k])
    dom_secs = stage_ms[dom] / 1e3
    achieved = alg[dom] / dom_secs / 1e9
    kernel_files = {"encode": "lz4_encode.hip", "cast_diff": "cast_diff.hip", "apply_patch": "apply.hip",
                    "receiver": "fp8_quant.hip",
                    "fp8_quant": "fp8_quant.hip",
                    "lz4_encode": "lz4_encode.hip", "lz4_decode": "lz4_decode.hip"}
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved * 1e9 / PEAK_HBM, 4), "traffic": None,
                "alg_bytes_per_launch": round(alg[dom] / launches[dom]),
                "avg_launch_ms": round(stage_ms[dom] / launches[dom], 4)}
    # measured HBM traffic, when profiles/ holds counters taken on this kernel's current source
    tfile = os.path.join(ROOT, "profiles", f"{dom}_qwen32b_traffic.json")
    if os.path.exists(tfile):
        try:
            tr = json.load(open(tfile))
            src = os.path.join(ROOT, "sparse_delta_codec_amd", "csrc", kernel_files[dom])
            if tr.get("source_sha") == src_hash(src):
                roofline["traffic"] = tr["bytes_per_launch"]
        except Exception:
            pass

    value = 2 * n / (ms_step / 1e3) / 1e9
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Qwen2.5-32B-shaped weight set ({args.layers} layers), one RL step at lr 3e-6, "
                               "full hot path: cast+diff+compact, patch apply, stacked FP8 quant, "
                               "LZ4 mask encode, LZ4 decode+XOR",
                   "params": n, "chunks": len(chunks), "lz4_block_bytes": BLOCK,
                   "encode_schedule": "one fused pass (pulse_cast_diff_lz4)" if fused
                   else "pulse_cast_diff, then lz4_encode_blocks",
                   "receiver": "one pass (pulse_apply_quant)" if recv_fused
                   else "pulse_apply_patch, then fp8_block_quant_groups",
                   "decode_schedule": SCHEDULES[sched],
                   "changed_fraction": round(d, 6), "lz4_bytes_per_param": round(c, 5),
                   "lz4_ratio_of_mask": round(comp_bytes / (2 * n), 5), "fp8_params": n_quant},
        "hbm_frac_step": round(alg_total / (ms_step / 1e3) / PEAK_HBM, 4),
        "alg_GB_per_step": round(alg_total / 1e9, 2),
        "stages": st_out,
        "decode_parse": None if sched == "serial" else {
            "ms": round(parse_ms, 3), "launches": len(parse_ev["lz4_decode"]) // args.steps,
            "stream": "second stream",
            "note": "lz4_decode above is the apply; the one-call decode is both"},
        "roofline": roofline,
        "step_ms_median": round(float(np.median(step_each)), 3),
        "step_ms_min": round(float(np.min(step_each)), 3),
        "setup_s": round(t_setup, 1),
        "env": run_env(torch),
    }

    # ---- the metric's own quantity: patch-path encode + apply (pulse_cast_diff,
    # then pulse_apply_patch), per chunk over the same set, outside the step
    if args.encode_apply_reps > 0:
        result["encode_apply"] = encode_apply_leg(pulse, chunks, W, b_old, b_recv, stage, idx, val, status, ws_cd,
                                                  args.encode_apply_reps, dev)
        log(f"encode+apply: {result['encode_apply']['ms']:.2f} ms, {result['encode_apply']['GBps_weights']:.1f} "
            "GB/s of weights")

    # ---- the same step at the pages' densities (lr sweep), then the masters at lr 3e-6 again
    lrs = [float(x) for x in args.lr_sweep.split(",") if x]
    if lrs:
        sweep = []
        tmp = torch.empty(max_tensor, dtype=torch.float32, device=dev)

        def masters_at(lr):
            for ti, s in enumerate(specs):
                w = W[offs[ti]: offs[ti] + s.numel]
                workload.fill_init(w, 2, ti, s.kind)
                workload.apply_step(w, 2, ti, 1, lr=lr, tmp=tmp)
            torch.cuda.synchronize()

        for lr in lrs:
            masters_at(lr)
            run_step(False)
            torch.cuda.synchronize()
            if int(status.item()) != 0 or not views_equal(b_recv, b_old):
                raise SystemExit(f"lr {lr}: status {int(status.item())} or the receiver did not return to v0")
            for k in ev:
                ev[k].clear()
            parse_ev["lz4_decode"].clear()
            ks = max(1, min(args.steps, 5))
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(ks):
                run_step(True)
            torch.cuda.synchronize()
            ms_lr = 1e3 * (time.perf_counter() - t0) / ks
            d_lr = int(cnt.sum().item()) / n
            c_lr = int(ctotal.sum().item()) / n
            sms = {k: round(sum(a.elapsed_time(b) for a, b in ev[k]) / ks, 3) for k in stages}
            if parse_ev["lz4_decode"]:
                sms["decode_parse"] = round(sum(a.elapsed_time(b) for a, b in parse_ev["lz4_decode"]) / ks, 3)
            sweep.append({"lr": lr, "changed_fraction": round(d_lr, 6), "lz4_bytes_per_param": round(c_lr, 5),
                          "ms_per_step": round(ms_lr, 3), "GBps_weights_step": round(2 * n / (ms_lr / 1e3) / 1e9, 1),
                          "stage_ms": sms, "steps": ks})
            log(f"lr {lr}: {ms_lr:.2f} ms per step, changed {100 * d_lr:.3f}%")
        masters_at(workload.LR)
        del tmp
        result["lr_sweep"] = sweep

    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(specs, offs, W, b_old, args.cpu_sample_frac)

    legs = set(x for x in args.next.split(",") if x and x != "none")
    nxt = {}
    if "patch" in legs:
        nxt.update(patch_stream_leg(pulse, chunks, W, b_old, stage, idx, val, cnt, status, ws_cd, dev,
                                    not args.no_cpu_baseline))
    if "fp8" in legs:
        nxt.update(fp8_view_leg(pulse, specs, chunks, offs, qplans, W, b_old, stage, dev,
                                not args.no_cpu_baseline))
    del stage, b_recv, idx, val, payload, codes, scales, gplans, tiles, bufs  # gplans holds views of b_recv
    if recv_fused:
        del aq_plans, ws_aq  # the plans hold the codes and scales they point into
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if "list" in legs:
        nxt.update(tensor_list_leg(pulse, specs, offs, W, b_old, changed, dev))
    del W, b_old
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if "loco" in legs:
        nxt.update(loco_leg(pulse, dev, not args.no_cpu_baseline))
    if nxt:
        result["next_rows"] = nxt
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ---- achievable bandwidth on this GPU, and each stage against the probe of its mix
    if args.probe_gib > 0:
        ach = achievable_probes(dev, gib=args.probe_gib)
        result["achievable"] = ach
        for k in stages:
            add_achievable(st_out[k], ach, READ_FRACTION[k](d, c))
        if "encode_apply" in result:
            add_achievable(result["encode_apply"], ach, READ_FRACTION["encode_apply"](d, c))
        rf = READ_FRACTION[dom](d, c)
        name, gbps = nearest_probe(ach, rf)
        roofline["achievable"] = {"probe": name, "GBps": gbps, "frac": round(roofline["achieved"] / gbps, 4)}

    # ---- the other configurations, each on its own
    cfgs = [x for x in args.configs.split(",") if x and x != "none"]
    if cfgs:
        per = {}
        fns = {"c1": config_c1, "c3": config_c3, "c4": config_c4, "c5": config_c5}
        for k in cfgs:
            log(f"configuration {k}")
            per[k] = fns[k](pulse, dev)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        result["configs"] = per
    print(json.dumps(result), flush=True)


def line_count(idx, count, base_elems, esz, line=64):
    """Distinct `line`-byte lines that the first `count` of an ascending index
    list land in (element size esz, the indexed view starting base_elems
    elements into a 256-byte aligned allocation)."""
    import torch

    if count <= 0:
        return 0
    l = torch.div(idx[:count].to(torch.int64) + base_elems, line // esz, rounding_mode="floor")
    return int((l[1:] != l[:-1]).sum().item()) + 1


def line_floor(ms, lines, stream_bytes):
    """A scatter's memory-side floor: every 64-byte line it touches is read
    and written whole (a partially written line costs the memory side a read
    of it), plus the entry stream it reads."""
    b = 2 * 64 * lines + stream_bytes
    return {"touched_lines": lines, "line_floor_GB": round(b / 1e9, 3),
            "line_floor_GBps": round(b / (ms / 1e3) / 1e9, 1) if ms > 0 else None}


def _leg(ms, launches, alg_bytes, **extra):
    secs = ms / 1e3
    out = {"ms": round(ms, 3), "launches": launches, "alg_GB": round(alg_bytes / 1e9, 3),
           "GBps": round(alg_bytes / secs / 1e9, 1), "frac_hbm": round(alg_bytes / secs / PEAK_HBM, 4)}
    out.update(extra)
    return out


def tensor_list_leg(pulse, specs, offs, W, b_old, changed, dev):
    """One launch over the whole tensor list (771 tensors of the Qwen2.5-32B
    shape, each addressed through the host-prepared table) against one
    pulse_cast_diff launch per tensor, both writing the patch only; then the
    list apply into the old views.  Checks: the two patch streams are equal
    tensor by tensor, their total is the main step's count, and the applied
    views equal the cast of the masters."""
    import torch

    nt = len(specs)
    views = [b_old[offs[i]: offs[i] + s.numel] for i, s in enumerate(specs)]
    masters = [W[offs[i]: offs[i] + s.numel] for i, s in enumerate(specs)]
    caps = [s.numel // 8 + 1024 for s in specs]  # 12.5% per tensor (+ slack for tiny ones)
    coff = [0]
    for c in caps:
        coff.append(coff[-1] + (c + 3) // 4 * 4)
    cap = coff[-1]
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    val = torch.empty(cap, dtype=torch.int16, device=dev)
    idx2 = torch.empty(cap, dtype=torch.int32, device=dev)
    val2 = torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(nt, dtype=torch.int64, device=dev)
    seg_off = torch.zeros(nt + 1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    table = pulse.SegmentTable(masters, views)
    ws_seg = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_SEGMENTS, table.ntiles, 0, dev)
    ws_cd = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, max(s.numel for s in specs), 0, dev)
    log(f"tensor-list leg: {nt} tensors, {table.ntiles} tiles")

    def per_tensor():
        for i in range(nt):
            pulse.pulse_cast_diff(masters[i], views[i], None, None, idx2[coff[i]: coff[i] + caps[i]],
                                  val2[coff[i]: coff[i] + caps[i]], cnt[i:i + 1], st, ws_cd)

    def one_launch():
        pulse.pulse_cast_diff_segments(table, idx, val, seg_off, st, ws_seg)

    times = {}
    for name, fn in (("per_tensor", per_tensor), ("list", one_launch)):
        fn()  # warm-up
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        fn()
        ev[1].record()
        torch.cuda.synchronize()
        times[name] = ev[0].elapsed_time(ev[1])
    if int(st.item()) != 0:
        raise SystemExit(f"tensor-list leg: device status {int(st.item())}")
    so = seg_off.cpu().tolist()
    cn = cnt.cpu().tolist()
    if so[-1] != changed:
        raise SystemExit(f"tensor-list leg: {so[-1]} entries, the main step found {changed}")
    for i in range(nt):
        m = so[i + 1] - so[i]
        if m != cn[i] or not (torch.equal(idx[so[i]: so[i + 1]], idx2[coff[i]: coff[i] + m]) and
                              torch.equal(val[so[i]: so[i + 1]], val2[coff[i]: coff[i] + m])):
            raise SystemExit(f"tensor-list leg: tensor {i} differs between the list call and its own call")
    del idx2, val2
    vt = pulse.ViewTable(views)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    pulse.pulse_apply_patch_segments(vt, idx, val, seg_off, st, max_count=so[-1])
    ev[1].record()
    torch.cuda.synchronize()
    t_apply = ev[0].elapsed_time(ev[1])
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.int16, device=dev)
    for i in range(nt):
        pulse.pulse_cast_diff(masters[i], b_new=tmp[: specs[i].numel])
        if not views_equal(views[i], tmp[: specs[i].numel]):
            raise SystemExit(f"tensor-list leg: view {i} differs from the cast of its masters after the apply")
    if int(st.item()) != 0:
        raise SystemExit(f"tensor-list leg: device status {int(st.item())} after the apply")
    n = sum(s.numel for s in specs)
    lines = sum(line_count(idx[so[i]:], so[i + 1] - so[i], offs[i], 2) for i in range(nt))
    log(f"tensor-list leg: one launch {times['list']:.2f} ms, {nt} launches {times['per_tensor']:.2f} ms")
    a_cd = n * 6 + 6 * changed  # read masters (4) + old view (2), write the patch
    return {"cast_diff_list": _leg(times["list"], 1, a_cd, tensors=nt, tiles=table.ntiles,
                                   checked="equal, tensor by tensor, to one pulse_cast_diff per tensor"),
            "cast_diff_per_tensor": _leg(times["per_tensor"], nt, a_cd),
            "apply_list": _leg(t_apply, 1, 8 * changed, checked="every view equals the cast of its masters",
                               **line_floor(t_apply, lines, 6 * changed))}


def patch_stream_leg(pulse, chunks, W, b_old, stage, idx, val, cnt, status, ws_cd, dev, with_oracle):
    """Compression of the patch stream over the whole weight set: per chunk the
    sender's patch (cast/diff/compact, untimed) is packed and LZ4-encoded (timed,
    the sender's side), then LZ4-decoded and unpacked (timed, the receiver's
    side); the unpacked patch must equal the original entry for entry."""
    import numpy as np
    import torch

    cap = idx.numel()
    nb = pulse.patch_packed_bytes(cap)
    packed = torch.empty(nb, dtype=torch.uint8, device=dev)
    back = torch.empty(nb, dtype=torch.uint8, device=dev)
    pcap = pulse.lz4_payload_bound(nb)
    payload = torch.empty(pcap, dtype=torch.uint8, device=dev)
    nblk = nb // BLOCK
    sizes = torch.empty(nblk, dtype=torch.int32, device=dev)
    offs = torch.empty(nblk, dtype=torch.int64, device=dev)
    tot = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    idx2 = torch.empty_like(idx)
    val2 = torch.empty_like(val)
    ws_en = pulse.workspace(pulse.PULSE_OP_LZ4_ENCODE, nb, BLOCK, dev)
    ws_de = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nblk, pcap, dev)
    ws_up = pulse.workspace(pulse.PULSE_OP_PATCH_UNPACK, cap, 0, dev)
    t = {"pack": 0.0, "encode": 0.0, "decode": 0.0, "unpack": 0.0}
    entries = 0
    packed_total = 0
    sample = None
    for k, (s0, e0, _) in enumerate(chunks):
        m = e0 - s0
        pulse.pulse_cast_diff(W[s0:e0], b_old[s0:e0], stage[:m], None, idx, val, cnt[k:k + 1], status, ws_cd)
        count = int(cnt[k].item())
        pb = pulse.patch_packed_bytes(count)
        nbk = pb // BLOCK
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record()
        pulse.patch_pack(idx, val, count, packed)
        ev[1].record()
        pulse.lz4_encode_blocks(packed, payload, sizes, offs, tot[k:k + 1], status, ws_en, nbytes=pb)
        ev[2].record()
        pulse.lz4_decode_blocks(payload, offs[:nbk], sizes[:nbk], back, status, ws_de, mode=0, nbytes=pb,
                                payload_bytes=pcap)
        ev[3].record()
        pulse.patch_unpack(back, count, idx2, val2, status, ws_up)
        ev[4].record()
        torch.cuda.synchronize()
        for i, key in enumerate(("pack", "encode", "decode", "unpack")):
            t[key] += ev[i].elapsed_time(ev[i + 1])
        if not (torch.equal(idx2[:count], idx[:count]) and torch.equal(val2[:count], val[:count])):
            raise SystemExit(f"patch-stream leg: chunk {k} did not round-trip")
        if k == 1 and with_oracle:
            n_s = min(count, 1 << 22)
            sample = (idx[:n_s].cpu().numpy(), val[:n_s].cpu().numpy().view(np.uint16))
        entries += count
        packed_total += pb
    if int(status.item()) != 0:
        raise SystemExit(f"patch-stream leg: device status {int(status.item())}")
    comp = int(tot.sum().item())
    cpe = comp / entries
    log(f"patch-stream leg: {entries} entries, {comp} compressed bytes ({cpe:.3f} B per entry)")
    L = len(chunks)
    out = {"patch_pack": _leg(t["pack"], L, 12 * entries, entries=entries),
           "patch_lz4_encode": _leg(t["encode"], L, packed_total + comp, compressed_bytes=comp,
                                    bytes_per_entry=round(cpe, 4), raw_bytes_per_entry=6,
                                    checked="decode + unpack == the patch, every chunk"),
           "patch_lz4_decode": _leg(t["decode"], L, comp + packed_total),
           "patch_unpack": _leg(t["unpack"], L, 12 * entries)}
    if sample is not None:  # the CPU baseline of this leg
        import oracle

        t0 = time.perf_counter()
        oracle.patch_compress(*sample)
        secs = time.perf_counter() - t0
        out["patch_lz4_encode"]["cpu_baseline"] = {
            "kind": "oracle", "GBps": round(6 * sample[0].size / secs / 1e9, 3), "cores": 1,
            "sample": f"first {sample[0].size} entries of chunk 1, pack + LZ4 encode, {secs:.2f} s"}
    return out


def fp8_view_leg(pulse, specs, chunks, offs, qplans, W, b_old, stage, dev, with_oracle):
    """Deltas of the FP8 served view over the whole weight set: per chunk, the
    old view and the sender's new view are quantised (untimed, FP8 groups laid
    end to end), then fp8_view_delta and fp8_view_apply are timed; the applied
    old quantisation must equal the new one bit for bit."""
    import torch

    max_q = max(sum(r * c for _, r, c in plan) for plan in qplans)
    max_s = max(sum(((r + 127) // 128) * ((c + 127) // 128) for _, r, c in plan) for plan in qplans)
    co = torch.empty(max_q, dtype=torch.uint8, device=dev)
    cn = torch.empty(max_q, dtype=torch.uint8, device=dev)
    so = torch.empty(max_s, dtype=torch.float32, device=dev)
    sn = torch.empty(max_s, dtype=torch.float32, device=dev)
    ccap = max_q // 10
    ci = torch.empty(ccap, dtype=torch.int32, device=dev)
    cv = torch.empty(ccap, dtype=torch.uint8, device=dev)
    si = torch.empty(max_s, dtype=torch.int32, device=dev)
    sv = torch.empty(max_s, dtype=torch.float32, device=dev)
    cc = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    sc = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = pulse.workspace(pulse.PULSE_OP_FP8_DELTA, max_q, 0, dev)
    t_delta = t_apply = 0.0
    lines = 0
    nq_tot = ns_tot = 0
    ok = True
    sample = None
    for k, (s0, e0, tids) in enumerate(chunks):
        m = e0 - s0
        pulse.pulse_cast_diff(W[s0:e0], b_new=stage[:m])
        qo = so_o = 0
        for (g, rows, cols) in qplans[k]:
            nq, ns = rows * cols, ((rows + 127) // 128) * ((cols + 127) // 128)
            pulse.fp8_block_quant([b_old[offs[i]: offs[i] + specs[i].numel].view(specs[i].shape) for i in g],
                                  co[qo:qo + nq], so[so_o:so_o + ns])
            pulse.fp8_block_quant([stage[offs[i] - s0: offs[i] - s0 + specs[i].numel].view(specs[i].shape)
                                   for i in g], cn[qo:qo + nq], sn[so_o:so_o + ns])
            qo, so_o = qo + nq, so_o + ns
        if k == 1 and with_oracle:  # a host copy of 64 Mi codes for the oracle's timing
            sample = (co[:1 << 26].cpu().numpy(), cn[:1 << 26].cpu().numpy())
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        pulse.fp8_view_delta(co[:qo], cn[:qo], so[:so_o], sn[:so_o], ci, cv, cc[k:k + 1], si, sv, sc[k:k + 1],
                             st, ws)
        ev[1].record()
        pulse.fp8_view_apply(co[:qo], so[:so_o], ci, cv, cc[k:k + 1], si, sv, sc[k:k + 1], st)
        ev[2].record()
        torch.cuda.synchronize()
        t_delta += ev[0].elapsed_time(ev[1])
        t_apply += ev[1].elapsed_time(ev[2])
        lines += line_count(ci, int(cc[k].item()), 0, 1) + line_count(si, int(sc[k].item()), 0, 4)
        ok = ok and views_equal(co[:qo], cn[:qo]) and views_equal(so[:so_o].view(torch.int32),
                                                                     sn[:so_o].view(torch.int32))
        nq_tot, ns_tot = nq_tot + qo, ns_tot + so_o
    if int(st.item()) != 0 or not ok:
        raise SystemExit(f"FP8-view delta leg failed (status {int(st.item())}, round trip {ok})")
    ncodes = int(cc.sum().item())
    nscales = int(sc.sum().item())
    dq = ncodes / nq_tot
    log(f"FP8-view delta leg: {nq_tot} codes, {ncodes} changed ({100 * dq:.3f}%), {nscales} scales changed")
    a_delta = 2 * nq_tot + 8 * ns_tot + 5 * ncodes + 8 * nscales
    a_apply = 6 * ncodes + 12 * nscales
    out = {"fp8_view_delta": _leg(t_delta, len(chunks), a_delta, changed_codes_fraction=round(dq, 6),
                                  changed_scales=nscales, codes=nq_tot,
                                  checked="apply(quant(old), delta) == quant(new) on every chunk"),
           "fp8_view_apply": _leg(t_apply, len(chunks), a_apply,
                                  **line_floor(t_apply, lines, 5 * ncodes + 8 * nscales))}
    if sample is not None:  # the CPU baseline of this leg
        import numpy as np

        import oracle

        ones = np.ones(1, np.float32)
        t = time.perf_counter()
        oracle.fp8_delta(sample[0], sample[1], ones, ones)
        secs = time.perf_counter() - t
        out["fp8_view_delta"]["cpu_baseline"] = {
            "kind": "oracle", "GBps": round(2 * sample[0].size / secs / 1e9, 3), "cores": 1,
            "sample": f"{sample[0].size} codes of chunk 1, {secs:.2f} s"}
    return out


LOCO_WORKLOAD = 6


def loco_leg(pulse, dev, with_oracle):
    """PULSELoCo gate over a Qwen2.5-7B-shaped FP32 checkpoint: round 1 (untimed)
    fills the error-feedback buffer, round 2 is timed, chunk by chunk, with the
    receiver's accumulation of each chunk's patch.  The round-2 entries of the
    first 2^22 elements are checked against the gate's defining properties
    (torch's float32 add and BF16 cast on the host copies)."""
    import torch

    import workload

    specs = workload.qwen25_7b_specs()
    n = workload.total_numel(specs)
    chunks, offs = build_plan(specs, layers_per_chunk=8)
    theta = torch.empty(n, dtype=torch.float32, device=dev)
    delta = torch.empty(n, dtype=torch.float32, device=dev)
    resid = torch.zeros(n, dtype=torch.float32, device=dev)
    acc = torch.zeros(n, dtype=torch.float32, device=dev)
    maxc = max(e - s for s, e, _ in chunks)
    cap = maxc // 2
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    val = torch.empty(cap, dtype=torch.float32, device=dev)
    cnt = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = pulse.workspace(pulse.PULSE_OP_LOCO_GATE, maxc, 0, dev)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    for ti, s in enumerate(specs):
        workload.fill_init(theta[offs[ti]: offs[ti] + s.numel], LOCO_WORKLOAD, ti, s.kind)
    log(f"LoCo leg: {n} params, checkpoint drawn")
    for rnd in (1, 2):
        for ti, s in enumerate(specs):
            workload.pseudo_gradient(delta[offs[ti]: offs[ti] + s.numel], LOCO_WORKLOAD, ti, rnd, tmp=tmp)
        torch.cuda.synchronize()
        log(f"LoCo leg: round {rnd} pseudo-gradient drawn")
        if rnd == 1:
            for k, (s0, e0, _) in enumerate(chunks):
                pulse.pulse_loco_gate(theta[s0:e0], delta[s0:e0], resid[s0:e0], idx, val, cnt[k:k + 1], st, ws)
            continue
        chk = 1 << 22
        host_in = (theta[:chk].cpu().numpy(), delta[:chk].cpu().numpy(), resid[:chk].cpu().numpy())
        t_gate = t_acc = 0.0
        acc_lines = 0
        first = None
        for k, (s0, e0, _) in enumerate(chunks):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            pulse.pulse_loco_gate(theta[s0:e0], delta[s0:e0], resid[s0:e0], idx, val, cnt[k:k + 1], st, ws)
            ev[1].record()
            pulse.pulse_loco_accumulate(acc[s0:e0], idx, val, cnt[k:k + 1], st)
            ev[2].record()
            torch.cuda.synchronize()
            t_gate += ev[0].elapsed_time(ev[1])
            t_acc += ev[1].elapsed_time(ev[2])
            acc_lines += line_count(idx, int(cnt[k].item()), s0, 4)
            if k == 0:
                m0 = int(cnt[0].item())
                first = (idx[:min(m0, chk)].cpu().numpy(), val[:min(m0, chk)].cpu().numpy(),
                         resid[:chk].cpu().numpy())
    del tmp
    if int(st.item()) != 0:
        raise SystemExit(f"LoCo leg: device status {int(st.item())}")
    sent = int(cnt.sum().item())
    dg = sent / n
    out = {}
    # properties of the first 2^22 elements (any size): the sent entries carry
    # a = resid + delta and leave 0 behind, the rest keep a, and exactly the
    # entries whose BF16 view a would move were sent
    th, de, r0 = (torch.from_numpy(x) for x in host_in)
    gi, gv, gr = (torch.from_numpy(x) for x in first)
    a = r0 + de
    vis = (th + a).to(torch.bfloat16).view(torch.int16) != th.to(torch.bfloat16).view(torch.int16)
    ref_idx = torch.nonzero(vis).flatten().to(torch.int32)
    kk = ref_idx.numel()
    keep = torch.where(vis, torch.zeros_like(a), a)
    if not (torch.equal(gi[:kk], ref_idx) and torch.equal(gv[:kk].view(torch.int32), a[vis].view(torch.int32))
            and torch.equal(gr.view(torch.int32), keep.view(torch.int32)) and (gi.numel() == kk or int(gi[kk]) >= chk)):
        raise SystemExit("LoCo leg: the first 2^22 elements break the gate's properties")
    log(f"LoCo leg: {n} params, {sent} entries sent ({100 * dg:.3f}%)")
    a_gate = 16 * n + 8 * sent     # read theta, delta, resid; write resid; write the entries
    a_acc = 16 * sent              # read the entries, read + write acc at them
    out["loco_gate"] = _leg(t_gate, len(chunks), a_gate, sent_fraction=round(dg, 6), params=n,
                            workload="Qwen2.5-7B-shaped FP32 checkpoint, round 2 of H=8 local steps at lr 3e-6",
                            checked="first 2^22 elements: sent = visible, values and buffer exact")
    out["loco_accumulate"] = _leg(t_acc, len(chunks), a_acc, **line_floor(t_acc, acc_lines, 8 * sent))
    if with_oracle:  # the CPU baseline of this leg
        import oracle

        t = time.perf_counter()
        oracle.loco_gate(*host_in)
        secs = time.perf_counter() - t
        out["loco_gate"]["cpu_baseline"] = {"kind": "oracle", "GBps": round(16 * chk / secs / 1e9, 3), "cores": 1,
                                            "sample": f"first {chk} elements of round 2, {secs:.3f} s"}
    return out


# ---------------------------------------------------------------------------
# read share of each stage's algorithmic bytes (d: changed fraction, c: LZ4
# bytes per element), to pick the probe with the same read:write mix
READ_FRACTION = {
    "encode": lambda d, c: 6 / (8 + 6 * d + c),
    "cast_diff": lambda d, c: 6 / (8 + 6 * d),
    "receiver": lambda d, c: (2 + 6 * d) / (3 + 8 * d),
    "apply_patch": lambda d, c: 0.75,
    "fp8_quant": lambda d, c: 2 / 3,
    "lz4_encode": lambda d, c: 4 / (4 + c),
    "lz4_decode": lambda d, c: (2 + c) / (4 + c),
    "encode_apply": lambda d, c: (6 + 6 * d) / (8 + 14 * d),
}


def encode_apply_leg(pulse, chunks, W, b_old, b_recv, stage, idx, val, status, ws_cd, reps, dev):
    """The metric's own quantity, the patch path alone: pulse_cast_diff (cast,
    diff and compaction against the old view, the new view written) then
    pulse_apply_patch into the receiver's view, chunk by chunk over the same
    set; one checked pass, then `reps` timed passes.  Every pass after the
    first writes the same values to the same positions (the same stores); the
    receiver's view is set back to the old view afterwards."""
    import torch

    cnt = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    cap = idx.numel()
    te = ta = 0.0
    lines = 0
    for r in range(reps + 1):
        ev = []
        for ci, (s0, e0, _) in enumerate(chunks):
            m = e0 - s0
            e = [_ev() for _ in range(3)]
            e[0].record()
            pulse.pulse_cast_diff(W[s0:e0], b_old[s0:e0], stage[:m], None, idx, val, cnt[ci:ci + 1], status, ws_cd)
            e[1].record()
            if r == 0:  # (the checked pass, untimed) the receiver view's lines this chunk's patch lands in
                lines += line_count(idx, int(cnt[ci].item()), s0, 2)
            pulse.pulse_apply_patch(b_recv[s0:e0], idx, val, cnt[ci:ci + 1], status, max_count=cap)
            e[2].record()
            ev.append(e)
            if r == 0 and not views_equal(b_recv[s0:e0], stage[:m]):
                raise SystemExit(f"encode+apply: chunk {ci}: the patched view differs from the new view")
        torch.cuda.synchronize()
        if r:
            te += sum(e[0].elapsed_time(e[1]) for e in ev)
            ta += sum(e[1].elapsed_time(e[2]) for e in ev)
    if int(status.item()) != 0:
        raise SystemExit(f"encode+apply: device status {int(status.item())}")
    b_recv.copy_(b_old)
    torch.cuda.synchronize()
    n = sum(e - s for s, e, _ in chunks)
    d = int(cnt.sum().item()) / n
    me, ma = te / reps, ta / reps
    a_enc, a_app = n * (8 + 6 * d), n * 8 * d
    secs = (me + ma) / 1e3
    return {"ms": round(me + ma, 3), "encode_ms": round(me, 3), "apply_ms": round(ma, 3),
            "apply_line_floor": line_floor(ma, lines, 6 * int(cnt.sum().item())),
            "GBps_weights": round(2 * n / secs / 1e9, 1), "alg_GB": round((a_enc + a_app) / 1e9, 3),
            "GBps": round((a_enc + a_app) / secs / 1e9, 1), "frac_hbm": round((a_enc + a_app) / secs / PEAK_HBM, 4),
            "encode_frac_hbm": round(a_enc / (me / 1e3) / PEAK_HBM, 4),
            "apply_frac_hbm": round(a_app / (ma / 1e3) / PEAK_HBM, 4), "launches": 2 * len(chunks),
            "calls": "pulse_cast_diff, then pulse_apply_patch, per chunk",
            "alg_bytes_per_element": "8 + 6 d (encode) + 8 d (apply)"}


# ---------------------------------------------------------------------------
# achievable bandwidth: our own 16-byte non-temporal streams
PROBE_MIXES = {"read": (1, 0), "write": (0, 1), "copy": (1, 1), "read2_write1": (2, 1), "read3_write1": (3, 1)}


def achievable_probes(dev, gib=4.0, reps=5, blocks=4096):
    """Plain streams (sparse_delta_codec_amd/csrc/probe.hip, 16-byte
    non-temporal loads and stores, 4 KiB per wave and stream per step) over
    `gib` GiB per stream, at the read:write mixes of the codec's kernels; the
    median of `reps` timed launches after one untimed.  A torch device copy is
    reported beside them."""
    import ctypes

    import torch

    L = ctypes.CDLL(os.path.join(ROOT, "sparse_delta_codec_amd", "libpulse_probe.so"))
    L.probe_stream.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.c_int32, ctypes.c_void_p]
    L.probe_stream.restype = ctypes.c_int
    n = int(gib * 2 ** 30) // 16
    bufs = [torch.full((n * 16,), k + 1, dtype=torch.uint8, device=dev) for k in range(4)]
    ptr = [ctypes.c_void_p(b.data_ptr()) for b in bufs]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}

    def timed(fn):
        ts = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    for name, (nr, w) in PROBE_MIXES.items():
        def fn():
            rc = L.probe_stream(ptr[0], ptr[1], ptr[2], ptr[3], n, nr, w, blocks, stream)
            if rc != 0:
                raise SystemExit(f"probe {name}: launch failed ({rc})")
        ms = timed(fn)
        out[name] = {"GBps": round((nr + w) * n * 16 / (ms / 1e3) / 1e9, 1), "read_fraction": round(nr / (nr + w), 3)}
    ms = timed(lambda: bufs[3].copy_(bufs[0]))
    out["torch_copy"] = {"GBps": round(2 * n * 16 / (ms / 1e3) / 1e9, 1), "read_fraction": 0.5}
    del bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def nearest_probe(achievable, read_fraction):
    """The probe whose read:write mix is closest to a kernel's (by read share of its bytes)."""
    name = min(PROBE_MIXES, key=lambda k: abs(PROBE_MIXES[k][0] / sum(PROBE_MIXES[k]) - read_fraction))
    return name, achievable[name]["GBps"]


def add_achievable(block, achievable, read_fraction):
    name, gbps = nearest_probe(achievable, read_fraction)
    block["achievable"] = {"probe": name, "GBps": gbps, "frac": round(block["GBps"] / gbps, 4)}


# ---------------------------------------------------------------------------
# the oracle on the host cores
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_sample_run(w, bo, groups, workers, block=BLOCK):
    """The whole hot path on the oracle over host arrays (w: float32 masters,
    bo: the old BF16 view, groups: FP8 stacks as [(offset, shape)]), its calls
    spread over `workers` threads, one independent piece per call: ranges of
    whole LZ4 blocks for cast + diff + compaction, apply, LZ4 encode and
    decode + XOR; 128-row bands for FP8.  Returns the seconds taken."""
    import concurrent.futures

    import numpy as np

    import oracle

    piece = 1 << 24
    rng = [(a, min(w.size, a + piece)) for a in range(0, w.size, piece)]
    pool = concurrent.futures.ThreadPoolExecutor(workers)
    recv = np.empty_like(bo)
    t = time.perf_counter()

    def step_patch(r):
        a, b = r
        res = oracle.cast_diff(w[a:b], bo[a:b], want_mask=False)
        recv[a:b] = oracle.apply_patch(bo[a:b], res["idx"], res["val"])[0]
        enc = oracle.lz4_encode_blocks(bo[a:b], block, src_xor=res["b_new"])
        oracle.lz4_decode_blocks(enc["payload"], enc["offsets"], enc["sizes"], recv[a:b], mode=1)
    list(pool.map(step_patch, rng))
    bands = []
    for g in groups:
        R, cols = sum(sh[0] for _, sh in g), g[0][1][1]
        for r0 in range(0, R, 128):
            bands.append((g, r0, min(R, r0 + 128), cols))

    def step_fp8(band):
        g, r0, r1, cols = band
        parts, base = [], 0
        for off, sh in g:
            a, b = max(r0, base), min(r1, base + sh[0])
            if a < b:
                parts.append(recv[off + (a - base) * cols: off + (b - base) * cols].reshape(b - a, cols))
            base += sh[0]
        oracle.fp8_block_quant([parts[0] if len(parts) == 1 else np.concatenate(parts, 0)])
    list(pool.map(step_fp8, bands))
    secs = time.perf_counter() - t
    pool.shutdown()
    return secs


def cpu_baseline(specs, offs, W, b_old, frac):
    """The oracle (plain single-threaded C calls) on a bounded sample of the same
    workload, decoder layer 0 (its 12 tensors, about 488 M parameters): all
    five steps over host copies of the same inputs, FP8 on the layer's stacked
    groups.  Timed with its calls on one host thread (about 13 s) and spread
    over every usable host core (one independent piece per call).  `frac` < 1
    shortens the sample (the FP8 step is then skipped)."""
    lay = [i for i, s in enumerate(specs) if s.name.startswith("l0.")]
    last = lay[-1]
    s0, e0 = offs[lay[0]], offs[last] + specs[last].numel
    m = int((e0 - s0) * min(frac, 1.0)) // 8 * 8
    import numpy as np

    w = W[s0:s0 + m].cpu().numpy()
    bo = b_old[s0:s0 + m].cpu().numpy().view(np.uint16)
    groups = []
    if frac >= 1.0:
        for g in quant_groups(specs, lay):
            groups.append([(offs[i] - s0, specs[i].shape) for i in g])
    cores = len(os.sched_getaffinity(0))
    log(f"oracle sample: {m} params, 1 thread")
    t1 = oracle_sample_run(w, bo, groups, 1)
    log(f"oracle sample: {t1:.1f} s on 1 thread; now {cores} threads")
    tn = oracle_sample_run(w, bo, groups, cores)
    log(f"oracle sample: {tn:.1f} s on {cores} threads")
    what = (f"decoder layer 0 of the same workload ({m} params{'' if frac >= 1 else ', FP8 step skipped'}), "
            f"all five steps")
    return {"value": round(2 * m / tn / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}, {tn:.2f} s on {cores} host threads", "cpu_model": cpu_model(),
            "one_core": {"value": round(2 * m / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "sample": f"{what}, {t1:.1f} s on one host thread"}}


# ---------------------------------------------------------------------------
# the other configurations (each on its own, after the main workload is freed)
def _ev():
    import torch

    return torch.cuda.Event(enable_timing=True)


def _flush(buf, k):
    buf.fill_(k & 0xFF)  # rewrites 512 MiB: the 256 MB MALL and the L2s hold none of the next inputs


def config_c1(pulse, dev, reps=20):
    """C1: one 4096 x 1024 FP32 tensor (numpy default_rng(0)), one step:
    pulse_cast_diff (cast, diff, patch; new view written) then
    pulse_apply_patch into a copy of the old view; caches flushed before each
    rep, median of `reps`."""
    import numpy as np
    import torch

    import workload

    w0, w1 = workload.c1_masters()
    n = w0.size
    W0 = torch.from_numpy(w0.reshape(-1)).to(dev)
    W1 = torch.from_numpy(w1.reshape(-1)).to(dev)
    b0 = torch.empty(n, dtype=torch.int16, device=dev)
    pulse.pulse_cast_diff(W0, b_new=b0)
    recv, stage = torch.empty_like(b0), torch.empty_like(b0)
    idx, val = torch.empty(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.int16, device=dev)
    cnt, st = torch.zeros(1, dtype=torch.int64, device=dev), torch.zeros(1, dtype=torch.int32, device=dev)
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, n, 0, dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    te, ta = [], []
    for r in range(reps + 2):
        recv.copy_(b0)
        _flush(flush, r)
        e = [_ev() for _ in range(3)]
        e[0].record()
        pulse.pulse_cast_diff(W1, b0, stage, None, idx, val, cnt, st, ws)
        e[1].record()
        pulse.pulse_apply_patch(recv, idx, val, cnt, st, max_count=n)
        e[2].record()
        torch.cuda.synchronize()
        if r >= 2:
            te.append(e[0].elapsed_time(e[1]))
            ta.append(e[1].elapsed_time(e[2]))
    if int(st.item()) != 0 or not torch.equal(recv, stage):
        raise SystemExit("C1: the patched old view differs from the new view")
    count = int(cnt.item())
    d = count / n
    me, ma = float(np.median(te)), float(np.median(ta))
    a = n * (8 + 6 * d) + n * 8 * d
    return {"workload": "C1: 4096x1024 FP32, one step at lr 3e-6", "params": n, "changed_fraction": round(d, 6),
            "encode_us": round(1e3 * me, 1), "apply_us": round(1e3 * ma, 1),
            "GBps_weights": round(2 * n / ((me + ma) / 1e3) / 1e9, 1),
            "alg_GB": round(a / 1e9, 4), "frac_hbm": round(a / ((me + ma) / 1e3) / PEAK_HBM, 4),
            "note": f"median of {reps}, caches flushed before each rep; launch-bound at this size"}


def config_c3(pulse, dev, steps=20):
    """C3: the Llama-3-8B-shaped set, 20 chained steps.  Per step and chunk:
    pulse_cast_diff against the sender's view (updated in place) and
    pulse_apply_patch into the receiver's view; after the last step the
    receiver's view must equal the sender's."""
    import torch

    import workload

    specs = workload.llama3_8b_specs()
    n = workload.total_numel(specs)
    chunks, offs = build_plan(specs)
    mc = max(e - s for s, e, _ in chunks)
    W = torch.empty(n, dtype=torch.float32, device=dev)
    prev = torch.empty(n, dtype=torch.int16, device=dev)
    for ti, s in enumerate(specs):
        workload.fill_init(W[offs[ti]: offs[ti] + s.numel], 3, ti, s.kind)
        pulse.pulse_cast_diff(W[offs[ti]: offs[ti] + s.numel], b_new=prev[offs[ti]: offs[ti] + s.numel])
    recv = prev.clone()
    cap = int(mc * PATCH_CAP_FRAC)
    idx, val = torch.empty(cap, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, mc, 0, dev)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    te = ta = 0.0
    changed = 0
    for step in range(1, steps + 1):
        for ti, s in enumerate(specs):
            workload.apply_step(W[offs[ti]: offs[ti] + s.numel], 3, ti, step, tmp=tmp)
        ev = []
        for ci, (s0, e0, _) in enumerate(chunks):
            e = [_ev() for _ in range(3)]
            e[0].record()
            pulse.pulse_cast_diff(W[s0:e0], prev[s0:e0], prev[s0:e0], None, idx, val, cnt[ci:ci + 1], st, ws)
            e[1].record()
            pulse.pulse_apply_patch(recv[s0:e0], idx, val, cnt[ci:ci + 1], st, max_count=cap)
            e[2].record()
            ev.append(e)
        torch.cuda.synchronize()
        te += sum(e[0].elapsed_time(e[1]) for e in ev)
        ta += sum(e[1].elapsed_time(e[2]) for e in ev)
        changed += int(cnt.sum().item())
    if int(st.item()) != 0 or not views_equal(recv, prev):
        raise SystemExit("C3: the chained receiver view differs from the sender's after the last step")
    d = changed / (n * steps)
    me, ma = te / steps, ta / steps
    a = n * (8 + 6 * d) + n * 8 * d
    return {"workload": f"C3: Llama-3-8B-shaped set, {steps} chained steps at lr 3e-6", "params": n,
            "changed_fraction": round(d, 6), "encode_ms_per_step": round(me, 3), "apply_ms_per_step": round(ma, 3),
            "GBps_weights": round(2 * n / ((me + ma) / 1e3) / 1e9, 1), "alg_GB_per_step": round(a / 1e9, 3),
            "frac_hbm": round(a / ((me + ma) / 1e3) / PEAK_HBM, 4),
            "checked": "receiver view == sender view after the last step"}


def config_c4(pulse, dev, reps=3):
    """C4: the first 16e9 elements of the C2 set as two BF16 views; the XOR
    mask LZ4-encoded in 64 KiB blocks (lz4_encode_blocks over both views, the
    mask never written), then decoded and XORed into the old view in place
    (lz4_decode_blocks); every second decode takes the view back."""
    import torch

    import workload

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
    payload = torch.empty(int(nbytes * PAYLOAD_CAP_FRAC), dtype=torch.uint8, device=dev)
    sizes = torch.empty(nb, dtype=torch.int32, device=dev)
    offsets = torch.empty(nb, dtype=torch.int64, device=dev)
    total = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = pulse.workspace(pulse.PULSE_OP_LZ4_ENCODE, nbytes, BLOCK, dev)
    te, td = [], []
    for r in range(reps + 1):
        e = [_ev() for _ in range(2)]
        e[0].record()
        pulse.lz4_encode_blocks(old, payload, sizes, offsets, total, st, ws, src_xor=new)
        e[1].record()
        torch.cuda.synchronize()
        if r:
            te.append(e[0].elapsed_time(e[1]))
    tot = int(total.item())
    dws = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nb, tot, dev)
    for r in range(2 * reps):
        e = [_ev() for _ in range(2)]
        e[0].record()
        pulse.lz4_decode_blocks(payload, offsets, sizes, old, st, dws, mode=1, payload_bytes=tot)
        e[1].record()
        torch.cuda.synchronize()
        td.append(e[0].elapsed_time(e[1]))
        if r == 0 and not views_equal(old, new):
            raise SystemExit("C4: decode + XOR did not rebuild the new view")
    if int(st.item()) != 0:
        raise SystemExit(f"C4: device status {int(st.item())}")
    c = tot / n
    me, md = sum(te) / len(te), sum(td) / len(td)
    a_enc, a_dec = n * (4 + c), n * (4 + c)
    return {"workload": "C4: first 16e9 elements of the C2 set, XOR mask LZ4 path", "params": n,
            "compressed_bytes": tot, "ratio_of_mask": round(tot / nbytes, 5),
            "encode_ms": round(me, 3), "encode_GBps_alg": round(a_enc / (me / 1e3) / 1e9, 1),
            "encode_frac_hbm": round(a_enc / (me / 1e3) / PEAK_HBM, 4),
            "decode_ms": round(md, 3), "decode_GBps_mask": round(nbytes / (md / 1e3) / 1e9, 1),
            "decode_frac_hbm": round(a_dec / (md / 1e3) / PEAK_HBM, 4),
            "GBps_weights": round(2 * n / ((me + md) / 1e3) / 1e9, 1),
            "checked": "decode + XOR rebuilds the new view"}


def config_c5(pulse, dev, reps=3, experts_per_chunk=48):
    """C5: the Kimi-K2-shaped MoE layer share.  The sender: pulse_cast_diff
    (new view written) per chunk of 48 experts (and one for q/k/v); the
    receiver: pulse_apply_quant per chunk, the patch applied and [gate; up]
    per expert, down per expert and [q; k; v] quantised to E4M3 with FP32
    128x128 scales in one read of the view."""
    import torch

    import workload

    specs = workload.kimi_k2_layer_specs()
    n = workload.total_numel(specs)
    offs = [0]
    for s in specs:
        offs.append(offs[-1] + s.numel)
    E = 384
    chunks = [(3 * e0, 3 * min(E, e0 + experts_per_chunk)) for e0 in range(0, E, experts_per_chunk)]
    chunks.append((3 * E, len(specs)))
    mc = max(offs[b] - offs[a] for a, b in chunks)
    W = torch.empty(n, dtype=torch.float32, device=dev)
    b = torch.empty(n, dtype=torch.int16, device=dev)
    tmp = torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev)
    for ti, s in enumerate(specs):
        w = W[offs[ti]: offs[ti + 1]]
        workload.fill_init(w, 5, ti, s.kind)
        pulse.pulse_cast_diff(w, b_new=b[offs[ti]: offs[ti + 1]])
        workload.apply_step(w, 5, ti, 1, tmp=tmp)
    del tmp
    recv = b.clone()
    stage = torch.empty(mc, dtype=torch.int16, device=dev)
    cap = int(mc * PATCH_CAP_FRAC)
    idx, val = torch.empty(cap, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int16, device=dev)
    cnt = torch.zeros(len(chunks), dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF, mc, 0, dev)
    ws_aq = pulse.workspace(pulse.PULSE_OP_APPLY_QUANT, mc, 0, dev)
    codes = torch.empty(mc, dtype=torch.uint8, device=dev)
    scales = torch.empty(mc // 16384 + 1024, dtype=torch.float32, device=dev)
    plans = []
    n_quant = 0
    for a, z in chunks:
        base = offs[a]
        groups, co, so = [], 0, 0
        ts = list(range(a, z))
        if specs[a].name == "q":
            srcs = [(offs[t] - base, specs[t].shape[0]) for t in ts]
            stacks = [(srcs, specs[a].shape[1])]
        else:
            stacks = []
            for t in range(a, z, 3):  # gate, up, down of one expert
                stacks.append(([(offs[t] - base, specs[t].shape[0]), (offs[t + 1] - base, specs[t + 1].shape[0])],
                               specs[t].shape[1]))
                stacks.append(([(offs[t + 2] - base, specs[t + 2].shape[0])], specs[t + 2].shape[1]))
        for srcs, cols in stacks:
            R = sum(r for _, r in srcs)
            nsc = ((R + 127) // 128) * ((cols + 127) // 128)
            groups.append((srcs, cols, codes[co: co + R * cols], scales[so: so + nsc]))
            co, so = co + R * cols, so + nsc
        n_quant += co
        plans.append(pulse.pulse_apply_quant_plan(groups, offs[z] - base, device=dev))
    te, tr = [], []
    for r in range(reps + 1):
        recv.copy_(b)
        torch.cuda.synchronize()
        ev = []
        for ci, (a, z) in enumerate(chunks):
            s0, e0 = offs[a], offs[z]
            e = [_ev() for _ in range(3)]
            e[0].record()
            pulse.pulse_cast_diff(W[s0:e0], b[s0:e0], stage[:e0 - s0], None, idx, val, cnt[ci:ci + 1], st, ws)
            e[1].record()
            pulse.pulse_apply_quant(recv[s0:e0], idx, val, cnt[ci:ci + 1], plans[ci], st, ws_aq, max_count=cap)
            e[2].record()
            ev.append(e)
        torch.cuda.synchronize()
        if r:
            te.append(sum(e[0].elapsed_time(e[1]) for e in ev))
            tr.append(sum(e[1].elapsed_time(e[2]) for e in ev))
    if int(st.item()) != 0:
        raise SystemExit(f"C5: device status {int(st.item())}")
    changed = int(cnt.sum().item())
    d = changed / n
    me, mr = sum(te) / len(te), sum(tr) / len(tr)
    a = n * (8 + 6 * d) + n * 8 * d + 3 * n_quant + 4 * n_quant / 16384
    return {"workload": "C5: Kimi-K2-shaped MoE layer share (384 experts + q/k/v), one step at lr 3e-6",
            "params": n, "changed_fraction": round(d, 6), "fp8_params": n_quant,
            "encode_ms": round(me, 3), "receiver_ms": round(mr, 3),
            "GBps_weights": round(2 * n / ((me + mr) / 1e3) / 1e9, 1), "alg_GB": round(a / 1e9, 3),
            "frac_hbm": round(a / ((me + mr) / 1e3) / PEAK_HBM, 4),
            "launches": 2 * len(chunks), "receiver": "pulse_apply_quant ([gate; up], down per expert; [q; k; v])"}


if __name__ == "__main__":
    main()
