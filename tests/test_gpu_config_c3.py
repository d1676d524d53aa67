"""Full-size parity of C3 on the GPU, every element against the oracle: the
Llama-3-8B-shaped set over 20 chained steps.  Every step's count and patch
entries, and the receiver's view after every step, against the oracle's own
chain (its cast of the initial host masters, then its patches); after step
20 that chain equals the oracle's direct cast of the step-20 masters.  Four
tests of five steps share the chain through a module-scoped fixture, so the
chain's GPU and host memory is released when this module ends."""
import numpy as np
import pytest
import torch

import workload
from bench import build_plan
from tests import fullsize as fs

pytestmark = pytest.mark.gpu

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise  # on a GPU machine the HIP library must be there
    pulse = None


def say(msg):
    print(f"[cfg] {msg}", flush=True)


def new_ws(op, n, aux=0):
    return pulse.workspace(op, n, aux, "cuda")


@pytest.fixture(scope="module")
def c3():
    """The C3 chain's state across its four tests: masters, the sender's
    previous view and the receiver's view on the GPU, the oracle's own chain
    on the host."""
    dev = torch.device("cuda")
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
    chain = np.empty(n, np.uint16)  # the oracle's chain: its cast of W_0, then its patches
    for s0, e0, _ in chunks:
        fs.oracle_cast(fs.to_host(W[s0:e0], "w"), out=chain[s0:e0])
        fs.check_equal(fs.to_host(prev[s0:e0], "v"), chain[s0:e0], f"C3 chunk at {s0}: initial view")
    st = dict(specs=specs, n=n, chunks=chunks, offs=offs, W=W, prev=prev, recv=prev.clone(), chain=chain, step=0,
              tmp=torch.empty(max(s.numel for s in specs), dtype=torch.float32, device=dev),
              stage=torch.empty(max_chunk, dtype=torch.int16, device=dev),
              idx=torch.empty(int(max_chunk * 0.125), dtype=torch.int32, device=dev),
              val=torch.empty(int(max_chunk * 0.125), dtype=torch.int16, device=dev),
              cnt=torch.zeros(1, dtype=torch.int64, device=dev), st=torch.zeros(1, dtype=torch.int32, device=dev),
              ws=new_ws(pulse.PULSE_OP_CAST_DIFF, max_chunk))
    yield st
    st.clear()
    fs.release()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("first,last", [(1, 5), (6, 10), (11, 15), (16, 20)])
def test_c3_llama8b_chain_every_element(c3, first, last):
    """C3, steps first .. last of 20: per chunk pulse_cast_diff against the
    sender's previous view and pulse_apply_patch into the receiver's view;
    every step's count and entries equal the oracle's cast + diff +
    compaction against its own chain, and the receiver's view equals the
    oracle's chain after every step.  After step 20 the oracle's chain equals
    the oracle's direct cast of the step-20 masters (no drift)."""
    assert c3["step"] == first - 1, "the C3 tests run in order on one chain"
    specs, chunks, offs, W = c3["specs"], c3["chunks"], c3["offs"], c3["W"]
    prev, recv, chain, stage = c3["prev"], c3["recv"], c3["chain"], c3["stage"]
    idx, val, cnt, st = c3["idx"], c3["val"], c3["cnt"], c3["st"]
    for step in range(first, last + 1):
        for ti, s in enumerate(specs):
            workload.apply_step(W[offs[ti]: offs[ti] + s.numel], 3, ti, step, tmp=c3["tmp"])
        changed = 0
        for ci, (s0, e0, _) in enumerate(chunks):
            m = e0 - s0
            pulse.pulse_cast_diff(W[s0:e0], prev[s0:e0], stage[:m], None, idx, val, cnt, st, c3["ws"])
            torch.cuda.synchronize()
            count = int(cnt.item())
            assert int(st.item()) == 0 and count <= idx.numel()
            ref = fs.OraclePatch(fs.to_host(W[s0:e0], "w"), chain[s0:e0])
            ref.check(count, fs.to_host(idx[:count], "idx"), fs.to_host(val[:count], "val"),
                      f"C3 step {step} chunk {ci}")
            pulse.pulse_apply_patch(recv[s0:e0], idx, val, cnt, st, max_count=max(count, 1))
            prev[s0:e0].copy_(stage[:m])
            ref.applied(chain[s0:e0], out=chain[s0:e0])  # the oracle's chain: B_t = apply(B_t-1, P_t)
            fs.check_equal(fs.to_host(recv[s0:e0], "v"), chain[s0:e0], f"C3 step {step} chunk {ci}: receiver")
            changed += count
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        c3["step"] = step
        say(f"C3 step {step}: {changed} changed ({changed / c3['n']:.4%}); patch and receiver view equal the oracle")
    if last == 20:
        for s0, e0, _ in chunks:
            direct = fs.oracle_cast(fs.to_host(W[s0:e0], "w"))
            fs.check_equal(chain[s0:e0], direct, f"C3 chunk at {s0}: oracle chain vs direct cast of W_20")
