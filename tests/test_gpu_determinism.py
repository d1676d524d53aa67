"""Repeatability of the hot path on the GPU: the same inputs through the fused
sender pass (pulse_cast_diff_lz4: new view, patch, tile index, LZ4 blocks of
the mask) and the LZ4 decode (lz4_decode_blocks, XOR into a copy of the old
view) give bit-identical outputs on every repetition, at several sizes, one
stream, one workspace per op reused across the repetitions.  The results
depend on the order in which workgroups take their tickets and finish their
look-backs only through the values they publish, so any dependence on timing
shows up here as a difference between repetitions."""
import numpy as np
import pytest
import torch

import workload

pytestmark = pytest.mark.gpu

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise
    pulse = None

from tests.gpu_util import dev, zeros  # noqa: E402

BLOCK = 65536
REPS = 4


@pytest.mark.parametrize("n", [1, 32768 * 3 + 5, 1 << 20, (1 << 24) + 4097])
def test_fused_pass_and_decode_repeat_bit_for_bit(n):
    w0, w1 = workload.host_masters(n, seed=4242 + n % 1000)
    W0, W1 = dev(w0), dev(w1)
    b0 = zeros(n, torch.int16)
    pulse.pulse_cast_diff(W0, b_new=b0)
    nb = (2 * n + BLOCK - 1) // BLOCK
    pcap = pulse.lz4_payload_bound(2 * n, BLOCK)
    ws_e = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_LZ4, n, BLOCK)
    ws_d = pulse.workspace(pulse.PULSE_OP_LZ4_DECODE, nb, pcap)
    first = None
    for rep in range(REPS):
        bn, idx, val = zeros(n, torch.int16), zeros(n, torch.int32), zeros(n, torch.int16)
        cnt, tot, st = zeros(1, torch.int64), zeros(1, torch.int64), zeros(1, torch.int32)
        tiles = zeros(pulse.patch_tile_count(n), torch.int64)
        payload, sizes, offs = zeros(pcap, torch.uint8), zeros(nb, torch.int32), zeros(nb, torch.int64)
        pulse.pulse_cast_diff_lz4(W1, b0, bn, idx, val, cnt, payload, sizes, offs, tot, st, ws_e, tile_first=tiles)
        rebuilt = b0.clone()
        pulse.lz4_decode_blocks(payload, offs, sizes, rebuilt, st, ws_d, mode=1, payload_bytes=pcap)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        c, t = int(cnt.item()), int(tot.item())
        out = [bn, idx[:c], val[:c], tiles, payload[:t], sizes, offs, rebuilt]
        assert torch.equal(rebuilt, bn)
        if first is None:
            first = (c, t, [x.clone() for x in out])
        else:
            assert (c, t) == first[:2], rep
            for k, (a, b) in enumerate(zip(out, first[2])):
                assert torch.equal(a, b), (rep, k)
