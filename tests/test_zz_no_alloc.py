"""The allocation-free form of the fused sender pass
(pulse_cast_diff_lz4_noalloc, the library's static per-GPU scratch instead of
a workspace) against pulse_cast_diff_lz4 with a workspace of its own: every
output bit for bit, on two calls in a row, the second with a smaller input,
for each block size.  The first call of the process on the GPU also sets the
scratch up; the second reuses the array as the first call left it."""
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

from tests.gpu_util import dev, host, zeros  # noqa: E402


def run(fn, w1, b0, block_bytes, ws=None):
    n = w1.size
    nb = (2 * n + block_bytes - 1) // block_bytes
    pcap = pulse.lz4_payload_bound(2 * n, block_bytes)
    W, B0 = dev(w1), dev(b0)
    out = dict(b_new=zeros(n, torch.int16), idx=zeros(n, torch.int32), val=zeros(n, torch.int16),
               cnt=zeros(1, torch.int64), tiles=torch.full((pulse.patch_tile_count(n),), -7, dtype=torch.int64,
                                                           device="cuda"),
               payload=zeros(pcap, torch.uint8), sizes=zeros(nb, torch.int32), offs=zeros(nb, torch.int64),
               tot=zeros(1, torch.int64), st=zeros(1, torch.int32))
    args = (W, B0, out["b_new"], out["idx"], out["val"], out["cnt"], out["payload"], out["sizes"], out["offs"],
            out["tot"], out["st"])
    if ws is None:
        fn(*args, block_bytes=block_bytes, tile_first=out["tiles"])
    else:
        fn(*args, ws, block_bytes=block_bytes, tile_first=out["tiles"])
    torch.cuda.synchronize()
    count = int(host(out["cnt"])[0])
    total = int(host(out["tot"])[0])
    return dict(status=int(host(out["st"])[0]), count=count, total=total, b_new=host(out["b_new"])[:n],
                idx=host(out["idx"])[:count], val=host(out["val"])[:count], tiles=host(out["tiles"]),
                payload=host(out["payload"])[:total], sizes=host(out["sizes"])[:nb], offs=host(out["offs"])[:nb])


@pytest.mark.parametrize("block_bytes", [65536, 16384])
def test_noalloc_equals_workspace_call_twice_shrinking(block_bytes):
    for i, n in enumerate((3 * 32768 * 5 + 4099, 70001)):
        w0, w1 = workload.host_masters(n, seed=1000 + i + block_bytes // 1024)
        b0 = np.frombuffer(torch.from_numpy(w0).to(torch.bfloat16).view(torch.int16).numpy().tobytes(), np.uint16)
        ws = pulse.workspace(pulse.PULSE_OP_CAST_DIFF_LZ4, n, block_bytes)
        ref = run(pulse.pulse_cast_diff_lz4, w1, b0, block_bytes, ws=ws)
        got = run(pulse.pulse_cast_diff_lz4_noalloc, w1, b0, block_bytes)
        assert ref["status"] == 0 and got["status"] == 0
        assert 0 < ref["count"] < n
        for k in ref:
            assert np.array_equal(np.asarray(got[k]), np.asarray(ref[k])), (n, k)
