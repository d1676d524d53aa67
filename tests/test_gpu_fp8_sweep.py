"""The FP8 quantiser on every finite BF16 block maximum, against the oracle.

The kernels reach the quotient x / s without a per-element division; their
codes must still equal the oracle's E4M3(fl32(x / s)) for every value a block
can hold.  A block's scale depends only on its maximum magnitude a, and every
block contains an element of magnitude a, so every a is its own case.  Here
each of the 32,639 positive finite BF16 patterns a (0x0001 .. 0x7F7F) gets a
[128, 256] matrix whose two 128x128 blocks both hold a, and which together
hold every BF16 magnitude pattern from 0 up to a, with every second element
negative.  The whole sweep (1.07e9 values) goes through fp8_block_quant and
through the receiver's pass (pulse_apply_quant with an empty patch), whose
quantiser is built on the same per-block code; codes and scales are compared
with the oracle's, every one of them.
"""
import numpy as np
import pytest
import torch

from tests import fullsize as fs

try:
    import sparse_delta_codec_amd as pulse
except ImportError:
    if torch.cuda.is_available():
        raise
    pulse = None

MAX_FINITE = 0x7F7F   # largest finite BF16 magnitude pattern
PER_CALL = 2048       # maxima per launch: a [128 * 2048, 256] matrix


def sweep_matrix(amaxes):
    """[128 * len(amaxes), 256] BF16 patterns: one [128, 256] matrix per
    maximum a, its two column blocks each starting with a and together
    holding the patterns 0 .. a (the rest filled with a), odd slots negated."""
    a = np.asarray(amaxes, np.int64)[:, None]
    mags = np.minimum(np.arange(2 * 16384 - 2, dtype=np.int64)[None, :], a)
    blk0 = np.concatenate([a, mags[:, :16383]], 1)
    blk1 = np.concatenate([a, mags[:, 16383:]], 1)
    both = np.stack([blk0, blk1], 1)                       # [K, 2, 16384]
    sign = (np.arange(16384) % 2 == 1).astype(np.int64) << 15
    both = (both | sign[None, None, :]).astype(np.uint16)
    both[:, :, 0] &= 0x7FFF                                # the maximum itself positive
    # block b of matrix k occupies rows [128 k, 128 k + 128), columns [128 b, 128 b + 128)
    m = both.reshape(len(amaxes), 2, 128, 128).transpose(0, 2, 1, 3).reshape(len(amaxes) * 128, 256)
    return np.ascontiguousarray(m)


def test_sweep_matrix_layout():
    m = sweep_matrix([5, 0x7F7F])
    assert m.shape == (256, 256)
    for k, a in enumerate((5, 0x7F7F)):
        for b in range(2):
            blk = m[128 * k:128 * k + 128, 128 * b:128 * b + 128] & 0x7FFF
            assert blk[0, 0] == a and blk.max() == a
        allm = m[128 * k:128 * k + 128] & 0x7FFF
        assert np.array_equal(np.unique(allm), np.arange(a + 1))


@pytest.mark.gpu
def test_fp8_every_bf16_block_maximum():
    dev = torch.device("cuda")
    amaxes = np.arange(1, MAX_FINITE + 1)
    rows = 128 * PER_CALL
    x = torch.empty(rows * 256, dtype=torch.int16, device=dev)
    codes = torch.empty(rows * 256, dtype=torch.uint8, device=dev)
    scales = torch.empty(2 * PER_CALL, dtype=torch.float32, device=dev)
    codes2 = torch.empty_like(codes)
    scales2 = torch.empty_like(scales)
    idx = torch.zeros(1, dtype=torch.int32, device=dev)
    val = torch.zeros(1, dtype=torch.int16, device=dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    checked = 0
    for k0 in range(0, amaxes.size, PER_CALL):
        am = amaxes[k0:k0 + PER_CALL]
        r = 128 * am.size
        host = sweep_matrix(am)
        xs = x[:r * 256]
        xs.copy_(torch.from_numpy(host.view(np.int16).reshape(-1)))
        pulse.fp8_block_quant([xs.view(r, 256)], codes[:r * 256], scales[:2 * am.size])
        plan = pulse.pulse_apply_quant_plan([([(0, r)], 256, codes2[:r * 256], scales2[:2 * am.size])], r * 256,
                                            device=dev)
        ws = pulse.workspace(pulse.PULSE_OP_APPLY_QUANT, r * 256, 0, dev)
        pulse.pulse_apply_quant(xs, idx, val, cnt, plan, st, ws, max_count=1)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        view = host.reshape(-1)
        fs.check_fp8(view, [(0, r)], 256, fs.to_host(codes[:r * 256], "codes"),
                     fs.to_host(scales[:2 * am.size], "scales"),
                     f"maxima {int(am[0]):#06x}..{int(am[-1]):#06x} (fp8_block_quant, then pulse_apply_quant)",
                     bands_per_task=64, more=[(fs.to_host(codes2[:r * 256], "codes2"),
                                               fs.to_host(scales2[:2 * am.size], "scales2"))])
        checked += am.size
    assert checked == MAX_FINITE
    print(f"[fp8] {checked} block maxima x every magnitude up to each: codes and scales equal the oracle's",
          flush=True)
    fs.release()
