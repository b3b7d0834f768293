"""Decode attention at the edges of its load schedule (needs an MI355X).

With one context split per (sequence, head), the kernel issues its first batch of K
loads before the barrier that orders the append of position pos, but only when that
batch ends before pos; otherwise the batch waits for the append.  Left padding moves
the first position, so pads of pos - batch - 1, pos - batch, pos - batch + 1 and pos
put the first batch just short of, exactly at and past the appended position (and a
sequence whose only position is the new one).  The cache is filled with random codes
and parameters (offsets N(0, 0.5), steps U(0.01, 0.1)); every (sequence, head) output
is compared with the oracle, and the appended codes and parameters bit for bit."""
import numpy as np
import pytest
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


# (head_dim, T): one split (8 x 128 = 1024 pairs); batch = UNR block steps of the launch
# (head_dim 64: 128 positions per block step, T 601 -> 5 steps, UNR 1; head_dim 128:
# 64 per block step, T 601 -> 10 steps, UNR 2), so the first batch covers 128 positions
@pytest.mark.parametrize("hd,batch_positions", [(64, 128), (128, 128)])
def test_decode_first_batch_at_the_appended_position(hd, batch_positions):
    F = require_gpu()
    B, nh, pos = 8, 128, 600
    T = pos + 1
    _say("decode edges", B, nh, hd, T)
    rng = np.random.default_rng(hd)
    pads = np.array([0, pos - batch_positions - 1, pos - batch_positions,
                     pos - batch_positions + 1, pos, 3, pos - 1, 200], np.int32)
    oc = O.KVCache(B, nh, hd, T)
    oc.pad[:] = pads
    for c in (oc.k_codes, oc.v_codes):
        c[:, :, :pos] = rng.integers(0, 256, size=c[:, :, :pos].shape, dtype=np.uint8)
    for p in (oc.k_params, oc.v_params):
        p[:, :, :pos, :, 0] = rng.normal(0.0, 0.5, size=p[:, :, :pos, :, 0].shape).astype(F16)
        p[:, :, :pos, :, 1] = rng.uniform(0.01, 0.1, size=p[:, :, :pos, :, 1].shape).astype(F16)
    kv = F.KV4(B, nh, hd, T, pad=torch.from_numpy(pads).cuda())
    for name in ("k_codes", "v_codes", "k_params", "v_params"):
        getattr(kv, name).copy_(torch.from_numpy(getattr(oc, name)))
    q1 = rng.normal(size=(B, 3 * nh * hd)).astype(F16)
    out = to_np(F.attn_decode(torch.from_numpy(q1).cuda(), pos, kv))
    torch.cuda.synchronize()
    ref = O.attn_decode(q1, pos, oc)
    for name in ("k_codes", "v_codes", "k_params", "v_params"):
        a, b = to_np(getattr(kv, name)), getattr(oc, name)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    vmax = 15 * 0.1 + np.abs(oc.v_params[..., 0].astype(np.float64)).max()
    for b in range(B):
        assert_close_fp16(out[b], ref[b], extra=2.0**-16 * vmax, what=f"seq {b} pad {pads[b]}")
