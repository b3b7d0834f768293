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


def _edge_groups(rng, n):
    """n fp16 64-groups covering the quantizer's special cases: constant, all-zero
    (with -0), a step that underflows fp16, a -0 minimum, exact ties (step 1, values
    on k + 1/2), the largest finite range, and ordinary N(0, 1) groups."""
    out = np.empty((n, 64))
    for i in range(n):
        kind = i % 7
        if kind == 0:
            out[i] = rng.choice([3.25, -7.5, 1024.0])
        elif kind == 1:
            out[i] = 0.0
        elif kind == 2:
            out[i] = rng.integers(0, 3, size=64) * 2.0**-24
        elif kind == 3:
            out[i] = np.abs(rng.normal(size=64))
            out[i, rng.integers(0, 64)] = 0.0          # made -0 below
        elif kind == 4:
            lo = rng.choice([0.0, -8.0, 32.0])
            out[i] = lo + rng.integers(0, 15, size=64) + 0.5
            out[i, 0], out[i, 1] = lo, lo + 15.0
        elif kind == 5:
            out[i] = rng.uniform(-60000, 60000, size=64)
            out[i, 0], out[i, 1] = -65504.0, 65504.0
        else:
            out[i] = rng.normal(size=64)
    x = out.astype(F16)
    x[3::7][x[3::7] == 0] = F16(-0.0)
    x[1::7][:, ::2] = F16(-0.0)
    return x


@pytest.mark.parametrize("B,nh,hd,pos", [(2, 4, 64, 300), (2, 4, 128, 300),
                                         (8, 128, 64, 40), (8, 128, 128, 40)])
def test_decode_append_edge_groups(B, nh, hd, pos):
    """The token's k and v, quantized by the decode kernel at position pos (by the last
    context split when the context is split, B x heads < 1024), equal the oracle's codes
    and (offset, scale) bit for bit on every special group; outputs stay in the bound."""
    F = require_gpu()
    T = pos + 1
    _say("decode append edges", B, nh, hd, pos)
    rng = np.random.default_rng(B * nh + hd + pos)
    h = nh * hd
    oc = O.KVCache(B, nh, hd, T)
    kv = F.KV4(B, nh, hd, T)
    prev = rng.normal(size=(B, nh, pos, hd)).astype(F16)
    for b in range(B):
        oc.store(b, 0, prev[b], prev[b])
    for name in ("k_codes", "v_codes", "k_params", "v_params"):
        getattr(kv, name).copy_(torch.from_numpy(getattr(oc, name)))
    q1 = (rng.normal(size=(B, 3 * h)) * 0.05).astype(F16)
    q1[:, h:2 * h] = _edge_groups(rng, B * h // 64).reshape(B, h)
    q1[:, 2 * h:] = _edge_groups(rng, B * h // 64).reshape(B, h)
    q1[:, 2 * h:][np.abs(q1[:, 2 * h:].astype(np.float64)) > 1e3] *= F16(1e-3)   # keep |v| modest
    out = to_np(F.attn_decode(torch.from_numpy(q1).cuda(), pos, kv))
    torch.cuda.synchronize()
    ref = O.attn_decode(q1, pos, oc)
    for name in ("k_codes", "v_codes", "k_params", "v_params"):
        a, b = to_np(getattr(kv, name))[:, :, pos], getattr(oc, name)[:, :, pos]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    # bound: the kernel's own 2^-16 max|v| plus the fp32 score error (hd 2^-23 sum|q||k|,
    # large where a K group spans the whole fp16 range) carried through the softmax
    q = q1[:, :h].astype(np.float64).reshape(B, nh, hd)
    kd = O.dequantize_kv(oc.k_codes, oc.k_params)             # [B][nh][T][hd]
    vmax = np.abs(O.dequantize_kv(oc.v_codes, oc.v_params)).max(axis=(2, 3))
    sabs = np.einsum("bhtd,bhd->bht", np.abs(kd), np.abs(q)).max(axis=2) / np.sqrt(hd)
    delta = hd * 2.0**-23 * sabs
    extra = (vmax * (2.0**-16 + 4 * delta))[:, :, None] * np.ones((1, 1, hd))
    assert_close_fp16(out, ref, extra=extra.reshape(B, h), what="decode over edge groups")


@pytest.mark.parametrize("B,S,nh,hd", [(2, 200, 3, 64), (2, 300, 3, 128), (1, 128, 8, 128)])
def test_prefill_store_edge_groups(B, S, nh, hd):
    """The prefill kernel's fused 4-bit store (one lane per 64-element group) turns K and
    V rows made of the quantizer's special groups into the oracle's codes and (offset,
    scale) bit for bit.  q = 0 makes every score 0, so the output is the plain causal
    mean of V and is checked within the usual prefill bound."""
    F = require_gpu()
    _say("prefill store edges", B, S, nh, hd)
    rng = np.random.default_rng(B * S + nh + hd)
    h = nh * hd
    qkv = np.zeros((B * S, 3 * h), F16)
    qkv[:, h:2 * h] = _edge_groups(rng, B * S * h // 64).reshape(B * S, h)
    qkv[:, 2 * h:] = _edge_groups(rng, B * S * h // 64).reshape(B * S, h)
    qkv[:, 2 * h:][np.abs(qkv[:, 2 * h:].astype(np.float64)) > 1e3] *= F16(1e-3)   # modest |v|
    kv = F.KV4(B, nh, hd, S)
    out = to_np(F.attn_prefill(torch.from_numpy(qkv).cuda(), B, S, kv))
    torch.cuda.synchronize()
    oc = O.KVCache(B, nh, hd, S)
    ref = O.attn_prefill(qkv, B, S, nh, hd, oc)
    for name in ("k_codes", "v_codes", "k_params", "v_params"):
        a, b = to_np(getattr(kv, name)), getattr(oc, name)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    vmax = np.abs(qkv[:, 2 * h:].astype(np.float64)).max()
    assert_close_fp16(out, ref, extra=2.0**-10 * vmax, what="prefill over edge groups")
