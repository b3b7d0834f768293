"""KV-compression stress at full size (OPT-30B attention shape), sampled parity.

Batch 64, prompt 2048, 56 heads x 128: fp16 Q/K/V ~N(0,1) with 1 % of the K/V
entries scaled by 8; prefill attention stores the whole cache in 4 bits, then 64
decode steps of attention over the 4-bit cache (fresh N(0,1) q/k/v each step,
same outlier rule).  The oracle follows sampled (sequence, head) pairs through all
of it from the same fp16 inputs: prefill rows, every cached code, every decode
output.  Also the standalone quantizer on a 4 GiB fp16 tensor, checked bit for bit
on sampled rows.
"""
import numpy as np
import pytest
import torch

from group_wise_bit_flexq_amd import synth
from group_wise_bit_flexq_amd.workloads import KV_STRESS, QUANT_4GIB
from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _stress_qkv(rows, h, seed, frac, factor):
    q = synth.normal_fp16((rows, h), 1.0, synth.sub_seed(seed, "q"), device="cuda")
    kv = synth.normal_fp16((rows, 2 * h), 1.0, synth.sub_seed(seed, "kv"), device="cuda")
    kv = synth.with_outliers(kv, frac, factor, synth.sub_seed(seed, "outliers"))
    return torch.cat([q, kv], dim=1).contiguous()


def _head(qkv_rows, head, hd, h):
    return np.concatenate([qkv_rows[:, head * hd:(head + 1) * hd],
                           qkv_rows[:, h + head * hd:h + (head + 1) * hd],
                           qkv_rows[:, 2 * h + head * hd:2 * h + (head + 1) * hd]], axis=1)


@pytest.mark.timeout(900)
def test_kv_stress_prefill_and_64_decode_steps():
    F = require_gpu()
    c = KV_STRESS
    B, nh, hd, S, steps = c["batch"], c["heads"], c["head_dim"], c["prompt"], c["steps"]
    h = nh * hd
    _say("kv stress", B, nh, hd, S, steps)
    rng = np.random.default_rng(2048)
    kv = F.KV4(B, nh, hd, S + steps)
    qkv = _stress_qkv(B * S, h, 1, c["outlier_frac"], c["outlier_factor"])
    att = F.attn_prefill(qkv, B, S, kv)
    torch.cuda.synchronize()
    pairs = [(int(rng.integers(0, B)), int(rng.integers(0, nh))) for _ in range(3)]
    caches = {}
    for (b, hh) in pairs:
        small = _head(to_np(qkv[b * S:(b + 1) * S]), hh, hd, h)
        oc = O.KVCache(1, 1, hd, S + steps)
        ref = O.attn_prefill(small, 1, S, 1, hd, oc)
        got = to_np(att[b * S:(b + 1) * S, hh * hd:(hh + 1) * hd])
        assert_close_fp16(got, ref, extra=2.0**-9 * np.abs(small.astype(np.float64)).max(),
                          what=f"prefill b={b} h={hh}")
        assert np.array_equal(to_np(kv.k_codes[b, hh, :S]), oc.k_codes[0, 0, :S])
        assert np.array_equal(to_np(kv.v_codes[b, hh, :S]), oc.v_codes[0, 0, :S])
        assert np.array_equal(to_np(kv.k_params[b, hh, :S]).view(np.uint16),
                              oc.k_params[0, 0, :S].view(np.uint16))
        assert np.array_equal(to_np(kv.v_params[b, hh, :S]).view(np.uint16),
                              oc.v_params[0, 0, :S].view(np.uint16))
        caches[(b, hh)] = oc
    del qkv, att
    for i in range(steps):
        pos = S + i
        q1 = _stress_qkv(B, h, 100 + i, c["outlier_frac"], c["outlier_factor"])
        out = F.attn_decode(q1, pos, kv)
        torch.cuda.synchronize()
        qn = to_np(q1)
        for (b, hh), oc in caches.items():
            ref = O.attn_decode(_head(qn[b:b + 1], hh, hd, h), pos, oc)
            got = to_np(out[b:b + 1, hh * hd:(hh + 1) * hd])
            vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
                np.abs(oc.v_params[..., 0].astype(np.float64)).max()
            assert_close_fp16(got, ref, extra=2.0**-16 * vmax, what=f"decode step {i} b={b} h={hh}")
            assert np.array_equal(to_np(kv.k_codes[b, hh, pos]), oc.k_codes[0, 0, pos])
            assert np.array_equal(to_np(kv.v_codes[b, hh, pos]), oc.v_codes[0, 0, pos])
        if i % 16 == 0:
            print(f"decode step {i} ok", flush=True)


@pytest.mark.timeout(600)
def test_quantize_4gib_sampled_rows():
    F = require_gpu()
    rows, cols = QUANT_4GIB["rows"], QUANT_4GIB["cols"]
    _say("quantize 4 GiB", rows, cols)
    x = synth.normal_fp16((rows, cols), 1.0, synth.sub_seed(0, "quant4g"), device="cuda")
    w = F.quantize(x)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    sel = np.concatenate([[0, rows - 1], rng.integers(0, rows, 62)])
    idx = torch.from_numpy(sel).cuda()
    codes, params = O.quantize(to_np(x[idx]))
    assert np.array_equal(to_np(w.codes[idx]), codes)
    assert np.array_equal(to_np(w.params[idx]).view(np.uint16), params.view(np.uint16))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("hd", [64, 128])
def test_long_context_split_merge_at_1024_pairs(hd):
    """Contexts past the 4096-position score buffer with enough (sequence, head) pairs
    that the context is split only to fit it: batch 16 x 64 heads = 1024 pairs, prompt
    4200, two decode steps (positions 4200, 4201 -> two splits and the merge).  Sampled
    pairs followed through prefill (cache bit-exact) and both decode outputs."""
    F = require_gpu()
    B, nh, S, steps = 16, 64, 4200, 2
    h = nh * hd
    _say("long context split", B, nh, hd, S, steps)
    assert F.attn_decode_ws_bytes(B, nh, hd, S) > 0   # the split path, not one work-group per pair
    rng = np.random.default_rng(4200 + hd)
    kv = F.KV4(B, nh, hd, S + steps)
    qkv = _stress_qkv(B * S, h, 7 + hd, 0.01, 8.0)
    att = F.attn_prefill(qkv, B, S, kv)
    torch.cuda.synchronize()
    pairs = [(0, 0), (B - 1, nh - 1), (int(rng.integers(0, B)), int(rng.integers(0, nh)))]
    caches = {}
    for (b, hh) in pairs:
        small = _head(to_np(qkv[b * S:(b + 1) * S]), hh, hd, h)
        oc = O.KVCache(1, 1, hd, S + steps)
        ref = O.attn_prefill(small, 1, S, 1, hd, oc)
        got = to_np(att[b * S:(b + 1) * S, hh * hd:(hh + 1) * hd])
        assert_close_fp16(got, ref, extra=2.0**-9 * np.abs(small.astype(np.float64)).max(),
                          what=f"prefill b={b} h={hh}")
        for name in ("k_codes", "v_codes"):
            assert np.array_equal(to_np(getattr(kv, name)[b, hh, :S]), getattr(oc, name)[0, 0, :S])
        for name in ("k_params", "v_params"):
            assert np.array_equal(to_np(getattr(kv, name)[b, hh, :S]).view(np.uint16),
                                  getattr(oc, name)[0, 0, :S].view(np.uint16))
        caches[(b, hh)] = oc
    del qkv, att
    for i in range(steps):
        pos = S + i
        q1 = _stress_qkv(B, h, 900 + i, 0.01, 8.0)
        out = F.attn_decode(q1, pos, kv)
        torch.cuda.synchronize()
        qn = to_np(q1)
        for (b, hh), oc in caches.items():
            ref = O.attn_decode(_head(qn[b:b + 1], hh, hd, h), pos, oc)
            got = to_np(out[b:b + 1, hh * hd:(hh + 1) * hd])
            vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
                np.abs(oc.v_params[..., 0].astype(np.float64)).max()
            assert_close_fp16(got, ref, extra=2.0**-16 * vmax, what=f"decode step {i} b={b} h={hh}")
