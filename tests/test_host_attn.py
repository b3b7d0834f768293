"""Decode attention on the host CPU over a host-memory 4-bit cache
(flexq_host_attn_decode_kv4, called through the C ABI; no GPU needed) against the oracle:
appended codes and params bit for bit (edge groups included: constant, underflowing
step, zero and negative-zero minimum), outputs within the GPU kernel's bound, left
padding, independence from the thread count, and argument rejection."""
import os

import numpy as np
import pytest
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16

pytestmark = pytest.mark.filterwarnings("ignore")


def _lib():
    from group_wise_bit_flexq_amd import flexq as F
    if not os.path.exists(F.LIB_PATH):
        pytest.skip("libflexq.so not built (run __graft_entry__.build())")
    F.lib()
    return F


def _fill(F, oc):
    kv = F.KV4(oc.batch, oc.heads, oc.head_dim, oc.max_len, device="cpu")
    kv.k_codes.copy_(torch.from_numpy(oc.k_codes))
    kv.v_codes.copy_(torch.from_numpy(oc.v_codes))
    kv.k_params.copy_(torch.from_numpy(oc.k_params))
    kv.v_params.copy_(torch.from_numpy(oc.v_params))
    return kv


def _check_cache(kv, oc):
    assert np.array_equal(kv.k_codes.numpy(), oc.k_codes)
    assert np.array_equal(kv.v_codes.numpy(), oc.v_codes)
    assert np.array_equal(kv.k_params.numpy().view(np.uint16), oc.k_params.view(np.uint16))
    assert np.array_equal(kv.v_params.numpy().view(np.uint16), oc.v_params.view(np.uint16))


def _vbound(oc):
    return 2.0**-16 * (15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() +
                       np.abs(oc.v_params[..., 0].astype(np.float64)).max())


@pytest.mark.parametrize("B,nh,hd,S,steps", [(3, 4, 128, 200, 3), (2, 3, 64, 65, 2),
                                             (1, 2, 128, 1, 2)])
def test_host_decode_matches_oracle(B, nh, hd, S, steps):
    F = _lib()
    rng = np.random.default_rng(B * 100 + S + hd)
    b0 = 1
    oc = O.KVCache(B + 2, nh, hd, S + steps)
    qkv = rng.normal(size=(B * S, 3 * nh * hd)).astype(F16)
    O.attn_prefill(qkv, B, S, nh, hd, oc, b0=b0)
    kv = _fill(F, oc)
    for i in range(steps):
        pos = S + i
        q1 = rng.normal(size=(B, 3 * nh * hd)).astype(F16)
        got = F.host_attn_decode(torch.from_numpy(q1), pos, kv, b0=b0, threads=4).numpy()
        ref = O.attn_decode(q1, pos, oc, b0=b0)
        _check_cache(kv, oc)
        assert_close_fp16(got, ref, extra=_vbound(oc), what=f"host decode pos {pos}")


def test_host_append_edge_groups():
    F = _lib()
    nh, hd = 2, 128
    oc = O.KVCache(1, nh, hd, 4)
    kv = _fill(F, oc)
    q1 = np.zeros((1, 3 * nh * hd), F16)
    h = nh * hd
    k = q1[0, h:2 * h].reshape(nh * 2, 64)
    v = q1[0, 2 * h:].reshape(nh * 2, 64)
    k[0] = 1.5                                   # constant group
    k[1] = np.linspace(0, 1, 64)                 # zero minimum
    k[2] = 2.0 ** -20                            # constant, tiny
    k[2, 5] = 2.0 ** -20 + 2.0 ** -24            # range that underflows the fp16 step
    k[3] = -0.0                                  # negative zero minimum, constant
    k[3, 7] = 1.0
    v[:] = np.random.default_rng(5).normal(size=(nh * 2, 64)) * 2.0 ** np.arange(-6, 2)[:4, None]
    got = F.host_attn_decode(torch.from_numpy(q1), 0, kv).numpy()
    ref = O.attn_decode(q1, 0, oc)
    _check_cache(kv, oc)
    assert_close_fp16(got, ref, extra=_vbound(oc), what="edge groups")


def test_host_decode_with_padding():
    F = _lib()
    rng = np.random.default_rng(7)
    B, nh, hd, S = 3, 2, 128, 50
    pads = np.array([0, 20, 49], np.int32)
    oc = O.KVCache(B, nh, hd, S + 2)
    oc.pad[:] = pads
    qkv = rng.normal(size=(B * S, 3 * nh * hd)).astype(F16)
    O.attn_prefill(qkv, B, S, nh, hd, oc)
    kv = _fill(F, oc)
    kv.pad = torch.from_numpy(pads.copy())
    for pos in (S, S + 1):
        q1 = rng.normal(size=(B, 3 * nh * hd)).astype(F16)
        got = F.host_attn_decode(torch.from_numpy(q1), pos, kv).numpy()
        ref = O.attn_decode(q1, pos, oc)
        assert_close_fp16(got, ref, extra=_vbound(oc), what=f"padded host decode pos {pos}")


def test_host_decode_independent_of_thread_count():
    F = _lib()
    rng = np.random.default_rng(8)
    B, nh, hd, S = 4, 5, 64, 100
    oc = O.KVCache(B, nh, hd, S + 1)
    O.attn_prefill(rng.normal(size=(B * S, 3 * nh * hd)).astype(F16), B, S, nh, hd, oc)
    q1 = torch.from_numpy(rng.normal(size=(B, 3 * nh * hd)).astype(F16))
    outs = []
    for t in (1, 3, 8, 64):
        kv = _fill(F, oc)
        outs.append(F.host_attn_decode(q1, S, kv, threads=t).numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))


def test_host_decode_rejects():
    F = _lib()
    kv = F.KV4(2, 2, 64, 8, device="cpu")
    q1 = torch.zeros(2, 3 * 128, dtype=torch.float16)
    for args in [(q1, 8, kv, 0), (q1, 3, kv, 1), (q1, -1, kv, 0)]:
        with pytest.raises(F.FlexqError):
            F.host_attn_decode(*args[:3], b0=args[3])
    bad = F.KV4(2, 2, 32, 8, device="cpu")
    with pytest.raises(F.FlexqError):
        F.host_attn_decode(torch.zeros(2, 3 * 64, dtype=torch.float16), 3, bad)
