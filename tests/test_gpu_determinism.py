"""Bitwise reruns (needs an MI355X).

Every reduction here has a fixed order: split-K partial sums are added in split order
by the reduce kernel, decode attention's context splits are merged in split order,
and nothing accumulates with atomics.  The same call on the same inputs must
therefore give the same bits every time, whatever the scheduling of its work-groups.
"""
import numpy as np
import pytest
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, require_gpu

pytestmark = pytest.mark.gpu

REPS = 4


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("M,N,K", [(144, 1024, 8192),    # decode kernel, split-K
                                   (144, 33792, 4096),   # decode kernel, two splits
                                   (32, 512, 8192),      # small-M kernel, split-K
                                   (512, 512, 4096),     # large-M kernel, split-K (few tiles)
                                   (1000, 768, 2048)])   # large-M kernel, no split
def test_linear_reruns_are_bitwise_identical(M, N, K):
    F = require_gpu()
    _say("linear rerun", M, N, K)
    rng = np.random.default_rng(M * N + K)
    w = (rng.normal(size=(N, K)) * 0.05).astype(F16)
    codes, params = O.quantize(w)
    wq = F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    x = torch.from_numpy(rng.normal(size=(M, K)).astype(F16)).cuda()
    b = torch.from_numpy((rng.normal(size=N) * 0.1).astype(F16)).cuda()
    ws = torch.empty(max(F.linear_ws_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
    first = F.linear_w4(x, wq, bias=b, relu=True, ws=ws).clone()
    lg = F.linear_w4_f32(x, wq, ws=ws).clone()
    for _ in range(REPS):
        ws.fill_(0x5A)                      # stale partials must not matter
        assert torch.equal(F.linear_w4(x, wq, bias=b, relu=True, ws=ws), first)
        assert torch.equal(F.linear_w4_f32(x, wq, ws=ws), lg)


@pytest.mark.parametrize("B,nh,hd,pos", [(2, 4, 128, 3000),   # 8 pairs: many context splits
                                         (3, 8, 64, 900),
                                         (144, 8, 128, 529)])  # one split per pair
def test_decode_attention_reruns_are_bitwise_identical(B, nh, hd, pos):
    F = require_gpu()
    _say("decode rerun", B, nh, hd, pos)
    rng = np.random.default_rng(B + nh + hd + pos)
    T = pos + 1
    kv = F.KV4(B, nh, hd, T)
    for c in (kv.k_codes, kv.v_codes):
        c.copy_(torch.from_numpy(rng.integers(0, 256, size=tuple(c.shape), dtype=np.uint8)))
    for p in (kv.k_params, kv.v_params):
        par = np.empty(tuple(p.shape), F16)
        par[..., 0] = rng.normal(0, 0.5, size=par.shape[:-1])
        par[..., 1] = rng.uniform(0.01, 0.1, size=par.shape[:-1])
        p.copy_(torch.from_numpy(par))
    q1 = torch.from_numpy(rng.normal(size=(B, 3 * nh * hd)).astype(F16)).cuda()
    ws = torch.empty(max(F.attn_decode_ws_bytes(B, nh, hd, pos), 16), dtype=torch.uint8,
                     device="cuda")
    first = F.attn_decode(q1, pos, kv, ws=ws).clone()
    cache = kv.k_codes.clone()
    for _ in range(REPS):
        ws.fill_(0xA5)
        assert torch.equal(F.attn_decode(q1, pos, kv, ws=ws), first)
        assert torch.equal(kv.k_codes, cache)      # the append rewrites the same codes


def test_prefill_attention_reruns_are_bitwise_identical():
    F = require_gpu()
    B, S, nh, hd = 3, 333, 4, 128
    _say("prefill rerun", B, S, nh, hd)
    rng = np.random.default_rng(7)
    qkv = torch.from_numpy(rng.normal(size=(B * S, 3 * nh * hd)).astype(F16)).cuda()
    kv = F.KV4(B, nh, hd, S)
    first = F.attn_prefill(qkv, B, S, kv).clone()
    for _ in range(REPS):
        assert torch.equal(F.attn_prefill(qkv, B, S, kv), first)
