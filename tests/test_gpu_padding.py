"""Ragged (left-padded) prompts through the C ABI against the oracle: the embedding's
shifted positions bit for bit; prefill attention with pad counts on either side of the
64-key blocks and 128-query work-groups (pad queries exactly 0, every cache code and
param bit-exact); decode attention whose context splits lie wholly, partly or not at
all in the padding; and greedy generation of a tiny OPT over a ragged batch in
micro-batches, teacher-forced against the oracle."""
import numpy as np
import pytest
import torch

from group_wise_bit_flexq_amd import synth
from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16, assert_logits_close, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _qkv(rng, rows, nh, hd):
    return rng.normal(size=(rows, 3 * nh * hd)).astype(F16)


def test_embed_with_padding():
    F = require_gpu()
    _say("embed with padding")
    rng = np.random.default_rng(21)
    V, h, S = 500, 192, 9
    e16 = (rng.normal(size=(V, h)) * 0.5).astype(F16)
    pos = rng.normal(size=(40, h)).astype(F16)
    codes, params = O.quantize(e16)
    ew = F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    toks = rng.integers(0, V, size=4 * S).astype(np.int32)
    pad = np.array([0, 3, 8, 5], np.int32)
    got = F.embed(torch.from_numpy(toks).cuda(), 0, S, ew, torch.from_numpy(pos).cuda(),
                  pad=torch.from_numpy(pad).cuda())
    positions = np.maximum(np.arange(S)[None, :] - pad[:, None], 0).reshape(-1)
    ref = O.embed(toks, positions, codes, params, pos)
    assert np.array_equal(to_np(got).view(np.uint16), ref.view(np.uint16))
    # decode form: one token per sequence at position 20
    got1 = F.embed(torch.from_numpy(toks[:4]).cuda(), 20, 1, ew, torch.from_numpy(pos).cuda(),
                   pad=torch.from_numpy(pad).cuda())
    ref1 = O.embed(toks[:4], 20 - pad, codes, params, pos)
    assert np.array_equal(to_np(got1).view(np.uint16), ref1.view(np.uint16))


PREFILL = [  # S, head_dim, heads, pad counts of the sequences
    (40, 64, 2, [0, 1, 39]),
    (300, 128, 2, [0, 63, 64, 65, 127, 128, 129, 200, 299]),
    (257, 64, 3, [255, 256, 100, 1]),
    (512, 128, 1, [511, 384, 130, 0]),
]


@pytest.mark.parametrize("case", range(len(PREFILL)))
def test_attn_prefill_with_padding(case):
    F = require_gpu()
    S, hd, nh, pads = PREFILL[case]
    B = len(pads)
    _say("attn_prefill padded", S, hd, nh, pads)
    rng = np.random.default_rng(case + 40)
    qkv = _qkv(rng, B * S, nh, hd)
    b0 = 1
    pad_rows = np.zeros(B + 2, np.int32)
    pad_rows[b0:b0 + B] = pads
    kv = F.KV4(B + 2, nh, hd, S + 3, pad=torch.from_numpy(pad_rows).cuda())
    out = F.attn_prefill(torch.from_numpy(qkv).cuda(), B, S, kv, b0=b0)
    torch.cuda.synchronize()
    oc = O.KVCache(B + 2, nh, hd, S + 3)
    oc.pad[:] = pad_rows
    ref = O.attn_prefill(qkv, B, S, nh, hd, oc, b0=b0)
    got = to_np(out)
    for b, p in enumerate(pads):
        assert not got[b * S:b * S + p].any(), f"pad queries of sequence {b} not 0"
    vmax = np.abs(qkv.astype(np.float64)).max()
    assert_close_fp16(got, ref, extra=2.0**-10 * vmax, what="padded prefill out")
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(to_np(getattr(kv, name)), getattr(oc, name)), name
    for name in ("k_params", "v_params"):
        assert np.array_equal(to_np(getattr(kv, name)).view(np.uint16),
                              getattr(oc, name).view(np.uint16)), name


DECODE = [  # B, heads, head_dim, prompt, steps, pads
    (4, 8, 128, 1000, 2, [0, 300, 700, 999]),     # 16 splits: some wholly in the padding
    (3, 2, 64, 130, 3, [129, 64, 5]),
    (2, 40, 128, 600, 2, [599, 0]),               # one split per (sequence, head)
]


@pytest.mark.parametrize("case", range(len(DECODE)))
def test_attn_decode_with_padding(case):
    F = require_gpu()
    B, nh, hd, S, steps, pads = DECODE[case]
    _say("attn_decode padded", B, nh, hd, S, steps, pads)
    rng = np.random.default_rng(case + 60)
    T = S + steps
    padt = torch.tensor(pads, dtype=torch.int32, device="cuda")
    kv = F.KV4(B, nh, hd, T, pad=padt)
    oc = O.KVCache(B, nh, hd, T)
    oc.pad[:] = pads
    qkv = _qkv(rng, B * S, nh, hd)
    F.attn_prefill(torch.from_numpy(qkv).cuda(), B, S, kv)
    O.attn_prefill(qkv, B, S, nh, hd, oc)
    for i in range(steps):
        pos = S + i
        q1 = _qkv(rng, B, nh, hd)
        out = F.attn_decode(torch.from_numpy(q1).cuda(), pos, kv)
        torch.cuda.synchronize()
        ref = O.attn_decode(q1, pos, oc)
        vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
            np.abs(oc.v_params[..., 0].astype(np.float64)).max()
        assert_close_fp16(to_np(out), ref, extra=2.0**-16 * vmax, what=f"padded decode pos {pos}")
        assert np.array_equal(to_np(kv.k_codes), oc.k_codes)
        assert np.array_equal(to_np(kv.v_params).view(np.uint16), oc.v_params.view(np.uint16))


def test_tiny_model_ragged_greedy():
    F = require_gpu()
    from tests.test_gpu_model import _gpu_model, _host_model, _oracle_model
    nh, B, S, G, mb = 4, 6, 40, 6, 3
    lens = [40, 1, 17, 39, 24, 2]
    pad = np.array([S - n for n in lens], np.int32)
    _say("tiny model ragged greedy", lens)
    parts = _host_model(256, nh, 1024, 1000, 2, 7)
    V = parts[1].shape[0]
    gm = _gpu_model(F, parts, nh, B, S + G - 1, mb * S)
    toks = synth.token_ids(B, S, V, synth.sub_seed(0, "tokens")).cuda()
    out = torch.empty(B, G, dtype=torch.int32, device="cuda")
    first = torch.empty(B, dtype=torch.int32, device="cuda")
    logits = torch.empty(G, B, V, dtype=torch.float32, device="cuda")
    for j in range(B // mb):
        sl = slice(j * mb, (j + 1) * mb)
        gm.prefill(toks[sl], b0=j * mb, logits=logits[0, sl], next_out=first[sl], pad=pad[sl])
    out[:, 0].copy_(first)
    cur = first
    for i in range(G - 1):
        nxt = gm.decode_step(cur, S + i, logits=logits[i + 1])
        out[:, i + 1].copy_(nxt)
        cur = nxt
    torch.cuda.synchronize()
    gl, go = to_np(logits), to_np(out).astype(np.int64)
    om = _oracle_model(parts, nh)
    caches = om.new_caches(B, S + G - 1)
    lg, nx = om.prefill(to_np(toks), caches, pad=pad)
    ties = 0
    for i in range(G):
        if i > 0:
            lg, nx = om.decode_step(go[:, i - 1], S + i - 1, caches)
        err, _ = assert_logits_close(gl[i], lg, f"ragged logits step {i}")
        for r in range(B):
            if nx[r] != go[r, i]:
                gap = lg[r].max() - lg[r, go[r, i]]
                assert gap <= 2 * err + 1e-6, f"step {i} seq {r}: token {go[r, i]} vs {nx[r]}"
                ties += 1
    assert ties == 0
