"""Full-size parity of the next rows on sampled outputs, at the OPT-175B attention shapes
(96 heads x 128): left-padded prefill attention of one micro-batch (48 x 512), top-k
sparse decode attention of the whole batch (144 sequences, 529 positions), and the
host-CPU decode attention of one micro-batch over the same cache moved to host memory.
The oracle recomputes sampled (sequence, head) pairs from the kernels' own inputs."""
import numpy as np
import pytest
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16, require_gpu, to_np

pytestmark = pytest.mark.gpu

NH, HD = 96, 128
H = NH * HD


def _say(*a):
    print("[case]", *a, flush=True)


def _pair_qkv(rows, head):
    """[n][3h] rows -> [n][3 hd] rows of one head (q | k | v)."""
    q = rows[:, head * HD:(head + 1) * HD]
    k = rows[:, H + head * HD:H + (head + 1) * HD]
    v = rows[:, 2 * H + head * HD:2 * H + (head + 1) * HD]
    return np.ascontiguousarray(np.concatenate([q, k, v], axis=1))


def _pair_cache(kv, b, head, T):
    """The cache rows of one (sequence, head) as a one-sequence, one-head oracle cache."""
    c = O.KVCache(1, 1, HD, T)
    for name in ("k_codes", "v_codes", "k_params", "v_params"):
        getattr(c, name)[0, 0, :T] = to_np(getattr(kv, name)[b, head, :T])
    return c


@pytest.mark.timeout(600)
def test_fullsize_padded_prefill_attention_sampled():
    F = require_gpu()
    B, S = 48, 512
    _say("full-size padded prefill attention", B, S, NH, HD)
    g = torch.Generator(device="cuda").manual_seed(5)
    qkv = torch.randn(B * S, 3 * H, generator=g, device="cuda").half()
    rng = np.random.default_rng(5)
    pads = rng.integers(0, S, B).astype(np.int32)
    pads[:4] = [0, 1, 255, 511]
    kv = F.KV4(B, NH, HD, S, pad=torch.from_numpy(pads).cuda())
    out = F.attn_prefill(qkv, B, S, kv)
    torch.cuda.synchronize()
    for b, head in [(0, 0), (1, 17), (2, 95), (3, 40), (int(rng.integers(4, B)), 63),
                    (int(rng.integers(4, B)), 7)]:
        rows = to_np(qkv[b * S:(b + 1) * S])
        pq = _pair_qkv(rows, head)
        oc = O.KVCache(1, 1, HD, S)
        ref = O.attn_prefill(pq, 1, S, 1, HD, oc, pad=[pads[b]])
        got = to_np(out[b * S:(b + 1) * S, head * HD:(head + 1) * HD])
        assert not got[:pads[b]].any()
        assert_close_fp16(got, ref, extra=2.0**-10 * np.abs(pq.astype(np.float64)).max(),
                          what=f"padded prefill seq {b} head {head}")
        for name in ("k_codes", "v_codes", "k_params", "v_params"):
            a = to_np(getattr(kv, name)[b, head])
            assert np.array_equal(a.view(np.uint8), getattr(oc, name)[0, 0].view(np.uint8)), name


@pytest.mark.timeout(600)
def test_fullsize_topk_and_host_decode_attention_sampled():
    F = require_gpu()
    B, S, sp = 144, 528, 0.25
    pos = S                      # 529 positions: the prompt + the new token
    _say("full-size sparse decode attention", B, NH, HD, pos + 1, sp)
    kv = F.KV4(B, NH, HD, S + 1)
    g = torch.Generator(device="cuda").manual_seed(6)
    for j in range(3):          # fill the cache one micro-batch at a time
        qkv = torch.randn(48 * S, 3 * H, generator=g, device="cuda").half()
        F.attn_prefill(qkv, 48, S, kv, b0=48 * j)
        del qkv
    q1 = torch.randn(B, 3 * H, generator=g, device="cuda").half()
    kv_before = {n: getattr(kv, n)[:48].cpu() for n in ("k_codes", "v_codes", "k_params",
                                                        "v_params")}
    out = to_np(F.attn_decode_topk(q1, pos, kv, sp))
    torch.cuda.synchronize()
    q1n = to_np(q1)
    rng = np.random.default_rng(6)
    vmax = None
    skipped = 0
    pairs = [(0, 0), (143, 95), (47, 48)] + [(int(rng.integers(0, B)), int(rng.integers(0, NH)))
                                            for _ in range(5)]
    for b, head in pairs:
        oc = _pair_cache(kv, b, head, pos + 1)
        pq = _pair_qkv(q1n[b:b + 1], head)
        # the oracle's boundary gap on the kept/dropped cut for this pair
        kh, _ = oc.read(0, 0, pos + 1)
        s = np.sort((kh @ pq[0, :HD].astype(np.float64)) / np.sqrt(HD))[::-1]
        k = O.topk_count(sp, pos + 1)
        # the append already happened on the GPU: recompute attention over its cache
        oc2 = _pair_cache(kv, b, head, pos + 1)
        ref = O.attn_decode(pq, pos, oc2, sparsity=sp)
        assert np.array_equal(oc2.k_codes, oc.k_codes), "append differs from the oracle's"
        if s[k - 1] - s[k] < 1e-4:
            skipped += 1
            continue
        vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
            np.abs(oc.v_params[..., 0].astype(np.float64)).max()
        assert_close_fp16(out[b, head * HD:(head + 1) * HD], ref[0], extra=2.0**-16 * vmax,
                          what=f"topk seq {b} head {head}")
    assert skipped <= 1

    # host-CPU attention for the first micro-batch over the same cache in host memory
    _say("full-size host decode attention", 48, NH, HD, pos + 1)
    hk = F.KV4(48, NH, HD, S + 1, device="cpu")
    for n, t in kv_before.items():
        getattr(hk, n).copy_(t)
    hq = q1[:48].cpu()
    hout = F.host_attn_decode(hq, pos, hk, threads=16).numpy()
    dense = to_np(F.attn_decode(q1, pos, kv))
    for name in ("k_codes", "v_codes", "k_params", "v_params"):   # identical appends
        a = getattr(hk, name).numpy()[:, :, pos]
        bb = to_np(getattr(kv, name)[:48, :, pos])
        assert np.array_equal(a.view(np.uint8), bb.view(np.uint8)), name
    for b, head in [(0, 0), (47, 95), (int(rng.integers(0, 48)), int(rng.integers(0, NH)))]:
        oc = _pair_cache(kv, b, head, pos + 1)
        ref = O.attn_decode(_pair_qkv(q1n[b:b + 1], head), pos, oc)[0]
        vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
            np.abs(oc.v_params[..., 0].astype(np.float64)).max()
        sl = slice(head * HD, (head + 1) * HD)
        assert_close_fp16(hout[b, sl], ref, extra=2.0**-16 * vmax, what=f"host seq {b} head {head}")
        assert_close_fp16(dense[b, sl], ref, extra=2.0**-16 * vmax, what=f"dense seq {b} head {head}")
