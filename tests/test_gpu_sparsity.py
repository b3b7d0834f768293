"""Sparse (top-k) decode attention through the C ABI against the oracle's
`attn_decode(..., sparsity)`: outputs within the dense kernel's bound wherever the kept
set is unambiguous (the oracle's gap between the last kept and the first dropped score
is above the fp32 score error), exact ties broken toward the lower position, the dense
limit, padding, argument rejection, the op on a real layer's activations, and a tiny
OPT decoding with sparse attention, teacher-forced against the oracle (logits max-abs
within 4e-2, relative Frobenius within 3e-2, and far below the sparse-vs-dense distance:
the kept sets are a discontinuous function of hidden states that the two sides compute
within the dense tolerance of each other)."""
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


def _boundary_gaps(oc, q1, pos, b0, sparsity):
    """Oracle score gap at the kept/dropped boundary for each (sequence, head)."""
    B = q1.shape[0]
    nh, hd = oc.heads, oc.head_dim
    q = q1[:, :nh * hd].reshape(B, nh, hd).astype(np.float64)
    gaps = np.full((B, nh), np.inf)
    for b in range(B):
        p0 = int(np.clip(oc.pad[b0 + b], 0, pos))
        for hh in range(nh):
            kh, _ = oc.read(b0 + b, hh, pos + 1)
            s = np.sort((kh[p0:] @ q[b, hh]) / np.sqrt(hd))[::-1]
            k = O.topk_count(sparsity, s.size)
            if k < s.size:
                gaps[b, hh] = s[k - 1] - s[k]
    return gaps


CASES = [  # B, heads, head_dim, prompt, steps, sparsity, pads
    (3, 4, 128, 200, 2, 0.25, None),
    (2, 3, 64, 100, 3, 0.05, None),
    (4, 2, 128, 529, 2, 0.5, [0, 100, 528, 3]),
    (2, 2, 64, 64, 2, 0.9, None),
    (1, 2, 128, 4000, 1, 0.1, None),          # near the 4096-position limit
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_attn_decode_topk_matches_oracle(case):
    F = require_gpu()
    B, nh, hd, S, steps, sp, pads = CASES[case]
    _say("attn_decode_topk", B, nh, hd, S, steps, sp, pads)
    rng = np.random.default_rng(case + 80)
    T = S + steps
    padt = None if pads is None else torch.tensor(pads, dtype=torch.int32, device="cuda")
    kv = F.KV4(B, nh, hd, T, pad=padt)
    oc = O.KVCache(B, nh, hd, T)
    if pads is not None:
        oc.pad[:] = pads
    qkv = _qkv(rng, B * S, nh, hd)
    F.attn_prefill(torch.from_numpy(qkv).cuda(), B, S, kv)
    O.attn_prefill(qkv, B, S, nh, hd, oc)
    skipped = 0
    for i in range(steps):
        pos = S + i
        q1 = _qkv(rng, B, nh, hd)
        out = to_np(F.attn_decode_topk(torch.from_numpy(q1).cuda(), pos, kv, sp))
        torch.cuda.synchronize()
        ref = O.attn_decode(q1, pos, oc, sparsity=sp)
        gaps = _boundary_gaps(oc, q1, pos, 0, sp)
        vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
            np.abs(oc.v_params[..., 0].astype(np.float64)).max()
        for b in range(B):
            for hh in range(nh):
                if gaps[b, hh] < 1e-4:       # ambiguous kept set: either choice is valid
                    skipped += 1
                    continue
                sl = slice(hh * hd, (hh + 1) * hd)
                assert_close_fp16(out[b, sl], ref[b, sl], extra=2.0**-16 * vmax,
                                  what=f"topk pos {pos} seq {b} head {hh}")
        assert np.array_equal(to_np(kv.k_codes), oc.k_codes)
    assert skipped <= max(1, B * nh * steps // 10)


def test_attn_decode_topk_ties_keep_lower_positions():
    F = require_gpu()
    _say("attn_decode_topk ties")
    rng = np.random.default_rng(90)
    nh, hd, S = 1, 128, 9
    k = (rng.normal(size=(S, hd)) * 0.01).astype(F16)
    big = rng.normal(size=hd).astype(F16)
    for t in (2, 5, 6, 8):
        k[t] = big
    v = rng.normal(size=(S, hd)).astype(F16)
    qkv = np.zeros((S, 3 * hd), F16)
    qkv[:, hd:2 * hd] = k
    qkv[:, 2 * hd:] = v
    kv = F.KV4(1, nh, hd, S + 1)
    oc = O.KVCache(1, nh, hd, S + 1)
    F.attn_prefill(torch.from_numpy(qkv).cuda(), 1, S, kv)
    O.attn_prefill(qkv, 1, S, nh, hd, oc)
    q1 = np.zeros((1, 3 * hd), F16)
    q1[0, :hd] = big
    q1[0, hd:2 * hd] = k[0]
    for sp in (2.5 / 10, 1.5 / 10):          # keep 3 (positions 2, 5, 6) and 2 (2, 5)
        got = to_np(F.attn_decode_topk(torch.from_numpy(q1).cuda(), S, kv, sp))
        kv_copy = O.KVCache(1, nh, hd, S + 1)
        for a in ("k_codes", "v_codes", "k_params", "v_params"):
            getattr(kv_copy, a)[...] = getattr(oc, a)
        ref = O.attn_decode(q1, S, kv_copy, sparsity=sp)
        vmax = np.abs(v.astype(np.float64)).max() * 1.1
        assert_close_fp16(got, ref, extra=2.0**-16 * vmax, what=f"ties sparsity {sp}")


def test_attn_decode_topk_dense_limit():
    F = require_gpu()
    _say("attn_decode_topk dense limit")
    rng = np.random.default_rng(91)
    B, nh, hd, S = 2, 4, 128, 300
    kv = F.KV4(B, nh, hd, S + 1)
    F.attn_prefill(torch.from_numpy(_qkv(rng, B * S, nh, hd)).cuda(), B, S, kv)
    q1 = torch.from_numpy(_qkv(rng, B, nh, hd)).cuda()
    a = to_np(F.attn_decode_topk(q1, S, kv, 1.0))
    b = to_np(F.attn_decode(q1, S, kv))
    assert_close_fp16(a, b, extra=2.0**-14, what="sparsity 1 vs dense")


def test_attn_decode_topk_rejects():
    F = require_gpu()
    kv = F.KV4(1, 1, 64, 5000)
    q1 = torch.zeros(1, 3 * 64, dtype=torch.float16, device="cuda")
    for sp in (0.0, -0.5, float("nan"), float("inf")):
        with pytest.raises(F.FlexqError):
            F.attn_decode_topk(q1, 3, kv, sp)
    with pytest.raises(F.FlexqError):
        F.attn_decode_topk(q1, 4096, kv, 0.5)     # 4097 positions: beyond the LDS scores


def test_opt125m_layer_qkv_topk_teacher_forced():
    # the attention op on the activations of a real layer: LN and QKV projection of
    # the OPT-125m layer on the GPU, then sparse decode attention on that qkv against
    # the oracle's on the same qkv
    F = require_gpu()
    from group_wise_bit_flexq_amd.workloads import WORKLOADS
    wl = WORKLOADS["opt125m-layer"]
    h, nh, hd, f, B, S, G = wl.hidden, wl.heads, wl.head_dim, wl.ffn, wl.batch, wl.prompt, wl.gen
    sp = 0.2
    _say("opt125m layer qkv, sparse decode attention", sp)
    w16 = synth.layer_weights_fp16(h, f, 0, 0)
    L = F.QLayer.from_fp16(w16, nh)
    v = {k: t.cuda() for k, t in w16.items() if k in F.QLayer.VECS}
    kv = F.KV4(B, nh, hd, S + G)
    oc = O.KVCache(B, nh, hd, S + G)

    def qkv_of(x):
        a = F.layernorm(torch.from_numpy(x).cuda(), v["ln1_g"], v["ln1_b"])
        return F.linear_w4(a, L.m["wqkv"], bias=v["bqkv"])

    x = synth.normal_fp16((B * S, h), 1.0, synth.sub_seed(0, "x", 0)).numpy()
    qp = qkv_of(x)
    F.attn_prefill(qp, B, S, kv)
    O.attn_prefill(to_np(qp), B, S, nh, hd, oc)
    skipped = compared = 0
    for i in range(G):
        pos = S + i
        q1 = qkv_of(synth.normal_fp16((B, h), 1.0, synth.sub_seed(0, "xd", i)).numpy())
        qn = to_np(q1)
        out = to_np(F.attn_decode_topk(q1, pos, kv, sp))
        ref = O.attn_decode(qn, pos, oc, sparsity=sp)
        gaps = _boundary_gaps(oc, qn, pos, 0, sp)
        vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
            np.abs(oc.v_params[..., 0].astype(np.float64)).max()
        for b in range(B):
            for hh in range(nh):
                if gaps[b, hh] < 1e-4:
                    skipped += 1
                    continue
                compared += 1
                sl = slice(hh * hd, (hh + 1) * hd)
                assert_close_fp16(out[b, sl], ref[b, sl], extra=2.0**-16 * vmax,
                                  what=f"layer topk pos {pos} seq {b} head {hh}")
    print(f"compared {compared}, ambiguous kept sets {skipped}", flush=True)
    assert skipped <= compared // 20


def test_tiny_model_sparse_decode():
    F = require_gpu()
    from tests.test_gpu_model import _gpu_model, _host_model, _oracle_model
    nh, B, S, G, mb, sp = 4, 4, 60, 5, 2, 0.3
    _say("tiny model sparse decode", sp)
    parts = _host_model(256, nh, 1024, 1000, 2, 9)
    V = parts[1].shape[0]
    gm = _gpu_model(F, parts, nh, B, S + G - 1, mb * S)
    gm.set_attn_sparsity(sp)
    toks = synth.token_ids(B, S, V, synth.sub_seed(0, "tokens")).cuda()
    out = torch.empty(B, G, dtype=torch.int32, device="cuda")
    first = torch.empty(B, dtype=torch.int32, device="cuda")
    logits = torch.empty(G, B, V, dtype=torch.float32, device="cuda")
    for j in range(B // mb):
        sl = slice(j * mb, (j + 1) * mb)
        gm.prefill(toks[sl], b0=j * mb, logits=logits[0, sl], next_out=first[sl])
    out[:, 0].copy_(first)
    cur = first
    for i in range(G - 1):
        nxt = gm.decode_step(cur, S + i, logits=logits[i + 1])
        out[:, i + 1].copy_(nxt)
        cur = nxt
    torch.cuda.synchronize()
    gl, go = to_np(logits), to_np(out).astype(np.int64)
    # the same decode steps with dense attention, on the same tokens
    gm.set_attn_sparsity(0.0)
    dense = torch.empty(G - 1, B, V, dtype=torch.float32, device="cuda")
    for j in range(B // mb):
        sl = slice(j * mb, (j + 1) * mb)
        gm.prefill(toks[sl], b0=j * mb)
    for i in range(G - 1):
        gm.decode_step(out[:, i].contiguous(), S + i, logits=dense[i])
    gd = to_np(dense)
    om = _oracle_model(parts, nh)
    caches = om.new_caches(B, S + G - 1)
    lg, nx = om.prefill(to_np(toks), caches)
    for i in range(G):
        if i > 0:
            lg, nx = om.decode_step(go[:, i - 1], S + i - 1, caches, sparsity=sp)
        # The kept sets are decided on scores computed from each side's hidden states,
        # which differ within the dense tolerance; a position near the boundary can be
        # kept on one side and dropped on the other, a jump no smooth bound covers.
        # Bounds twice the dense ones (max-abs 4e-2, relative Frobenius 3e-2; measured up
        # to 2.03e-2 / 1.08e-2), and the error must stay far below the sparse-vs-dense
        # distance (measured 0.39-0.44), so the sparse path is what matches.
        err, rf = assert_logits_close(gl[i], lg, f"sparse logits step {i}", atol=4e-2,
                                    rel_frob=3e-2)
        if i > 0:
            d = np.linalg.norm(gd[i - 1] - lg) / np.linalg.norm(lg)
            print(f"step {i}: sparse rel-frob {rf:.3g}, dense-vs-sparse {d:.3g}", flush=True)
            assert rf < d / 4, (rf, d)
        for r in range(B):
            if nx[r] != go[r, i]:
                assert lg[r].max() - lg[r, go[r, i]] <= 2 * err + 1e-6, (i, r)


def test_attn_decode_topk_single_position():
    # pos 0: one candidate, kept whatever the sparsity; the output is that position's value
    F = require_gpu()
    _say("attn_decode_topk at pos 0")
    rng = np.random.default_rng(92)
    nh, hd = 2, 64
    kv = F.KV4(1, nh, hd, 4)
    oc = O.KVCache(1, nh, hd, 4)
    q1 = _qkv(rng, 1, nh, hd)
    got = to_np(F.attn_decode_topk(torch.from_numpy(q1).cuda(), 0, kv, 0.01))
    ref = O.attn_decode(q1, 0, oc, sparsity=0.01)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
