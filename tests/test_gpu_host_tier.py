"""The host-DRAM cache tier through the C ABI (flexq_model.host): a tiny OPT whose last
sequences keep their 4-bit caches in pinned host memory, attended on the CPU while the
GPU attends the rest.  The prefill of host rows (through the device stage) leaves the
same codes and params as an all-device run, bit for bit; greedy generation, ragged
prompts included, follows the oracle teacher-forced (logits within 2e-2 max-abs /
1e-2 relative Frobenius, tokens identical except where the oracle's own top-2 gap is
within twice the logit error); unsupported combinations are rejected; and sampling with
a stop token over a ragged batch half in the host tier picks what the oracle picks."""
import numpy as np
import pytest
import torch

from group_wise_bit_flexq_amd import synth
from oracle import flexq_oracle as O
from tests.gpu_helpers import assert_logits_close, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _model(F, parts, nh, B, max_len, mb, S, host_rows):
    layers16, emb, pos, g, b = parts
    layers = [F.QLayer.from_fp16(w, nh) for w in layers16]
    return F.QModel(layers, F.quantize_weight(emb.cuda()), pos.cuda(), g.cuda(), b.cuda(), nh, B,
                    max_len, mb * S, host_rows=host_rows, host_threads=4, max_prefill_batch=mb)


def _generate(gm, toks, S, G, mb, V, pad=None):
    B = toks.shape[0]
    out = torch.empty(B, G, dtype=torch.int32, device="cuda")
    first = torch.empty(B, dtype=torch.int32, device="cuda")
    logits = torch.empty(G, B, V, dtype=torch.float32, device="cuda")
    for j in range(B // mb):
        sl = slice(j * mb, (j + 1) * mb)
        gm.prefill(toks[sl], b0=j * mb, logits=logits[0, sl], next_out=first[sl],
                   pad=None if pad is None else pad[sl])
    out[:, 0].copy_(first)
    cur = first
    for i in range(G - 1):
        nxt = gm.decode_step(cur, S + i, logits=logits[i + 1])
        out[:, i + 1].copy_(nxt)
        cur = nxt
    torch.cuda.synchronize()
    return to_np(logits), to_np(out).astype(np.int64)


def _follow_oracle(parts, nh, toks, gl, go, S, G, pad=None):
    from tests.test_gpu_model import _oracle_model
    om = _oracle_model(parts, nh)
    B = toks.shape[0]
    caches = om.new_caches(B, S + G - 1)
    lg, nx = om.prefill(to_np(toks), caches, pad=pad)
    ties = 0
    for i in range(G):
        if i > 0:
            lg, nx = om.decode_step(go[:, i - 1], S + i - 1, caches)
        err, _ = assert_logits_close(gl[i], lg, f"host-tier logits step {i}")
        for r in range(B):
            if nx[r] != go[r, i]:
                assert lg[r].max() - lg[r, go[r, i]] <= 2 * err + 1e-6, (i, r)
                ties += 1
    return ties


@pytest.mark.parametrize("ragged", [False, True])
def test_tiny_model_host_tier_greedy(ragged):
    F = require_gpu()
    from tests.test_gpu_model import _host_model
    nh, B, S, G, mb, host_rows = 4, 6, 40, 6, 3, 3
    _say("tiny model, host tier", host_rows, "ragged" if ragged else "")
    parts = _host_model(256, nh, 1024, 1000, 2, 11)
    V = parts[1].shape[0]
    toks = synth.token_ids(B, S, V, synth.sub_seed(0, "tokens")).cuda()
    pad = np.array([0, 5, 39, 0, 12, 38], np.int32) if ragged else None
    gm = _model(F, parts, nh, B, S + G - 1, mb, S, host_rows)
    gl, go = _generate(gm, toks, S, G, mb, V, pad)
    ties = _follow_oracle(parts, nh, toks, gl, go, S, G, pad)
    print(f"near-tie token differences: {ties}", flush=True)
    assert ties <= 2
    # the prefill K/V of the host rows equal an all-device run's, bit for bit
    ref = _model(F, parts, nh, B, S + G - 1, mb, S, 0)
    for j in range(B // mb):
        sl = slice(j * mb, (j + 1) * mb)
        ref.prefill(toks[sl], b0=j * mb, pad=None if pad is None else pad[sl])
    torch.cuda.synchronize()
    gm2 = _model(F, parts, nh, B, S + G - 1, mb, S, host_rows)
    for j in range(B // mb):
        sl = slice(j * mb, (j + 1) * mb)
        gm2.prefill(toks[sl], b0=j * mb, pad=None if pad is None else pad[sl])
    torch.cuda.synchronize()
    for l in range(len(parts[0])):
        for name in ("k_codes", "v_codes", "k_params", "v_params"):
            dev = to_np(getattr(ref.caches[l], name))[B - host_rows:, :, :S]
            host = getattr(gm2.host_caches[l], name).numpy()[:, :, :S]
            assert np.array_equal(dev.view(np.uint8), host.view(np.uint8)), (l, name)


def test_host_tier_rejects():
    F = require_gpu()
    from tests.test_gpu_model import _host_model
    nh, B, S, mb = 4, 6, 16, 3
    parts = _host_model(256, nh, 1024, 1000, 1, 12)
    gm = _model(F, parts, nh, B, S + 2, mb, S, 4)        # host rows 2..5
    toks = torch.zeros(3, S, dtype=torch.int32, device="cuda")
    with pytest.raises(F.FlexqError):
        gm.prefill(toks, b0=1)                          # straddles row 2
    gm.prefill(toks, b0=3)
    gm.set_attn_sparsity(0.5)
    with pytest.raises(F.FlexqError):
        gm.decode_step(torch.zeros(B, dtype=torch.int32, device="cuda"), S)


def test_host_tier_sampling_stop_and_padding_together():
    # every generation feature at once: temperature sampling with a stop token over a
    # ragged batch whose last micro-batch lives in the host tier; each step's tokens are
    # the oracle's pick on the GPU's own logits, and the logits follow the oracle model
    F = require_gpu()
    from tests.test_gpu_model import _host_model
    nh, B, S, G, mb, host_rows = 4, 6, 40, 6, 3, 3
    _say("host tier + sampling + stop + padding")
    parts = _host_model(256, nh, 1024, 1000, 2, 13)
    V = parts[1].shape[0]
    toks = synth.token_ids(B, S, V, synth.sub_seed(0, "tokens")).cuda()
    pad = np.array([3, 0, 30, 7, 0, 25], np.int32)
    gm = _model(F, parts, nh, B, S + G - 1, mb, S, host_rows)
    free = _model(F, parts, nh, B, S + G - 1, mb, S, host_rows)
    cfg = dict(do_sample=True, temperature=0.9, seed=77, stop=-1)
    free.set_generation(F.gen_config(**cfg))
    _, fo = _generate(free, toks, S, G, mb, V, pad)
    stop = int(fo[4, 1])                      # a host-tier row's second token
    cfg["stop"] = stop
    gm.set_generation(F.gen_config(**cfg))
    gl, go = _generate(gm, toks, S, G, mb, V, pad)
    from tests.test_gpu_sampling import _assert_same_picks
    stopped = np.zeros(B, bool)
    for i in range(G):
        want = O.pick(gl[i], cfg, S - 1 + i, 0, stopped)
        _assert_same_picks(go[:, i], want, gl[i], cfg, S - 1 + i, 0)
        stopped |= go[:, i] == stop
    assert np.all(go[4, 1:] == stop)
    from tests.test_gpu_model import _oracle_model
    om = _oracle_model(parts, nh)
    caches = om.new_caches(B, S + G - 1)
    lg, _ = om.prefill(to_np(toks), caches, pad=pad)
    for i in range(G):
        if i > 0:
            lg, _ = om.decode_step(go[:, i - 1], S + i - 1, caches)
        assert_logits_close(gl[i], lg, f"combined logits step {i}")


def test_all_rows_in_the_host_tier():
    # no device cache rows at all: every prefill goes through the stage, every decode
    # attention runs on the CPU
    F = require_gpu()
    from tests.test_gpu_model import _host_model
    nh, B, S, G, mb = 4, 2, 24, 4, 2
    _say("all rows in the host tier")
    parts = _host_model(256, nh, 1024, 1000, 1, 14)
    V = parts[1].shape[0]
    toks = synth.token_ids(B, S, V, synth.sub_seed(0, "tokens")).cuda()
    gm = _model(F, parts, nh, B, S + G - 1, mb, S, B)
    gl, go = _generate(gm, toks, S, G, mb, V)
    assert _follow_oracle(parts, nh, toks, gl, go, S, G) <= 1
