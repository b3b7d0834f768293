"""Argument checks of the C ABI, forced from the host (needs an MI355X).

Every call checks its arguments before it enqueues anything: a rejected call returns
its status and leaves the output buffers untouched.  Each case here is a real call
through the library with one argument made invalid; nothing is launched."""
import numpy as np
import pytest
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16, require_gpu, to_np

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E01          # an fp16 NaN pattern that no kernel writes


def _say(*a):
    print("[case]", *a, flush=True)


def _sentinel(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.float16)


def _untouched(t):
    torch.cuda.synchronize()
    return bool((t.view(torch.int16) == SENTINEL).all())


def _status(F, fn):
    try:
        fn()
    except F.FlexqError as e:
        return e.status
    return F.OK


def _weight(F, rng, N, K):
    w = (rng.normal(size=(N, K)) * 0.05).astype(F16)
    codes, params = O.quantize(w)
    return F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda()), \
        codes, params


def test_linear_rejects_k_not_multiple_of_64():
    F = require_gpu()
    _say("linear K % 64")
    rng = np.random.default_rng(1)
    wq, _, _ = _weight(F, rng, 128, 128)
    bad = F.W4(wq.codes, wq.params, wq.rows)
    bad.cols = 100                                    # the struct says K = 100
    x = torch.zeros(4, 128, dtype=torch.float16, device="cuda")
    y = _sentinel((4, 128))
    assert _status(F, lambda: F.linear_w4(x, bad, out=y)) == F.ERR_INVALID
    assert _untouched(y)


@pytest.mark.parametrize("M,N,K", [(144, 1024, 8192), (32, 512, 8192), (512, 512, 4096)])
def test_linear_short_workspace_runs_fewer_splits(M, N, K):
    """A workspace below flexq_linear_w4_workspace_size is accepted: the call runs with
    as many split-K partials as fit (none with NULL), within the same bound."""
    F = require_gpu()
    _say("linear short ws", M, N, K)
    rng = np.random.default_rng(M + N + K)
    wq, codes, params = _weight(F, rng, N, K)
    x = rng.normal(size=(M, K)).astype(F16)
    xt = torch.from_numpy(x).cuda()
    need = F.linear_ws_bytes(M, N, K)
    assert need > 0, "shape must use split-K"
    ref = O.linear_w4(x, codes, params)
    wd = O.dequantize_weight(codes, params).astype(np.float64)
    bound = 1e-7 + K * 2.0**-24 * (np.abs(x.astype(np.float64)) @ np.abs(wd).T)
    import ctypes as C
    buf = torch.empty(need, dtype=torch.uint8, device="cuda")
    wc = wq.c()
    for ws_bytes in (need, need // 2, M * N * 4 * 2, 0):
        y = torch.empty(M, N, dtype=torch.float16, device="cuda")
        st = F.lib().flexq_linear_w4(xt.data_ptr(), M, C.byref(wc), None, None, 0, y.data_ptr(),
                                     buf.data_ptr() if ws_bytes else None, ws_bytes, F._stream())
        assert st == F.OK, (ws_bytes, st)
        assert_close_fp16(to_np(y), ref, extra=bound, what=f"ws {ws_bytes} of {need}")


def test_attn_decode_rejects_short_workspace_and_bad_head_dim():
    F = require_gpu()
    _say("attn_decode ws / head_dim")
    B, nh, hd, pos = 2, 4, 128, 1500
    need = F.attn_decode_ws_bytes(B, nh, hd, pos)
    assert need > 0, "a split context needs the merge workspace"
    kv = F.KV4(B, nh, hd, pos + 1)
    q = torch.zeros(B, 3 * nh * hd, dtype=torch.float16, device="cuda")
    import ctypes as C
    k_before = kv.k_codes.clone()
    buf = torch.empty(need, dtype=torch.uint8, device="cuda")
    kc = kv.c()
    for ptr, nbytes in ((None, 0), (None, need), (buf.data_ptr(), need - 16)):
        y = _sentinel((B, nh * hd))
        st = F.lib().flexq_attn_decode_kv4(q.data_ptr(), B, 0, pos, C.byref(kc), y.data_ptr(),
                                           ptr, nbytes, F._stream())
        assert st == F.ERR_INVALID, (ptr, nbytes, st)
        assert _untouched(y)
    assert torch.equal(kv.k_codes, k_before), "a rejected call must not append"
    # head_dim 96 is not a whole number of 64-groups: unsupported
    kv96 = F.KV4(B, nh, 96, 64)
    q96 = torch.zeros(B, 3 * nh * 96, dtype=torch.float16, device="cuda")
    y = _sentinel((B, nh * 96))
    assert _status(F, lambda: F.attn_decode(q96, 10, kv96, out=y,
                                            ws=torch.empty(1 << 20, dtype=torch.uint8,
                                                           device="cuda"))) == F.ERR_UNSUPPORTED
    assert _untouched(y)
    # position past the cache
    y = _sentinel((B, nh * hd))
    assert _status(F, lambda: F.attn_decode(q, pos + 1, kv, out=y)) == F.ERR_INVALID
    assert _untouched(y)


def test_prefill_attention_rejects_prompt_longer_than_cache():
    F = require_gpu()
    _say("attn_prefill S > max_len")
    B, S, nh, hd = 2, 65, 2, 64
    kv = F.KV4(B, nh, hd, 64)
    qkv = torch.zeros(B * S, 3 * nh * hd, dtype=torch.float16, device="cuda")
    y = _sentinel((B * S, nh * hd))
    assert _status(F, lambda: F.attn_prefill(qkv, B, S, kv, out=y)) == F.ERR_INVALID
    assert _untouched(y)


def test_quantize_and_layernorm_reject_bad_shapes():
    F = require_gpu()
    _say("quantize / layernorm shapes")
    x = torch.zeros(4, 96, dtype=torch.float16, device="cuda")
    assert _status(F, lambda: F.quantize(x)) == F.ERR_INVALID          # 96 % 64 != 0
    x = torch.zeros(4, 128, dtype=torch.float16, device="cuda")
    lib = F.lib()
    q = F.Q4.empty(4, 128)
    st = lib.flexq_quantize(x.data_ptr(), 4, 128, F.QConfig(3, 64, 0), q.codes.data_ptr(),
                            q.params.data_ptr(), F._stream())
    assert st == F.ERR_UNSUPPORTED                                      # 3-bit: quantize_ex
    g = torch.ones(100, dtype=torch.float16, device="cuda")
    y = _sentinel((4, 100))
    xl = torch.zeros(4, 100, dtype=torch.float16, device="cuda")
    assert _status(F, lambda: F.layernorm(xl, g, g, out=y)) == F.ERR_INVALID   # 100 % 8
    assert _untouched(y)


def _tiny_model(F, layers=2, h=128, nh=2, f=256, V=256, B=3, max_len=12):
    from group_wise_bit_flexq_amd import synth
    Ls = [F.QLayer.from_fp16(synth.layer_weights_fp16(h, f, 5, l), nh) for l in range(layers)]
    emb = F.quantize_weight(synth.normal_fp16((V, h), 0.5, 3).cuda())
    pos = synth.normal_fp16((2050, h), 0.1, 4).cuda()
    g = torch.ones(h, dtype=torch.float16, device="cuda")
    b = torch.zeros(h, dtype=torch.float16, device="cuda")
    return F.QModel(Ls, emb, pos, g, b, nh, B, max_len, B * max_len)


def test_model_calls_reject_positions_and_rows_outside_the_caches():
    F = require_gpu()
    _say("model bounds")
    m = _tiny_model(F)
    toks = torch.zeros(3, 8, dtype=torch.int32, device="cuda")
    m.prefill(toks)
    cur = torch.zeros(3, dtype=torch.int32, device="cuda")
    nxt = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    # pos >= max_len
    assert _status(F, lambda: m.decode_step(cur, 12, next_out=nxt)) == F.ERR_INVALID
    # more sequences than cache rows
    cur4 = torch.zeros(4, dtype=torch.int32, device="cuda")
    nxt4 = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    assert _status(F, lambda: m.decode_step(cur4, 9, next_out=nxt4)) == F.ERR_INVALID
    # prompt longer than the cache
    long = torch.zeros(1, 13, dtype=torch.int32, device="cuda")
    nxt1 = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    assert _status(F, lambda: m.prefill(long, next_out=nxt1)) == F.ERR_INVALID
    torch.cuda.synchronize()
    assert (nxt == -7).all() and (nxt4 == -7).all() and (nxt1 == -7).all()
    # the last valid position still runs
    m.decode_step(cur, 11, next_out=nxt)
    torch.cuda.synchronize()
    assert ((nxt >= 0) & (nxt < 256)).all()
