"""flexq_attn_decode_kv4_static (the decode attention that allocates nothing) against
flexq_attn_decode_kv4 with a caller workspace (needs an MI355X).

Two calls in a row on split contexts, the second smaller, so the second reads the
static array after a larger call left other partials in it: outputs and appended
cache entries must equal the workspace entry point's bit for bit.  A request whose
partials exceed the array is refused before any work."""
import ctypes as C

import numpy as np
import pytest
import torch

from tests.gpu_helpers import F16, require_gpu

pytestmark = pytest.mark.gpu

STATIC_BYTES = 4 << 20


def _say(*a):
    print("[case]", *a, flush=True)


def _filled_cache(F, rng, B, nh, hd, T):
    kv = F.KV4(B, nh, hd, T)
    for c in (kv.k_codes, kv.v_codes):
        c.copy_(torch.from_numpy(rng.integers(0, 256, size=tuple(c.shape), dtype=np.uint8)))
    for p in (kv.k_params, kv.v_params):
        par = np.empty(tuple(p.shape), F16)
        par[..., 0] = rng.normal(0, 0.5, size=par.shape[:-1])
        par[..., 1] = rng.uniform(0.01, 0.1, size=par.shape[:-1])
        p.copy_(torch.from_numpy(par))
    return kv


def _clone(F, kv):
    c = F.KV4(kv.batch, kv.heads, kv.head_dim, kv.max_len)
    for n in ("k_codes", "v_codes", "k_params", "v_params"):
        getattr(c, n).copy_(getattr(kv, n))
    return c


def _static_call(F, q, pos, kv, out):
    kc = kv.c()
    return F.lib().flexq_attn_decode_kv4_static(q.data_ptr(), q.shape[0], 0, pos, C.byref(kc),
                                                out.data_ptr(), F._stream())


@pytest.mark.parametrize("first,second", [((8, 16, 128, 3000), (2, 4, 64, 700)),
                                          ((4, 8, 64, 5000), (1, 3, 128, 200))])
def test_static_scratch_matches_workspace_entry_point(first, second):
    F = require_gpu()
    rng = np.random.default_rng(sum(first) + sum(second))
    for B, nh, hd, pos in (first, second):
        _say("static decode", B, nh, hd, pos)
        need = F.attn_decode_ws_bytes(B, nh, hd, pos)
        assert 0 < need <= STATIC_BYTES, "the case must use the static partials"
        kv_a = _filled_cache(F, rng, B, nh, hd, pos + 1)
        kv_b = _clone(F, kv_a)
        q = torch.from_numpy(rng.normal(size=(B, 3 * nh * hd)).astype(F16)).cuda()
        ref = F.attn_decode(q, pos, kv_a)
        out = torch.full((B, nh * hd), float("nan"), dtype=torch.float16, device="cuda")
        assert _static_call(F, q, pos, kv_b, out) == F.OK
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "outputs differ from the workspace entry point"
        for n in ("k_codes", "v_codes", "k_params", "v_params"):
            assert torch.equal(getattr(kv_a, n), getattr(kv_b, n)), n


def test_static_scratch_refuses_oversize_partials():
    F = require_gpu()
    B, nh, hd, pos = 64, 64, 64, 12288          # 4096 pairs x 4 splits x 66 floats > 4 MiB
    need = F.attn_decode_ws_bytes(B, nh, hd, pos)
    assert need > STATIC_BYTES
    _say("static decode oversize", need)
    kv = F.KV4(B, nh, hd, pos + 1)              # real memory of the claimed size
    q = torch.zeros(B, 3 * nh * hd, dtype=torch.float16, device="cuda")
    out = torch.full((B, nh * hd), 7.0, dtype=torch.float16, device="cuda")
    assert _static_call(F, q, pos, kv, out) == F.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out == 7.0).all()
