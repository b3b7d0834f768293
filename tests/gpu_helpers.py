"""Shared pieces of the GPU parity tests (comparison bounds, device guards)."""
import numpy as np
import pytest
import torch

F16 = np.float16


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from group_wise_bit_flexq_amd import flexq as F
    F.lib()            # loads libflexq.so or raises: no silent fallback
    return F


def to_np(t):
    return t.detach().cpu().numpy()


def ulp16(x):
    """fp16 ulp at |x| (the gap above |x| in fp16)."""
    return np.spacing(np.abs(np.asarray(x, dtype=np.float64)).astype(F16)).astype(np.float64)


def assert_close_fp16(got, ref, extra=0.0, what=""):
    """|got - ref| <= 1 fp16 ulp of ref + extra (both arrays, fp16 or wider)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    bound = ulp16(r) + extra
    bad = np.abs(g - r) > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements off; first at {tuple(i)}: "
                             f"got {g[tuple(i)]} ref {r[tuple(i)]} bound {np.broadcast_to(bound, r.shape)[tuple(i)]}")


def assert_logits_close(got, ref, what="", atol=2e-2, rel_frob=1e-2):
    """Layer outputs / logits: max-abs <= 2e-2 and relative Frobenius <= 1e-2."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    rf = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    assert err.max() <= atol, f"{what}: max-abs {err.max():.3g} > {atol} (rel-frob {rf:.3g})"
    assert rf <= rel_frob, f"{what}: rel-frob {rf:.3g} > {rel_frob}"
    return err.max(), rf
