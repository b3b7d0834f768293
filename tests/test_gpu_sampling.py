"""Token choice through the C ABI (flexq_pick, and the model's output head under a
generation config) against the oracle's `pick`: greedy bit-exact with ties, Gumbel-max
sampling on the same logits identical except where two fp64 scores agree to 1e-12
(the two sides' log functions may differ in the last bit), keyed by sequence and step
(batch splits do not change a draw), the stop rule, and sampled generation of a tiny
OPT with a stop token, teacher-forced against the oracle."""
import numpy as np
import pytest
import torch

from group_wise_bit_flexq_amd import synth
from oracle import flexq_oracle as O
from tests.gpu_helpers import assert_logits_close, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _scores(lg, gen, step, m0):
    u = O.sample_uniform(gen["seed"], step, np.arange(m0, m0 + lg.shape[0]), lg.shape[1])
    return lg.astype(np.float64) / np.float64(np.float32(gen["temperature"])) - np.log(-np.log(u))


def _assert_same_picks(got, want, lg, gen, step, m0):
    """Identical tokens, except at fp64 near-ties of the sampling scores."""
    diff = np.nonzero(got != want)[0]
    if diff.size == 0:
        return 0
    assert gen is not None and gen["do_sample"], f"greedy picks differ at rows {diff[:8]}"
    for r in diff:
        sr = _scores(lg[r:r + 1], gen, step, m0 + r)[0]
        a, b = sr[want[r]], sr[got[r]]
        assert abs(a - b) <= 1e-12 * max(1.0, abs(a)), (f"row {r}: GPU {got[r]} vs oracle "
                                                         f"{want[r]}, scores {b!r} vs {a!r}")
    return diff.size


def _gen(do_sample, temperature=1.0, seed=0, stop=-1):
    return dict(do_sample=do_sample, temperature=temperature, seed=seed, stop=stop)


@pytest.mark.parametrize("M,N", [(1, 1), (5, 64), (37, 1000), (144, 50272), (3, 250000)])
@pytest.mark.parametrize("mode", ["greedy", "t0.7", "t1.0", "t1.6"])
def test_pick_matches_oracle(M, N, mode):
    F = require_gpu()
    _say("pick", M, N, mode)
    rng = np.random.default_rng(M * 7 + N)
    lg = (rng.normal(size=(M, N)) * 3).astype(np.float32)
    # a few exact ties at the maximum
    if N > 8:
        lg[:, 5] = lg[:, 3] = lg.max(axis=1) + 1
    gen = None if mode == "greedy" else _gen(True, float(mode[1:]), seed=0xDEADBEEF12345, stop=-1)
    step, m0 = 511, 17
    g = F.pick(torch.from_numpy(lg).cuda(), None if gen is None else F.gen_config(**gen),
               step=step, m0=m0)
    torch.cuda.synchronize()
    want = O.pick(lg, gen, step, m0)
    ties = _assert_same_picks(to_np(g).astype(np.int64), want, lg, gen, step, m0)
    assert ties <= max(1, M // 50)
    if gen is None and N > 8:
        assert np.all(to_np(g) == 3)


def test_pick_greedy_config_equals_argmax():
    F = require_gpu()
    _say("pick greedy config")
    rng = np.random.default_rng(1)
    lg = torch.from_numpy(rng.normal(size=(64, 5000)).astype(np.float32)).cuda()
    a = F.argmax(lg)
    b = F.pick(lg, F.gen_config(False, 0.5, 9, -1))
    c = F.pick(lg)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_pick_draw_is_keyed_by_sequence_not_batch_slot():
    F = require_gpu()
    _say("pick batch split")
    rng = np.random.default_rng(2)
    lg = torch.from_numpy(rng.normal(size=(40, 3000)).astype(np.float32)).cuda()
    gen = F.gen_config(True, 1.0, 77, -1)
    whole = F.pick(lg, gen, step=9, m0=100)
    parts = torch.cat([F.pick(lg[:13], gen, step=9, m0=100), F.pick(lg[13:], gen, step=9, m0=113)])
    assert torch.equal(whole, parts)
    other = F.pick(lg, gen, step=10, m0=100)
    assert not torch.equal(whole, other)


def test_pick_stop_rule():
    F = require_gpu()
    _say("pick stop rule")
    lg = np.zeros((4, 10), np.float32)
    lg[0, 2] = lg[1, 4] = lg[2, 4] = lg[3, 2] = 1
    stopped = torch.tensor([0, 0, 1, 0], dtype=torch.int32, device="cuda")
    gen = F.gen_config(False, 1.0, 0, 2)
    nxt = F.pick(torch.from_numpy(lg).cuda(), gen, stopped=stopped)
    assert to_np(nxt).tolist() == [2, 4, 2, 2]
    assert to_np(stopped).tolist() == [1, 0, 1, 1]
    ost = np.array([False, False, True, False])
    assert O.pick(lg, _gen(False, stop=2), stopped=ost).tolist() == [2, 4, 2, 2]
    # no stop token: the flags are left alone
    st2 = torch.tensor([0, 1, 0, 1], dtype=torch.int32, device="cuda")
    nxt2 = F.pick(torch.from_numpy(lg).cuda(), F.gen_config(False), stopped=st2)
    assert to_np(nxt2).tolist() == [2, 4, 4, 2] and to_np(st2).tolist() == [0, 1, 0, 1]


def test_pick_rejects_bad_configs():
    F = require_gpu()
    lg = torch.zeros(4, 10, dtype=torch.float32, device="cuda")
    for gen, step, m0 in [(F.gen_config(True, 0.0), 0, 0), (F.gen_config(True, -1.0), 0, 0),
                          (F.gen_config(True, float("inf")), 0, 0),
                          (F.gen_config(True, float("nan")), 0, 0),
                          (F.gen_config(False, 1.0, 0, 10), 0, 0),
                          (F.gen_config(True, 1.0), 65536, 0), (F.gen_config(True, 1.0), 0, 65533)]:
        with pytest.raises(F.FlexqError):
            F.pick(lg, gen, step=step, m0=m0)


def _run(gm, toks, S, G, mb, logits):
    B = toks.shape[0]
    out = torch.empty(B, G, dtype=torch.int32, device="cuda")
    first = torch.empty(B, dtype=torch.int32, device="cuda")
    for j in range(B // mb):
        gm.prefill(toks[j * mb:(j + 1) * mb], b0=j * mb, logits=logits[0, j * mb:(j + 1) * mb],
                   next_out=first[j * mb:(j + 1) * mb])
    out[:, 0].copy_(first)
    cur = first
    for i in range(G - 1):
        nxt = gm.decode_step(cur, S + i, logits=logits[i + 1])
        out[:, i + 1].copy_(nxt)
        cur = nxt
    torch.cuda.synchronize()
    return to_np(out).astype(np.int64)


def test_tiny_model_sampled_generation_with_stop():
    F = require_gpu()
    from tests.test_gpu_model import _gpu_model, _host_model, _oracle_model
    _say("tiny model sampled generation with stop")
    nh, B, S, G, mb = 4, 6, 40, 8, 3
    parts = _host_model(256, nh, 1024, 1000, 2, 5)
    V = parts[1].shape[0]
    gm = _gpu_model(F, parts, nh, B, S + G - 1, mb * S)
    toks = synth.token_ids(B, S, V, synth.sub_seed(0, "tokens")).cuda()
    logits = torch.empty(G, B, V, dtype=torch.float32, device="cuda")
    free_cfg = _gen(True, 0.8, seed=123, stop=-1)
    gm.set_generation(F.gen_config(**free_cfg))
    free = _run(gm, toks, S, G, mb, logits)
    stop = int(free[0, 2])
    cfg = _gen(True, 0.8, seed=123, stop=stop)
    gm.set_generation(F.gen_config(**cfg))
    out = _run(gm, toks, S, G, mb, logits)
    gl = to_np(logits)
    # the stop rule on top of the free run: identical up to the first stop, then stop
    for r in range(B):
        hit = np.nonzero(free[r] == stop)[0]
        k = hit[0] if hit.size else G
        assert np.array_equal(out[r, :k], free[r, :k]), r
        assert np.all(out[r, k:] == stop), r
    assert np.all(out[0, 2:] == stop)
    assert np.array_equal(to_np(gm.stopped) != 0, np.any(out == stop, axis=1))
    # every step's choice is the oracle's pick on the same logits
    stopped = np.zeros(B, bool)
    for i in range(G):
        want = O.pick(gl[i], cfg, S - 1 + i, 0, stopped)
        _assert_same_picks(out[:, i], want, gl[i], cfg, S - 1 + i, 0)
        stopped |= out[:, i] == stop
    # and the logits follow the oracle model teacher-forced on the GPU's tokens
    sample = [0, 4]
    om = _oracle_model(parts, nh)
    caches = om.new_caches(len(sample), S + G - 1)
    lg, _ = om.prefill(to_np(toks)[sample], caches)
    for i in range(G):
        if i > 0:
            lg, _ = om.decode_step(out[sample, i - 1], S + i - 1, caches)
        assert_logits_close(gl[i, sample], lg, f"logits step {i}")
    # a greedy config through the same head gives the greedy tokens
    gm.set_generation(F.gen_config(False))
    g1 = _run(gm, toks, S, G, mb, logits)
    gm.set_generation(None)
    g2 = _run(gm, toks, S, G, mb, logits)
    assert np.array_equal(g1, g2)
