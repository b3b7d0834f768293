"""Pins of the oracle's token choice (`pick`) and its counter-based generator: the
SplitMix64 generator against its published output sequences, the uniforms' range and
distribution, the Gumbel-max draw against softmax(logits / T) by a chi-square test,
the greedy and low-temperature limits, tie order, and the stop rule."""
import numpy as np
import pytest

from oracle import flexq_oracle as O


def test_splitmix64_published_sequences():
    # the first outputs of the SplitMix64 reference generator for seeds 0 and 1234567
    assert [int(v) for v in O.splitmix64(0, np.arange(3))] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [int(v) for v in O.splitmix64(1234567, np.arange(5))] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_uniforms_are_open_interval_and_uniform():
    u = O.sample_uniform(7, 3, np.arange(64), 4096).reshape(-1)
    assert np.all(u > 0) and np.all(u < 1)
    # u is the generator's top 52 bits, centred: output number 3 * 2^48 + 5 * 2^32 + 7
    # for step 3, sequence 5, token 7
    z = int(O.splitmix64(7, np.array([3 * 2**48 + 5 * 2**32 + 7], np.uint64))[0])
    assert O.sample_uniform(7, 3, [5], 8)[0, 7] == ((z >> 12) + 0.5) / 2.0**52
    # Kolmogorov-Smirnov statistic of 262144 draws against U(0, 1)
    s = np.sort(u)
    n = s.size
    d = max(np.max(np.arange(1, n + 1) / n - s), np.max(s - np.arange(n) / n))
    assert d < 1.63 / np.sqrt(n)                      # the 1% critical value
    # the counter separates steps, sequences and tokens
    a = O.sample_uniform(7, 3, [5], 8)
    assert not np.array_equal(a, O.sample_uniform(7, 4, [5], 8))
    assert not np.array_equal(a, O.sample_uniform(7, 3, [6], 8))
    assert not np.array_equal(a, O.sample_uniform(8, 3, [5], 8))
    assert np.array_equal(a[0, 1:], O.sample_uniform(7, 3, [5], 9)[0, 1:8])


@pytest.mark.parametrize("temp", [0.5, 1.0, 2.0])
def test_gumbel_max_draws_follow_softmax(temp):
    logits = np.array([[0.0, 1.0, -0.5, 2.0, 0.3, -3.0]], np.float32)
    gen = dict(do_sample=True, temperature=temp, seed=11, stop=-1)
    draws = np.array([O.pick(logits, gen, step=s, m0=0)[0] for s in range(20000)])
    counts = np.bincount(draws, minlength=6)
    p = np.exp(logits[0].astype(np.float64) / temp)
    p /= p.sum()
    exp = p * draws.size
    chi2 = np.sum((counts - exp) ** 2 / exp)
    assert chi2 < 20.5                               # 5 degrees of freedom, p = 0.001


def test_greedy_is_argmax_with_lowest_index_on_ties():
    lg = np.array([[1.0, 3.0, 3.0, 2.0], [-1.0, -1.0, -2.0, -1.0]], np.float32)
    assert list(O.pick(lg)) == [1, 0]
    assert list(O.pick(lg, dict(do_sample=False, temperature=1.0, seed=0, stop=-1))) == [1, 0]


def test_low_temperature_sampling_is_greedy(rng):
    # logits on a 1/64 grid with distinct maxima: at T = 1e-6 the gap over T dwarfs the
    # Gumbel noise, which stays within [-3.7, 36.8] for uniforms in [2^-53, 1 - 2^-53]
    lg = (rng.permutation(np.arange(300 * 50)) / 64.0).astype(np.float32).reshape(300, 50)
    gen = dict(do_sample=True, temperature=1e-6, seed=3, stop=-1)
    assert np.array_equal(O.pick(lg, gen, step=9), lg.argmax(axis=1))


def test_sampling_depends_on_sequence_index_not_batch_slot(rng):
    lg = rng.normal(size=(8, 1000)).astype(np.float32)
    gen = dict(do_sample=True, temperature=1.0, seed=5, stop=-1)
    whole = O.pick(lg, gen, step=4, m0=0)
    part = O.pick(lg[3:], gen, step=4, m0=3)
    assert np.array_equal(whole[3:], part)


def test_stop_token_rule():
    lg = np.zeros((3, 5), np.float32)
    lg[0, 2] = 1          # row 0 picks 2 (the stop token)
    lg[1, 4] = 1          # row 1 picks 4
    lg[2, 4] = 1          # row 2 picks 4 but was already stopped
    gen = dict(do_sample=False, temperature=1.0, seed=0, stop=2)
    stopped = np.array([False, False, True])
    nxt = O.pick(lg, gen, stopped=stopped)
    assert list(nxt) == [2, 4, 2]
    assert list(stopped) == [True, False, True]
    lg2 = np.zeros((3, 5), np.float32)
    lg2[:, 1] = 1
    assert list(O.pick(lg2, gen, stopped=stopped)) == [2, 1, 2]


def test_generate_with_stop_then_repeats_stop(rng):
    from tests.test_oracle_model import _tiny_model
    m = _tiny_model(rng, L=1, h=128, nh=2, f=256, V=40)
    tok = rng.integers(0, 40, size=(4, 5))
    free = m.generate(tok, 6, dict(do_sample=True, temperature=1.0, seed=2, stop=-1))
    greedy = m.generate(tok, 6)
    assert np.array_equal(m.generate(tok, 6, dict(do_sample=False, temperature=1.0, seed=0,
                                                  stop=-1)), greedy)
    stop = int(free[0, 1])
    out = m.generate(tok, 6, dict(do_sample=True, temperature=1.0, seed=2, stop=stop))
    for r in range(4):
        hit = np.nonzero(free[r] == stop)[0]
        if hit.size:
            k = hit[0]
            assert np.array_equal(out[r, :k + 1], free[r, :k + 1])
            assert np.all(out[r, k:] == stop)
        else:
            assert np.array_equal(out[r], free[r])
