"""Pins of the oracle's sampled drafting and lossless verification
(oracle/sampling.py) against facts that do not come from the oracle: the
generator's published reference outputs, the distributions the method must
produce (checked statistically over many draws), and special cases that
reduce to the greedy rule or to a forced decision."""
import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import sampling as S


def test_splitmix64_reference_outputs():
    # Reference outputs of SplitMix64 (Steele, Lea, Flood 2014; the public C
    # reference implementation): seed 0 and seed 1234567, outputs 1..3.
    assert [S.splitmix64(0, n) for n in (1, 2, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [S.splitmix64(1234567, n) for n in (1, 2, 3)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_uniform23_and_vector_generator_agree_with_scalar():
    n = np.array([1, 2, 3, 1 << 40, (5 << 40) | (3 << 32) | 77], dtype=np.uint64)
    u = S.uniform23(99, n)
    for i, c in enumerate(n):
        assert u[i] == ((S.splitmix64(99, int(c)) >> 41) + 0.5) / 2 ** 23
    assert np.all((u > 0) & (u < 1))


def test_uniforms_are_exact_in_fp32_and_below_one():
    # the extreme numerators of (bits + 1/2) / 2^23 survive a cast to fp32
    for bits in (0, 1, (1 << 22) + 1, (1 << 23) - 2, (1 << 23) - 1):
        u = (bits + 0.5) / 2 ** 23
        assert float(np.float32(u)) == u and np.float32(u) < np.float32(1.0)
    u = S.uniform23(7, np.arange(1, 20001, dtype=np.uint64))
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)


def _chi2_pvalue(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    expected = counts.sum() * np.asarray(probs)
    return stats.chisquare(counts, expected).pvalue


def test_gumbel_max_draws_follow_the_softmax():
    # Gumbel-max with the counter stream must draw token v with probability
    # softmax(logits)[v]; every (sequence, position) gives a fresh draw.
    logits = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4])
    p = S.softmax(logits)
    counts = np.zeros(len(logits))
    for seq in range(400):
        for pos in range(1, 51):
            counts[int(np.argmax(logits + S.gumbel(12345, seq, pos, len(logits))))] += 1
    assert _chi2_pvalue(counts, p) > 1e-3
    # and a wrong sign on the noise would be caught
    bad = np.zeros(len(logits))
    for seq in range(100):
        for pos in range(1, 51):
            bad[int(np.argmax(logits - S.gumbel(12345, seq, pos, len(logits))))] += 1
    assert _chi2_pvalue(bad, p) < 1e-6


def _random_logits(rng, rows, V, scale=1.5):
    return rng.normal(0.0, scale, size=(rows, V))


@pytest.mark.parametrize("gamma", [2, 4])
def test_first_emitted_token_follows_the_target(gamma):
    # Losslessness: whatever the drafter proposes, the first token the
    # verification emits is distributed as the target's row 0.
    rng = np.random.default_rng(5)
    V = 6
    draft = _random_logits(rng, gamma, V)
    target = _random_logits(rng, gamma, V)
    counts = np.zeros(V)
    n = 12000
    for t in range(n):
        block = S.sample_block(draft, anchor=0, seed=777, seq=t)
        u = rng.random(gamma)
        tau, out, _ = S.verify_stochastic(block, draft, target, u)
        assert 1 <= tau <= gamma and out[tau - 1] >= 0 and np.all(out[tau:] == -1)
        counts[out[0]] += 1
    assert _chi2_pvalue(counts, S.softmax(target[0])) > 1e-3
    # the drafter's own distribution is a different one: the test can tell
    assert _chi2_pvalue(counts, S.softmax(draft[1])) < 1e-6


def test_accept_probability_is_min_of_one_and_the_ratio():
    # One proposal: it survives with probability min(1, p_t(x) / p_d(x))
    # averaged over the drafter's draws = sum_x min(p_d(x), p_t(x)).
    rng = np.random.default_rng(9)
    V = 5
    draft = _random_logits(rng, 2, V)
    target = _random_logits(rng, 2, V)
    kept = 0
    n = 20000
    for t in range(n):
        block = S.sample_block(draft, anchor=0, seed=31, seq=t)
        tau, _, acc = S.verify_stochastic(block, draft, target, rng.random(2))
        kept += acc
    expect = np.sum(np.minimum(S.softmax(draft[1]), S.softmax(target[0])))
    assert abs(kept / n - expect) < 4 * np.sqrt(expect * (1 - expect) / n)


def test_equal_distributions_accept_every_proposal():
    rng = np.random.default_rng(3)
    gamma, V = 5, 7
    target = _random_logits(rng, gamma, V)
    draft = np.vstack([target[:1], target[:-1]])   # draft row k == target row k-1
    for t in range(200):
        block = S.sample_block(draft, anchor=2, seed=5, seq=t)
        u = rng.random(gamma)
        tau, out, acc = S.verify_stochastic(block, draft, target, u)
        assert tau == gamma and acc == gamma - 1
        assert np.array_equal(out[:gamma - 1], block[1:])
        assert out[gamma - 1] == S.draw(S.softmax(target[gamma - 1]), u[0])


def test_one_hot_target_reduces_to_greedy_verification():
    # At temperature 0 the target is one-hot at its argmax: the stochastic
    # rule then keeps a proposal exactly when it equals that argmax and
    # corrects with it, which is the greedy rule of the oracle's C code.
    rng = np.random.default_rng(11)
    gamma, V = 6, 9
    for t in range(100):
        target = np.zeros((gamma, V), dtype=np.float32)
        top = rng.integers(0, V, size=gamma)
        target[np.arange(gamma), top] = 2000.0       # softmax is exactly one-hot in fp64
        block = rng.integers(0, V, size=gamma).astype(np.int32)
        n = rng.integers(0, gamma)
        block[1:n + 1] = top[:n]                     # a planted matching prefix
        draft = _random_logits(rng, gamma, V)
        tau, out, _ = S.verify_stochastic(block, draft, target, rng.random(gamma))
        g_tau, g_out, _ = oracle.verify(block, target, False)
        assert tau == g_tau and np.array_equal(out[:tau], g_out[:tau])


def test_proposal_the_target_excludes_is_always_rejected():
    rng = np.random.default_rng(13)
    gamma, V = 4, 6
    draft = _random_logits(rng, gamma, V)
    target = _random_logits(rng, gamma, V)
    for t in range(100):
        block = S.sample_block(draft, anchor=0, seed=9, seq=t)
        tg = target.copy()
        tg[0, block[1]] = -2000.0                    # p_t(x_1) = 0
        tau, out, acc = S.verify_stochastic(block, draft, tg, rng.random(gamma))
        assert tau == 1 and acc == 0 and out[0] != block[1]


def test_rejection_with_an_empty_residual_draws_from_the_target():
    # equal rows and a proposal both give probability zero: the check
    # rejects it and the residual has no mass, so the target row decides
    rng = np.random.default_rng(17)
    gamma, V = 3, 6
    target = _random_logits(rng, gamma, V)
    target[0, 4] = -2000.0
    draft = np.vstack([target[:1], target[:-1]])
    block = np.array([1, 4, 2], dtype=np.int32)
    for u0 in (0.05, 0.5, 0.95):
        u = np.array([u0, 0.3, 0.3])
        tau, out, acc = S.verify_stochastic(block, draft, target, u)
        assert tau == 1 and acc == 0
        assert out[0] == S.draw(S.softmax(target[0]), u0) and out[0] != 4


def test_residual_draw_uses_only_the_positive_part():
    # the correction comes from max(0, p_t - p_d): a token where the draft
    # already puts at least the target's mass is never drawn
    pt = np.array([0.5, 0.3, 0.2])
    pd = np.array([0.1, 0.6, 0.3])
    r = np.maximum(pt - pd, 0.0)
    draws = {S.draw(r, u) for u in np.linspace(0.0, 0.999, 500)}
    assert draws == {0}
    assert S.draw(np.array([0.0, 1.0, 1.0]), 0.49) == 1 and S.draw(np.array([0.0, 1.0, 1.0]), 0.51) == 2
