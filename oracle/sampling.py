"""Sampled drafting and lossless (stochastic) verification, in numpy fp64.

TEST INFRASTRUCTURE ONLY, like the rest of the oracle package: the tests,
the package smoke check and the CPU baseline leg of the benchmark use it.

Follows the DFlash summary page, section "The Target Verifier Remains the
Correctness Anchor": a proposal x_k drawn from the drafter's distribution
p_k^d is kept with probability min(1, p_k^t(x_k) / p_k^d(x_k)); checking
stops at the first rejection, where the target draws a correction from the
residual distribution and the rest of the block is dropped; a block that
survives whole earns one bonus token from the target.

Readings where the page leaves a step open (listed in the design doc):
  * p^d and p^t are softmax distributions of the drafter's and the target's
    logits at temperature 1.
  * Proposal k (block position k >= 1) is checked against target row k - 1,
    the row that predicts position k (as in the greedy rule).
  * "Kept with probability a" means kept iff u_k < a for an input uniform u_k
    in [0, 1); the comparison is made as u_k * p^d < p^t.
  * The residual distribution is max(0, p^t - p^d), normalised.  When it has
    no mass (the two rows agree and the proposal has probability zero under
    both, so the check could not keep it), the correction is drawn from p^t.
  * A draw from a discrete distribution r with uniform u is the smallest
    token v whose cumulative mass exceeds u * sum(r).
  * The drafter draws x_k by Gumbel-max: x_k = argmax_v (logit_k(v) + g),
    g = -log(-log(w)), w a uniform from a counter-based generator (the
    SplitMix64 stream below), so that the draw is reproducible.
"""
from __future__ import annotations

import numpy as np

_GAMMA = 0x9E3779B97F4A7C15
_MASK = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> int:
    """n-th output (n >= 1) of the SplitMix64 generator started at `seed`
    (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): the state advances by the golden-ratio
    constant, and each output is the state put through the finaliser
    (xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31)."""
    z = (seed + n * _GAMMA) & _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def _splitmix64_vec(seed: int, n: np.ndarray) -> np.ndarray:
    """splitmix64 over an array of counters (uint64 arithmetic wraps)."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + n.astype(np.uint64) * np.uint64(_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def draw_counter(seq: int, pos: int, tok: np.ndarray) -> np.ndarray:
    """Counter of the drafter's draw for (sequence, block position, token):
    seq in bits 40.., pos in bits 32..39, token in bits 0..31, plus one (the
    stream's first output is n = 1)."""
    return ((np.uint64(seq) << np.uint64(40)) | (np.uint64(pos) << np.uint64(32))
            | np.asarray(tok, dtype=np.uint64)) + np.uint64(1)


def uniform23(seed: int, n: np.ndarray) -> np.ndarray:
    """Uniforms in (0, 1) from the top 23 bits of the SplitMix64 outputs:
    (bits + 1/2) / 2^23.  The numerator 2 * bits + 1 has at most 24
    significant bits, so every value is exact in fp32 as well as in fp64 and
    the largest one stays below 1."""
    bits = _splitmix64_vec(seed, n) >> np.uint64(41)
    return (bits.astype(np.float64) + 0.5) / float(1 << 23)


def gumbel(seed: int, seq: int, pos: int, vocab: int) -> np.ndarray:
    """Gumbel noise -log(-log(w)) for every token of one block position."""
    w = uniform23(seed, draw_counter(seq, pos, np.arange(vocab, dtype=np.uint64)))
    return -np.log(-np.log(w))


def sample_block(logits: np.ndarray, anchor: int, seed: int, seq: int) -> np.ndarray:
    """Block tokens of one sequence drawn from the drafter: position 0 is the
    anchor, position k >= 1 the Gumbel-max draw from logits[k]
    (lowest index on ties)."""
    logits = np.asarray(logits, dtype=np.float64)
    gamma, V = logits.shape
    block = np.empty(gamma, dtype=np.int32)
    block[0] = anchor
    for k in range(1, gamma):
        block[k] = int(np.argmax(logits[k] + gumbel(seed, seq, k, V)))
    return block


def softmax(logits: np.ndarray) -> np.ndarray:
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - np.max(x, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def draw(r: np.ndarray, u: float) -> int:
    """Smallest v with cumsum(r)[v] > u * sum(r)."""
    c = np.cumsum(np.asarray(r, dtype=np.float64))
    return int(np.searchsorted(c, u * c[-1], side="right"))


def verify_stochastic(block, draft_logits, target_logits, uniforms):
    """Lossless verification of one block.

    block [gamma] (block[0] the anchor), draft_logits [gamma][V] (row k
    predicts position k), target_logits [gamma][V] (row k predicts position
    k + 1), uniforms [gamma]: uniforms[k] decides proposal k (k >= 1),
    uniforms[0] draws the correction or the bonus token.
    Returns (tau, out [gamma] (positions >= tau are -1), accepted count)."""
    block = np.asarray(block)
    gamma = block.shape[0]
    pd = softmax(draft_logits)
    pt = softmax(target_logits)
    out = np.full(gamma, -1, dtype=np.int32)
    for k in range(1, gamma):
        x = int(block[k])
        p, q = pt[k - 1][x], pd[k][x]
        if uniforms[k] * q < p:
            out[k - 1] = x
            continue
        resid = np.maximum(pt[k - 1] - pd[k], 0.0)
        out[k - 1] = draw(resid if resid.sum() > 0.0 else pt[k - 1], float(uniforms[0]))
        return k, out, k - 1
    out[gamma - 1] = draw(pt[gamma - 1], float(uniforms[0]))
    return gamma, out, gamma - 1
