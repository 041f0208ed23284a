"""Pins of the oracle's autoregressive drafting (oracle/ar.py) against the
block drafter and against causality, facts that do not come from the
composition itself."""
import numpy as np

import oracle
from oracle import ar
from synth.configs import CONFIGS, context_kv, make_weights


def _setup(L=12):
    s = CONFIGS[1]
    m = oracle.Model(s, make_weights(s))
    ck, cv = context_kv(s, 0, max(L, 1))
    return s, m, ck, cv


def test_first_pass_is_a_block_of_one():
    # one row that sees the context and itself: the block drafter at
    # block size 1 computes exactly this
    s, m, ck, cv = _setup()
    for L in (0, 5, 12):
        block, logits = ar.draft_ar(m, ck, cv, L, 77, 2)
        ref, _ = m.draft(ck, cv, L, np.array([77], np.int32))
        assert np.array_equal(logits[0], ref[0])
        assert block[1] == int(np.argmax(ref[0]))


def test_passes_are_causal():
    # the last pass, over all proposed tokens, reproduces every earlier
    # pass's last row: earlier rows cannot see later tokens
    s, m, ck, cv = _setup()
    L, g = 12, 6
    block, logits = ar.draft_ar(m, ck, cv, L, 5, g)
    last = m.forward(ck, cv, L, block[:g - 1], L + np.arange(g - 1), ar.causal_visibility(L, g - 1))
    assert np.array_equal(last, logits)
    assert [int(np.argmax(r)) for r in last] == list(block[1:])


def test_the_mask_matters():
    # a bidirectional pass over the same tokens changes row 0 (a missing
    # causal mask would be caught by the test above)
    s, m, ck, cv = _setup()
    L, g = 12, 5
    block, logits = ar.draft_ar(m, ck, cv, L, 5, g)
    vis = np.ones((g - 1, L + g - 1), np.uint8)
    bi = m.forward(ck, cv, L, block[:g - 1], L + np.arange(g - 1), vis)
    assert not np.array_equal(bi[0], logits[0])


def test_no_context_and_block_of_one():
    s, m, ck, cv = _setup()
    block, logits = ar.draft_ar(m, ck, cv, 0, 9, 1)
    assert list(block) == [9] and logits.shape == (0, s.vocab)
    block, logits = ar.draft_ar(m, ck, cv, 0, 9, 4)
    assert block[0] == 9 and logits.shape == (3, s.vocab)
