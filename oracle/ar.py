"""DFlash-AR: the drafter with per-layer K/V injection, drafting
autoregressively.  Composed from the oracle's general masked forward.

TEST INFRASTRUCTURE ONLY, like the rest of the oracle package: the tests,
the package smoke check and the CPU baseline leg of the benchmark use it.

Follows the paper page, §5.5.5 ("KV Injection vs. Input Fusion", where
DFlash-AR keeps the K/V injection and drafts autoregressively), and the
summary page's section "Block Diffusion Makes Draft Cost Nearly Independent
of Block Length" (an autoregressive drafter pays one forward pass per
proposed token, T_draft = gamma * t_step).

Readings where the pages leave a step open (listed in the design doc):
  * Pass i (i = 1 .. gamma-1) runs the drafter over the tokens
    [anchor, d_1, ..., d_{i-1}] at positions L .. L+i-1; inside them the mask
    is causal (row j sees the context and rows 0..j); d_i is the
    lowest-index argmax of the pass's last row (next-token prediction).
  * Each pass recomputes all its rows: the drafter keeps no cache of its own
    tokens, so pass i costs one forward of i rows.
  * The logits reported for d_i are the last row of pass i.
"""
from __future__ import annotations

import numpy as np


def causal_visibility(L: int, R: int) -> np.ndarray:
    """[R][L+R]: every row sees the L context keys and the rows up to itself."""
    vis = np.zeros((R, L + R), dtype=np.uint8)
    vis[:, :L] = 1
    for j in range(R):
        vis[j, L:L + j + 1] = 1
    return vis


def draft_ar(model, ctx_k, ctx_v, L: int, anchor: int, gamma: int):
    """Block [gamma] = [anchor, d_1, ..., d_{gamma-1}] and the logits that
    chose each d_i, [gamma-1][V] float64."""
    tokens = [int(anchor)]
    chosen = []
    for i in range(1, gamma):
        toks = np.array(tokens, dtype=np.int32)
        lg = model.forward(ctx_k, ctx_v, L, toks, L + np.arange(i, dtype=np.int32),
                           causal_visibility(L, i))
        chosen.append(lg[i - 1])
        tokens.append(int(np.argmax(lg[i - 1])))
    V = model.shape.vocab
    return np.array(tokens, dtype=np.int32), (np.array(chosen) if chosen else np.empty((0, V)))
