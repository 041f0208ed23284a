"""Autoregressive drafting (DFlash-AR) on the GPU vs the oracle's passes
(oracle/ar.py): each pass is causal inside the block and proposes the
argmax of its last row.

Tolerances as in the draft tests: the logits that chose each token within
1e-4 of the largest reference logit (fp32 models) or 2e-2 (bf16 models);
a token may differ from the oracle's only where the oracle's top-2 gap is
below that tolerance, and since later passes then see different tokens,
checking stops at such a tie.

Covers: the tiny fp32 workload, a mini bf16 model (batch 3, ragged and
empty contexts, fused and plain paths as the pass grows), the Qwen3-8B
shape at batch 1 and 2048 context tokens, attention splits run longest
first (batch 8, a 1002-page table), a block of one, and agreement of
the GPU's last-pass logits with its own earlier choices."""
import numpy as np
import pytest

from oracle import ar
import oracle
from gpu_util import log, logits_tolerance, make_drafter
from synth.configs import CONFIGS, anchors, context_lengths, make_weights
from test_gpu_draft import MINI, _c2_weights, pages_for, setup_cache

pytestmark = pytest.mark.gpu


def run_ar(s, ctx_lens, gamma, weights=None):
    import torch
    log(f"AR draft {s.name}: batch {len(ctx_lens)} block {gamma} contexts {list(ctx_lens)[:8]}")
    w = weights if weights is not None else make_weights(s)
    drafter, w, _ = make_drafter(s, w)
    pps = pages_for(max(ctx_lens))
    cache, kv, dense = setup_cache(s, ctx_lens, pps)
    B = len(ctx_lens)
    anc = anchors(s, B, tag=f"ar.anchor.{gamma}")
    ws = torch.empty(drafter.ar_workspace_bytes(B, gamma, pps), dtype=torch.uint8, device="cuda")
    a = torch.from_numpy(np.asarray(anc, np.int32)).cuda()
    blk = torch.full((B, gamma), -5, dtype=torch.int32, device="cuda")
    lg = torch.full((B, max(gamma - 1, 1), s.vocab), float("nan"), device="cuda")
    drafter.draft_ar(kv, a, gamma, blk, ws, logits=lg if gamma > 1 else None)
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    return blk.cpu().numpy(), lg.cpu().numpy(), anc, dense, w


def check(s, ctx_lens, gamma, res):
    blk, lg, anc, dense, w = res
    model = oracle.Model(s, w)
    for b, L in enumerate(ctx_lens):
        k, v = dense[b]
        ref_blk, ref_lg = ar.draft_ar(model, k, v, int(L), int(anc[b]), gamma)
        assert blk[b, 0] == anc[b]
        tol = logits_tolerance(s, ref_lg) if gamma > 1 else 0.0
        tok_tol = 2e-2 if s.bf16 else tol
        checked = 0
        for i in range(1, gamma):
            row = ref_lg[i - 1]
            err = float(np.max(np.abs(lg[b, i - 1].astype(np.float64) - row)))
            assert err <= tol, (b, i, err, tol)
            checked += 1
            if blk[b, i] != ref_blk[i]:
                top = int(np.argmax(row))
                gap = row[top] - row[int(blk[b, i])]
                assert gap < tok_tol, (b, i, blk[b, i], ref_blk[i], gap)
                break
        log(f"  seq {b} (L={L}): {checked} passes checked, block {blk[b, :6].tolist()}...")
        # causality on the GPU: the last pass's rows chose the earlier tokens
        # (the passes differ in row count and so in summation order: ties
        # within the tolerance may go either way)
        for j in range(gamma - 1):
            row = lg[b, j].astype(np.float64)
            top = int(np.argmax(row))
            if top != blk[b, j + 1]:
                assert row[top] - row[int(blk[b, j + 1])] < tok_tol, (b, j)


def test_ar_tiny_fp32_workload():
    s = CONFIGS[1]
    L = context_lengths(s)
    check(s, L, s.block, run_ar(s, L, s.block))


def test_ar_mini_bf16_batch():
    s = MINI
    ctx = [0, 40, 133]
    check(s, ctx, 16, run_ar(s, ctx, 16))


def test_ar_mini_bf16_longest_first_order():
    # causal block keys when the attention runs its splits longest first
    from test_gpu_draft import LONGEST_FIRST
    s = MINI
    ctx = LONGEST_FIRST[0]
    check(s, ctx, 5, run_ar(s, ctx, 5))


def test_ar_block_of_one():
    s = MINI
    blk, lg, anc, dense, w = run_ar(s, [7], 1)
    assert blk[0, 0] == anc[0]


def test_ar_qwen3_8b_batch1():
    s = CONFIGS[2]
    L = context_lengths(s)
    check(s, L, 16, run_ar(s, L, 16, weights=_c2_weights()))
