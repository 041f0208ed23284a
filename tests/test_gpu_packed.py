"""Packed multi-block forward on the GPU vs the oracle's packed forward
(block b sees the context keys before its anchor and its own block only),
plus the position-decayed weighted cross-entropy vs the oracle's.

Tolerances: logits as in the draft tests (fp32 models 1e-4 of the largest
reference logit, bf16 models 2e-2 absolute); proposals as in the draft
tests; a block's loss within twice the logits tolerance plus 1e-5 relative
(a cross-entropy moves by at most twice the largest logit error).

Covers: blocks at anchor position 0 (no context) and at the full context,
unsorted anchor positions, both the fused (<= 64 rows) and the plain
(> 64 rows) draft paths, the large-product kernel (8 and 24 blocks of 16 on
the Qwen3-8B shape), fp32 and bf16 models, and the device error for an anchor
past the context."""
import numpy as np
import pytest

import oracle
from gpu_util import check_tokens, log, logits_tolerance, make_drafter
from synth import Gen
from synth.configs import CONFIGS, make_weights
from test_gpu_draft import MINI, _c2_weights, pages_for, setup_cache

pytestmark = pytest.mark.gpu


def run_packed(s, L, anchor_pos, gamma, decay, weights=None, tag="pk"):
    import torch
    anchor_pos = np.asarray(anchor_pos, np.int32)
    n = len(anchor_pos)
    log(f"packed {s.name}: {n} blocks of {gamma} over {L} context tokens, anchors at "
        f"{anchor_pos.tolist()[:8]}")
    w = weights if weights is not None else make_weights(s)
    drafter, w, _ = make_drafter(s, w)
    pps = pages_for(L)
    cache, kv, dense = setup_cache(s, [L], pps)
    g = Gen(s.seed + 77)
    anchors = g.uniform_int(f"{tag}.anchor", n, 0, s.vocab - 2).astype(np.int32)
    targets = g.uniform_int(f"{tag}.target", n * gamma, 0, s.vocab - 1).reshape(n, gamma)
    targets = targets.astype(np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = torch.empty(drafter.packed_workspace_bytes(n, gamma, pps), dtype=torch.uint8,
                     device="cuda")
    lg = torch.full((n, gamma, s.vocab), float("nan"), device="cuda")
    bt = torch.full((n, gamma), -5, dtype=torch.int32, device="cuda")
    bl = torch.full((n,), float("nan"), device="cuda")
    loss = torch.full((1,), float("nan"), device="cuda")
    drafter.packed_forward(kv, dev(anchors), dev(anchor_pos), gamma, lg, ws, targets=dev(targets),
                           decay=decay, block_tokens=bt, block_loss=bl, loss=loss)
    torch.cuda.synchronize()
    err_word = drafter.device_error()
    out = dict(logits=lg.cpu().numpy().reshape(n * gamma, s.vocab), tokens=bt.cpu().numpy(),
               block_loss=bl.cpu().numpy().astype(np.float64), loss=float(loss.cpu().numpy()[0]),
               err=err_word, anchors=anchors, targets=targets, dense=dense[0], weights=w)
    return out


def check_against_oracle(s, L, anchor_pos, gamma, decay, res):
    n = len(anchor_pos)
    model = oracle.Model(s, res["weights"])
    k, v = res["dense"]
    toks = np.full((n, gamma), s.mask_id, np.int32)
    toks[:, 0] = res["anchors"]
    ref = model.draft_packed(k, v, toks, np.asarray(anchor_pos, np.int32))
    tol = logits_tolerance(s, ref)
    err = float(np.max(np.abs(res["logits"].astype(np.float64) - ref)))
    log(f"  max|dlogit| {err:.3e} (tol {tol:.1e})")
    assert np.all(np.isfinite(res["logits"])) and err <= tol
    wts = oracle.loss_weights(decay, gamma - 1)
    ref_bl = np.empty(n)
    for b in range(n):
        rows = ref[b * gamma:(b + 1) * gamma]
        assert res["tokens"][b, 0] == res["anchors"][b]
        check_tokens(res["tokens"][b], rows, 2e-2 if s.bf16 else tol)
        ref_bl[b] = oracle.weighted_ce(rows[1:], res["targets"][b, 1:], wts)
    dl = np.abs(res["block_loss"] - ref_bl)
    log(f"  block losses {np.round(ref_bl[:4], 4).tolist()}..., max|dloss| {dl.max():.2e}")
    assert np.all(dl <= 2 * tol + 1e-5 * np.abs(ref_bl))
    assert abs(res["loss"] - ref_bl.mean()) <= 2 * tol + 1e-5 * abs(ref_bl.mean())


def test_packed_tiny_fp32():
    s = CONFIGS[1]
    L = 64
    ap = [0, 17, 64, 5, 40]
    res = run_packed(s, L, ap, s.block, 2.0)
    assert res["err"] == 0
    check_against_oracle(s, L, ap, s.block, 2.0, res)


@pytest.mark.parametrize("n_blocks", [3, 6])     # 48 rows: fused path; 96: plain path
def test_packed_mini_bf16(n_blocks):
    s = MINI
    L = 133
    ap = [0, 133, 64, 1, 100, 17][:n_blocks]
    res = run_packed(s, L, ap, 16, 7.0)
    assert res["err"] == 0
    check_against_oracle(s, L, ap, 16, 7.0, res)


# 64 rows fused; 128 rows on the large-product kernel's 8-wave 128-row tile;
# 384 rows on its other tiles
@pytest.mark.parametrize("n_blocks", [4, 8, 24])
def test_packed_qwen3_8b(n_blocks):
    s = CONFIGS[2]
    L = 2048
    g = Gen(4242 + n_blocks)
    ap = np.sort(g.uniform_int("pk.pos", n_blocks, 0, L)).astype(np.int32)
    ap[0], ap[-1] = 0, L
    res = run_packed(s, L, ap, 16, 7.0, weights=_c2_weights())
    assert res["err"] == 0
    check_against_oracle(s, L, ap, 16, 7.0, res)


def test_packed_anchor_past_the_context_sets_the_error_word():
    from block_diffusion_drafter_fc_amd import DEVERR_POS
    s = MINI
    res = run_packed(s, 40, [3, 41], 8, 4.0, tag="pkerr")
    assert res["err"] & DEVERR_POS
    assert np.all(np.isfinite(res["logits"]))
