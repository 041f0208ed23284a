"""Single-pass block draft on the GPU vs the oracle, per call: both sides get
the same seeded weights, the same synthetic context cache and the same
anchors.  Logits must agree within the stated tolerance (fp32 models: 1e-4 of
the largest reference logit; bf16 models: 2e-2 absolute) and every proposed
token must be the oracle's argmax unless the oracle's top-2 gap there is
below that tolerance.

Covers: the five workloads (every sequence of the long-context and wide
ones; the first, last and every fourth sequence of the batch-32 one, plus
its longest and shortest contexts), block sizes 4, 8 and 10 at the batch-1 Qwen3-8B shape, every GEMM path (1, 2, 4 row tiles and the tiled kernel,
packed and row-major weights),
ragged and empty contexts, several context splits, ragged blocks, a block of
one, determinism, batch invariance, other streams, replays from a captured
HIP graph, the two-wave-set LM head with fewer groups than workgroups, the
greedy LM heads without a logits output (their branch-free argmax, against
the oracle-checked run with logits), and the device error word."""
import numpy as np
import pytest

import oracle
from gpu_util import (PagedCache, check_tokens, log, logits_tolerance, make_drafter, workspace)
from synth.configs import CONFIGS, Shape, anchors, context_kv, context_lengths, make_weights

pytestmark = pytest.mark.gpu

MINI = Shape("mini-bf16", 512, 2, 4, 2, 128, 768, 1000, 16, 1, True, seed=991)
MINI_F32 = Shape("mini-f32", 256, 2, 4, 2, 64, 768, 1001, 5, 1, False, seed=992)


_C2_WEIGHTS = []


def _c2_weights():
    # generated once per session: the Qwen3-8B-shaped weights take seconds
    if not _C2_WEIGHTS:
        _C2_WEIGHTS.append(make_weights(CONFIGS[2]))
    return _C2_WEIGHTS[0]


def pages_for(L_max, extra=2):
    return (int(L_max) + 15) // 16 + extra


def setup_cache(s, ctx_lens, pages_per_seq):
    cache = PagedCache(s, len(ctx_lens), pages_per_seq)
    dense = {}
    for b, L in enumerate(ctx_lens):
        k, v = context_kv(s, b, int(L))
        cache.write_dense(b, k, v)
        dense[b] = (k, v)
    kv = cache.upload(ctx_lens)
    return cache, kv, dense


def gpu_draft(drafter, kv, anc, gamma, pages_per_seq, logits=True):
    import torch
    B = len(anc)
    ws = workspace(drafter, B, gamma, 1, pages_per_seq)
    a = torch.from_numpy(np.asarray(anc, np.int32)).cuda()
    blk = torch.full((B, gamma), -5, dtype=torch.int32, device="cuda")
    lg = torch.full((B, gamma, drafter.cfg.vocab), float("nan"), device="cuda") if logits else None
    drafter.draft(kv, a, gamma, blk, ws, logits=lg)
    torch.cuda.synchronize()
    return blk.cpu().numpy(), (lg.cpu().numpy() if logits else None)


def check_seq(s, model, dense, L, anchor, gamma, gpu_block, gpu_logits):
    k, v = dense
    toks = np.full(gamma, s.mask_id, np.int32)
    toks[0] = anchor
    ref, ref_block = model.draft(k, v, int(L), toks)
    tol = logits_tolerance(s, ref)
    err = float(np.max(np.abs(gpu_logits.astype(np.float64) - ref)))
    log(f"  L={L} gamma={gamma}: max|dlogit|={err:.3e} (tol {tol:.1e}), ref max {np.max(np.abs(ref)):.2f}")
    assert np.all(np.isfinite(gpu_logits))
    assert err <= tol
    assert gpu_block[0] == anchor
    tolerated = check_tokens(gpu_block, ref, 2e-2 if s.bf16 else tol)
    return err, tolerated


def run_case(s, ctx_lens, gamma, sample=None, weights=None, pack=True):
    log(f"draft {s.name}: batch {len(ctx_lens)} block {gamma} contexts {list(ctx_lens)[:8]}"
        f"{'' if pack else ' (unpacked weights)'}")
    w = weights if weights is not None else make_weights(s)
    drafter, w, _ = make_drafter(s, w, pack=pack)
    pps = pages_for(max(ctx_lens))
    cache, kv, dense = setup_cache(s, ctx_lens, pps)
    anc = anchors(s, len(ctx_lens), tag=f"draft.anchor.{gamma}")
    blk, lg = gpu_draft(drafter, kv, anc, gamma, pps)
    assert drafter.device_error() == 0
    model = oracle.Model(s, w)
    seqs = range(len(ctx_lens)) if sample is None else sample
    for b in seqs:
        check_seq(s, model, dense[b], ctx_lens[b], anc[b], gamma, blk[b], lg[b])
    return drafter, kv, anc, blk, lg, pps


# ---------------------------------------------------------------- workloads
def test_draft_tiny_fp32_workload():
    s = CONFIGS[1]
    run_case(s, context_lengths(s), s.block)


def test_draft_qwen3_8b_batch1_workload():
    s = CONFIGS[2]
    run_case(s, context_lengths(s), s.block, weights=_c2_weights())


@pytest.mark.parametrize("gamma", [4, 8, 10])
def test_draft_qwen3_8b_batch1_block_sizes(gamma):
    # the block-size sweep's shapes: fewer mask positions, same weights
    s = CONFIGS[2]
    run_case(s, context_lengths(s), gamma, weights=_c2_weights())


def test_draft_qwen3_8b_batch32_workload_sampled():
    # every fourth sequence, the last one, and the longest and shortest
    # contexts: a batch-offset mistake shows in any of them
    s = CONFIGS[3]
    L = context_lengths(s)
    seqs = sorted(set(range(0, s.batch, 4)) | {s.batch - 1, int(np.argmax(L)), int(np.argmin(L))})
    run_case(s, L, s.block, sample=seqs)


def test_draft_qwen3_8b_long_context_workload():
    s = CONFIGS[4]
    run_case(s, context_lengths(s), s.block)        # all four sequences


def test_draft_wide_workload():
    s = CONFIGS[5]
    run_case(s, context_lengths(s), s.block)        # all eight sequences


# --------------------------------------------------------------- edge cases
@pytest.mark.parametrize("ctx", [[37], [0, 300], [5, 0, 129], [64, 17, 300, 31, 96]])
def test_draft_mini_bf16_paths_and_ragged_contexts(ctx):
    # batch 1/2/3/5 -> 16/32/48/80 block rows: 1, 2 and 4 row tiles of the
    # skinny product, then the tiled product; contexts include 0, non-multiples
    # of 16 and of 32, and several context splits.
    run_case(MINI, ctx, 16)


@pytest.mark.parametrize("ctx", [[37], [5, 0, 129]])
def test_draft_mini_bf16_unpacked_weights(ctx):
    # the row-major weight path of the skinny products (no packed copy)
    run_case(MINI, ctx, 16, pack=False)


@pytest.mark.parametrize("gamma", [1, 7])
def test_draft_mini_bf16_ragged_block(gamma):
    run_case(MINI, [45, 200], gamma)


def test_draft_mini_f32_batch():
    run_case(MINI_F32, [3, 0, 70], MINI_F32.block)


def test_draft_is_deterministic_and_batch_invariant():
    s = MINI
    w = make_weights(s)
    ctx = [33, 250, 7]
    drafter, kv, anc, blk, lg, pps = run_case(s, ctx, 16, weights=w)
    blk2, lg2 = gpu_draft(drafter, kv, anc, 16, pps)
    assert np.array_equal(blk, blk2) and np.array_equal(lg, lg2)        # bit-identical rerun
    for b in range(len(ctx)):                                           # one sequence at a time
        cache1 = PagedCache(s, 1, pps, tag=f"single{b}")
        k, v = context_kv(s, b, ctx[b])
        cache1.write_dense(0, k, v)
        kv1 = cache1.upload([ctx[b]])
        b1, l1 = gpu_draft(drafter, kv1, [anc[b]], 16, pps)
        assert np.max(np.abs(l1[0] - lg[b])) <= 2e-2
        check_tokens(b1[0], lg[b].astype(np.float64), 2e-2)


def test_draft_on_other_streams_is_bit_identical():
    # Each hardware queue starts the workgroup -> XCD round robin at its own
    # XCD; the split-K products learn the rotation from the previous launch.
    # Switching streams (a stale rotation) and repeating on one stream must
    # give exactly the default stream's results, with no device error.
    import torch
    s = MINI
    w = make_weights(s)
    ctx = [33, 250, 7]
    drafter, kv, anc, blk, lg, pps = run_case(s, ctx, 16, weights=w)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in (streams + streams[::-1]) * 3:
        with torch.cuda.stream(st):
            b2, l2 = gpu_draft(drafter, kv, anc, 16, pps)
        assert np.array_equal(blk, b2) and np.array_equal(lg, l2)
        assert drafter.device_error() == 0


@pytest.mark.parametrize("vocab", [1000, 130])
def test_draft_lm_head_wave_sets_few_groups(vocab):
    # Hidden 4096 at one row tile runs the LM head with two wave sets per
    # 64-column group.  A small vocabulary leaves fewer groups than
    # workgroups and a ragged last group (1000 = 15 x 64 + 40, 130 = 2 x 64
    # + 2); blocks of 16 and 5 rows.
    s = Shape(f"ks-bf16-v{vocab}", 4096, 1, 32, 8, 128, 1024, vocab, 16, 1, True,
              seed=995 + vocab)
    w = make_weights(s)
    for ctx, gamma in (([70], 16), ([37], 5)):
        drafter, kv, anc, blk, _, pps = run_case(s, ctx, gamma, weights=w)
        blk2, _ = gpu_draft(drafter, kv, anc, gamma, pps, logits=False)   # branch-free fold
        assert np.array_equal(blk, blk2)


@pytest.mark.parametrize("which", ["mini", "qwen3-8b-bs1"])
def test_draft_replays_from_a_captured_graph(which):
    # The draft call allocates nothing, never waits on the host and records no
    # memset, so a HIP graph can capture it.  Each replay (with eager draft
    # calls and host synchronisation between replays) must reproduce the eager
    # call's tokens and logits exactly.  The full-size case runs the dynamic
    # LM head and the split-K products at their benchmark launch shapes.
    import torch
    if which == "mini":
        s, w, ctx = MINI, make_weights(MINI), [33, 250, 7]
    else:
        s = CONFIGS[2]
        w, ctx = _c2_weights(), list(context_lengths(s))
    drafter, _, _ = make_drafter(s, w)
    pps = pages_for(max(ctx))
    cache, kv, _ = setup_cache(s, ctx, pps)
    anc = anchors(s, len(ctx), tag="draft.graph")
    blk, lg = gpu_draft(drafter, kv, anc, s.block, pps)
    B, gamma = len(ctx), s.block
    ws = workspace(drafter, B, gamma, 1, pps)
    a = torch.from_numpy(np.asarray(anc, np.int32)).cuda()
    b2 = torch.full((B, gamma), -5, dtype=torch.int32, device="cuda")
    l2 = torch.full((B, gamma, drafter.cfg.vocab), float("nan"), device="cuda")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        drafter.draft(kv, a, gamma, b2, ws, logits=l2)   # first use of the capture stream
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        drafter.draft(kv, a, gamma, b2, ws, logits=l2)
    for r in range(4):
        b2.fill_(-7)
        l2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  {which}: replay {r}")
        assert np.array_equal(b2.cpu().numpy(), blk)
        assert np.array_equal(l2.cpu().numpy(), lg)
        b3, l3 = gpu_draft(drafter, kv, anc, gamma, pps)      # eager work between replays
        assert np.array_equal(b3, blk) and np.array_equal(l3, lg)
    assert drafter.device_error() == 0


def test_draft_device_error_word_reports_bad_page_and_anchor():
    import torch
    s = MINI
    drafter, _, _ = make_drafter(s)
    cache = PagedCache(s, 2, 4)
    kv = cache.allocate_empty()
    cache.ctx_dev.copy_(torch.tensor([20, 10], dtype=torch.int32))
    bad = torch.from_numpy(cache.table.copy())
    bad[0, 1] = cache.n_pages + 5            # outside the pool: reads are skipped
    kv_bad = cache.KVCache(cache.pages, bad.cuda(), cache.ctx_dev)
    ws = workspace(drafter, 2, 16, 1, 4)
    blk = torch.zeros((2, 16), dtype=torch.int32, device="cuda")
    drafter.draft(kv_bad, torch.tensor([1, 2], dtype=torch.int32, device="cuda"), 16, blk, ws)
    assert drafter.device_error() & 1
    assert drafter.device_error() == 0       # cleared by the read
    drafter.draft(kv, torch.tensor([1, s.vocab + 3], dtype=torch.int32, device="cuda"), 16, blk, ws)
    assert drafter.device_error() & 4


def test_draft_device_error_word_reports_context_beyond_the_page_table():
    # 8 pages of 16 keys: the attention's splits cover 128 keys, so a context
    # of 130 cannot be read whole and must be reported (not silently cut).
    import torch
    s = MINI
    drafter, _, _ = make_drafter(s)
    cache = PagedCache(s, 2, 8)
    kv = cache.allocate_empty()
    ws = workspace(drafter, 2, 16, 1, 8)
    blk = torch.zeros((2, 16), dtype=torch.int32, device="cuda")
    anc = torch.tensor([1, 2], dtype=torch.int32, device="cuda")
    cache.ctx_dev.copy_(torch.tensor([20, 128], dtype=torch.int32))
    drafter.draft(kv, anc, 16, blk, ws)
    assert drafter.device_error() == 0       # a full page table is fine
    cache.ctx_dev.copy_(torch.tensor([20, 130], dtype=torch.int32))
    drafter.draft(kv, anc, 16, blk, ws)
    assert drafter.device_error() & 2


# Several sequences whose split grid exceeds one round of resident
# workgroups (a 1002-page table: 64 splits x 2 KV heads x 8 sequences) run
# their splits longest first: full splits, partly filled ones, block keys,
# empty splits.  Empty sequences, sequences shorter than a tile and a mix of
# full and partial splits occur.
LONGEST_FIRST = [[0, 5, 33, 16000, 700, 0, 9999, 64], [16000, 15999] + [1] * 6]


@pytest.mark.parametrize("ctx", LONGEST_FIRST)
@pytest.mark.parametrize("gamma", [16, 7])
def test_draft_mini_bf16_longest_first_order(ctx, gamma):
    run_case(MINI, ctx, gamma)


GREEDY_NO_LOGITS = [[37], [5, 129], [64, 17, 300, 31], [5, 0, 129, 64, 17], [40] * 8,
                    [3 + 19 * b for b in range(17)], [250, 0] * 16]


@pytest.mark.parametrize("zero_norm", [False, True])
@pytest.mark.parametrize("ctx", GREEDY_NO_LOGITS)
def test_draft_greedy_without_logits_matches_with_logits(ctx, zero_norm):
    # Without a logits output the LM-head kernels take their branch-free
    # argmax (the fused skinny head at 16, 32 and 64 rows folds each group
    # with selects; the tiled product at 80 rows and the large product at
    # 128, 272 and 512 rows scan their fragments in order with columns past
    # the vocabulary masked); with one
    # they take the general path that run_case checks against the oracle.
    # The tokens must agree exactly, with a ragged last column group or tile
    # (vocabulary 1000), and with a zero final-norm gain, where every row is
    # one tie resolved to column 0.
    w = make_weights(MINI)
    if zero_norm:
        w["final_norm"] = np.zeros_like(w["final_norm"])
    drafter, kv, anc, blk, lg, pps = run_case(MINI, ctx, 16, weights=w,
                                              sample=[0, len(ctx) - 1])
    blk2, _ = gpu_draft(drafter, kv, anc, 16, pps, logits=False)
    assert drafter.device_error() == 0
    assert np.array_equal(blk, blk2)
    if zero_norm:
        for b in range(len(ctx)):
            assert list(blk2[b][1:]) == [0] * 15


def test_draft_qwen3_8b_batch1_greedy_without_logits():
    # the headline configuration's LM head (two wave sets, dynamic groups)
    # without a logits output
    s = CONFIGS[2]
    drafter, kv, anc, blk, lg, pps = run_case(s, context_lengths(s), s.block,
                                              weights=_c2_weights())
    blk2, _ = gpu_draft(drafter, kv, anc, s.block, pps, logits=False)
    assert drafter.device_error() == 0
    assert np.array_equal(blk, blk2)


def test_draft_qwen3_8b_batch32_greedy_without_logits():
    # the measured configuration: batch-32 LM head over the full vocabulary
    # (151936 = 593 x 256 + 128: a ragged last tile) without a logits output
    s = CONFIGS[3]
    L = context_lengths(s)
    drafter, kv, anc, blk, lg, pps = run_case(s, L, s.block, sample=[0, s.batch - 1])
    blk2, _ = gpu_draft(drafter, kv, anc, s.block, pps, logits=False)
    assert drafter.device_error() == 0
    assert np.array_equal(blk, blk2)


@pytest.mark.parametrize("ctx", [[37], [5, 0, 129, 64, 17], [40] * 8])
def test_draft_lm_head_ties_take_the_lowest_index(ctx):
    # A zero final-norm gain makes every logit exactly zero, so each row is
    # one tie across the vocabulary; the argmax must resolve it to column 0
    # on every LM-head path (16 rows: the fused skinny head; 80 rows: the
    # tiled product; 128 rows: the large product and its finalize kernel),
    # as the oracle does.
    w = make_weights(MINI)
    w["final_norm"] = np.zeros_like(w["final_norm"])
    _, _, _, blk, lg, _ = run_case(MINI, ctx, 16, weights=w)
    assert np.all(lg == 0.0)
    for b in range(len(ctx)):
        assert list(blk[b][1:]) == [0] * 15
