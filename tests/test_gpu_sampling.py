"""Sampled drafting and lossless (stochastic) verification on the GPU vs the
oracle (oracle/sampling.py).

Sampled draft: the logits must agree with the oracle's as in the greedy
draft tests, and every proposal must be the oracle's Gumbel-max draw (the
oracle's logits plus the oracle's noise) unless that draw's top-2 gap is
below the logits tolerance plus 1e-4 (the kernel evaluates the noise in
fp32).

Stochastic verification: both sides take every decision in fp64 from the
same fp32/bf16 inputs, so accepted lengths and output tokens must match
exactly; a mismatch is tolerated only where the oracle's own decision
margin (relative) is below 1e-10, i.e. where summation order alone can flip
it.  Inputs: seeded drafter logits N(0, 2), target rows equal to the next
drafter row plus N(0, 1) (so acceptance is frequent but not certain),
proposals that are the drafter's argmax for most positions, uniforms from
the seeded generator."""
import numpy as np
import pytest

import oracle
from oracle import sampling as S
from gpu_util import check_tokens, log, logits_tolerance, make_drafter, to_dev, workspace
from synth import Gen
from synth.configs import CONFIGS, anchors, context_lengths, make_weights
from test_gpu_draft import MINI, _c2_weights, pages_for, setup_cache

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ verification
def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (input construction)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + r) >> np.uint64(16)).astype(np.uint16)


def make_inputs(seed, B, gamma, V, bf16, p_argmax=0.75):
    g = Gen(seed)
    draft = g.normal("sv.draft", (B, gamma, V), std=2.0)
    noise = g.normal("sv.noise", (B, gamma, V), std=1.0)
    target = np.empty_like(draft)
    target[:, :-1] = draft[:, 1:] + noise[:, :-1]
    target[:, -1] = noise[:, -1] * 2.0
    pick = g.uniform("sv.pick", B * gamma).reshape(B, gamma) < p_argmax
    rnd = g.uniform_int("sv.tok", B * gamma, 0, V - 1).reshape(B, gamma)
    blocks = np.where(pick, np.argmax(draft, axis=-1), rnd).astype(np.int32)
    blocks[:, 0] = g.uniform_int("sv.anchor", B, 0, V - 1)
    u = g.uniform("sv.u", B * gamma).reshape(B, gamma).astype(np.float32)
    tgt = round_bf16(target) if bf16 else target
    return blocks, draft, tgt, u


def run_stochastic(blocks, draft, target, uniforms, bf16):
    import torch
    from block_diffusion_drafter_fc_amd import verify_stochastic, verify_stochastic_workspace_bytes
    B, gamma = blocks.shape
    V = draft.shape[-1]
    ws = torch.empty(verify_stochastic_workspace_bytes(B, gamma, V), dtype=torch.uint8,
                     device="cuda")
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, gamma), -7, dtype=torch.int32, device="cuda")
    verify_stochastic(torch.from_numpy(np.ascontiguousarray(blocks)).cuda(),
                      to_dev(np.ascontiguousarray(draft, dtype=np.float32), False),
                      to_dev(target, bf16),
                      torch.from_numpy(np.ascontiguousarray(uniforms)).cuda(), acc, out, ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def host64(target, bf16):
    if bf16:
        return (target.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return target.astype(np.float64)


def decision_margin(block, draft, target, u):
    """Smallest relative margin of the oracle's decisions on this block: each
    accept/reject comparison and the final draw's threshold."""
    pd, pt = S.softmax(draft), S.softmax(target)
    gamma = len(block)
    m = np.inf
    for k in range(1, gamma):
        x = int(block[k])
        p, q = pt[k - 1][x], pd[k][x]
        lhs = float(u[k]) * q
        m = min(m, abs(lhs - p) / max(p, lhs, 1e-300))
        if not lhs < p:
            r = np.maximum(pt[k - 1] - pd[k], 0.0)
            break
    else:
        r = pt[gamma - 1]
    if r.sum() <= 0.0:
        r = pt[k - 1]
    c = np.cumsum(r)
    T = float(u[0]) * c[-1]
    v = int(np.searchsorted(c, T, side="right"))
    lo = T - (c[v - 1] if v > 0 else 0.0)
    hi = c[min(v, len(c) - 1)] - T
    return min(m, lo / c[-1], hi / c[-1])


def compare_stochastic(blocks, draft, target, u, bf16, max_tolerated=1):
    acc, out = run_stochastic(blocks, draft, target, u, bf16)
    t64 = host64(target, bf16)
    d64 = draft.astype(np.float64)
    u64 = u.astype(np.float64)
    tolerated = 0
    taus = []
    for b in range(blocks.shape[0]):
        tau, o, _ = S.verify_stochastic(blocks[b], d64[b], t64[b], u64[b])
        taus.append(tau)
        if acc[b] == tau and np.array_equal(out[b], o):
            continue
        m = decision_margin(blocks[b], d64[b], t64[b], u64[b])
        log(f"  seq {b}: gpu tau {acc[b]} {out[b].tolist()} vs oracle {tau} {o.tolist()}, "
            f"margin {m:.3e}")
        assert m < 1e-10, f"seq {b}: gpu tau {acc[b]} {out[b]} vs oracle {tau} {o}, margin {m:.3e}"
        tolerated += 1
    assert tolerated <= max_tolerated
    return np.array(taus), acc, out


@pytest.mark.parametrize("B,gamma,V,bf16", [
    (4, 16, 1000, False),        # several chunks of units, fp32 scores
    (3, 5, 4097, True),          # one column past a 4096-column chunk
    (2, 1, 777, True),           # block of one: bonus token only
    (5, 7, 8, False),            # vocabulary smaller than one unit
    (2, 64, 300, False),         # the largest block
    (1, 16, 151936, True),       # Qwen3-8B vocabulary, batch 1
    (8, 16, 151936, True),       # wide workload's batch
    (32, 16, 151936, True),      # batch-32 workload
])
def test_stochastic_verify_matches_oracle(B, gamma, V, bf16):
    log(f"stochastic verify: batch {B} block {gamma} vocab {V} {'bf16' if bf16 else 'f32'}")
    blocks, draft, target, u = make_inputs(1000 + B * 131 + gamma * 7 + V, B, gamma, V, bf16)
    taus, _, _ = compare_stochastic(blocks, draft, target, u, bf16)
    log(f"  accepted lengths {np.bincount(taus, minlength=gamma + 1)[1:].tolist()}")
    if gamma > 1 and B >= 4:
        assert len(set(taus.tolist())) > 1      # the inputs reach more than one outcome


@pytest.mark.parametrize("bf16", [False, True])
def test_stochastic_verify_decisions_near_the_boundary(bf16):
    # uniforms planted a relative 1e-6 below or above p_t / p_d of one
    # proposal per sequence: inside the margin where fp32 normalisers could
    # decide wrongly, far outside fp64 rounding, so the outcome is fixed
    B, gamma, V = 12, 8, 5000
    blocks, draft, target, u = make_inputs(4321 + bf16, B, gamma, V, bf16)
    pd = S.softmax(draft.astype(np.float64))
    pt = S.softmax(host64(target, bf16))
    planted = 0
    for b in range(B):
        for k in range(1, gamma):
            x = blocks[b, k]
            ratio = pt[b, k - 1, x] / pd[b, k, x]
            if ratio < 0.9:
                side = 1.0 - 1e-6 if b % 2 == 0 else 1.0 + 1e-6
                u[b, 1:k] = 0.0                      # keep the proposals before it
                u[b, k] = np.float32(ratio * side)
                planted += 1
                break
    assert planted >= 8
    taus, acc, out = compare_stochastic(blocks, draft, target, u, bf16, max_tolerated=0)
    log(f"  near-boundary accepted lengths {acc.tolist()}")


def test_stochastic_verify_out_of_range_proposals_are_rejected():
    B, gamma, V = 4, 6, 500
    blocks, draft, target, u = make_inputs(77, B, gamma, V, False, p_argmax=1.0)
    u[:] = 0.0                               # every in-range proposal with p_t > 0 is kept
    bad_k = [1, 3, 5, 2]
    for b, k in enumerate(bad_k):
        blocks[b, k] = -1 if b % 2 else V
    acc, out = run_stochastic(blocks, draft, target, u, False)
    pd, pt = S.softmax(draft.astype(np.float64)), S.softmax(target.astype(np.float64))
    for b, k in enumerate(bad_k):
        assert acc[b] == k
        assert np.array_equal(out[b, :k - 1], blocks[b, 1:k])
        r = np.maximum(pt[b, k - 1] - pd[b, k], 0.0)
        assert out[b, k - 1] == S.draw(r, 0.0)
        assert np.all(out[b, k:] == -1)


def test_stochastic_verify_empty_residual_draws_from_the_target():
    # drafter row k equal to target row k - 1 and a proposal of probability
    # zero under both: rejected, and the correction comes from p_t
    B, gamma, V = 3, 4, 300
    g = Gen(31)
    target = g.normal("er.t", (B, gamma, V), std=1.5)
    draft = np.concatenate([target[:, :1], target[:, :-1]], axis=1).copy()
    blocks = np.argmax(draft, axis=-1).astype(np.int32)
    blocks[:, 2] = 17
    target[:, 1, 17] = -3000.0
    draft[:, 2, 17] = -3000.0
    u = np.array([[0.1, 0.5, 0.5, 0.5], [0.6, 0.5, 0.5, 0.5], [0.99, 0.5, 0.5, 0.5]],
                 dtype=np.float32)
    taus, acc, out = compare_stochastic(blocks, draft, target, u, False, max_tolerated=0)
    assert np.all(acc == 2)
    pt = S.softmax(target.astype(np.float64))
    for b in range(B):
        assert out[b, 1] == S.draw(pt[b, 1], float(u[b, 0]))


def test_stochastic_verify_first_token_follows_the_target():
    # Losslessness on the GPU: over many sequences with the same logits and
    # fresh proposals and uniforms, the first emitted token is distributed
    # as the target's row 0, whatever the drafter proposed.
    from scipy import stats
    B, gamma, V = 8192, 3, 6
    g = Gen(2024)
    d1 = g.normal("ft.d", (gamma, V), std=1.5).astype(np.float64)
    t1 = g.normal("ft.t", (gamma, V), std=1.5).astype(np.float64)
    draft = np.broadcast_to(d1.astype(np.float32), (B, gamma, V)).copy()
    target = np.broadcast_to(t1.astype(np.float32), (B, gamma, V)).copy()
    # proposals drawn from the drafter's rows by inverse CDF of seeded uniforms
    e = np.exp(d1 - d1.max(axis=-1, keepdims=True))
    cdf = np.cumsum(e / e.sum(axis=-1, keepdims=True), axis=-1)
    w = g.uniform("ft.w", B * gamma).reshape(B, gamma)
    blocks = np.stack([np.minimum(np.searchsorted(cdf[k], w[:, k], side="right"), V - 1)
                       for k in range(gamma)], axis=1).astype(np.int32)
    blocks[:, 0] = 0
    u = g.uniform("ft.u", B * gamma).reshape(B, gamma).astype(np.float32)
    acc, out = run_stochastic(blocks, draft, target, u, False)
    counts = np.bincount(out[:, 0], minlength=V)
    expected = B * S.softmax(t1[0])
    p = stats.chisquare(counts, expected).pvalue
    log(f"  first tokens {counts.tolist()} expected {np.round(expected).tolist()} p={p:.3g}")
    assert p > 1e-4
    assert stats.chisquare(counts, B * S.softmax(d1[1])).pvalue < 1e-6


# ----------------------------------------------------------- sampled draft
SEED = 0xC0FFEE1234567897


def sampled_case(s, ctx_lens, gamma, seed=SEED, weights=None, sample=None):
    import torch
    log(f"sampled draft {s.name}: batch {len(ctx_lens)} block {gamma} seed {seed:#x}")
    w = weights if weights is not None else make_weights(s)
    drafter, w, _ = make_drafter(s, w)
    pps = pages_for(max(ctx_lens))
    cache, kv, dense = setup_cache(s, ctx_lens, pps)
    B = len(ctx_lens)
    anc = anchors(s, B, tag=f"sampled.anchor.{gamma}")
    ws = workspace(drafter, B, gamma, 1, pps)
    a = torch.from_numpy(np.asarray(anc, np.int32)).cuda()
    blk = torch.full((B, gamma), -5, dtype=torch.int32, device="cuda")
    lg = torch.full((B, gamma, s.vocab), float("nan"), device="cuda")
    drafter.draft_sampled(kv, a, gamma, seed, blk, lg, ws)
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    blk, lg = blk.cpu().numpy(), lg.cpu().numpy()
    model = oracle.Model(s, w)
    for b in (range(B) if sample is None else sample):
        k, v = dense[b]
        toks = np.full(gamma, s.mask_id, np.int32)
        toks[0] = anc[b]
        ref, _ = model.draft(k, v, int(ctx_lens[b]), toks)
        tol = logits_tolerance(s, ref)
        err = float(np.max(np.abs(lg[b].astype(np.float64) - ref)))
        assert np.all(np.isfinite(lg[b])) and err <= tol, (b, err, tol)
        assert blk[b, 0] == anc[b]
        noisy = ref.copy()
        for j in range(1, gamma):
            noisy[j] += S.gumbel(seed, b, j, s.vocab)
        ref_block = S.sample_block(ref, anc[b], seed, b)
        assert np.array_equal(np.argmax(noisy[1:], axis=-1), ref_block[1:])
        n_tol = check_tokens(blk[b], noisy, (2e-2 if s.bf16 else tol) + 1e-4)
        log(f"  seq {b}: max|dlogit| {err:.2e}, proposals {blk[b, 1:6].tolist()}..., "
            f"near-tie rows {n_tol}")
    return drafter, kv, a, ws, blk, lg


def test_sampled_draft_tiny_fp32_workload():
    s = CONFIGS[1]
    sampled_case(s, context_lengths(s), s.block)


def test_sampled_draft_mini_bf16():
    sampled_case(MINI, [0, 5, 40, 133], 16)


def test_sampled_draft_qwen3_8b_batch1_workload():
    s = CONFIGS[2]
    sampled_case(s, context_lengths(s), s.block, weights=_c2_weights())


def test_sampled_draft_qwen3_8b_batch32_workload_sampled():
    s = CONFIGS[3]
    L = context_lengths(s)
    sampled_case(s, L, s.block, sample=[0, int(np.argmax(L)), 31])


def test_sampled_draft_seed_and_logits():
    # the draw leaves the logits untouched; the same seed repeats the block,
    # another seed changes it, and the greedy call still takes the argmax
    import torch
    s = MINI
    ctx = [3, 60]
    drafter, kv, a, ws, blk, lg = sampled_case(s, ctx, 8)
    blk2 = torch.empty((2, 8), dtype=torch.int32, device="cuda")
    lg2 = torch.empty((2, 8, s.vocab), device="cuda")
    drafter.draft_sampled(kv, a, 8, SEED, blk2, lg2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(blk2.cpu().numpy(), blk)
    assert np.array_equal(lg2.cpu().numpy(), lg)
    drafter.draft_sampled(kv, a, 8, SEED ^ 1, blk2, lg2, ws)
    torch.cuda.synchronize()
    assert not np.array_equal(blk2.cpu().numpy(), blk)
    drafter.draft(kv, a, 8, blk2, ws, logits=lg2)
    torch.cuda.synchronize()
    assert np.array_equal(lg2.cpu().numpy(), lg)
    greedy = blk2.cpu().numpy()
    assert np.array_equal(greedy[:, 1:], np.argmax(lg[:, 1:], axis=-1))
    assert not np.array_equal(greedy, blk)
