"""Greedy verification on the GPU vs the oracle: bit-exact accepted lengths,
output tokens and target argmax tokens, on all five workloads and on edge
cases (block of one, ties, ties between -0.0 and +0.0, vocab sizes off the
vector width, fp32 scores)."""
import numpy as np
import pytest

import oracle
from gpu_util import log
from synth import Gen
from synth.configs import CONFIGS, planted_tau

pytestmark = pytest.mark.gpu


def run_verify(blocks, target, bf16):
    import torch
    from block_diffusion_drafter_fc_amd import verify_greedy, verify_greedy_workspace_bytes
    B, g = blocks.shape
    bt = torch.from_numpy(np.ascontiguousarray(blocks, dtype=np.int32)).cuda()
    tt = torch.from_numpy(np.ascontiguousarray(target))
    tt = (tt.view(torch.bfloat16) if bf16 else tt).cuda()
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, g), -7, dtype=torch.int32, device="cuda")
    ta = torch.full((B, g), -7, dtype=torch.int32, device="cuda")
    # the exact size the call asks for, filled with junk: nothing in it may
    # need clearing
    ws = torch.full((verify_greedy_workspace_bytes(B, g, target.shape[-1]),), 0xA5,
                    dtype=torch.uint8, device="cuda")
    verify_greedy(bt, tt, acc, out, ws, target_argmax=ta)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), ta.cpu().numpy()


def compare(blocks, target, bf16, tau_expect=None):
    acc, out, ta = run_verify(blocks, target, bf16)
    for b in range(blocks.shape[0]):
        tau, o, T = oracle.verify(blocks[b], target[b], bf16)
        assert acc[b] == tau, (b, acc[b], tau)
        assert np.array_equal(out[b], o), b
        assert np.array_equal(ta[b], T), b
        if tau_expect is not None:
            assert tau == tau_expect[b]
    return acc


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_verify_matches_oracle_on_workload(k):
    s = CONFIGS[k]
    log(f"verify workload {s.name}: batch {s.batch} block {s.block} vocab {s.vocab}")
    g = Gen(s.seed)
    blocks = g.uniform_int("verify.block", s.batch * s.block, 0, s.vocab - 1)
    blocks = blocks.reshape(s.batch, s.block).astype(np.int32)
    tau = planted_tau(s, s.batch, "verify.tau")
    tgt = g.plant_target("verify.target", blocks, tau, s.vocab, dtype=s.dtype)
    compare(blocks, tgt, s.bf16, tau)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("V", [8, 1000, 1001, 20003])
def test_verify_edge_vocab_sizes_and_all_lengths(bf16, V):
    gamma = 16
    g = Gen(5 + V)
    blocks = g.uniform_int("b", gamma * gamma, 0, V - 1).reshape(gamma, gamma).astype(np.int32)
    tau = np.arange(1, gamma + 1)
    tgt = g.plant_target("t", blocks, tau, V, dtype="bf16" if bf16 else "f32")
    compare(blocks, tgt, bf16, tau)


def test_verify_block_of_one_and_ties():
    V = 4096
    tgt = np.zeros((3, 1, V), np.float32)        # all-equal rows: argmax is index 0
    tgt[1, 0, [17, 4000]] = 2.0                  # tie between 17 and 4000
    tgt[2, 0, V - 1] = 1.0
    blocks = np.array([[5], [6], [7]], np.int32)
    acc = compare(blocks, tgt, False)
    assert list(acc) == [1, 1, 1]
    _, out, _ = run_verify(blocks, tgt, False)
    assert list(out[:, 0]) == [0, 17, V - 1]


def test_verify_large_batch_bf16():
    V, gamma, B = 3000, 16, 96
    g = Gen(77)
    blocks = g.uniform_int("b", B * gamma, 0, V - 1).reshape(B, gamma).astype(np.int32)
    tau = g.uniform_int("tau", B, 1, gamma)
    tgt = g.plant_target("t", blocks, tau, V, dtype="bf16")
    compare(blocks, tgt, True, tau)


@pytest.mark.parametrize("bf16,V", [(True, 20000), (True, 20003), (False, 20004), (False, 20003)])
def test_verify_signed_zero_ties_take_the_lower_index(bf16, V):
    # -0.0 and +0.0 are equal scores, so the lower index wins whichever sign
    # it carries: within one 16-byte load, within one argmax chunk (8192
    # columns), and across chunks; on the vector and the scalar load paths.
    # The rest of each row is -1.
    gamma = 6
    neg, pos, minus_one = (0x8000, 0x0000, 0xBF80) if bf16 else (-0.0, 0.0, -1.0)
    dt = np.uint16 if bf16 else np.float32
    pairs = [(100, 200, neg, pos), (5, 6, pos, neg), (30, 19000, pos, neg),
             (7, 15000, neg, pos), (2, 3, neg, pos), (16390, 16391, neg, pos)]
    tgt = np.full((2, gamma, V), minus_one, dt)
    for j, (lo, hi, a, b) in enumerate(pairs):
        tgt[:, j, lo], tgt[:, j, hi] = a, b
    T = [lo for lo, _, _, _ in pairs]
    blocks = np.array([[9] + T[:5], [9] + T[:2] + [11, 12, 13]], np.int32)
    acc = compare(blocks, tgt, bf16)
    assert list(acc) == [6, 3]
    _, out, ta = run_verify(blocks, tgt, bf16)
    assert list(ta[0]) == T and list(out[0]) == T
    assert list(out[1]) == T[:3] + [-1, -1, -1]
