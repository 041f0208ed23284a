"""One whole speculative cycle on the GPU -- inject the prompt's target
features, draft a block, verify it -- against the oracle's own cycle on the
same seeded inputs.  The verification targets are planted from the oracle's
proposed block, so when the GPU proposes the same block the accepted length
must be the planted one, and the output tokens must be the target's greedy
tokens."""
import numpy as np
import pytest

import oracle
from gpu_util import PagedCache, check_tokens, log, logits_tolerance, make_drafter, to_dev, workspace
from synth import Gen
from synth.configs import CONFIGS, Shape, anchors, hidden_states, planted_tau

pytestmark = pytest.mark.gpu

MINI = Shape("mini-bf16", 512, 2, 4, 2, 128, 768, 1000, 16, 1, True, seed=991)


def oracle_cycle(s, model, prompt_lens, anc, gamma):
    """Oracle inject of every prompt token, then a draft per sequence."""
    out = []
    for b, L in enumerate(prompt_lens):
        hid = hidden_states(s, b, 0, L)
        k, v = model.inject(hid, np.arange(L, dtype=np.int32))         # [L][layer][Hkv][dh]
        dt = np.float32
        ck = np.ascontiguousarray(np.transpose(k, (1, 0, 2, 3)))
        cv = np.ascontiguousarray(np.transpose(v, (1, 0, 2, 3)))
        if s.bf16:   # the values are bf16 already; store their bit patterns
            ck = (ck.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            cv = (cv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        else:
            ck, cv = ck.astype(dt), cv.astype(dt)
        toks = np.full(gamma, s.mask_id, np.int32)
        toks[0] = anc[b]
        out.append(model.draft(ck, cv, L, toks))
    return out


@pytest.mark.parametrize("s,prompt_lens", [(CONFIGS[1], [64]), (MINI, [40, 75]),
                                           (CONFIGS[2], [48])])
def test_cycle_matches_oracle(s, prompt_lens):
    import torch
    from block_diffusion_drafter_fc_amd import verify_greedy
    gamma = s.block
    B = len(prompt_lens)
    log(f"cycle {s.name}: prompts {prompt_lens} block {gamma}")
    drafter, w, _ = make_drafter(s)
    pps = max(prompt_lens) // 16 + 2
    cache = PagedCache(s, B, pps)
    kv = cache.allocate_empty()
    hid = np.concatenate([hidden_states(s, b, 0, L) for b, L in enumerate(prompt_lens)])
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(prompt_lens)]).astype(np.int32)).cuda()
    ws = workspace(drafter, B, gamma, int(sum(prompt_lens)), pps)
    drafter.inject(kv, to_dev(hid, s.bf16), cu, ws)
    anc = anchors(s, B, tag="cycle.anchor")
    a = torch.from_numpy(anc).cuda()
    blk = torch.zeros((B, gamma), dtype=torch.int32, device="cuda")
    lg = torch.zeros((B, gamma, s.vocab), dtype=torch.float32, device="cuda")
    drafter.draft(kv, a, gamma, blk, ws, logits=lg)
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    assert np.array_equal(cache.ctx_dev.cpu().numpy(), prompt_lens)
    model = oracle.Model(s, w)
    cache.fetch()
    for b, L in enumerate(prompt_lens):
        rk, rv = model.inject(hidden_states(s, b, 0, L), np.arange(L, dtype=np.int32))
        gk, gv = cache.read_dense(b, 0, L)
        dk = np.abs(np.transpose(gk, (1, 0, 2, 3)) - rk)
        dv = np.abs(np.transpose(gv, (1, 0, 2, 3)) - rv)
        log(f"  seq {b}: cache max|dK| {dk.max():.3e} max|dV| {dv.max():.3e}, "
            f"fraction of K/V values that differ {np.mean(dk > 0):.3f}/{np.mean(dv > 0):.3f}")
    ref = oracle_cycle(s, model, prompt_lens, anc, gamma)
    gblk = blk.cpu().numpy()
    glg = lg.cpu().numpy()
    same_block = []
    for b in range(B):
        rl, rb = ref[b]
        err = float(np.max(np.abs(glg[b] - rl)))
        log(f"  seq {b}: max|dlogit| {err:.3e}")
        assert err <= logits_tolerance(s, rl)
        check_tokens(gblk[b], rl, 2e-2 if s.bf16 else logits_tolerance(s, rl))
        same_block.append(np.array_equal(gblk[b], rb))
    # verification, targets planted from the oracle's blocks
    tau = planted_tau(s, B, "cycle.tau")
    oblocks = np.stack([r[1] for r in ref])
    tgt = Gen(s.seed).plant_target("cycle.target", oblocks, tau, s.vocab, dtype=s.dtype)
    tt = torch.from_numpy(tgt)
    tt = (tt.view(torch.bfloat16) if s.bf16 else tt).cuda()
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, gamma), dtype=torch.int32, device="cuda")
    verify_greedy(blk, tt, acc, out, ws)
    torch.cuda.synchronize()
    acc = acc.cpu().numpy()
    out = out.cpu().numpy()
    for b in range(B):
        t_o, o_o, T_o = oracle.verify(gblk[b], tgt[b], s.bf16)
        assert acc[b] == t_o and np.array_equal(out[b], o_o)
        assert list(out[b][:acc[b]]) == list(T_o[:acc[b]])
        if same_block[b]:
            assert acc[b] == tau[b]
