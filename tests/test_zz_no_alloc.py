"""dflash_draft_block_noalloc (the draft with the library's static per-GPU
scratch, for callers that cannot allocate) against dflash_draft_block with a
caller workspace: same inputs, bit-identical block tokens and logits, on two
calls in a row with the second one smaller; and the capacity error for a
call whose scratch need exceeds the array."""
import numpy as np
import pytest

from gpu_util import PagedCache, log, make_drafter, workspace
from synth.configs import CONFIGS, Shape, anchors, context_kv, make_weights

pytestmark = pytest.mark.gpu

MINI = Shape("mini-bf16", 512, 2, 4, 2, 128, 768, 1000, 16, 1, True, seed=991)
MINI_F32 = Shape("mini-f32", 256, 2, 4, 2, 64, 768, 1001, 5, 1, False, seed=992)


def _cache(s, ctx, pps, tag):
    cache = PagedCache(s, len(ctx), pps, tag=tag)
    for b, L in enumerate(ctx):
        k, v = context_kv(s, b, int(L))
        cache.write_dense(b, k, v)
    return cache.upload(ctx)


def _both(drafter, s, ctx, gamma, tag):
    import torch
    pps = (max(ctx) + 15) // 16 + 2
    kv = _cache(s, ctx, pps, tag)
    B = len(ctx)
    anc = torch.from_numpy(anchors(s, B, tag=f"noalloc.{tag}")).cuda()
    V = drafter.cfg.vocab
    blk_a = torch.full((B, gamma), -5, dtype=torch.int32, device="cuda")
    lg_a = torch.full((B, gamma, V), float("nan"), device="cuda")
    drafter.draft(kv, anc, gamma, blk_a, workspace(drafter, B, gamma, 1, pps), logits=lg_a)
    blk_b = torch.full((B, gamma), -7, dtype=torch.int32, device="cuda")
    lg_b = torch.full((B, gamma, V), float("nan"), device="cuda")
    drafter.draft_noalloc(kv, anc, gamma, blk_b, logits=lg_b)
    blk_c = torch.full((B, gamma), -9, dtype=torch.int32, device="cuda")
    drafter.draft_noalloc(kv, anc, gamma, blk_c)            # without logits
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    a, b = lg_a.cpu().numpy(), lg_b.cpu().numpy()
    log(f"noalloc {s.name} batch {B} block {gamma}: max|dlogit| "
        f"{float(np.max(np.abs(a - b))):.3e}")
    assert np.all(np.isfinite(b))
    assert np.array_equal(a, b)
    assert np.array_equal(blk_a.cpu().numpy(), blk_b.cpu().numpy())
    assert np.array_equal(blk_a.cpu().numpy(), blk_c.cpu().numpy())


@pytest.mark.parametrize("s", [MINI, MINI_F32], ids=["bf16", "f32"])
def test_noalloc_draft_equals_workspace_draft_twice_second_smaller(s):
    drafter, _, _ = make_drafter(s, make_weights(s))
    _both(drafter, s, [33, 250, 7], min(16, s.block if not s.bf16 else 16), "first")
    _both(drafter, s, [37], 3, "second")                    # fewer rows, shorter block
    drafter.close()


def test_noalloc_draft_qwen3_8b_batch1_shape():
    s = CONFIGS[2]
    drafter, _, _ = make_drafter(s, make_weights(s))
    _both(drafter, s, [2048, 1500], 16, "q8-first")         # 32 rows: two row tiles
    _both(drafter, s, [2048], 10, "q8-second")
    drafter.close()


def test_noalloc_draft_rejects_a_call_beyond_the_scratch():
    import torch
    from block_diffusion_drafter_fc_amd import DFlashError
    s = MINI
    drafter, _, _ = make_drafter(s, make_weights(s))
    from block_diffusion_drafter_fc_amd import KVCache
    # a page table of 64 x 4096 pages: ~130 MB of attention partials alone.
    # The call is refused on the host, so a one-page pool is enough.
    B, pps = 64, 4096
    pages = torch.zeros((s.n_layers, 1, 2, s.n_kv_heads, 16, s.head_dim), dtype=torch.bfloat16,
                        device="cuda")
    kv = KVCache(pages, torch.zeros((B, pps), dtype=torch.int32, device="cuda"),
                 torch.zeros(B, dtype=torch.int32, device="cuda"))
    assert drafter.workspace_bytes(B, 16, 1, pps) > (48 << 20)
    anc = torch.zeros(B, dtype=torch.int32, device="cuda")
    blk = torch.zeros((B, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(DFlashError) as e:
        drafter.draft_noalloc(kv, anc, 16, blk)
    assert e.value.status == -4 and "scratch" in str(e.value)
    # nothing was launched: a fitting call still works
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    drafter.close()
