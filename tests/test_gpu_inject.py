"""Context injection on the GPU vs the oracle: the keys and values written
into the paged cache (after fusion, RMSNorm, projection and rotary embedding
at the token's absolute position) and the advanced context lengths.

Tolerance: fp32 models 1e-4 of the largest reference value; bf16 models one
bf16 unit in the last place of the reference value plus 2e-3 (both sides round
the stored value to bf16; an input that lands on the other side of a
rounding boundary moves the result by one unit)."""
import numpy as np
import pytest

import oracle
from gpu_util import PagedCache, log, make_drafter, to_dev, workspace
from synth.configs import CONFIGS, Shape, hidden_states
from synth import Gen

pytestmark = pytest.mark.gpu

MINI = Shape("mini-bf16", 512, 2, 4, 2, 128, 768, 1000, 16, 1, True, seed=991)


def check_kv(s, got, ref, what):
    if s.bf16:
        tol = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7) + 2e-3
        bad = np.abs(got - ref) > tol
        err = float(np.max(np.abs(got - ref)))
        assert not np.any(bad), f"{what}: {int(bad.sum())} values off, max |d| {err}"
    else:
        err = float(np.max(np.abs(got - ref)))
        assert err <= 1e-4 * float(np.max(np.abs(ref))), f"{what}: max |d| {err}"
    return err


def run_inject(s, drafter, cache, kv, starts, counts, hidden_rows):
    """One inject call: sequence b gets counts[b] new tokens at positions
    starts[b]..; hidden_rows is the concatenated [n_tok][m*D] input."""
    import torch
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n_tok = int(cu[-1])
    ws = workspace(drafter, len(counts), 1, max(n_tok, 1), cache.pages_per_seq)
    cache.ctx_dev.copy_(torch.from_numpy(np.asarray(starts, np.int32)))
    drafter.inject(kv, to_dev(hidden_rows, s.bf16), torch.from_numpy(cu).cuda(), ws)
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    got_lens = cache.ctx_dev.cpu().numpy()
    assert np.array_equal(got_lens, np.asarray(starts) + np.asarray(counts))
    return cu


def inject_case(s, starts, counts, sample_tokens=None, pages_per_seq=None):
    log(f"inject {s.name}: starts {list(starts)[:6]} counts {list(counts)[:6]}")
    drafter, w, _ = make_drafter(s)
    B = len(starts)
    pps = pages_per_seq or (int(max(np.asarray(starts) + np.asarray(counts))) + 15) // 16 + 1
    cache = PagedCache(s, B, pps)
    kv = cache.allocate_empty()
    rows = [hidden_states(s, b, int(starts[b]), int(counts[b])) for b in range(B)]
    hid = np.ascontiguousarray(np.concatenate(rows, axis=0))
    run_inject(s, drafter, cache, kv, starts, counts, hid)
    cache.fetch()
    model = oracle.Model(s, w)
    worst = 0.0
    for b in range(B):
        n = int(counts[b])
        if n == 0:
            continue
        idx = np.arange(n) if sample_tokens is None else np.unique(
            np.clip(np.asarray(sample_tokens), 0, n - 1))
        pos = (int(starts[b]) + idx).astype(np.int32)
        rk, rv = model.inject(np.ascontiguousarray(rows[b][idx]), pos)   # [t][layer][Hkv][dh]
        for t, i in enumerate(idx):
            gk, gv = cache.read_dense(b, int(starts[b] + i), 1)         # [layer][1][Hkv][dh]
            worst = max(worst, check_kv(s, gk[:, 0], rk[t], f"K seq {b} tok {i}"),
                        check_kv(s, gv[:, 0], rv[t], f"V seq {b} tok {i}"))
    log(f"  worst |dK|,|dV| = {worst:.3e}")
    return drafter, cache


def test_inject_tiny_fp32_workload_prefill():
    s = CONFIGS[1]
    inject_case(s, [0], [64])


def test_inject_mini_bf16_ragged_batch_and_zero_counts():
    inject_case(MINI, [3, 10, 0, 40], [5, 0, 17, 1])


def test_inject_mini_bf16_many_tokens_uses_tiled_product():
    inject_case(MINI, [0, 16], [70, 33])


def test_inject_qwen3_8b_prefill_sampled():
    s = CONFIGS[2]
    inject_case(s, [0], [2048], sample_tokens=[0, 1, 777, 1024, 2047])


def test_inject_qwen3_8b_batch32_step():
    s = CONFIGS[3]
    g = Gen(s.seed)
    starts = g.uniform_int("ctx_len", s.batch, 1024, 4096)
    counts = g.uniform_int("inject.step0", s.batch, 1, 16)
    inject_case(s, starts, counts, sample_tokens=list(range(16)), pages_per_seq=(4096 + 16) // 16 + 1)


def test_inject_long_context_chunk_high_positions():
    s = CONFIGS[4].replace(batch=1)
    inject_case(s, [28672], [4096], sample_tokens=[0, 100, 4095], pages_per_seq=32768 // 16 + 1)


def test_inject_wide_step_sampled():
    s = CONFIGS[5]
    g = Gen(s.seed)
    starts = g.uniform_int("ctx_len", s.batch, 2048, 8192)
    counts = g.uniform_int("inject.step0", s.batch, 1, 16)
    inject_case(s, starts, counts, sample_tokens=[0, 15], pages_per_seq=(8192 + 16) // 16 + 1)


def test_inject_reports_positions_beyond_the_page_table():
    import torch
    s = MINI
    drafter, _, _ = make_drafter(s)
    cache = PagedCache(s, 1, 2)             # room for 32 positions
    kv = cache.allocate_empty()
    hid = hidden_states(s, 0, 30, 4)
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    cache.ctx_dev.fill_(30)
    ws = workspace(drafter, 1, 1, 4, 2)
    drafter.inject(kv, to_dev(hid, True), cu, ws)
    assert drafter.device_error() & 2
