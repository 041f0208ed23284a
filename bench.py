#!/usr/bin/env python3
"""Throughput of the DFlash draft hot path on one MI355X.

One step is one speculative cycle of the hot path for every sequence of the
batch: inject the target features of the tokens accepted in the previous
cycle (context fusion, per-layer K/V projection, rotary embedding, paged
store), draft a block of 16 (anchor + 15 masks, one forward pass, LM-head
argmax), and verify it greedily against planted target scores.  All inputs
of all steps are resident in HBM before the timed region starts.

The printed JSON line reports draft blocks/s (value) and draft tokens/s for
the whole step, the LM-head kernel's achieved HBM bandwidth against the
MI355X peak (timed live with HIP events on the launch stream), the whole
step's algorithmic bytes as a fraction of the HBM roofline, and the CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload qwen3-8b-bs1|qwen3-8b-bs32|qwen3-8b-long|wide-8layer|tiny-fp32]
                       [--block-sweep 4,8,10,16]

HBM traffic of the LM-head kernel (the "traffic" field) comes from rocprofv3
counter runs summarised into profiles/lm_head_traffic_<workload>.json:
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d D1 -o c -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-bs32 --replays 3
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d D2 -o c -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-bs32 --replays 3
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d D3 -o c -- python3 bench.py --read-calibration
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d D4 -o c -- python3 bench.py --copy-calibration
  python3 bench.py --counter-summary D1 D2 D3 D4
A pure read of known size with the LM head's own load pattern (16-byte
non-temporal loads, one contiguous run per workgroup) calibrates FETCH_SIZE,
a device copy of known size WRITE_SIZE (bytes per counted KiB); the record
carries a hash of the kernel sources and is ignored once they change.

Matrix-core use of the batch-32 draft (profiles/mfma_util_qwen3-8b-bs32.md):
  rocprofv3 --kernel-trace --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d D5 -o c -- python3 bench.py --workload qwen3-8b-bs32 --steps 2 --warmup 1 --no-cpu-baseline --replays 2
  python3 bench.py --mfma-summary D5
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft blocks/s & draft tokens/s (block 16, Qwen3-8B-shaped, bs 1/32); %HBM peak"
# LM head at M <= 16 rows: packed, norm-staged, argmax, 16-block batches, column
# groups taken dynamically
LM_KERNEL = {"bf16-skinny": "k_skinny<1, 2, 1, true, 16, true, 2>"}
COPY_BYTES = 1 << 30                               # calibration copy size
KERNEL_SOURCES = ("block_diffusion_drafter_fc_amd/csrc/skinny.hip",
                  "block_diffusion_drafter_fc_amd/csrc/common.h",
                  "block_diffusion_drafter_fc_amd/csrc/kernels.h",
                  "block_diffusion_drafter_fc_amd/csrc/calibrate.hip")
READ_CAL_WORKGROUPS = 512   # the LM head's workgroup count
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, vendor peak
BF16_MFMA_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------- bytes model
def fc_memory(hidden: int, n_tokens: int, n_feats: int = 5, elem: int = 2):
    """Context projection memory (paper §7.3): W_c [D][m*D], the projection's
    input [n][m*D] and output [n][D], in bytes."""
    return (hidden * n_feats * hidden * elem, n_tokens * n_feats * hidden * elem,
            n_tokens * hidden * elem)


def algorithmic_bytes(s, ctx_lens_at_draft, n_new_total: int, batch: int, gamma: int) -> dict:
    """Bytes the hot path must move once per step: every weight once, every
    cached context K/V read once, the new K/V written once, the inputs read
    and outputs written once.  Transient activations are small and counted
    at 4 bytes per element where they cross kernels of the LM head."""
    e = 2 if s.bf16 else 4
    D, NL, V, I = s.hidden, s.n_layers, s.vocab, s.inter
    QD, KVD = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    M = batch * gamma
    layer_w = ((QD + 2 * KVD) * D + D * QD + 2 * I * D + D * I) * e
    lm_w = V * D * e
    kv_read = int(np.sum(ctx_lens_at_draft)) * NL * 2 * KVD * e
    lm_head = lm_w + M * D * 4 + M * 8
    draft = NL * (layer_w + 2 * s.hidden * e) + lm_head + kv_read + M * D * e + M * 4
    w_fc, in_fc, _ = fc_memory(D, n_new_total, s.n_feats, e)
    inject = w_fc + NL * 2 * KVD * D * e + in_fc + n_new_total * NL * 2 * KVD * e
    verify = M * V * e + M * 4 * 3
    return {"draft": draft, "inject": inject, "verify": verify, "lm_head": lm_head,
            "step": draft + inject + verify, "kv_read": kv_read}


def draft_phase_roofline(s, ctx_lens, batch, gamma) -> float:
    """Per-phase roofline time (s) of one draft step: the sum over its phases
    (each layer's QKV, attention, O, gate/up and down products, then the LM
    head) of max(bytes / HBM peak, flops / bf16 MFMA peak).  Bytes of a
    product: its weights once, fp32 activations in and out; of attention:
    the layer's cached K/V once."""
    e = 2 if s.bf16 else 4
    D, NL, V, I = s.hidden, s.n_layers, s.vocab, s.inter
    QD, KVD = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    M = batch * gamma
    hbm, mfma = HBM_PEAK_GBS * 1e9, BF16_MFMA_PEAK_TFLOPS * 1e12

    def product(N, K):
        return max((N * K * e + M * (N + K) * 4) / hbm, 2.0 * M * N * K / mfma)

    L = np.asarray(ctx_lens, dtype=np.float64)
    attn_bytes = float(L.sum()) * 2 * KVD * e
    attn_flops = 4.0 * float(np.sum(L + gamma)) * gamma * s.n_q_heads * s.head_dim
    layer = (product(QD + 2 * KVD, D) + max(attn_bytes / hbm, attn_flops / mfma) +
             product(D, QD) + product(2 * I, D) + product(D, I))
    return NL * layer + product(V, D)


def draft_flops(s, ctx_lens, batch, gamma):
    D, NL, V, I = s.hidden, s.n_layers, s.vocab, s.inter
    QD, KVD = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    M = batch * gamma
    gemm = 2 * M * (NL * ((QD + 2 * KVD) * D + D * QD + 3 * I * D) + V * D)
    attn = 4 * int(np.sum(np.asarray(ctx_lens) + gamma)) * gamma * s.n_q_heads * s.head_dim * NL
    return gemm + attn


# ------------------------------------------------------------------ workload
class Workload:
    """Seeded inputs of every step, resident on the device."""

    def __init__(self, s, n_steps: int):
        import torch
        from synth import Gen
        from synth.configs import context_lengths, planted_tau, anchors
        self.s = s
        self.B, self.gamma = s.batch, s.block
        g = Gen(s.seed)
        self.L0 = context_lengths(s).astype(np.int64)
        B, S = self.B, n_steps
        self.S = S
        self.tau = np.stack([planted_tau(s, B, f"bench.tau.{k}") for k in range(S)])
        if s.name == "qwen3-8b-bs32":      # 1..16 newly accepted tokens per step
            self.n_new = np.stack([g.uniform_int(f"bench.new.{k}", B, 1, 16) for k in range(S)])
        else:                               # the previous cycle's accepted length
            first = planted_tau(s, B, "bench.tau.first")
            self.n_new = np.concatenate([first[None], self.tau[:-1]], axis=0)
        self.anchor = np.stack([anchors(s, B, tag=f"bench.anchor.{k}") for k in range(S)])
        self.L_at = np.zeros((S, B), np.int64)      # context length seen by each draft
        L = self.L0.copy()
        for k in range(S):
            L = L + self.n_new[k]
            self.L_at[k] = L
        self.Lmax = int(self.L_at[-1].max())
        self.dev = torch.device("cuda")

    def step_hidden(self, k):
        from synth.configs import hidden_states
        rows = []
        start = self.L_at[k] - self.n_new[k]
        for b in range(self.B):
            rows.append(hidden_states(self.s, b, int(start[b]), int(self.n_new[k][b])))
        return np.ascontiguousarray(np.concatenate(rows, axis=0))


def to_dev(a, bf16):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def percentiles(ms) -> dict:
    """Median and 10th/90th percentiles of per-call times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"n": int(a.size), "median_ms": round(float(np.median(a)), 4),
            "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4)}


def event_times(fn, n):
    """Device time (ms) of each of n calls fn(i), from a HIP event pair
    recorded around each call on the current stream (where the binding
    launches)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def run_gpu(s, steps, warmup, sampled=False, replays=50):
    """Time `steps` whole steps.  sampled: the draft draws its proposals
    (fresh seed per step, logits written) and the verification is the
    lossless stochastic one with seeded uniforms.  Afterwards, for the
    spread: `replays` steps timed one by one (the context rewound and
    replayed from the first step), then `replays` draft calls and verify
    calls timed one by one."""
    import torch
    from block_diffusion_drafter_fc_amd import (Drafter, DrafterConfig, KVCache, verify_greedy,
                                                verify_stochastic,
                                                verify_stochastic_workspace_bytes)
    from synth import Gen
    from synth.configs import hidden_states, make_weights, page_pool

    t0 = time.time()
    S = warmup + max(steps, replays)
    wl = Workload(s, S)
    B, gamma = wl.B, wl.gamma
    w_host = make_weights(s)
    wdev = {k: to_dev(v, s.bf16) for k, v in w_host.items()}
    cfg = DrafterConfig(hidden=s.hidden, n_layers=s.n_layers, n_q_heads=s.n_q_heads,
                        n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, intermediate=s.inter,
                        vocab=s.vocab, n_target_feats=s.n_feats, max_block=16,
                        mask_token_id=s.mask_id, dtype=s.dtype, rope_theta=s.rope_theta,
                        rms_eps=s.eps)
    drafter = Drafter(cfg, wdev)
    log(f"weights ready ({time.time() - t0:.1f}s)")

    pps = (wl.Lmax + 15) // 16 + 1
    n_pages, table = page_pool(s, pps, extra=4, tag="bench.pages")
    dt = torch.bfloat16 if s.bf16 else torch.float32
    pages = torch.zeros((s.n_layers, n_pages, 2, s.n_kv_heads, 16, s.head_dim), dtype=dt,
                        device="cuda")
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv = KVCache(pages, torch.from_numpy(table).cuda(), ctx)
    chunk = 4096
    ws = torch.empty(drafter.workspace_bytes(B, gamma, max(chunk, B * 16), pps),
                     dtype=torch.uint8, device="cuda")

    # prefill: inject each prompt in chunks of up to 4096 tokens
    torch.cuda.synchronize()
    tp = time.time()
    prefill_tokens = 0
    for b in range(B):
        for c0 in range(0, int(wl.L0[b]), chunk):
            n = min(chunk, int(wl.L0[b]) - c0)
            cu = np.zeros(B + 1, np.int32)
            cu[b + 1:] = n
            drafter.inject(kv, to_dev(hidden_states(s, b, c0, n), s.bf16),
                           torch.from_numpy(cu).cuda(), ws)
            prefill_tokens += n
    torch.cuda.synchronize()
    prefill_s = time.time() - tp
    assert np.array_equal(ctx.cpu().numpy(), wl.L0), "prefill did not advance the context"
    log(f"prefill of {prefill_tokens} tokens: {prefill_s * 1e3:.1f} ms (incl. host input upload)")

    # per-step inputs, resident on the device
    hid = [to_dev(wl.step_hidden(k), s.bf16) for k in range(S)]
    cus = [torch.from_numpy(np.concatenate([[0], np.cumsum(wl.n_new[k])]).astype(np.int32)).cuda()
           for k in range(S)]
    anc = [torch.from_numpy(wl.anchor[k]).cuda() for k in range(S)]
    blk = [torch.zeros((B, gamma), dtype=torch.int32, device="cuda") for _ in range(S)]
    acc = [torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(S)]
    out = [torch.zeros((B, gamma), dtype=torch.int32, device="cuda") for _ in range(S)]
    L0_dev = torch.from_numpy(wl.L0.astype(np.int32)).cuda()

    # pre-pass: the drafted blocks decide the planted target scores
    for k in range(S):
        drafter.inject(kv, hid[k], cus[k], ws)
        drafter.draft(kv, anc[k], gamma, blk[k], ws)
    torch.cuda.synchronize()
    assert drafter.device_error() == 0
    g = Gen(s.seed)
    tgt = []
    for k in range(S):
        t = g.plant_target(f"bench.target.{k}", blk[k].cpu().numpy(), wl.tau[k], s.vocab,
                           dtype=s.dtype)
        tgt.append(to_dev(t, s.bf16))
    log(f"inputs of {S} steps resident ({time.time() - t0:.1f}s)")

    if sampled:
        logits = torch.empty((B, gamma, s.vocab), dtype=torch.float32, device="cuda")
        uni = [torch.from_numpy(g.uniform(f"bench.u.{k}", B * gamma).astype(np.float32)
                                .reshape(B, gamma)).cuda() for k in range(S)]
        vws = torch.empty(verify_stochastic_workspace_bytes(B, gamma, s.vocab), dtype=torch.uint8,
                          device="cuda")
        seed0 = 0x5EED_0000_0000_0000

        def draft_call(k):
            drafter.draft_sampled(kv, anc[k], gamma, seed0 + k, blk[k], logits, ws)

        def verify_call(k):
            verify_stochastic(blk[k], logits, tgt[k], uni[k], acc[k], out[k], vws)
    else:
        def draft_call(k):
            drafter.draft(kv, anc[k], gamma, blk[k], ws)

        def verify_call(k):
            verify_greedy(blk[k], tgt[k], acc[k], out[k], ws)

    def step(k):
        drafter.inject(kv, hid[k], cus[k], ws)
        draft_call(k)
        verify_call(k)

    # The timed region: exactly `steps` steps after `warmup` untimed ones.
    # The LM-head timing events are created by profile_enable, before it.
    ctx.copy_(L0_dev)
    for k in range(warmup):
        step(k)
    drafter.profile_enable(True)
    drafter.profile_read(reset=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(warmup, warmup + steps):
        step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    drafter.profile_enable(False)
    lm_ms, lm_count = drafter.profile_read(reset=True)
    assert drafter.device_error() == 0
    timed = range(warmup, warmup + steps)
    accepted = np.stack([acc[k].cpu().numpy() for k in timed])
    replay_ok = float(np.mean(accepted == wl.tau[warmup:warmup + steps]))
    taus = accepted

    # Spread: the context rewound to the prompt, the warm-up steps replayed,
    # then `replays` steps timed one by one (each re-injects what the first
    # pass injected, so the cache ends as it did).
    ctx.copy_(L0_dev)
    for k in range(warmup):
        step(k)
    step_ms = event_times(lambda i: step(warmup + i), replays)
    assert drafter.device_error() == 0
    replay_ok = min(replay_ok, float(np.mean(
        np.stack([acc[warmup + i].cpu().numpy() for i in range(replays)])
        == wl.tau[warmup:warmup + replays])))
    # the draft call alone, and verification alone, on the final context
    draft_ms = event_times(lambda i: draft_call(i % S), replays)
    verify_ms = event_times(lambda i: verify_call(i % S), replays)
    assert drafter.device_error() == 0

    res = dict(elapsed=elapsed, steps=steps, warmup=warmup, lm_ms=lm_ms, lm_count=lm_count,
               replay_ok=replay_ok, draft_only_ms=float(np.mean(draft_ms)),
               draft_spread=percentiles(draft_ms), step_spread=percentiles(step_ms),
               verify_spread=percentiles(verify_ms), prefill_s=prefill_s,
               verify_only_ms=float(np.mean(verify_ms)), mean_tau=float(taus.mean()),
               prefill_tokens=prefill_tokens, wl=wl, draft_ctx_step=warmup + replays - 1)
    drafter.close()
    return res, w_host


def host_description() -> dict:
    """CPU model, logical CPUs and those this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count() or 1, "usable_cpus": usable,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def hipblaslt_lm_head(s, rows):
    """Vendor-library comparison for the LM head: torch.mm (hipBLASLt on
    ROCm) of random bf16 activations [rows][hidden] with a random bf16
    weight [vocab][hidden] (bf16 logits out), alone and followed by the row
    argmax that the fused kernel also does, at the workload's rows and at
    twice as many.  A measurement beside the product path, not part of it."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(s.seed)
    w = (torch.randn(s.vocab, s.hidden, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    out = {}
    for m in (rows, 2 * rows):
        a = torch.randn(m, s.hidden, device="cuda", generator=g).to(torch.bfloat16)
        flops = 2.0 * m * s.vocab * s.hidden
        rec = {}
        for name, fn in (("mm", lambda: torch.mm(a, w.t())),
                         ("mm_argmax", lambda: torch.mm(a, w.t()).argmax(dim=1))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            rec[name] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        out[f"rows_{m}"] = rec
        del a
    del w
    torch.cuda.empty_cache()
    return out


def lm_roofline(s, rows, lm_bytes, lm_avg_ms, launches):
    """Roofline object of the LM head, the dominant kernel.  Up to 64 rows it
    is the fused weight-streaming product (HBM-bound: the bytes it must read
    over the launch time against 8 TB/s); from 128 rows on it is the
    large-tile MFMA product (2 * rows * vocab * hidden flops against the
    2.5 PFLOP/s bf16 peak).  Counter traffic is recorded for the first."""
    if rows >= 128:
        flops = 2.0 * rows * s.vocab * s.hidden
        tf = flops / (lm_avg_ms * 1e-3) / 1e12
        return {"kernel": "LM head: bf16 MFMA 256 x 256 tiles + argmax (k_gemm_big)",
                "bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                "avg_launch_ms": round(lm_avg_ms, 5), "launches": launches,
                "flops_per_launch": flops, "traffic": None}
    gbs = lm_bytes / (lm_avg_ms * 1e-3) / 1e9
    return {"kernel": "LM head: final RMSNorm staged + bf16 MFMA + argmax (k_skinny)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "avg_launch_ms": round(lm_avg_ms, 5), "launches": launches,
            "bytes_per_launch": lm_bytes, "traffic": recorded_traffic(s.name)}


def cpu_baseline(s, w_host, budget_s=15.0):
    """The oracle, as committed, on a bounded sample of the same step: per
    block, inject the new context tokens of a step (their target features),
    draft the block over the sequence's context (its real length, synthetic
    cached context) and verify it greedily.  About budget_s of work on all
    the oracle's threads, then one block on a single thread."""
    import oracle
    from synth import Gen
    from synth.configs import anchors, context_kv, context_lengths, hidden_states, planted_tau
    L = int(context_lengths(s)[0])
    ck, cv = context_kv(s, 0, L)
    m = oracle.Model(s, w_host)
    toks = np.full(s.block, s.mask_id, np.int32)

    def one_block(n):
        # the previous cycle's accepted tokens enter the context first
        n_new = int(planted_tau(s, 1, f"cpu.new.{n}")[0])
        m.inject(hidden_states(s, 0, L, n_new), np.arange(L, L + n_new, dtype=np.int32))
        toks[0] = anchors(s, 1, tag=f"cpu.anchor.{n}")[0]
        _, block = m.draft(ck, cv, L, toks)
        tgt = Gen(s.seed).plant_target(f"cpu.target.{n}", block[None], np.array([4]), s.vocab,
                                       dtype=s.dtype)
        oracle.verify(block, tgt[0], s.bf16)
        return n_new

    threads = oracle.threads()
    n = tokens = 0
    t0 = time.perf_counter()
    while True:
        tokens += one_block(n)
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= 50:
            break
    dt = time.perf_counter() - t0
    oracle.set_threads(1)
    t1 = time.perf_counter()
    one_block(n)
    dt1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    out = {"value": round(n / dt, 4), "unit": "blocks/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} steps of one sequence with a {L}-token synthetic context: inject "
                     f"{tokens} new context tokens in all, draft a block of {s.block}, verify it "
                     f"greedily; {dt:.1f} s on {threads} threads",
           "single_thread": {"value": round(1.0 / dt1, 4), "unit": "blocks/s",
                             "sample": f"1 step, {dt1:.1f} s"}}
    out.update(host_description())
    return out


# ------------------------------------------------------------ HBM counters
def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"lm_head_traffic_{workload}.json")


def copy_calibration(reps: int = 5):
    """A plain device-to-device copy of COPY_BYTES, reps times (calibrates
    the HBM byte counters: the copy reads and writes exactly COPY_BYTES)."""
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": reps}), flush=True)


def read_calibration(reps: int = 5):
    """A pure read of COPY_BYTES with the LM head's load pattern, reps times
    (calibrates FETCH_SIZE: the kernel reads exactly COPY_BYTES and writes 16
    bytes per workgroup)."""
    import torch
    from block_diffusion_drafter_fc_amd import read_calibration as rc
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    out = torch.empty(16 * READ_CAL_WORKGROUPS, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    rc(src, out, READ_CAL_WORKGROUPS)   # warm-up
    ts = event_times(lambda i: rc(src, out, READ_CAL_WORKGROUPS), reps)
    # (this is also the read ceiling of the LM head's load pattern)
    print(json.dumps({"read_bytes": COPY_BYTES, "reps": reps, "workgroups": READ_CAL_WORKGROUPS,
                      "ms_median": round(float(np.median(ts)), 4),
                      "read_GBps": round(COPY_BYTES / (float(np.median(ts)) * 1e-3) / 1e9, 1)}),
          flush=True)


def _csv_files(d: str, suffix: str):
    import glob
    return glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)


def _counter_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no counter_collection.csv under {d}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                key = (fn, r["Dispatch_Id"])
                e = per.setdefault(key, {"name": r["Kernel_Name"], "value": 0.0})
                e["value"] += float(r["Counter_Value"])
    return list(per.values())


def counter_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the LM-head kernel,
    scaled by what the same counters read for the calibration copy."""
    kname = LM_KERNEL["bf16-skinny"]

    def mean_for(rows, pred):
        v = [r["value"] for r in rows if pred(r)]
        if not v:
            sys.exit("no matching dispatches in the counter files")
        return float(np.mean(v)), len(v)

    def cal_kib(d, key):
        # the calibration dispatches: the largest ones of the calibration kernel
        rows = [r for r in _counter_rows(d) if key in r["name"].lower()]
        if not rows:
            sys.exit(f"no '{key}' dispatches in {d}")
        top = max(r["value"] for r in rows)
        return mean_for(rows, lambda r: r["value"] >= 0.5 * top)[0]

    f_kib, nf = mean_for(_counter_rows(fetch_dir), lambda r: kname in r["name"])
    w_kib, nw = mean_for(_counter_rows(write_dir), lambda r: kname in r["name"])
    # FETCH_SIZE from the pure read with the LM head's pattern, WRITE_SIZE
    # from the copy (the read's own writes are 16 bytes per workgroup)
    cf_kib, cw_kib = cal_kib(cfetch_dir, "read_calibration"), cal_kib(cwrite_dir, "copy")
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    rec = {"workload": workload, "kernel": kname, "source_sha256_16": kernel_source_hash(),
           "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
           "dispatches": [nf, nw],
           "calibration_bytes": COPY_BYTES,
           "read_calibration_fetch_kib": round(cf_kib, 1), "copy_write_kib": round(cw_kib, 1),
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "traffic_bytes_per_launch": int(round(f_kib * 1024 * f_scale + w_kib * 1024 * w_scale))}
    with open(traffic_path(workload), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)


def mfma_summary(d: str, workload: str):
    """Per kernel of a --kernel-trace --pmc MfmaUtil MfmaFlopsBF16 run:
    dispatches, mean duration, matrix-core busy share (MfmaUtil: MFMA busy
    cycles over active cycles x SIMDs) and counted bf16 TFLOP/s.  Printed as
    a markdown table."""
    import csv
    util, flops, dur = {}, {}, {}
    for fn in _csv_files(d, "counter_collection.csv"):
        with open(fn) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], fn, r["Dispatch_Id"])
                if r["Counter_Name"] == "MfmaUtil":
                    util[key] = float(r["Counter_Value"])
                elif r["Counter_Name"] == "MfmaFlopsBF16":
                    flops[key] = float(r["Counter_Value"])
    for fn in _csv_files(d, "kernel_trace.csv"):
        with open(fn) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], fn.replace("kernel_trace", "counter_collection"),
                       r["Dispatch_Id"])
                dur[key] = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3
    per = {}
    for key, u in util.items():
        name = key[0]
        e = per.setdefault(name, {"n": 0, "util": 0.0, "flops": 0.0, "us": 0.0, "nd": 0})
        e["n"] += 1
        e["util"] += u
        e["flops"] += flops.get(key, 0.0)
        if key in dur:
            e["us"] += dur[key]
            e["nd"] += 1
    rows = sorted(per.items(), key=lambda kv: -kv[1]["us"])
    print(f"| kernel | dispatches | mean us | MFMA busy % | bf16 TFLOP/s (counted) |")
    print("|---|---:|---:|---:|---:|")
    for name, e in rows:
        if e["flops"] == 0 and e["util"] == 0:
            continue
        mean_us = e["us"] / max(e["nd"], 1)
        tf = e["flops"] / (e["us"] * 1e-6) / 1e12 if e["us"] > 0 else float("nan")
        short = name.replace("void ", "").replace("(anonymous namespace)::", "")
        print(f"| `{short[:90]}` | {e['n']} | {mean_us:.1f} | {e['util'] / e['n']:.1f} | {tf:.0f} |")


def stats_summary(d: str):
    """Markdown table of a rocprofv3 --stats run's kernel_stats.csv: calls,
    average / min / max duration and share of kernel time, per kernel."""
    import csv
    rows = []
    for fn in _csv_files(d, "kernel_stats.csv"):
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        name = r["Name"].replace("void ", "").replace("(anonymous namespace)::", "")
        print(f"| `{name[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f}% |")


def recorded_traffic(workload: str):
    """Counter-derived HBM bytes per LM-head launch, if recorded for the
    current kernel sources; else None."""
    try:
        with open(traffic_path(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def block_sweep(s, gammas, steps, warmup):
    """Draft cost against block size on one workload: each block size gets
    its own seeded steps (planted accepted lengths within the block), the
    same context, weights and shapes otherwise.  Proposals per block are
    gamma - 1 (the anchor is given)."""
    import dataclasses
    rows = []
    for gamma in gammas:
        if not 2 <= gamma <= 16:
            sys.exit(f"block size {gamma} outside 2..16")
        sg = dataclasses.replace(s, block=gamma)
        res, _ = run_gpu(sg, steps, warmup)
        wl = res["wl"]
        B = wl.B
        timed = range(warmup, warmup + steps)
        draft_bytes = float(np.mean([algorithmic_bytes(sg, wl.L_at[k], int(wl.n_new[k].sum()), B,
                                                       gamma)["draft"] for k in timed]))
        blocks_per_s = B * steps / res["elapsed"]
        d_ms = res["draft_only_ms"]
        rows.append({"block": gamma,
                     "step_blocks_per_s": round(blocks_per_s, 2),
                     "step_tokens_per_s": round(blocks_per_s * (gamma - 1), 1),
                     "draft_ms": round(d_ms, 4),
                     "draft_blocks_per_s": round(B * 1e3 / d_ms, 2),
                     "draft_tokens_per_s": round(B * 1e3 / d_ms * (gamma - 1), 1),
                     "draft_hbm_frac": round(draft_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "replay_accept_match": res["replay_ok"]})
        log(f"block {gamma}: draft {d_ms:.4f} ms, step {blocks_per_s:.1f} blocks/s")
    print(json.dumps({"block_sweep": rows, "workload": s.name, "batch": s.batch,
                      "steps": steps, "warmup": warmup, "dtype": s.dtype}), flush=True)


def sampled_bench(s, steps, warmup):
    """The step with sampled drafting and lossless verification, next to the
    greedy step on the same inputs (one JSON line)."""
    rows = {}
    for mode in ("greedy", "sampled"):
        res, _ = run_gpu(s, steps, warmup, sampled=mode == "sampled")
        wl = res["wl"]
        B, gamma = wl.B, wl.gamma
        rows[mode] = {"step_ms": round(res["elapsed"] * 1e3 / steps, 4),
                      "step_blocks_per_s": round(B * steps / res["elapsed"], 2),
                      "draft_ms": round(res["draft_only_ms"], 4),
                      "verify_ms": round(res["verify_only_ms"], 4),
                      "mean_accept_len": round(res["mean_tau"], 3)}
        log(f"{mode}: {rows[mode]}")
    elem = 2 if s.bf16 else 4
    v_bytes = B * gamma * s.vocab * elem + B * (gamma - 1) * s.vocab * 4
    rows["sampled"]["verify_logit_bytes"] = v_bytes
    rows["sampled"]["verify_hbm_frac"] = round(
        v_bytes / (rows["sampled"]["verify_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    print(json.dumps({"sampled_vs_greedy": rows, "workload": s.name, "batch": s.batch,
                      "block": s.block, "steps": steps, "warmup": warmup, "dtype": s.dtype}),
          flush=True)


def packed_bench(s, n_blocks, steps, warmup):
    """Packed multi-block forward with the weighted loss: n_blocks blocks of
    one sequence (anchor positions spread over its context, seeded targets)
    in one pass per step, after the context is injected (one JSON line)."""
    import torch
    from block_diffusion_drafter_fc_amd import Drafter, DrafterConfig, KVCache
    from synth import Gen
    from synth.configs import context_lengths, hidden_states, make_weights, page_pool
    t0 = time.time()
    w_host = make_weights(s)
    wdev = {k: to_dev(v, s.bf16) for k, v in w_host.items()}
    cfg = DrafterConfig(hidden=s.hidden, n_layers=s.n_layers, n_q_heads=s.n_q_heads,
                        n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, intermediate=s.inter,
                        vocab=s.vocab, n_target_feats=s.n_feats, max_block=16,
                        mask_token_id=s.mask_id, dtype=s.dtype, rope_theta=s.rope_theta,
                        rms_eps=s.eps)
    drafter = Drafter(cfg, wdev)
    L = int(context_lengths(s)[0])
    gamma = s.block
    pps = (L + 15) // 16 + 1
    s1 = s.replace(batch=1)
    n_pages, table = page_pool(s1, pps, extra=4, tag="bench.packed.pages")
    dt = torch.bfloat16 if s.bf16 else torch.float32
    pages = torch.zeros((s.n_layers, n_pages, 2, s.n_kv_heads, 16, s.head_dim), dtype=dt,
                        device="cuda")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv = KVCache(pages, torch.from_numpy(table[:1]).cuda(), ctx)
    ws = torch.empty(max(drafter.workspace_bytes(1, gamma, 4096, pps),
                         drafter.packed_workspace_bytes(n_blocks, gamma, pps)),
                     dtype=torch.uint8, device="cuda")
    for c0 in range(0, L, 4096):
        n = min(4096, L - c0)
        drafter.inject(kv, to_dev(hidden_states(s, 0, c0, n), s.bf16),
                       torch.tensor([0, n], dtype=torch.int32, device="cuda"), ws)
    torch.cuda.synchronize()
    g = Gen(s.seed + 5)
    S = warmup + steps
    anc, pos, tgt = [], [], []
    for k in range(S):
        anc.append(torch.from_numpy(g.uniform_int(f"bench.pk.anchor.{k}", n_blocks, 0,
                                                  s.vocab - 2).astype(np.int32)).cuda())
        pos.append(torch.from_numpy(g.uniform_int(f"bench.pk.pos.{k}", n_blocks, 0,
                                                  L).astype(np.int32)).cuda())
        tgt.append(torch.from_numpy(g.uniform_int(f"bench.pk.tgt.{k}", n_blocks * gamma, 0,
                                                  s.vocab - 1).astype(np.int32)
                                    .reshape(n_blocks, gamma)).cuda())
    logits = torch.empty((n_blocks, gamma, s.vocab), dtype=torch.float32, device="cuda")
    bl = torch.empty(n_blocks, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    log(f"packed set-up ({time.time() - t0:.1f}s): {n_blocks} blocks of {gamma}, context {L}")

    def step(k):
        drafter.packed_forward(kv, anc[k], pos[k], gamma, logits, ws, targets=tgt[k], decay=7.0,
                               block_loss=bl, loss=loss)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for k in range(warmup, S):
        step(k)
    torch.cuda.synchronize()
    el = time.perf_counter() - t
    assert drafter.device_error() == 0
    ms = el * 1e3 / steps
    flops = draft_flops(s, np.asarray([p for p in pos[-1].cpu().numpy()]), n_blocks, gamma)
    print(json.dumps({"packed_forward": {
        "blocks": n_blocks, "block": gamma, "context": L, "ms_per_pass": round(ms, 4),
        "blocks_per_s": round(n_blocks * 1e3 / ms, 2),
        "tokens_per_s": round(n_blocks * (gamma - 1) * 1e3 / ms, 1),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "loss": float(loss.cpu().numpy()[0])},
        "workload": s.name, "steps": steps, "warmup": warmup, "dtype": s.dtype}), flush=True)
    drafter.close()


def ar_bench(s, gammas, steps, warmup):
    """Autoregressive drafting (block_size - 1 causal passes) next to the
    one-pass block draft on the same model, context and anchors, per block
    size (one JSON line): the pages' draft-cost argument measured here."""
    import torch
    from block_diffusion_drafter_fc_amd import Drafter, DrafterConfig, KVCache
    from synth.configs import anchors, context_lengths, hidden_states, make_weights, page_pool
    w_host = make_weights(s)
    wdev = {k: to_dev(v, s.bf16) for k, v in w_host.items()}
    cfg = DrafterConfig(hidden=s.hidden, n_layers=s.n_layers, n_q_heads=s.n_q_heads,
                        n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, intermediate=s.inter,
                        vocab=s.vocab, n_target_feats=s.n_feats, max_block=16,
                        mask_token_id=s.mask_id, dtype=s.dtype, rope_theta=s.rope_theta,
                        rms_eps=s.eps)
    drafter = Drafter(cfg, wdev)
    B = s.batch
    L0 = context_lengths(s).astype(np.int64)
    pps = int(L0.max() + 15) // 16 + 1
    n_pages, table = page_pool(s, pps, extra=4, tag="bench.ar.pages")
    dt = torch.bfloat16 if s.bf16 else torch.float32
    pages = torch.zeros((s.n_layers, n_pages, 2, s.n_kv_heads, 16, s.head_dim), dtype=dt,
                        device="cuda")
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv = KVCache(pages, torch.from_numpy(table).cuda(), ctx)
    ws = torch.empty(max(drafter.workspace_bytes(B, 16, 4096, pps),
                         drafter.ar_workspace_bytes(B, 16, pps)), dtype=torch.uint8, device="cuda")
    for b in range(B):
        for c0 in range(0, int(L0[b]), 4096):
            n = min(4096, int(L0[b]) - c0)
            cu = np.zeros(B + 1, np.int32)
            cu[b + 1:] = n
            drafter.inject(kv, to_dev(hidden_states(s, b, c0, n), s.bf16),
                           torch.from_numpy(cu).cuda(), ws)
    a = torch.from_numpy(anchors(s, B, tag="bench.ar.anchor")).cuda()
    rows = []
    for gamma in gammas:
        res = {}
        blk = torch.empty((B, gamma), dtype=torch.int32, device="cuda")
        for mode in ("block", "ar"):
            call = ((lambda: drafter.draft(kv, a, gamma, blk, ws)) if mode == "block" else
                    (lambda: drafter.draft_ar(kv, a, gamma, blk, ws)))
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            res[mode] = (time.perf_counter() - t) * 1e3 / steps
        rows.append({"block": gamma, "block_draft_ms": round(res["block"], 4),
                     "ar_draft_ms": round(res["ar"], 4),
                     "ar_over_block": round(res["ar"] / res["block"], 2),
                     "block_tokens_per_s": round(B * (gamma - 1) * 1e3 / res["block"], 1),
                     "ar_tokens_per_s": round(B * (gamma - 1) * 1e3 / res["ar"], 1)})
        log(f"block {gamma}: {rows[-1]}")
    assert drafter.device_error() == 0
    print(json.dumps({"ar_vs_block": rows, "workload": s.name, "batch": B, "steps": steps,
                      "warmup": warmup, "dtype": s.dtype}), flush=True)
    drafter.close()


def workload_report(s, res) -> dict:
    """Draft-alone figures of a run: mean time over the replays, the spread,
    blocks and tokens per second, HBM fraction, achieved TFLOP/s and the
    per-phase roofline fraction (roofline time / measured time)."""
    wl = res["wl"]
    B, gamma = wl.B, wl.gamma
    k_last = res["draft_ctx_step"]
    timed = range(res["warmup"], res["warmup"] + res["steps"])
    step_bytes = [algorithmic_bytes(s, wl.L_at[k], int(wl.n_new[k].sum()), B, gamma)
                  for k in timed]
    # the draft-alone calls run on the final context
    d_bytes = algorithmic_bytes(s, wl.L_at[k_last], 0, B, gamma)["draft"]
    d_ms = res["draft_only_ms"]
    t_roof = draft_phase_roofline(s, wl.L_at[k_last], B, gamma)
    flops = draft_flops(s, wl.L_at[k_last], B, gamma)
    draft = {"ms": round(d_ms, 4), **res["draft_spread"],
             "blocks_per_s": round(B * 1e3 / d_ms, 3),
             "tokens_per_s": round(B * (gamma - 1) * 1e3 / d_ms, 1),
             "hbm_frac": round(d_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "algorithmic_GB": round(d_bytes / 1e9, 4),
             "tflops": round(flops / (d_ms * 1e-3) / 1e12, 2),
             "roofline_ms": round(t_roof * 1e3, 4),
             "roofline_frac": round(t_roof * 1e3 / d_ms, 4)}
    return {"draft_only": draft, "step_bytes": float(np.mean([b["step"] for b in step_bytes])),
            "lm_bytes": step_bytes[0]["lm_head"]}


def workload_object(k: int, steps: int, warmup: int, replays: int, contexts: str) -> dict:
    """One more workload of the default run, in the batch-1 line: `steps`
    whole steps timed after `warmup`, then the spread of `replays` steps,
    draft calls and verify calls, and the draft's per-phase roofline."""
    from synth.configs import CONFIGS
    s = CONFIGS[k]
    log(f"workload {s.name}")
    res, _ = run_gpu(s, steps, warmup, replays=replays)
    rep = workload_report(s, res)
    wl = res["wl"]
    B, gamma = wl.B, wl.gamma
    ms_step = res["elapsed"] * 1e3 / steps
    lm_ms = res["lm_ms"] / max(res["lm_count"], 1)
    M = B * gamma
    return {"workload": s.name, "batch": B, "block": gamma,
            "contexts": f"{contexts} at the start, {int(wl.L_at[-1].mean())} mean at the end",
            "steps": steps, "warmup": warmup,
            "step_ms": round(ms_step, 4), "step_blocks_per_s": round(B * 1e3 / ms_step, 2),
            "step_spread": res["step_spread"],
            "draft_only": rep["draft_only"], "verify_only": res["verify_spread"],
            "lm_head": {"avg_launch_ms": round(lm_ms, 4),
                        "tflops": round(2.0 * M * s.vocab * s.hidden / (lm_ms * 1e-3) / 1e12, 1)},
            "replay_accept_match": res["replay_ok"], "mean_accept_len": round(res["mean_tau"], 3)}


def bs32_report(replays: int) -> dict:
    """The Qwen3-8B-shaped drafter at batch 32 (concurrency-32 serving
    shape): 10 whole steps timed after 2, then the spreads."""
    return workload_object(3, 10, 2, replays, "U[1024,4096]")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-8b-bs1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bs32", action="store_true",
                    help="skip the batch-32 object of the default batch-1 run")
    ap.add_argument("--no-long-wide", action="store_true",
                    help="skip the long-context and wide-drafter objects of the default run")
    ap.add_argument("--replays", type=int, default=50,
                    help="steps and calls timed one by one for the spread")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the counter-calibration copy")
    ap.add_argument("--read-calibration", action="store_true",
                    help="only run the pure-read counter calibration")
    ap.add_argument("--counter-summary", nargs=4,
                    metavar=("FETCH", "WRITE", "READ_CAL_FETCH", "COPY_WRITE"),
                    help="summarise rocprofv3 --pmc output directories into profiles/")
    ap.add_argument("--stats-summary", metavar="DIR",
                    help="markdown table of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="per-kernel matrix-core use from a rocprofv3 MfmaUtil/MfmaFlopsBF16 run")
    ap.add_argument("--sampled", action="store_true",
                    help="time the sampled-draft + lossless-verify step next to the greedy one")
    ap.add_argument("--ar", default=None, metavar="G1,G2,...",
                    help="time autoregressive drafting next to the block draft at these block sizes")
    ap.add_argument("--packed", type=int, default=0, metavar="N",
                    help="time the packed forward + loss of N blocks of one sequence instead")
    ap.add_argument("--block-sweep", default=None, metavar="G1,G2,...",
                    help="time the step at each block size instead (one JSON line)")
    ap.add_argument("--lm-head-hipblaslt", action="store_true",
                    help="also time hipBLASLt (torch.mm) on the LM-head shape, bare and with "
                         "the row argmax, at the workload's rows and twice as many")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_calibration:
        read_calibration()
        return
    if args.stats_summary:
        stats_summary(args.stats_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, args.workload)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the DFlash hot path here is built for and timed on a "
              f"single MI355X (sequences shard across GPUs with no exchange); --gpus {args.gpus} "
              f"is not run.", file=sys.stderr)
        sys.exit(2)
    from synth.configs import CONFIGS
    by_name = {c.name: c for c in CONFIGS.values()}
    if args.workload not in by_name:
        sys.exit(f"unknown workload {args.workload}; one of {sorted(by_name)}")
    s = by_name[args.workload]
    if args.ar:
        ar_bench(s, [int(g) for g in args.ar.split(",")], args.steps, args.warmup)
        return
    if args.packed:
        packed_bench(s, args.packed, args.steps, args.warmup)
        return
    if args.sampled:
        sampled_bench(s, args.steps, args.warmup)
        return
    if args.block_sweep:
        block_sweep(s, [int(g) for g in args.block_sweep.split(",")], args.steps, args.warmup)
        return

    res, w_host = run_gpu(s, args.steps, args.warmup, replays=args.replays)
    rep = workload_report(s, res)
    wl = res["wl"]
    B, gamma = wl.B, wl.gamma
    ms_step = res["elapsed"] * 1e3 / args.steps
    blocks_per_s = B * args.steps / res["elapsed"]
    lm_bytes = rep["lm_bytes"]
    lm_avg_ms = res["lm_ms"] / max(res["lm_count"], 1)
    line = {
        "metric": METRIC,
        "value": round(blocks_per_s, 3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "batch": B, "block": gamma, "hidden": s.hidden,
                   "draft_layers": s.n_layers, "heads": f"{s.n_q_heads}/{s.n_kv_heads}",
                   "intermediate": s.inter, "vocab": s.vocab,
                   "context_start": int(wl.L0.mean()), "context_end": int(wl.L_at[-1].mean()),
                   "step": "inject accepted tokens + draft block + greedy verify",
                   "parallelism": "single GPU"},
        "draft_tokens_per_s": round(blocks_per_s * (gamma - 1), 2),
        "step_hbm_frac": round(rep["step_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_GB": round(rep["step_bytes"] / 1e9, 4),
        "step_spread": res["step_spread"],
        "draft_only": rep["draft_only"],
        "verify_only": res["verify_spread"],
        "replay_accept_match": res["replay_ok"],
        "prefill": {"tokens": res["prefill_tokens"], "s": round(res["prefill_s"], 4)},
        "roofline": lm_roofline(s, B * gamma, lm_bytes, lm_avg_ms, res["lm_count"]),
    }
    if args.lm_head_hipblaslt:
        line["lm_head_hipblaslt"] = hipblaslt_lm_head(s, B * gamma)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(s, w_host, args.cpu_budget)
    del w_host
    if s.name == "qwen3-8b-bs1" and not args.no_bs32:
        line["bs32"] = bs32_report(args.replays)
    if s.name == "qwen3-8b-bs1" and not args.no_long_wide:
        # the other two workloads of the survey's configurations, shorter runs
        line["long"] = workload_object(4, 5, 2, min(args.replays, 20), "4 x 32768")
        line["wide"] = workload_object(5, 5, 2, min(args.replays, 20), "U[2048,8192]")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
