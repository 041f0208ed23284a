"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
filling and reading the paged cache, and the parity checks themselves.
Inputs come from synth/ only; expected values from oracle/ only."""
from __future__ import annotations

import math
import sys
import time

import numpy as np

from synth.configs import Shape, make_weights


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, bf16: bool):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        assert a.dtype == np.uint16
        t = t.view(torch.bfloat16)
    else:
        assert a.dtype == np.float32
    return t.to("cuda")


def values_view(pages: np.ndarray) -> np.ndarray:
    """The value halves of a [layers][pages][2][Hkv][page_size][dh] page
    array, seen as [layers][pages][Hkv][dh][page_size]: each page stores its
    values transposed (dimension-major), its keys row-major."""
    nl, n_pages, _, hkv, ps, dh = pages.shape
    v = pages[:, :, 1].reshape(nl, n_pages, hkv, dh, ps)
    assert np.shares_memory(v, pages)
    return v


def to_host(t, bf16: bool) -> np.ndarray:
    import torch
    t = t.detach().to("cpu").contiguous()
    if bf16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def host_values(a: np.ndarray, bf16: bool) -> np.ndarray:
    return bf16_to_f64(a) if bf16 else a.astype(np.float64)


def drafter_config(s: Shape, max_block=None):
    from block_diffusion_drafter_fc_amd import DrafterConfig
    return DrafterConfig(hidden=s.hidden, n_layers=s.n_layers, n_q_heads=s.n_q_heads,
                         n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, intermediate=s.inter,
                         vocab=s.vocab, n_target_feats=s.n_feats,
                         max_block=max_block or max(s.block, 16), mask_token_id=s.mask_id,
                         page_size=s.page_size, dtype=s.dtype, rope_theta=s.rope_theta,
                         rms_eps=s.eps)


def make_drafter(s: Shape, weights_np: dict | None = None, pack: bool = True):
    """(Drafter, host weights) with device copies of the seeded weights; bf16
    models get packed weights unless pack is False."""
    from block_diffusion_drafter_fc_amd import Drafter
    w = weights_np if weights_np is not None else make_weights(s)
    dev = {k: to_dev(v, s.bf16) for k, v in w.items()}
    return Drafter(drafter_config(s), dev, pack=pack), w, dev


class PagedCache:
    """Host mirror + device tensors of a paged cache for `batch` sequences."""

    def __init__(self, s: Shape, batch: int, pages_per_seq: int, extra_pages: int = 3,
                 tag: str = "pages"):
        import torch
        from block_diffusion_drafter_fc_amd import KVCache
        from synth.configs import page_pool
        self.s = s
        self.batch = batch
        s2 = s.replace(batch=batch)
        self.n_pages, table = page_pool(s2, pages_per_seq, extra_pages, tag)
        self.table = table
        self.pages_per_seq = pages_per_seq
        dt = np.uint16 if s.bf16 else np.float32
        self.host = np.zeros((s.n_layers, self.n_pages, 2, s.n_kv_heads, s.page_size, s.head_dim),
                             dtype=dt)
        self.pages = None
        self.table_dev = torch.from_numpy(table).to("cuda")
        self.ctx_dev = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.KVCache = KVCache

    def write_dense(self, b: int, k: np.ndarray, v: np.ndarray, start: int = 0):
        """Put dense [n_layers][L][Hkv][dh] keys/values of sequence b at
        positions start.. into the host mirror."""
        L = k.shape[1]
        pos = np.arange(start, start + L)
        pg = self.table[b][pos // self.s.page_size]
        slot = pos % self.s.page_size
        self.host[:, pg, 0, :, slot, :] = np.transpose(k, (1, 0, 2, 3))
        values_view(self.host)[:, pg, :, :, slot] = np.transpose(v, (1, 0, 2, 3))

    def upload(self, ctx_lens):
        import torch
        self.pages = to_dev(self.host, self.s.bf16)
        self.ctx_dev.copy_(torch.from_numpy(np.asarray(ctx_lens, dtype=np.int32)))
        return self.kv()

    def allocate_empty(self):
        import torch
        dt = torch.bfloat16 if self.s.bf16 else torch.float32
        self.pages = torch.zeros(self.host.shape, dtype=dt, device="cuda")
        self.ctx_dev.zero_()
        return self.kv()

    def kv(self):
        return self.KVCache(self.pages, self.table_dev, self.ctx_dev)

    def fetch(self):
        """Copy the device cache to the host once; read_dense uses the copy."""
        self.snapshot = to_host(self.pages, self.s.bf16)
        return self.snapshot

    def read_dense(self, b: int, start: int, n: int):
        """Cache of sequence b (as of the last fetch()), positions
        start..start+n-1, as dense float64 (k, v) [n_layers][n][Hkv][dh]."""
        host = self.snapshot
        pos = np.arange(start, start + n)
        pg = self.table[b][pos // self.s.page_size]
        slot = pos % self.s.page_size
        k = host[:, pg, 0, :, slot, :]   # [n][layers][Hkv][dh]
        v = values_view(host)[:, pg, :, :, slot]
        return (np.transpose(host_values(k, self.s.bf16), (1, 0, 2, 3)),
                np.transpose(host_values(v, self.s.bf16), (1, 0, 2, 3)))


def logits_tolerance(s: Shape, ref: np.ndarray) -> float:
    """fp32 models: 1e-4 of the largest reference magnitude; bf16 models:
    2e-2 absolute on the fp32 logits."""
    return 2e-2 if s.bf16 else 1e-4 * float(np.max(np.abs(ref)))


def check_tokens(gpu_tokens, ref_logits, gap_tol: float):
    """Each GPU proposal must equal the oracle's argmax, unless the oracle's
    top-2 gap at that row is below gap_tol and the GPU picked one of the
    near-tied candidates.  Returns the number of tolerated mismatches."""
    tolerated = 0
    for j in range(1, len(gpu_tokens)):
        row = ref_logits[j]
        top = int(np.argmax(row))       # lowest index among maxima
        if int(gpu_tokens[j]) == top:
            continue
        gap = row[top] - row[int(gpu_tokens[j])]
        assert gap < gap_tol, f"row {j}: gpu {gpu_tokens[j]} vs oracle {top}, gap {gap}"
        tolerated += 1
    return tolerated


def workspace(drafter, max_batch, max_block, max_new, max_pages):
    import torch
    n = drafter.workspace_bytes(max_batch, max_block, max_new, max_pages)
    return torch.empty(n, dtype=torch.uint8, device="cuda")
