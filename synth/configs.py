"""Drafter shapes and workload recipes used by the parity tests and the
benchmark.  Test and benchmark infrastructure: it draws inputs, it computes
nothing of the method.

Five workloads (seed 20261200 + k for workload k):
  k=1 tiny-fp32      D=256, 2 layers, 4/2 heads, dh 64, I 768, V 1024,
                     block 4, batch 1, 64 context tokens, fp32
  k=2 qwen3-8b-bs1   D=4096, 5 layers, 32/8 heads, dh 128, I 12288,
                     V 151936, block 16, batch 1, 2048 context tokens, bf16
  k=3 qwen3-8b-bs32  same drafter, batch 32, context U[1024, 4096] in
                     16-token pages, 1..16 new context tokens per step,
                     planted accepted length min(Geom(1/6), 16)
  k=4 qwen3-8b-long  same drafter, batch 4, 32768 context tokens each
  k=5 wide-8layer    D=5120, 8 layers, 40/8 heads, dh 128, I 17408,
                     V 151936, batch 8, context U[2048, 8192], bf16
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import Gen


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    block: int
    batch: int
    bf16: bool
    n_feats: int = 5
    rope_theta: float = 1.0e6
    eps: float = 1.0e-6
    page_size: int = 16
    seed: int = 0

    @property
    def dtype(self) -> str:
        return "bf16" if self.bf16 else "f32"

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


TINY = Shape("tiny-fp32", 256, 2, 4, 2, 64, 768, 1024, 4, 1, False, seed=20261201)
Q8_BS1 = Shape("qwen3-8b-bs1", 4096, 5, 32, 8, 128, 12288, 151936, 16, 1, True, seed=20261202)
Q8_BS32 = Shape("qwen3-8b-bs32", 4096, 5, 32, 8, 128, 12288, 151936, 16, 32, True, seed=20261203)
Q8_LONG = Shape("qwen3-8b-long", 4096, 5, 32, 8, 128, 12288, 151936, 16, 4, True, seed=20261204)
WIDE = Shape("wide-8layer", 5120, 8, 40, 8, 128, 17408, 151936, 16, 8, True, seed=20261205)

CONFIGS = {1: TINY, 2: Q8_BS1, 3: Q8_BS32, 4: Q8_LONG, 5: WIDE}


def context_lengths(s: Shape) -> np.ndarray:
    """Per-sequence context length before the first draft."""
    g = Gen(s.seed)
    if s.name == "tiny-fp32":
        return np.full(s.batch, 64, dtype=np.int64)
    if s.name == "qwen3-8b-bs1":
        return np.full(s.batch, 2048, dtype=np.int64)
    if s.name == "qwen3-8b-bs32":
        return g.uniform_int("ctx_len", s.batch, 1024, 4096)
    if s.name == "qwen3-8b-long":
        return np.full(s.batch, 32768, dtype=np.int64)
    if s.name == "wide-8layer":
        return g.uniform_int("ctx_len", s.batch, 2048, 8192)
    return np.full(s.batch, 64, dtype=np.int64)


def planted_tau(s: Shape, n: int, tag: str = "tau") -> np.ndarray:
    """Accepted lengths to plant: U{1..block} for every workload except the
    batch-32 one, which draws min(Geom(1/6), block) on {1, 2, ...}."""
    g = Gen(s.seed)
    if s.name == "qwen3-8b-bs32":
        u = g.uniform(tag, n)
        k = 1 + np.floor(np.log1p(-u) / math.log(5.0 / 6.0)).astype(np.int64)
        return np.minimum(k, s.block)
    return g.uniform_int(tag, n, 1, s.block)


def anchors(s: Shape, n: int | None = None, tag: str = "anchor") -> np.ndarray:
    """Clean anchor tokens, drawn from [0, V-2] (V-1 is the mask token)."""
    return Gen(s.seed).uniform_int(tag, s.batch if n is None else n, 0, s.vocab - 2).astype(np.int32)


def weight_names(s: Shape):
    """(name, shape, kind) for every drafter tensor; kind 'mat' ~ N(0, 0.02^2),
    kind 'gain' ~ 1 + 0.02 N(0, 1)."""
    D, I, V = s.hidden, s.inter, s.vocab
    QD, KV = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    out = [("fc_w", (D, s.n_feats * D), "mat"), ("fc_norm", (D,), "gain"),
           ("embed", (V, D), "mat"), ("lm_head", (V, D), "mat"), ("final_norm", (D,), "gain")]
    for l in range(s.n_layers):
        out += [(f"l{l}.attn_norm", (D,), "gain"), (f"l{l}.wq", (QD, D), "mat"),
                (f"l{l}.wk", (KV, D), "mat"), (f"l{l}.wv", (KV, D), "mat"),
                (f"l{l}.wo", (D, QD), "mat"), (f"l{l}.mlp_norm", (D,), "gain"),
                (f"l{l}.w_gate", (I, D), "mat"), (f"l{l}.w_up", (I, D), "mat"),
                (f"l{l}.w_down", (D, I), "mat")]
    return out


def make_weights(s: Shape) -> dict:
    """All drafter weights as numpy arrays (uint16 bf16 bits or float32)."""
    g = Gen(s.seed)
    w = {}
    for name, shape, kind in weight_names(s):
        if kind == "mat":
            w[name] = g.normal("w." + name, shape, std=0.02, dtype=s.dtype)
        else:
            w[name] = g.normal("w." + name, shape, std=0.02, mean=1.0, dtype=s.dtype)
    return w


def hidden_states(s: Shape, seq: int, start: int, n: int) -> np.ndarray:
    """Target features [n][n_feats*D] for tokens start..start+n-1 of
    sequence `seq`, N(0, 1); a token's values depend only on (seq, position)."""
    F = s.n_feats * s.hidden
    return Gen(s.seed).normal(f"hidden.s{seq}", (n, F), dtype=s.dtype, offset=start * F)


def kv_std(s: Shape) -> float:
    """Scale of a synthetic injected key/value: an RMS-normalised context
    vector times N(0, 0.02^2) weights has per-element std 0.02*sqrt(D)."""
    return 0.02 * math.sqrt(s.hidden)


def context_kv(s: Shape, seq: int, L: int, start: int = 0):
    """Synthetic context cache of one sequence, as if injected:
    (k, v) each [n_layers][L][Hkv][dh] for positions start..start+L-1."""
    KV = s.n_kv_heads * s.head_dim
    g = Gen(s.seed)
    k = np.empty((s.n_layers, L, s.n_kv_heads, s.head_dim),
                 dtype=np.uint16 if s.bf16 else np.float32)
    v = np.empty_like(k)
    for l in range(s.n_layers):
        k[l] = g.normal(f"ctxk.l{l}.s{seq}", (L, s.n_kv_heads, s.head_dim), std=kv_std(s),
                        dtype=s.dtype, offset=start * KV)
        v[l] = g.normal(f"ctxv.l{l}.s{seq}", (L, s.n_kv_heads, s.head_dim), std=kv_std(s),
                        dtype=s.dtype, offset=start * KV)
    return k, v


def page_pool(s: Shape, pages_per_seq: int, extra: int = 0, tag: str = "pages"):
    """A shuffled page pool: returns (n_pages, page_table [batch][pages_per_seq])."""
    n_pages = s.batch * pages_per_seq + extra
    keys = Gen(s.seed).uniform(tag, n_pages)
    perm = np.argsort(keys, kind="stable").astype(np.int32)
    table = perm[: s.batch * pages_per_seq].reshape(s.batch, pages_per_seq)
    return n_pages, np.ascontiguousarray(table)
