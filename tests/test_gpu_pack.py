"""Packed weights (dflash_pack_weights) against the layout the header defines:
for every fused product, its rows in kernel order (gate/up: 64-row groups of
gate and up alternating), padded to a multiple of 64 with zeros, cut into
16-row x 32-column tiles of 512 bf16, in which 16-byte piece l holds row
l % 16 and columns 8 (l // 16) .. + 7 of the tile, the tiles ordered
[64-row group][32-column block][16-row group].  The products follow one
another in the order fc, K/V of all layers, LM head, then per layer QKV, O,
gate/up, down, each starting at a multiple of 128 elements.  Bit-exact."""
import numpy as np
import pytest

from gpu_util import log, make_drafter
from synth.configs import Shape, make_weights

pytestmark = pytest.mark.gpu

MINI = Shape("mini-bf16-pack", 512, 2, 4, 2, 128, 768, 1000, 16, 1, True, seed=993)


def tiles(rows):
    """rows [N][K] uint16 -> packed uint16 vector of the defined tile order."""
    N, K = rows.shape
    Np = (N + 63) // 64 * 64
    pad = np.zeros((Np, K), np.uint16)
    pad[:N] = rows
    # [g][w][r][kb][q][8] -> [g][kb][w][q][r][8]   (piece l = 16 q + r)
    t = pad.reshape(Np // 64, 4, 16, K // 32, 4, 8).transpose(0, 3, 1, 4, 2, 5)
    return t.reshape(-1)


def test_packed_layout_matches_definition():
    import torch
    s = MINI
    w = make_weights(s)
    drafter, w, _ = make_drafter(s, w)
    assert drafter.packed is not None
    got = drafter.packed.view(torch.int16).cpu().numpy().view(np.uint16)
    b = w                                   # bf16 bit patterns, as uploaded
    assert all(v.dtype == np.uint16 for v in b.values())
    D, I, NL = s.hidden, s.inter, s.n_layers
    prods = [("fc", b["fc_w"]),
             ("kv", np.concatenate([b[f"l{l}.{k}"] for l in range(NL) for k in ("wk", "wv")])),
             ("lm", b["lm_head"])]
    for l in range(NL):
        g, u = b[f"l{l}.w_gate"], b[f"l{l}.w_up"]
        gu = np.concatenate([np.concatenate([g[64 * j:64 * j + 64], u[64 * j:64 * j + 64]])
                             for j in range(I // 64)])
        prods += [(f"qkv{l}", np.concatenate([b[f"l{l}.wq"], b[f"l{l}.wk"], b[f"l{l}.wv"]])),
                  (f"o{l}", b[f"l{l}.wo"]), (f"gu{l}", gu), (f"down{l}", b[f"l{l}.w_down"])]
    off = 0
    for name, rows in prods:
        exp = tiles(rows)
        seg = got[off:off + exp.size]
        bad = int(np.count_nonzero(seg != exp))
        log(f"  {name}: {rows.shape[0]}x{rows.shape[1]} -> {exp.size} elements, {bad} mismatches")
        assert bad == 0, name
        off += (exp.size + 127) // 128 * 128
    assert off * 2 <= drafter.packed.numel()
