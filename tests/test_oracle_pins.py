"""Pins of the CPU oracle against facts that do not come from the oracle
itself: library routines for special cases, closed forms, invariants of the
method, and the worked example / constants printed on the pages.

Each test would fail for a plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a wrong mask).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import Gen
from synth.configs import Shape, context_kv, hidden_states, make_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(bf16=False, **kw):
    base = dict(name="pin", hidden=32, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                inter=48, vocab=64, block=4, batch=1, bf16=bf16, seed=7)
    base.update(kw)
    return Shape(**base)


# --------------------------------------------------------------------- bf16
def test_round_bf16_matches_library_rounding():
    import torch
    x = Gen(1).normal("x", 4000, std=10.0)
    ours = oracle.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_round_bf16_ties_to_even():
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0            # halfway, even is 1.0
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6  # halfway, even is up
    assert oracle.round_bf16(-(1 + 2 ** -8 + 2 ** -20)) == -(1 + 2 ** -7)
    assert oracle.round_bf16(0.0) == 0.0


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    g = Gen(2).normal("g", 16, std=0.1, mean=1.0)
    for c in (3.0, -2.0, 0.5):
        out = oracle.rmsnorm(np.full(16, c), g, 1e-6)
        expect = np.sign(c) * g.astype(np.float64) / math.sqrt(1.0 + 1e-6 / c ** 2)
        np.testing.assert_allclose(out, expect, rtol=1e-14)


def test_rmsnorm_scale_invariant_with_unit_rms():
    x = Gen(3).normal("x", 64).astype(np.float64)
    ones = np.ones(64, np.float32)
    a = oracle.rmsnorm(x, ones, 0.0)
    b = oracle.rmsnorm(7.5 * x, ones, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-14)
    assert abs(np.mean(a ** 2) - 1.0) < 1e-14


# --------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = Gen(4).normal("x", 3 * 8).astype(np.float64)
    assert np.array_equal(oracle.rope(x, 3, 8, 0.0, 1e6), x)


def test_rope_two_dims_rotates_by_position():
    for p in (1.0, 2.5, 1000.0):
        np.testing.assert_allclose(oracle.rope([1.0, 0.0], 1, 2, p, 1e6),
                                   [math.cos(p), math.sin(p)], atol=1e-15)
        np.testing.assert_allclose(oracle.rope([0.0, 1.0], 1, 2, p, 1e6),
                                   [-math.sin(p), math.cos(p)], atol=1e-15)


def test_rope_pairs_dimension_i_with_i_plus_half():
    p, theta = 3.0, 100.0
    # dh = 4: pair (0, 2) turns at p * theta^0, pair (1, 3) at p * theta^(-1/2)
    np.testing.assert_allclose(oracle.rope([1, 0, 0, 0], 1, 4, p, theta),
                               [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    a = p / math.sqrt(theta)
    np.testing.assert_allclose(oracle.rope([0, 1, 0, 0], 1, 4, p, theta),
                               [0, math.cos(a), 0, math.sin(a)], atol=1e-15)


def test_rope_preserves_norm_and_depends_on_relative_position():
    q = Gen(5).normal("q", 16).astype(np.float64)
    k = Gen(5).normal("k", 16).astype(np.float64)
    theta = 1e6
    rq = oracle.rope(q, 1, 16, 123.0, theta)
    assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
    d1 = np.dot(oracle.rope(q, 1, 16, 40.0, theta), oracle.rope(k, 1, 16, 17.0, theta))
    d2 = np.dot(oracle.rope(q, 1, 16, 40.0 + 5000, theta), oracle.rope(k, 1, 16, 17.0 + 5000, theta))
    assert abs(d1 - d2) < 1e-9 * max(1.0, abs(d1))


# ---------------------------------------------------------------- attention
def _qkv(seed, nq, nk, dh):
    g = Gen(seed)
    return (g.normal("q", (nq, dh)).astype(np.float64), g.normal("k", (nk, dh)).astype(np.float64),
            g.normal("v", (nk, dh)).astype(np.float64))


def test_attention_equal_keys_give_mean_of_values():
    q, k, v = _qkv(6, 3, 5, 8)
    k[:] = k[0]
    o = oracle.attention_dense(q, k, v, np.ones((3, 5)))
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-13, atol=1e-15)


def test_attention_two_keys_closed_form_with_scale():
    q, k, v = _qkv(7, 2, 2, 8)
    o = oracle.attention_dense(q, k, v, np.ones((2, 2)))
    for i in range(2):
        s = q[i] @ k.T / math.sqrt(8.0)
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        np.testing.assert_allclose(o[i], w0 * v[0] + (1 - w0) * v[1], rtol=1e-13)


def test_attention_masked_key_equals_removed_key_and_empty_row_is_zero():
    q, k, v = _qkv(8, 4, 6, 8)
    vis = np.ones((4, 6), np.uint8)
    vis[:, 2] = 0
    vis[3, :] = 0
    o = oracle.attention_dense(q, k, v, vis)
    keep = [0, 1, 3, 4, 5]
    o2 = oracle.attention_dense(q[:3], k[keep], v[keep], np.ones((3, 5)))
    assert np.array_equal(o[:3], o2)
    assert np.array_equal(o[3], np.zeros(8))


def test_attention_single_visible_key_returns_its_value():
    q, k, v = _qkv(9, 2, 4, 8)
    vis = np.zeros((2, 4), np.uint8)
    vis[0, 1] = 1
    vis[1, 3] = 1
    o = oracle.attention_dense(q, k, v, vis)
    assert np.array_equal(o[0], v[1]) and np.array_equal(o[1], v[3])


# ------------------------------------------------------------------- SwiGLU
def test_swiglu_diagonal_special_case():
    from scipy.special import expit
    g = Gen(10)
    a = g.normal("a", 6, std=2.0)
    b = g.normal("b", 6, std=2.0)
    z = g.normal("z", (3, 6)).astype(np.float64)
    out = oracle.swiglu(np.diag(a), np.diag(b), np.eye(6, dtype=np.float32), z)
    gate = z * a.astype(np.float64)
    expect = gate * expit(gate) * (z * b.astype(np.float64))
    np.testing.assert_allclose(out, expect, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------- inject
@pytest.mark.parametrize("which", [0, 2, 4])
def test_inject_fuses_feature_blocks_in_order(which):
    s = tiny()
    D, KV = s.hidden, s.n_kv_heads * s.head_dim
    w = make_weights(s)
    fc = np.zeros((D, 5 * D), np.float32)
    fc[:, which * D:(which + 1) * D] = np.eye(D, dtype=np.float32)
    w["fc_w"] = fc
    for l in range(s.n_layers):
        wk = np.zeros((KV, D), np.float32)
        wk[:, l * KV:(l + 1) * KV] = np.eye(KV, dtype=np.float32)   # layer l keeps dims l*KV..
        wv = np.zeros((KV, D), np.float32)
        wv[:, (1 - l) * KV:(2 - l) * KV] = np.eye(KV, dtype=np.float32)
        w[f"l{l}.wk"], w[f"l{l}.wv"] = wk, wv
    m = oracle.Model(s, w)
    hid = hidden_states(s, 0, 0, 5)
    k, v = m.inject(hid, np.zeros(5, np.int32))      # position 0: RoPE is the identity
    for t in range(5):
        c = oracle.rmsnorm(hid[t, which * D:(which + 1) * D].astype(np.float64), w["fc_norm"], s.eps)
        for l in range(s.n_layers):
            assert np.array_equal(k[t, l].reshape(-1), c[l * KV:(l + 1) * KV])
            assert np.array_equal(v[t, l].reshape(-1), c[(1 - l) * KV:(2 - l) * KV])


def test_inject_rounds_the_fused_context_to_bf16_before_projecting():
    # Paper §7.3 sizes the fc output at two bytes per value, so in bf16 mode
    # c is rounded before W_K/W_V.  With W_c selecting the first feature and
    # a key that adds two entries of c, k_j = bf16(bf16(c_j) + bf16(c_j+16)):
    # rounding only the stored key would give bf16(c_j + c_j+16).
    s = tiny(bf16=True)
    D, KV = s.hidden, s.n_kv_heads * s.head_dim
    one = np.uint16(0x3F80)
    w = make_weights(s)
    fc = np.zeros((D, 5 * D), np.uint16)
    fc[np.arange(D), np.arange(D)] = one
    w["fc_w"] = fc
    for l in range(s.n_layers):
        wk = np.zeros((KV, D), np.uint16)
        wk[np.arange(KV), np.arange(KV)] = one
        wk[np.arange(KV), KV + np.arange(KV)] = one
        w[f"l{l}.wk"] = wk
    hid = hidden_states(s, 0, 0, 4)
    k, _ = oracle.Model(s, w).inject(hid, np.zeros(4, np.int32))   # position 0: no rotation
    gain = (w["fc_norm"].astype(np.uint32) << 16).view(np.float32)
    f1 = (hid[:, :D].astype(np.uint32) << 16).view(np.float32)
    differs = 0
    for t in range(4):
        c = oracle.rmsnorm(f1[t], gain, s.eps)
        cr = oracle.round_bf16(c)
        expect = oracle.round_bf16(cr[:KV] + cr[KV:2 * KV])
        for l in range(s.n_layers):
            assert np.array_equal(k[t, l].reshape(-1), expect)
        differs += int(np.sum(expect != oracle.round_bf16(c[:KV] + c[KV:2 * KV])))
    assert differs > 0          # the construction tells the two readings apart


@pytest.mark.parametrize("bf16", [False, True])
def test_inject_is_per_token_chunk_invariant(bf16):
    s = tiny(bf16=bf16)
    m = oracle.Model(s, make_weights(s))
    hid = hidden_states(s, 0, 0, 9)
    pos = np.arange(9, dtype=np.int32) + 11
    k, v = m.inject(hid, pos)
    for lo, hi in ((0, 1), (1, 5), (5, 9)):
        k2, v2 = m.inject(np.ascontiguousarray(hid[lo:hi]), pos[lo:hi])
        assert np.array_equal(k[lo:hi], k2) and np.array_equal(v[lo:hi], v2)
    if bf16:
        assert np.array_equal(oracle.round_bf16(k[:2]), k[:2])


# -------------------------------------------------------------------- draft
def _ctx_from_inject(m, s, L, start):
    hid = hidden_states(s, 0, 0, L)
    k, v = m.inject(hid, np.arange(start, start + L, dtype=np.int32))
    dt = np.float32
    return (np.ascontiguousarray(k.transpose(1, 0, 2, 3)).astype(dt),
            np.ascontiguousarray(v.transpose(1, 0, 2, 3)).astype(dt))


def test_draft_is_invariant_to_a_common_position_shift_without_context():
    s = tiny()
    m = oracle.Model(s, make_weights(s))
    toks = np.array([5, 63, 63, 63], np.int32)
    empty = np.zeros((s.n_layers, 1, s.n_kv_heads, s.head_dim), np.float32)
    vis = np.ones((4, 4), np.uint8)
    a = m.forward(empty, empty, 0, toks, np.arange(4), vis)
    b = m.forward(empty, empty, 0, toks, np.arange(4) + 777, vis)
    assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(a))


def test_draft_is_invariant_to_a_common_position_shift_with_context():
    s = tiny()
    m = oracle.Model(s, make_weights(s))
    L, shift = 12, 4321
    toks = np.array([9, 63, 63, 63], np.int32)
    vis = np.ones((4, L + 4), np.uint8)
    k0, v0 = _ctx_from_inject(m, s, L, 0)
    k1, v1 = _ctx_from_inject(m, s, L, shift)
    a = m.forward(k0, v0, L, toks, L + np.arange(4), vis)
    b = m.forward(k1, v1, L, toks, shift + L + np.arange(4), vis)
    # the context is stored in fp32, so the shift changes it by fp32 rounding only
    assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(a))


def test_packed_blocks_equal_separate_drafts():
    s = tiny()
    m = oracle.Model(s, make_weights(s))
    Lc = 20
    ck, cv = context_kv(s, 0, Lc)
    anchors_pos = np.array([0, 7, 13, 20], np.int32)
    toks = np.array([[3, 63, 63, 63], [17, 63, 63, 63], [40, 63, 63, 63], [2, 63, 63, 63]], np.int32)
    packed = m.draft_packed(ck, cv, toks, anchors_pos)
    for b in range(4):
        lg, _ = m.draft(ck, cv, int(anchors_pos[b]), toks[b])
        assert np.array_equal(packed[4 * b:4 * b + 4], lg)


def test_no_leakage_from_cache_slots_after_the_context_or_later_blocks():
    s = tiny()
    m = oracle.Model(s, make_weights(s))
    L = 10
    ck, cv = context_kv(s, 0, 16)
    toks = np.array([8, 63, 63, 63], np.int32)
    a, _ = m.draft(ck, cv, L, toks)
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, L:] = 1e3
    cv2[:, L:] = -1e3
    b, _ = m.draft(ck2, cv2, L, toks)
    assert np.array_equal(a, b)
    t1 = np.array([[3, 63, 63, 63], [17, 63, 63, 63]], np.int32)
    t2 = t1.copy()
    t2[1] = [50, 1, 2, 3]
    p1 = m.draft_packed(ck, cv, t1, np.array([4, 9], np.int32))
    p2 = m.draft_packed(ck, cv, t2, np.array([4, 9], np.int32))
    assert np.array_equal(p1[:4], p2[:4])
    assert not np.array_equal(p1[4:], p2[4:])


def test_block_attention_is_bidirectional():
    s = tiny()
    m = oracle.Model(s, make_weights(s))
    ck, cv = context_kv(s, 0, 6)
    a, _ = m.draft(ck, cv, 6, np.array([8, 63, 63, 63], np.int32))
    b, _ = m.draft(ck, cv, 6, np.array([8, 63, 63, 12], np.int32))
    assert np.max(np.abs(a[0] - b[0])) > 1e-6       # row 0 sees the last row


def test_gqa_equals_mha_with_duplicated_kv_heads():
    sa = tiny(n_kv_heads=2)
    sb = tiny(n_kv_heads=4)
    wa = make_weights(sa)
    wb = dict(wa)
    dh = sa.head_dim
    dup = np.repeat(np.arange(2), 2)     # MHA head h reuses GQA kv head h // 2
    for l in range(sa.n_layers):
        for key in ("wk", "wv"):
            src = wa[f"l{l}.{key}"].reshape(2, dh, -1)
            wb[f"l{l}.{key}"] = np.ascontiguousarray(src[dup].reshape(4 * dh, -1))
    ka, va = context_kv(sa, 0, 9)
    kb = np.ascontiguousarray(ka[:, :, dup])
    vb = np.ascontiguousarray(va[:, :, dup])
    toks = np.array([30, 63, 63, 63], np.int32)
    la, _ = oracle.Model(sa, wa).draft(ka, va, 9, toks)
    lb, _ = oracle.Model(sb, wb).draft(kb, vb, 9, toks)
    assert np.array_equal(la, lb)


def test_zero_sublayers_with_tied_orthogonal_embedding_propose_own_tokens():
    s = tiny(vocab=32)
    D = s.hidden
    w = make_weights(s)
    E = (0.5 * np.eye(D)).astype(np.float32)
    w["embed"] = E
    w["lm_head"] = E
    w["final_norm"] = np.ones(D, np.float32)
    for l in range(s.n_layers):
        w[f"l{l}.wo"] = np.zeros_like(w[f"l{l}.wo"])
        w[f"l{l}.w_down"] = np.zeros_like(w[f"l{l}.w_down"])
    m = oracle.Model(s, w)
    ck, cv = context_kv(s, 0, 5)
    toks = np.array([7, 31, 31, 31], np.int32)
    logits, block = m.draft(ck, cv, 5, toks)
    assert list(block) == [7, 31, 31, 31]
    expect = np.zeros((4, D))
    expect[np.arange(4), toks] = 0.5 * 0.5 / math.sqrt(0.25 / D + s.eps)
    np.testing.assert_allclose(logits, expect, rtol=1e-13, atol=1e-15)


def test_argmax_ties_resolve_to_the_lowest_index():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax([-1.0, -1.0]) == 0
    assert oracle.argmax([0.0, 0.0, 5.0, 5.0, 5.0]) == 2


def test_argmax_signed_zeros_tie_and_take_the_lowest_index():
    # -0.0 == +0.0, so whichever comes first wins
    assert oracle.argmax([-1.0, -0.0, 0.0, -2.0]) == 1
    assert oracle.argmax([-1.0, 0.0, -0.0, -2.0]) == 1
    tgt = np.full((2, 6), 0xBF80, np.uint16)     # bf16 -1.0
    tgt[0, [2, 4]] = [0x8000, 0x0000]            # -0.0 before +0.0
    tgt[1, [1, 3]] = [0x0000, 0x8000]
    tau, out, T = oracle.verify(np.array([9, 2], np.int32), tgt, True)
    assert list(T) == [2, 1] and tau == 2 and list(out) == [2, 1]


# ------------------------------------------------- norm gains and their wiring
# A zero RMSNorm gain zeroes exactly what that norm feeds, so each gain can be
# tied to its sub-layer by an independent construction: zeroing the gain must
# give bit for bit what zeroing that sub-layer's output projection gives.  A
# gain wired to the wrong sub-layer (or layer) breaks the equality.

def _draft_with(s, w, L, toks):
    m = oracle.Model(s, w)
    ck, cv = context_kv(s, 0, max(L, 1))
    return m.draft(ck, cv, L, toks)


def _zero(a):
    return np.zeros_like(a)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("layer", [0, 1])
def test_attention_norm_gain_feeds_only_the_attention_sublayer(bf16, layer):
    # Empty context: with a zero input the block queries/keys/values are zero,
    # the attention output is the mean of zero values, and the sub-layer adds
    # nothing -- exactly as with W_O = 0.
    s = tiny(bf16=bf16)
    toks = np.array([11, 63, 63, 63], np.int32)
    w = make_weights(s)
    a = dict(w)
    a[f"l{layer}.attn_norm"] = _zero(w[f"l{layer}.attn_norm"])
    b = dict(w)
    b[f"l{layer}.wo"] = _zero(w[f"l{layer}.wo"])
    la, _ = _draft_with(s, a, 0, toks)
    lb, _ = _draft_with(s, b, 0, toks)
    ln, _ = _draft_with(s, w, 0, toks)
    assert np.array_equal(la, lb)
    assert np.max(np.abs(la - ln)) > 1e-6      # the sub-layer did contribute


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("layer", [0, 1])
def test_mlp_norm_gain_feeds_only_the_mlp_sublayer(bf16, layer):
    s = tiny(bf16=bf16)
    toks = np.array([29, 63, 63, 63], np.int32)
    w = make_weights(s)
    a = dict(w)
    a[f"l{layer}.mlp_norm"] = _zero(w[f"l{layer}.mlp_norm"])
    b = dict(w)
    b[f"l{layer}.w_down"] = _zero(w[f"l{layer}.w_down"])
    la, _ = _draft_with(s, a, 7, toks)
    lb, _ = _draft_with(s, b, 7, toks)
    ln, _ = _draft_with(s, w, 7, toks)
    assert np.array_equal(la, lb)
    assert np.max(np.abs(la - ln)) > 1e-6


@pytest.mark.parametrize("bf16", [False, True])
def test_final_norm_gain_feeds_the_lm_head(bf16):
    s = tiny(bf16=bf16)
    toks = np.array([40, 63, 63, 63], np.int32)
    w = make_weights(s)
    w["final_norm"] = _zero(w["final_norm"])
    logits, block = _draft_with(s, w, 5, toks)
    assert np.all(logits == 0.0)
    assert list(block) == [40, 0, 0, 0]        # all-zero rows: the lowest index


@pytest.mark.parametrize("bf16", [False, True])
def test_fc_norm_gain_feeds_the_injected_keys_and_values(bf16):
    s = tiny(bf16=bf16)
    w = make_weights(s)
    w["fc_norm"] = _zero(w["fc_norm"])
    hid = hidden_states(s, 0, 0, 6)
    k, v = oracle.Model(s, w).inject(hid, np.arange(6, dtype=np.int32))
    assert np.all(k == 0.0) and np.all(v == 0.0)


# ------------------------------------------------------------------- verify
def test_verify_worked_example_from_the_pages():
    fx = json.load(open(os.path.join(GOLDEN, "verify_worked_example.json")))
    n = fx["n_proposals"]
    g = Gen(11)
    block = np.concatenate([[5], g.uniform_int("d", n, 0, 998)]).astype(np.int32)
    tgt = g.plant_target("t", block[None], np.array([fx["n_matching"] + 1]), 1000)[0]
    tau, out, T = oracle.verify(block, tgt, False)
    assert tau == fx["expect_tau"]
    names = {f"d{i}": block[i] for i in range(1, n + 1)}
    names.update({f"T{i}": T[i] for i in range(n + 1)})
    assert list(out[:tau]) == [names[x] for x in fx["expect_out"]]
    assert np.all(out[tau:] == -1)
    assert T[fx["n_matching"]] != block[fx["n_matching"] + 1]    # the fourth is rejected
    assert len(fx["expect_discarded"]) == n - fx["n_matching"] - 1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_recovers_every_planted_length(dtype):
    gamma, V = 16, 500
    g = Gen(12)
    for trial in range(3):
        blocks = g.uniform_int(f"b{trial}", gamma * gamma, 0, V - 1).reshape(gamma, gamma)
        taus = np.arange(1, gamma + 1)
        tgt = g.plant_target(f"t{trial}", blocks, taus, V, dtype=dtype)
        for i in range(gamma):
            tau, out, T = oracle.verify(blocks[i], tgt[i], dtype == "bf16")
            assert tau == taus[i]
            assert list(out[:tau]) == list(T[:tau])           # greedy output equality
            assert list(out[:tau - 1]) == list(blocks[i][1:tau])
            assert np.all(out[tau:] == -1)


def test_verify_all_match_and_first_mismatch():
    g = Gen(13)
    block = g.uniform_int("b", 8, 0, 99).astype(np.int32)
    tgt = np.zeros((8, 100), np.float32)
    for j in range(7):
        tgt[j, block[j + 1]] = 1.0
    tgt[7, 42] = 1.0
    tau, out, T = oracle.verify(block, tgt, False)
    assert tau == 8 and list(out) == list(block[1:]) + [42]
    tgt[0, :] = 0.0
    tgt[0, (block[1] + 1) % 100] = 1.0
    tau, out, T = oracle.verify(block, tgt, False)
    assert tau == 1 and out[0] == (block[1] + 1) % 100 and np.all(out[1:] == -1)


def test_verify_block_of_one_returns_the_target_token():
    tgt = np.zeros((1, 10), np.float32)
    tgt[0, 3] = 2.0
    tau, out, T = oracle.verify(np.array([7], np.int32), tgt, False)
    assert tau == 1 and out[0] == 3


def test_verify_ties_in_target_scores_take_the_lowest_index():
    tgt = np.zeros((2, 10), np.float32)
    tgt[0, [4, 6]] = 1.0
    tgt[1, [2, 9]] = 3.0
    tau, out, T = oracle.verify(np.array([0, 4], np.int32), tgt, False)
    assert list(T) == [4, 2] and tau == 2 and list(out) == [4, 2]


# --------------------------------------------------------- loss weighting
def test_loss_weights_closed_form_and_page_constants():
    fx = json.load(open(os.path.join(GOLDEN, "loss_decay.json")))
    for block, gd in fx["decay_by_block_size"].items():
        K = int(block) - 1
        w = oracle.loss_weights(gd, K)
        assert w[0] == 1.0
        np.testing.assert_allclose(w[1:] / w[:-1], math.exp(-1.0 / gd), rtol=1e-14)
        if gd + 1 <= K:
            assert abs(w[gd] - math.exp(-1.0)) < 1e-15       # k = gamma + 1 gives 1/e
        assert np.all(np.diff(w) < 0)


def test_weighted_ce_uniform_logits_give_log_vocab():
    w = oracle.loss_weights(7, 15)
    V = 1000
    ce = oracle.weighted_ce(np.zeros((15, V)), np.arange(15), w)
    assert abs(ce - math.log(V)) < 1e-12


def test_weighted_ce_penalises_early_errors_more():
    w = oracle.loss_weights(7, 15)
    good = np.zeros((15, 50))
    good[np.arange(15), np.arange(15)] = 30.0
    early, late = good.copy(), good.copy()
    early[0] = 0.0
    late[14] = 0.0
    t = np.arange(15)
    assert oracle.weighted_ce(early, t, w) > oracle.weighted_ce(late, t, w) > oracle.weighted_ce(good, t, w)
