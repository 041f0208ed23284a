"""ctypes binding of the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the CPU
baseline leg of the benchmark use it.  The product path never imports it,
and it imports nothing from the product package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
# DFLASH_ORACLE_LIB points the loader at another build (the sanitizer test's)
_LIB = os.environ.get("DFLASH_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None
MAX_LAYERS = 32
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile liboracle.so (g++ -O2, strict IEEE double, OpenMP); with
    sanitize, an AddressSanitizer + UndefinedBehaviorSanitizer build at `out`."""
    out = out or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared"] +
                              (SANITIZE if sanitize else []) + ["-o", tmp, _SRC])
        os.replace(tmp, out)
    return out


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("n_feats", ctypes.c_int32),
                ("bf16", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("eps", ctypes.c_double)]


_PA = ctypes.c_void_p * MAX_LAYERS


class Weights(ctypes.Structure):
    _fields_ = [("fc_w", ctypes.c_void_p), ("fc_norm", ctypes.c_void_p),
                ("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PA), ("wq", _PA), ("wk", _PA), ("wv", _PA), ("wo", _PA),
                ("mlp_norm", _PA), ("w_gate", _PA), ("w_up", _PA), ("w_down", _PA)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
        lib.oracle_round_bf16.argtypes = [dbl]
        lib.oracle_round_bf16.restype = dbl
        lib.oracle_rmsnorm.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, dbl, vp]
        lib.oracle_rope.argtypes = [vp, ctypes.c_int, ctypes.c_int, dbl, dbl]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_argmax.argtypes = [vp, ctypes.c_int]
        lib.oracle_argmax.restype = ctypes.c_int
        lib.oracle_attention_dense.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                               ctypes.c_int, vp, vp]
        lib.oracle_inject.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp]
        lib.oracle_draft.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int,
                                     vp, vp]
        lib.oracle_forward.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                       ctypes.c_int, vp, vp]
        lib.oracle_swiglu.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                      ctypes.c_int, vp]
        lib.oracle_draft_packed.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                            ctypes.c_int, ctypes.c_int, vp]
        lib.oracle_verify.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        lib.oracle_verify.restype = ctypes.c_int
        lib.oracle_loss_weights.argtypes = [dbl, ctypes.c_int, vp]
        lib.oracle_weighted_ce.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int]
        lib.oracle_weighted_ce.restype = dbl
        for f in (lib.oracle_rmsnorm, lib.oracle_rope, lib.oracle_attention_dense,
                  lib.oracle_inject, lib.oracle_draft, lib.oracle_draft_packed,
                  lib.oracle_forward, lib.oracle_swiglu,
                  lib.oracle_loss_weights):
            f.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


class Model:
    """Dimensions + weights of one drafter, as the oracle sees them.

    shape: any object with hidden, n_layers, n_q_heads, n_kv_heads, head_dim,
    inter, vocab, n_feats, bf16, rope_theta, eps.
    weights: dict name -> numpy array (uint16 bf16 bits or float32), names as
    in synth.configs.weight_names.
    """

    def __init__(self, shape, weights: dict):
        self.shape = shape
        self.bf16 = bool(shape.bf16)
        exp_dt = np.uint16 if self.bf16 else np.float32
        self._keep = {}
        for k, a in weights.items():
            a = np.ascontiguousarray(a)
            assert a.dtype == exp_dt, (k, a.dtype)
            self._keep[k] = a
        self.dims = Dims(shape.hidden, shape.n_layers, shape.n_q_heads, shape.n_kv_heads,
                         shape.head_dim, shape.inter, shape.vocab, shape.n_feats,
                         1 if self.bf16 else 0, 0, float(shape.rope_theta), float(shape.eps))
        w = Weights()
        for k in ("fc_w", "fc_norm", "embed", "lm_head", "final_norm"):
            setattr(w, k, _p(self._keep[k]))
        for l in range(shape.n_layers):
            for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
                getattr(w, k)[l] = _p(self._keep[f"l{l}.{k}"])
        self.w = w

    def _dtype_check(self, a):
        a = np.ascontiguousarray(a)
        assert a.dtype == (np.uint16 if self.bf16 else np.float32), a.dtype
        return a

    def inject(self, hidden, pos):
        """hidden [n][n_feats*D], pos [n] -> (k, v) [n][n_layers][Hkv][dh] float64."""
        s = self.shape
        hidden = self._dtype_check(hidden)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        n = pos.shape[0]
        assert hidden.shape == (n, s.n_feats * s.hidden)
        k = np.empty((n, s.n_layers, s.n_kv_heads, s.head_dim))
        v = np.empty_like(k)
        _load().oracle_inject(ctypes.byref(self.dims), ctypes.byref(self.w), _p(hidden),
                              _p(pos), n, _p(k), _p(v))
        return k, v

    def draft(self, ctx_k, ctx_v, L, tokens):
        """ctx_k/v [n_layers][>=L][Hkv][dh] (model dtype); tokens [gamma]
        -> (logits [gamma][V] float64, block [gamma] int32)."""
        s = self.shape
        ctx_k = self._dtype_check(ctx_k)
        ctx_v = self._dtype_check(ctx_v)
        assert ctx_k.shape[0] == s.n_layers and ctx_k.shape[2:] == (s.n_kv_heads, s.head_dim)
        assert ctx_v.shape == ctx_k.shape
        Lbuf = ctx_k.shape[1]
        assert Lbuf >= L
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        g = tokens.shape[0]
        logits = np.empty((g, s.vocab))
        block = np.empty(g, dtype=np.int32)
        _load().oracle_draft(ctypes.byref(self.dims), ctypes.byref(self.w), _p(ctx_k), _p(ctx_v),
                             int(L), int(Lbuf), _p(tokens), g, _p(logits), _p(block))
        return logits, block

    def forward(self, ctx_k, ctx_v, L, tokens, pos, visible):
        """General forward of R rows: tokens [R], pos [R], visible [R][L+R]
        over [context keys 0..L) ++ [the rows' keys] -> logits [R][V]."""
        s = self.shape
        ctx_k = self._dtype_check(ctx_k)
        ctx_v = self._dtype_check(ctx_v)
        Lbuf = ctx_k.shape[1]
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        R = tokens.shape[0]
        visible = np.ascontiguousarray(visible, dtype=np.uint8)
        assert visible.shape == (R, L + R)
        logits = np.empty((R, s.vocab))
        _load().oracle_forward(ctypes.byref(self.dims), ctypes.byref(self.w), _p(tokens), _p(pos),
                               R, _p(ctx_k), _p(ctx_v), int(L), int(Lbuf), _p(visible),
                               _p(logits))
        return logits

    def draft_packed(self, ctx_k, ctx_v, tokens, anchors_pos):
        """Packed multi-block forward: tokens [n_blocks][gamma],
        anchors_pos [n_blocks] -> logits [n_blocks*gamma][V]."""
        s = self.shape
        ctx_k = self._dtype_check(ctx_k)
        ctx_v = self._dtype_check(ctx_v)
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        anchors_pos = np.ascontiguousarray(anchors_pos, dtype=np.int32)
        nb, g = tokens.shape
        logits = np.empty((nb * g, s.vocab))
        _load().oracle_draft_packed(ctypes.byref(self.dims), ctypes.byref(self.w), _p(ctx_k),
                                    _p(ctx_v), ctx_k.shape[1], _p(tokens), _p(anchors_pos),
                                    nb, g, _p(logits))
        return logits


def verify(block, target, tgt_bf16: bool):
    """block [gamma] int, target [gamma][V] (uint16 bf16 bits or float32)
    -> (tau, out_tokens [gamma], target_argmax [gamma])."""
    block = np.ascontiguousarray(block, dtype=np.int32)
    target = np.ascontiguousarray(target)
    assert target.dtype == (np.uint16 if tgt_bf16 else np.float32)
    g, V = target.shape
    out = np.empty(g, dtype=np.int32)
    T = np.empty(g, dtype=np.int32)
    tau = _load().oracle_verify(_p(block), _p(target), 1 if tgt_bf16 else 0, g, V, _p(out), _p(T))
    return tau, out, T


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Set the oracle's OpenMP thread count (its results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def round_bf16(x):
    f = _load().oracle_round_bf16
    return np.vectorize(lambda v: f(float(v)), otypes=[np.float64])(np.asarray(x, dtype=np.float64))


def rmsnorm(x, g, eps):
    x = _f64(x)
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty_like(x)
    _load().oracle_rmsnorm(_p(x), x.shape[0], _p(g), 0, float(eps), _p(out))
    return out


def rope(x, heads, dh, pos, theta):
    x = _f64(x).copy()
    _load().oracle_rope(_p(x), int(heads), int(dh), float(pos), float(theta))
    return x


def argmax(row):
    row = _f64(row)
    return _load().oracle_argmax(_p(row), row.shape[0])


def attention_dense(q, k, v, visible):
    q, k, v = _f64(q), _f64(k), _f64(v)
    visible = np.ascontiguousarray(visible, dtype=np.uint8)
    nq, dh = q.shape
    nk = k.shape[0]
    o = np.empty((nq, dh))
    _load().oracle_attention_dense(_p(q), nq, _p(k), _p(v), nk, dh, _p(visible), _p(o))
    return o


def swiglu(w_gate, w_up, w_down, z):
    """fp32 weights: W_gate, W_up [I][D], W_down [D][I]; z [R][D] -> [R][D]."""
    w_gate, w_up, w_down = (np.ascontiguousarray(a, dtype=np.float32) for a in (w_gate, w_up, w_down))
    z = _f64(z)
    R, D = z.shape
    I = w_gate.shape[0]
    out = np.empty((R, D))
    _load().oracle_swiglu(_p(w_gate), _p(w_up), _p(w_down), 0, D, I, _p(z), R, _p(out))
    return out


def loss_weights(gamma_decay, K):
    w = np.empty(int(K))
    _load().oracle_loss_weights(float(gamma_decay), int(K), _p(w))
    return w


def weighted_ce(logits, targets, w):
    logits = _f64(logits)
    targets = np.ascontiguousarray(targets, dtype=np.int32)
    w = _f64(w)
    K, V = logits.shape
    return _load().oracle_weighted_ce(_p(logits), _p(targets), _p(w), K, V)
