"""ctypes declarations mirroring include/dflash.h."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB points the loader at another build (the sanitizer test's)
LIB_PATH = os.environ.get("DFLASH_LIB") or os.path.join(HERE, "libdflash.so")

DFLASH_OK = 0
STATUS_NAMES = {0: "DFLASH_OK", -1: "DFLASH_E_INVAL", -2: "DFLASH_E_SHAPE", -3: "DFLASH_E_DTYPE",
                -4: "DFLASH_E_CAPACITY", -5: "DFLASH_E_HIP", -6: "DFLASH_E_DEVICE"}
DFLASH_F32, DFLASH_BF16 = 0, 1
DEVERR_PAGE, DEVERR_POS, DEVERR_TOKEN, DEVERR_XCD = 1, 2, 4, 8
MAX_LAYERS = 16
MAX_BLOCK = 16
STATE_BYTES = 16384

EXPORTED = ["dflash_model_create", "dflash_model_destroy", "dflash_workspace_bytes",
            "dflash_packed_weight_bytes", "dflash_pack_weights",
            "dflash_inject_ctx", "dflash_draft_block", "dflash_draft_block_noalloc",
            "dflash_verify_greedy",
            "dflash_draft_block_sampled", "dflash_verify_greedy_workspace_bytes",
            "dflash_verify_stochastic_workspace_bytes",
            "dflash_verify_stochastic", "dflash_packed_workspace_bytes", "dflash_packed_forward",
            "dflash_ar_workspace_bytes", "dflash_draft_block_ar",
            "dflash_last_error", "dflash_device_error", "dflash_profile_enable",
            "dflash_profile_read", "dflash_read_calibration"]


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("n_target_feats", ctypes.c_int32),
                ("max_block", ctypes.c_int32), ("mask_token_id", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class Weights(ctypes.Structure):
    _fields_ = [("fc_w", ctypes.c_void_p), ("fc_norm", ctypes.c_void_p),
                ("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layer", LayerWeights * MAX_LAYERS)]


class KV(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("n_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("ctx_lens", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libdflash.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with block_diffusion_drafter_fc_amd.build"
                          " (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    lib.dflash_model_create.argtypes = [P(Config), P(Weights), vp, P(vp)]
    lib.dflash_model_create.restype = ctypes.c_int
    lib.dflash_model_destroy.argtypes = [vp]
    lib.dflash_model_destroy.restype = None
    lib.dflash_workspace_bytes.argtypes = [vp, i32, i32, i32, i32]
    lib.dflash_workspace_bytes.restype = sz
    lib.dflash_packed_weight_bytes.argtypes = [vp]
    lib.dflash_packed_weight_bytes.restype = sz
    lib.dflash_pack_weights.argtypes = [vp, vp, sz, vp]
    lib.dflash_pack_weights.restype = ctypes.c_int
    lib.dflash_inject_ctx.argtypes = [vp, P(KV), vp, vp, i32, i32, vp, sz, vp]
    lib.dflash_inject_ctx.restype = ctypes.c_int
    lib.dflash_draft_block.argtypes = [vp, P(KV), vp, i32, i32, vp, vp, vp, sz, vp]
    lib.dflash_draft_block.restype = ctypes.c_int
    lib.dflash_read_calibration.argtypes = [vp, sz, vp, i32, vp]
    lib.dflash_read_calibration.restype = ctypes.c_int
    lib.dflash_draft_block_noalloc.argtypes = [vp, P(KV), vp, i32, i32, vp, vp, vp]
    lib.dflash_draft_block_noalloc.restype = ctypes.c_int
    lib.dflash_verify_greedy.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.dflash_verify_greedy.restype = ctypes.c_int
    lib.dflash_draft_block_sampled.argtypes = [vp, P(KV), vp, i32, i32, ctypes.c_uint64, vp, vp,
                                               vp, sz, vp]
    lib.dflash_draft_block_sampled.restype = ctypes.c_int
    lib.dflash_verify_greedy_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dflash_verify_greedy_workspace_bytes.restype = sz
    lib.dflash_verify_stochastic_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dflash_verify_stochastic_workspace_bytes.restype = sz
    lib.dflash_verify_stochastic.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, vp, vp, vp, sz,
                                             vp]
    lib.dflash_verify_stochastic.restype = ctypes.c_int
    lib.dflash_packed_workspace_bytes.argtypes = [vp, i32, i32, i32]
    lib.dflash_packed_workspace_bytes.restype = sz
    lib.dflash_packed_forward.argtypes = [vp, P(KV), vp, vp, i32, i32, vp, ctypes.c_float, vp, vp,
                                          vp, vp, vp, sz, vp]
    lib.dflash_packed_forward.restype = ctypes.c_int
    lib.dflash_ar_workspace_bytes.argtypes = [vp, i32, i32, i32]
    lib.dflash_ar_workspace_bytes.restype = sz
    lib.dflash_draft_block_ar.argtypes = [vp, P(KV), vp, i32, i32, vp, vp, vp, sz, vp]
    lib.dflash_draft_block_ar.restype = ctypes.c_int
    lib.dflash_last_error.argtypes = []
    lib.dflash_last_error.restype = ctypes.c_char_p
    lib.dflash_device_error.argtypes = [vp, vp, P(i32)]
    lib.dflash_device_error.restype = ctypes.c_int
    lib.dflash_profile_enable.argtypes = [vp, i32]
    lib.dflash_profile_enable.restype = ctypes.c_int
    lib.dflash_profile_read.argtypes = [vp, P(ctypes.c_double), P(i64), i32]
    lib.dflash_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib
