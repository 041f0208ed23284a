"""DFlash draft hot path on MI355X (gfx950): thin Python binding of libdflash.so.

The three calls of one speculative cycle -- context injection, the
single-pass block draft and greedy verification -- run entirely in the HIP
kernels of libdflash.so.  This module only marshals arguments: it checks that
tensors are CUDA-resident and contiguous, passes their data pointers, the
current HIP stream and the sizes through the C ABI declared in
include/dflash.h, and raises DFlashError for a non-OK status.  PyTorch is used
for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import dataclasses

from . import _abi
from ._abi import (DEVERR_PAGE, DEVERR_POS, DEVERR_TOKEN, DEVERR_XCD, DFLASH_BF16, DFLASH_F32,
                   MAX_BLOCK, MAX_LAYERS, STATE_BYTES)

__all__ = ["DFlashError", "DrafterConfig", "Drafter", "KVCache", "verify_greedy",
           "verify_greedy_workspace_bytes",
           "verify_stochastic", "verify_stochastic_workspace_bytes", "load_library",
           "read_calibration",
           "DEVERR_PAGE", "DEVERR_POS", "DEVERR_TOKEN", "DEVERR_XCD", "MAX_BLOCK", "MAX_LAYERS"]

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")
GLOBAL_KEYS = ("fc_w", "fc_norm", "embed", "lm_head", "final_norm")


def load_library():
    return _abi.load()


class DFlashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_abi.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(rc: int):
    if rc != _abi.DFLASH_OK:
        raise DFlashError(rc, _abi.load().dflash_last_error().decode(errors="replace"))


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


@dataclasses.dataclass
class DrafterConfig:
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_target_feats: int = 5
    max_block: int = 16
    mask_token_id: int | None = None     # default: vocab - 1
    page_size: int = 16
    dtype: str = "bf16"                  # "bf16" or "f32"
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def to_c(self) -> _abi.Config:
        mask = self.vocab - 1 if self.mask_token_id is None else self.mask_token_id
        return _abi.Config(self.hidden, self.n_layers, self.n_q_heads, self.n_kv_heads,
                           self.head_dim, self.intermediate, self.vocab, self.n_target_feats,
                           self.max_block, mask, self.page_size,
                           DFLASH_BF16 if self.dtype == "bf16" else DFLASH_F32,
                           float(self.rope_theta), float(self.rms_eps))


class KVCache:
    """Paged draft cache: pages [n_layers][n_pages][2][Hkv][page_size][dh],
    page_table int32 [batch][max_pages_per_seq], ctx_lens int32 [batch]."""

    def __init__(self, pages, page_table, ctx_lens):
        import torch
        self.pages, self.page_table, self.ctx_lens = pages, page_table, ctx_lens
        _dev_ptr(pages, "pages")
        _dev_ptr(page_table, "page_table", torch.int32)
        _dev_ptr(ctx_lens, "ctx_lens", torch.int32)
        if pages.dim() != 6 or page_table.dim() != 2 or ctx_lens.dim() != 1:
            raise ValueError("KVCache: pages must be 6-D, page_table 2-D, ctx_lens 1-D")
        self.c = _abi.KV(pages.data_ptr(), pages.shape[1], page_table.shape[1],
                         page_table.data_ptr(), ctx_lens.data_ptr())

    @property
    def batch(self):
        return self.page_table.shape[0]

    @property
    def max_pages_per_seq(self):
        return self.page_table.shape[1]


class Drafter:
    """A drafter whose weights live in device tensors (names: fc_w, fc_norm,
    embed, lm_head, final_norm and l{i}.{attn_norm, wq, wk, wv, wo, mlp_norm,
    w_gate, w_up, w_down})."""

    def __init__(self, cfg: DrafterConfig, weights: dict, pack: bool = True):
        import torch
        self.lib = _abi.load()
        self.cfg = cfg
        dt = cfg.torch_dtype()
        self._weights = weights
        w = _abi.Weights()
        for k in GLOBAL_KEYS:
            setattr(w, k, _dev_ptr(weights[k], k, dt).value)
        if cfg.n_layers > MAX_LAYERS:
            raise ValueError(f"at most {MAX_LAYERS} layers")
        for l in range(cfg.n_layers):
            for k in LAYER_KEYS:
                setattr(w.layer[l], k, _dev_ptr(weights[f"l{l}.{k}"], f"l{l}.{k}", dt).value)
        dev = weights["embed"].device
        self.state = torch.zeros(STATE_BYTES, dtype=torch.uint8, device=dev)
        self._c_cfg = cfg.to_c()
        self._c_w = w
        h = ctypes.c_void_p()
        _check(self.lib.dflash_model_create(ctypes.byref(self._c_cfg), ctypes.byref(w),
                                            ctypes.c_void_p(self.state.data_ptr()), ctypes.byref(h)))
        self.handle = h
        self.packed = None
        nbytes = self.lib.dflash_packed_weight_bytes(self.handle)
        if pack and nbytes:
            # weights in matrix-core tile order for the <= 64-row products
            self.packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            stream = torch.cuda.current_stream(dev).cuda_stream
            _check(self.lib.dflash_pack_weights(self.handle, ctypes.c_void_p(self.packed.data_ptr()),
                                                nbytes, ctypes.c_void_p(stream)))

    def close(self):
        if getattr(self, "handle", None):
            self.lib.dflash_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, max_batch, max_block, max_new_tokens, max_pages_per_seq) -> int:
        n = self.lib.dflash_workspace_bytes(self.handle, max_batch, max_block, max_new_tokens,
                                            max_pages_per_seq)
        if n == 0:
            raise DFlashError(-1, "workspace_bytes: invalid arguments")
        return int(n)

    def inject(self, kv: KVCache, hidden, cu_new, workspace, stream=None):
        import torch
        n_tok = int(hidden.shape[0]) if hidden is not None else 0
        _check(self.lib.dflash_inject_ctx(
            self.handle, ctypes.byref(kv.c), _dev_ptr(hidden, "hidden", self.cfg.torch_dtype()),
            _dev_ptr(cu_new, "cu_new", torch.int32), int(cu_new.numel()) - 1, n_tok,
            _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream)))

    def draft(self, kv: KVCache, anchor, block_size, block_tokens, workspace, logits=None,
              stream=None):
        import torch
        _check(self.lib.dflash_draft_block(
            self.handle, ctypes.byref(kv.c), _dev_ptr(anchor, "anchor", torch.int32),
            int(anchor.numel()), int(block_size), _dev_ptr(block_tokens, "block_tokens", torch.int32),
            _dev_ptr(logits, "logits", torch.float32), _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)))

    def draft_noalloc(self, kv: KVCache, anchor, block_size, block_tokens, logits=None,
                      stream=None):
        """dflash_draft_block_noalloc: the draft with the library's static
        per-GPU scratch instead of a workspace (allocates nothing)."""
        import torch
        _check(self.lib.dflash_draft_block_noalloc(
            self.handle, ctypes.byref(kv.c), _dev_ptr(anchor, "anchor", torch.int32),
            int(anchor.numel()), int(block_size), _dev_ptr(block_tokens, "block_tokens", torch.int32),
            _dev_ptr(logits, "logits", torch.float32), _stream(stream)))

    def draft_sampled(self, kv: KVCache, anchor, block_size, seed, block_tokens, logits,
                      workspace, stream=None):
        """dflash_draft_block_sampled: proposals drawn by Gumbel-max from the
        drafter's logits with the counter stream of `seed` (logits required)."""
        import torch
        if logits is None:
            raise ValueError("draft_sampled: logits are required")
        _check(self.lib.dflash_draft_block_sampled(
            self.handle, ctypes.byref(kv.c), _dev_ptr(anchor, "anchor", torch.int32),
            int(anchor.numel()), int(block_size), int(seed) & ((1 << 64) - 1),
            _dev_ptr(block_tokens, "block_tokens", torch.int32),
            _dev_ptr(logits, "logits", torch.float32), _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)))

    def packed_workspace_bytes(self, max_blocks, max_block, max_pages_per_seq) -> int:
        n = self.lib.dflash_packed_workspace_bytes(self.handle, max_blocks, max_block,
                                                   max_pages_per_seq)
        if n == 0:
            raise DFlashError(-1, "packed_workspace_bytes: invalid arguments")
        return int(n)

    def packed_forward(self, ctx: KVCache, anchors, anchor_pos, block_size, logits, workspace,
                       targets=None, decay=7.0, block_tokens=None, block_loss=None, loss=None,
                       stream=None):
        """dflash_packed_forward: the blocks of one sequence (ctx has batch 1)
        in one pass, with the weighted cross-entropy when targets is given."""
        import torch
        _check(self.lib.dflash_packed_forward(
            self.handle, ctypes.byref(ctx.c), _dev_ptr(anchors, "anchors", torch.int32),
            _dev_ptr(anchor_pos, "anchor_pos", torch.int32), int(anchors.numel()),
            int(block_size), _dev_ptr(targets, "targets", torch.int32), float(decay),
            _dev_ptr(logits, "logits", torch.float32),
            _dev_ptr(block_tokens, "block_tokens", torch.int32),
            _dev_ptr(block_loss, "block_loss", torch.float32),
            _dev_ptr(loss, "loss", torch.float32), _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)))

    def ar_workspace_bytes(self, max_batch, max_block, max_pages_per_seq) -> int:
        n = self.lib.dflash_ar_workspace_bytes(self.handle, max_batch, max_block, max_pages_per_seq)
        if n == 0:
            raise DFlashError(-1, "ar_workspace_bytes: invalid arguments")
        return int(n)

    def draft_ar(self, kv: KVCache, anchor, block_size, block_tokens, workspace, logits=None,
                 stream=None):
        """dflash_draft_block_ar: block_size - 1 causal passes, one token each."""
        import torch
        _check(self.lib.dflash_draft_block_ar(
            self.handle, ctypes.byref(kv.c), _dev_ptr(anchor, "anchor", torch.int32),
            int(anchor.numel()), int(block_size), _dev_ptr(block_tokens, "block_tokens", torch.int32),
            _dev_ptr(logits, "logits", torch.float32), _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)))

    def device_error(self, stream=None) -> int:
        code = ctypes.c_int32(0)
        rc = self.lib.dflash_device_error(self.handle, _stream(stream), ctypes.byref(code))
        if rc not in (0, -6):
            _check(rc)
        return int(code.value)

    def profile_enable(self, on: bool = True):
        _check(self.lib.dflash_profile_enable(self.handle, 1 if on else 0))

    def profile_read(self, reset: bool = False):
        ms = ctypes.c_double(0.0)
        cnt = ctypes.c_int64(0)
        _check(self.lib.dflash_profile_read(self.handle, ctypes.byref(ms), ctypes.byref(cnt),
                                            1 if reset else 0))
        return ms.value, cnt.value


def verify_greedy(block_tokens, target_logits, accept_len, out_tokens, workspace,
                  target_argmax=None, stream=None):
    """Greedy verification through dflash_verify_greedy.  block_tokens int32
    [B][gamma]; target_logits [B][gamma][V] bf16 or fp32."""
    import torch
    lib = _abi.load()
    if target_logits.dtype == torch.bfloat16:
        dt = DFLASH_BF16
    elif target_logits.dtype == torch.float32:
        dt = DFLASH_F32
    else:
        raise ValueError("target_logits must be bf16 or fp32")
    B, gamma = block_tokens.shape
    _check(lib.dflash_verify_greedy(
        _dev_ptr(block_tokens, "block_tokens", torch.int32), _dev_ptr(target_logits, "target_logits"),
        dt, int(B), int(gamma), int(target_logits.shape[-1]),
        _dev_ptr(accept_len, "accept_len", torch.int32), _dev_ptr(out_tokens, "out_tokens", torch.int32),
        _dev_ptr(target_argmax, "target_argmax", torch.int32), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def read_calibration(src, out, workgroups=512, stream=None):
    """dflash_read_calibration: stream all of `src` (a device tensor, size a
    multiple of 16 bytes) with the LM head's load pattern; `out` receives
    16 bytes per workgroup."""
    lib = _abi.load()
    nbytes = src.numel() * src.element_size()
    if out.numel() * out.element_size() < 16 * workgroups:
        raise ValueError("read_calibration: out needs 16 bytes per workgroup")
    _check(lib.dflash_read_calibration(_dev_ptr(src, "src"), nbytes, _dev_ptr(out, "out"),
                                       int(workgroups), _stream(stream)))


def verify_greedy_workspace_bytes(batch, block_size, vocab) -> int:
    n = _abi.load().dflash_verify_greedy_workspace_bytes(int(batch), int(block_size), int(vocab))
    if n == 0:
        raise DFlashError(-1, "verify_greedy_workspace_bytes: invalid arguments")
    return int(n)


def verify_stochastic_workspace_bytes(batch, block_size, vocab) -> int:
    n = _abi.load().dflash_verify_stochastic_workspace_bytes(int(batch), int(block_size), int(vocab))
    if n == 0:
        raise DFlashError(-1, "verify_stochastic_workspace_bytes: invalid arguments")
    return int(n)


def verify_stochastic(block_tokens, draft_logits, target_logits, uniforms, accept_len, out_tokens,
                      workspace, stream=None):
    """Lossless verification through dflash_verify_stochastic.  block_tokens
    int32 [B][gamma]; draft_logits fp32 and target_logits bf16 or fp32
    [B][gamma][V]; uniforms fp32 [B][gamma]."""
    import torch
    lib = _abi.load()
    if target_logits.dtype == torch.bfloat16:
        dt = DFLASH_BF16
    elif target_logits.dtype == torch.float32:
        dt = DFLASH_F32
    else:
        raise ValueError("target_logits must be bf16 or fp32")
    B, gamma = block_tokens.shape
    _check(lib.dflash_verify_stochastic(
        _dev_ptr(block_tokens, "block_tokens", torch.int32),
        _dev_ptr(draft_logits, "draft_logits", torch.float32),
        _dev_ptr(target_logits, "target_logits"), dt,
        _dev_ptr(uniforms, "uniforms", torch.float32), int(B), int(gamma),
        int(target_logits.shape[-1]), _dev_ptr(accept_len, "accept_len", torch.int32),
        _dev_ptr(out_tokens, "out_tokens", torch.int32), _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
