"""Python binding of libtalker_moe.so (ctypes): argument marshalling only.

Every function has the name of the C entry point it calls and takes torch
tensors that live on the GPU; torch supplies device memory and the current HIP
stream, all arithmetic runs in the library's kernels.  Outputs not passed in
are allocated with ``torch.empty``.  A nonzero status raises :class:`MoeError`.

Loading fails loudly when the library has not been built; there is no CPU or
PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtalker_moe.so")

MOE_F32, MOE_BF16 = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP"}

EXPORTS = ("moe_status_string", "moe_check_config", "moe_workspace_size", "moe_route", "moe_permute",
           "moe_grouped_swiglu", "moe_shared_swiglu", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_timed", "moe_rmsnorm",
           "moe_codec_head_argmax", "moe_codec_head_workspace_size", "moe_stack_forward",
           "moe_stack_workspace_size", "moe_codec_head_sample", "moe_attention_decode",
           "moe_attention_workspace_size", "moe_predictor_frame", "moe_predictor_workspace_size",
           "moe_talker_decode", "moe_talker_decode_workspace_size", "moe_layer_forward_static",
           "moe_talker_frame", "moe_talker_frame_workspace_size")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), text))
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_experts_per_tok", ctypes.c_int32), ("moe_intermediate_size", ctypes.c_int32),
                ("shared_expert_intermediate_size", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class moe_attn_config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_sections", ctypes.c_int32 * 3), ("rope_theta", ctypes.c_float),
                ("eps", ctypes.c_float), ("max_len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class moe_attn_weights(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p)]


@dataclasses.dataclass
class AttnConfig:
    """The attention shape (defaults: the Talker's 16 query / 2 KV heads of 128, TM-RoPE 24/20/20)."""
    max_len: int
    hidden_size: int = 1024
    num_heads: int = 16
    num_kv_heads: int = 2
    head_dim: int = 128
    rope_sections: tuple = (24, 20, 20)
    rope_theta: float = 1.0e6
    eps: float = 1e-6

    def c(self) -> moe_attn_config:
        return moe_attn_config(self.hidden_size, self.num_heads, self.num_kv_heads, self.head_dim,
                               (ctypes.c_int32 * 3)(*self.rope_sections), self.rope_theta, self.eps, self.max_len,
                               MOE_BF16)


class moe_predictor_config(ctypes.Structure):
    _fields_ = [("attn", moe_attn_config), ("num_layers", ctypes.c_int32), ("intermediate_size", ctypes.c_int32),
                ("num_codes", ctypes.c_int32), ("codebook_size", ctypes.c_int32), ("c0_vocab", ctypes.c_int32),
                ("eps", ctypes.c_float)]


class moe_predictor_layer(ctypes.Structure):
    _fields_ = [("attn", moe_attn_weights), ("in_norm", ctypes.c_void_p), ("post_norm", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


class moe_predictor_weights(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(moe_predictor_layer)), ("final_norm", ctypes.c_void_p),
                ("c0_embedding", ctypes.c_void_p), ("codec_embedding", ctypes.c_void_p), ("lm_head", ctypes.c_void_p)]


@dataclasses.dataclass
class PredictorConfig:
    """The depth code predictor (defaults: 5 layers, 16 query / 8 KV heads, MLP 3072, 16 codes of 2048, c_0
    vocabulary 3072)."""
    num_layers: int = 5
    hidden_size: int = 1024
    num_heads: int = 16
    num_kv_heads: int = 8
    intermediate_size: int = 3072
    num_codes: int = 16
    codebook_size: int = 2048
    c0_vocab: int = 3072
    eps: float = 1e-6
    rope_sections: tuple = (24, 20, 20)
    rope_theta: float = 1.0e6

    def c(self) -> moe_predictor_config:
        a = AttnConfig(max_len=32, hidden_size=self.hidden_size, num_heads=self.num_heads,
                       num_kv_heads=self.num_kv_heads, rope_sections=self.rope_sections, rope_theta=self.rope_theta,
                       eps=self.eps)
        return moe_predictor_config(a.c(), self.num_layers, self.intermediate_size, self.num_codes,
                                    self.codebook_size, self.c0_vocab, self.eps)


class moe_weights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p),
                ("shared_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p)]


class moe_talker_layer(ctypes.Structure):
    _fields_ = [("moe", moe_weights), ("attn", moe_attn_weights), ("in_norm", ctypes.c_void_p),
                ("post_norm", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


@dataclasses.dataclass(frozen=True)
class Config:
    """Layer configuration (field names as in the model configuration)."""
    hidden_size: int
    num_experts: int
    num_experts_per_tok: int
    moe_intermediate_size: int
    shared_expert_intermediate_size: int
    norm_topk_prob: bool = True
    dtype: torch.dtype = torch.bfloat16

    def c(self) -> moe_config:
        if self.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dtype must be torch.bfloat16 or torch.float32")
        return moe_config(self.hidden_size, self.num_experts, self.num_experts_per_tok,
                          self.moe_intermediate_size, self.shared_expert_intermediate_size,
                          1 if self.norm_topk_prob else 0,
                          MOE_BF16 if self.dtype == torch.bfloat16 else MOE_F32)


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it is missing: build it first."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libtalker_moe.so not found at %s; build it with "
                           "`python -m sparse_moe_transformer_talker_amd.build`" % p)
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(moe_config)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_check_config": (ctypes.c_int, [cfgp]),
        "moe_workspace_size": (sz, [cfgp, i64]),
        "moe_route": (ctypes.c_int, [cfgp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "moe_permute": (ctypes.c_int, [cfgp, vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_grouped_swiglu": (ctypes.c_int, [cfgp, vp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp]),
        "moe_shared_swiglu": (ctypes.c_int, [cfgp, vp, i64, vp, vp, vp, vp, vp, sz, vp]),
        "moe_combine": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, i64, vp, vp]),
        "moe_layer_forward": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), vp, vp, i64, vp, vp, vp, vp,
                                             vp, sz, vp]),
        "moe_layer_forward_timed": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), vp, vp, i64, vp, vp, vp,
                                                   vp, vp, sz, vp, ctypes.POINTER(vp)]),
        "moe_layer_forward_static": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), vp, vp, i64, vp, vp, vp,
                                                    vp, vp]),
        "moe_rmsnorm": (ctypes.c_int, [cfgp, vp, vp, ctypes.c_float, i64, vp, vp]),
        "moe_codec_head_argmax": (ctypes.c_int, [cfgp, vp, vp, i32, i64, vp, vp, vp, sz, vp]),
        "moe_codec_head_workspace_size": (sz, [cfgp, i32, i64]),
        "moe_stack_forward": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), i32, vp, i64, vp, ctypes.c_float,
                                             vp, i32, vp, vp, vp, vp, sz, vp]),
        "moe_stack_workspace_size": (sz, [cfgp, i64, i32]),
        "moe_codec_head_sample": (ctypes.c_int, [cfgp, vp, vp, i32, i64, ctypes.c_float, vp, vp, vp, vp, sz, vp]),
        "moe_attention_decode": (ctypes.c_int, [ctypes.POINTER(moe_attn_config), ctypes.POINTER(moe_attn_weights),
                                                vp, i64, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, sz, vp]),
        "moe_attention_workspace_size": (sz, [ctypes.POINTER(moe_attn_config), i64]),
        "moe_predictor_frame": (ctypes.c_int, [ctypes.POINTER(moe_predictor_config),
                                               ctypes.POINTER(moe_predictor_weights), vp, vp, i64, vp, vp, vp, sz,
                                               vp]),
        "moe_predictor_workspace_size": (sz, [ctypes.POINTER(moe_predictor_config), i64]),
        "moe_talker_decode": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_attn_config), ctypes.POINTER(moe_talker_layer),
                                             i32, vp, i64, vp, vp, vp, ctypes.c_float, vp, i32, vp, vp, vp, vp, sz,
                                             vp]),
        "moe_talker_decode_workspace_size": (sz, [cfgp, ctypes.POINTER(moe_attn_config), i64, i32]),
        "moe_talker_frame": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_attn_config), ctypes.POINTER(moe_talker_layer),
                                            i32, vp, ctypes.c_float, vp, i32, ctypes.POINTER(moe_predictor_config),
                                            ctypes.POINTER(moe_predictor_weights), vp, i64, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]),
        "moe_talker_frame_workspace_size": (sz, [cfgp, ctypes.POINTER(moe_attn_config),
                                                 ctypes.POINTER(moe_predictor_config), i64, i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_cache: Dict[int, torch.Tensor] = {}


def workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """A cached device workspace of at least nbytes (one per device, stream-ordered use)."""
    dev = torch.device(device).index or 0
    buf = _ws_cache.get(dev)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=torch.device("cuda", dev))
        _ws_cache[dev] = buf
    return buf


def moe_check_config(cfg: Config) -> int:
    return load_library().moe_check_config(ctypes.byref(cfg.c()))


def moe_workspace_size(cfg: Config, T: int) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(cfg.c()), T))


def _ws(cfg: Config, T: int, device, ws: Optional[torch.Tensor]):
    n = moe_workspace_size(cfg, T)
    buf = ws if ws is not None else workspace(n, device)
    return buf, n if ws is None else buf.numel()


def moe_route(cfg: Config, x: torch.Tensor, router: torch.Tensor, bias: Optional[torch.Tensor] = None,
              want_probs: bool = False, topk_idx=None, topk_w=None, probs=None, ws=None):
    """Router + softmax + exact Top-k + renormalisation.  Returns (idx, w, probs or None)."""
    T = x.shape[0]
    k, E = cfg.num_experts_per_tok, cfg.num_experts
    dev = x.device
    topk_idx = topk_idx if topk_idx is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = topk_w if topk_w is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    if want_probs and probs is None:
        probs = torch.empty((T, E), dtype=torch.float32, device=dev)
    buf, n = _ws(cfg, T, dev, ws)
    _check("moe_route", load_library().moe_route(
        ctypes.byref(cfg.c()), _ptr(x), _ptr(router), _ptr(bias), T, _ptr(topk_idx), _ptr(topk_w), _ptr(probs),
        _ptr(buf), n, _stream(dev)))
    return topk_idx, topk_w, probs


def moe_permute(cfg: Config, topk_idx: torch.Tensor, x: Optional[torch.Tensor] = None, ws=None):
    """Stable grouping by expert.  Returns dict(counts, offsets, row_token, row_of[, x_perm])."""
    T, k = topk_idx.shape
    E, dev = cfg.num_experts, topk_idx.device
    out = {"counts": torch.empty(E, dtype=torch.int32, device=dev),
           "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "row_token": torch.empty(T * k, dtype=torch.int32, device=dev),
           "row_of": torch.empty((T, k), dtype=torch.int32, device=dev)}
    if x is not None:
        out["x_perm"] = torch.empty((T * k, x.shape[1]), dtype=x.dtype, device=dev)
    buf, n = _ws(cfg, T, dev, ws)
    _check("moe_permute", load_library().moe_permute(
        ctypes.byref(cfg.c()), _ptr(topk_idx), T, _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["row_token"]), _ptr(out["row_of"]), _ptr(x), _ptr(out.get("x_perm")), _ptr(buf), n,
        _stream(dev)))
    return out


def moe_grouped_swiglu(cfg: Config, x: torch.Tensor, row_token: Optional[torch.Tensor], offsets: torch.Tensor,
                       T: int, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor, y_perm=None, ws=None):
    """Routed experts on their grouped rows (unweighted).  Returns y_perm [T*k, H]."""
    dev = x.device
    y_perm = y_perm if y_perm is not None else torch.empty((T * cfg.num_experts_per_tok, cfg.hidden_size),
                                                           dtype=x.dtype, device=dev)
    buf, n = _ws(cfg, T, dev, ws)
    _check("moe_grouped_swiglu", load_library().moe_grouped_swiglu(
        ctypes.byref(cfg.c()), _ptr(x), _ptr(row_token), _ptr(offsets), T, _ptr(gate), _ptr(up), _ptr(down),
        _ptr(y_perm), _ptr(buf), n, _stream(dev)))
    return y_perm


def moe_shared_swiglu(cfg: Config, x: torch.Tensor, sg: torch.Tensor, su: torch.Tensor, sd: torch.Tensor,
                      y_shared=None, ws=None):
    """The shared expert on every token.  Returns y_shared [T, H]."""
    T, dev = x.shape[0], x.device
    y_shared = y_shared if y_shared is not None else torch.empty_like(x)
    buf, n = _ws(cfg, T, dev, ws)
    _check("moe_shared_swiglu", load_library().moe_shared_swiglu(
        ctypes.byref(cfg.c()), _ptr(x), T, _ptr(sg), _ptr(su), _ptr(sd), _ptr(y_shared), _ptr(buf), n,
        _stream(dev)))
    return y_shared


def moe_combine(cfg: Config, y_perm: torch.Tensor, row_of: torch.Tensor, topk_w: torch.Tensor,
                y_shared: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None, y=None):
    """Weighted combine of expert outputs (+ shared, + residual).  Returns y [T, H]."""
    T = row_of.shape[0]
    dev = y_perm.device
    y = y if y is not None else torch.empty((T, cfg.hidden_size), dtype=y_perm.dtype, device=dev)
    _check("moe_combine", load_library().moe_combine(
        ctypes.byref(cfg.c()), _ptr(y_perm), _ptr(row_of), _ptr(topk_w), _ptr(y_shared), _ptr(residual), T,
        _ptr(y), _stream(dev)))
    return y


def weights_struct(w: Dict[str, Optional[torch.Tensor]]) -> moe_weights:
    """moe_weights from a dict of device tensors (keys as in the C struct)."""
    p = lambda name: (None if w.get(name) is None else _ptr(w[name]))
    return moe_weights(p("router"), p("router_bias"), p("gate"), p("up"), p("down"), p("shared_gate"),
                       p("shared_up"), p("shared_down"))


def moe_layer_forward(cfg: Config, weights, x: torch.Tensor, residual: Optional[torch.Tensor] = None,
                      y=None, topk_idx=None, topk_w=None, counts=None, ws=None, stream=None, stage_events=None):
    """The whole MoE layer.  ``weights``: dict of device tensors or a prebuilt moe_weights.
    Returns y [T, H] (routing copies are written to the optional tensors).  With
    ``stage_events`` (up to 8 torch.cuda.Event or None: six stage boundaries, then
    the gate/up kernel's own start and end) it calls moe_layer_forward_timed."""
    T, dev = x.shape[0], x.device
    y = y if y is not None else torch.empty_like(x)
    ws_struct = weights if isinstance(weights, moe_weights) else weights_struct(weights)
    buf, n = _ws(cfg, T, dev, ws)
    st = stream if stream is not None else _stream(dev)
    lib = load_library()
    args = (ctypes.byref(cfg.c()), ctypes.byref(ws_struct), _ptr(x), _ptr(residual), T, _ptr(y), _ptr(topk_idx),
            _ptr(topk_w), _ptr(counts), _ptr(buf), n, st)
    if stage_events is None:
        _check("moe_layer_forward", lib.moe_layer_forward(*args))
    else:
        if len(stage_events) > 8:
            raise ValueError("at most 8 stage events")
        evs = (ctypes.c_void_p * 8)(*[None if e is None else e.cuda_event for e in stage_events])
        _check("moe_layer_forward_timed", lib.moe_layer_forward_timed(*args, evs))
    return y


# MOE_STATIC_SCRATCH_BYTES of include/talker_moe.h
STATIC_SCRATCH_BYTES = 8 << 20
MOE_ERR_SCRATCH = -5


def moe_layer_forward_static(cfg: Config, weights, x: torch.Tensor, residual: Optional[torch.Tensor] = None,
                             y=None, topk_idx=None, topk_w=None, counts=None, stream=None, check=True):
    """moe_layer_forward on the library's static per-GPU scratch (no workspace
    argument; the library allocates nothing).  Returns y, or the raw status when
    check is False."""
    T, dev = x.shape[0], x.device
    y = y if y is not None else torch.empty_like(x)
    ws_struct = weights if isinstance(weights, moe_weights) else weights_struct(weights)
    st = stream if stream is not None else _stream(dev)
    r = load_library().moe_layer_forward_static(ctypes.byref(cfg.c()), ctypes.byref(ws_struct), _ptr(x),
                                                _ptr(residual), T, _ptr(y), _ptr(topk_idx), _ptr(topk_w),
                                                _ptr(counts), st)
    if not check:
        return r
    _check("moe_layer_forward_static", r)
    return y


def moe_rmsnorm(cfg: Config, x: torch.Tensor, gain: torch.Tensor, eps: float = 1e-6, out=None):
    """Row RMSNorm.  Returns out [T, H]."""
    T, dev = x.shape[0], x.device
    out = out if out is not None else torch.empty_like(x)
    _check("moe_rmsnorm", load_library().moe_rmsnorm(
        ctypes.byref(cfg.c()), _ptr(x), _ptr(gain), eps, T, _ptr(out), _stream(dev)))
    return out


def moe_codec_head_argmax(cfg: Config, x: torch.Tensor, w_head: torch.Tensor, want_logits: bool = False,
                          c0=None, logits=None, ws=None):
    """codec_head + exact argmax.  Returns (c0 [T] int32, logits [T, V] fp32 or None)."""
    T, dev = x.shape[0], x.device
    V = w_head.shape[0]
    c0 = c0 if c0 is not None else torch.empty(T, dtype=torch.int32, device=dev)
    if want_logits and logits is None:
        logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    lib = load_library()
    need = int(lib.moe_codec_head_workspace_size(ctypes.byref(cfg.c()), V, T))
    buf = ws if ws is not None else workspace(need, dev)
    _check("moe_codec_head_argmax", lib.moe_codec_head_argmax(
        ctypes.byref(cfg.c()), _ptr(x), _ptr(w_head), V, T, _ptr(logits), _ptr(c0), _ptr(buf), buf.numel(),
        _stream(dev)))
    return c0, logits


def moe_codec_head_sample(cfg: Config, x: torch.Tensor, w_head: torch.Tensor, u: torch.Tensor,
                          temperature: float = 1.0, want_logits: bool = False, c0=None, logits=None, ws=None):
    """c_0 drawn from softmax(logits / temperature) with the uniforms u [T] (fp64).
    Returns (c0 [T] int32, logits [T, V] fp32 or None)."""
    T, dev = x.shape[0], x.device
    V = w_head.shape[0]
    if u.dtype != torch.float64 or u.numel() < T:
        raise ValueError("u must hold T float64 values")
    c0 = c0 if c0 is not None else torch.empty(T, dtype=torch.int32, device=dev)
    if want_logits and logits is None:
        logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    lib = load_library()
    need = int(lib.moe_codec_head_workspace_size(ctypes.byref(cfg.c()), V, T))
    buf = ws if ws is not None else workspace(need, dev)
    _check("moe_codec_head_sample", lib.moe_codec_head_sample(
        ctypes.byref(cfg.c()), _ptr(x), _ptr(w_head), V, T, temperature, _ptr(u), _ptr(logits), _ptr(c0),
        _ptr(buf), buf.numel(), _stream(dev)))
    return c0, logits


def moe_stack_workspace_size(cfg: Config, T: int, V: int = 0) -> int:
    return int(load_library().moe_stack_workspace_size(ctypes.byref(cfg.c()), T, V))


def moe_stack_forward(cfg: Config, layers, x: torch.Tensor, gains: Optional[torch.Tensor] = None,
                      eps: float = 1e-6, codec_head: Optional[torch.Tensor] = None, h_out=None, xn_out=None,
                      c0=None, want_c0: bool = True, ws=None, stream=None):
    """L stacked layers, then the final RMSNorm and (with ``codec_head``) the head
    argmax.  ``layers``: list of weight dicts or moe_weights; ``gains`` [L + 1, H]
    fp32.  Returns (h_out [T, H], xn_out [T, H] or None, c0 [T] int32 or None)."""
    T, dev = x.shape[0], x.device
    L = len(layers)
    arr = (moe_weights * max(L, 1))(*[w if isinstance(w, moe_weights) else weights_struct(w) for w in layers])
    h_out = h_out if h_out is not None else torch.empty_like(x)
    V = 0 if codec_head is None else codec_head.shape[0]
    if c0 is None and want_c0 and codec_head is not None:
        c0 = torch.empty(T, dtype=torch.int32, device=dev)
    lib = load_library()
    need = int(lib.moe_stack_workspace_size(ctypes.byref(cfg.c()), T, V if c0 is not None else 0))
    buf = ws if ws is not None else workspace(need, dev)
    st = stream if stream is not None else _stream(dev)
    _check("moe_stack_forward", lib.moe_stack_forward(
        ctypes.byref(cfg.c()), arr, L, _ptr(x), T, _ptr(gains), eps, _ptr(codec_head), V, _ptr(h_out),
        _ptr(xn_out), _ptr(c0), _ptr(buf), buf.numel(), st))
    return h_out, xn_out, c0


def moe_attention_workspace_size(acfg: AttnConfig, T: int) -> int:
    return int(load_library().moe_attention_workspace_size(ctypes.byref(acfg.c()), T))


def attn_weights_struct(w: Dict[str, torch.Tensor]) -> moe_attn_weights:
    return moe_attn_weights(_ptr(w["w_qkv"]), _ptr(w["q_norm"]), _ptr(w["k_norm"]), _ptr(w["w_o"]))


def moe_attention_decode(acfg: AttnConfig, weights, x: torch.Tensor, pos: torch.Tensor, cache_len: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, residual: Optional[torch.Tensor] = None,
                         y=None, norm_gain: Optional[torch.Tensor] = None, norm_eps: float = 1e-6, norm_out=None,
                         ws=None, stream=None):
    """One decode step of the attention block (caches updated in place).  Returns y [T, H]."""
    T, dev = x.shape[0], x.device
    y = y if y is not None else torch.empty_like(x)
    w = weights if isinstance(weights, moe_attn_weights) else attn_weights_struct(weights)
    lib = load_library()
    c = acfg.c()
    buf = ws if ws is not None else workspace(int(lib.moe_attention_workspace_size(ctypes.byref(c), T)), dev)
    st = stream if stream is not None else _stream(dev)
    _check("moe_attention_decode", lib.moe_attention_decode(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), T, _ptr(pos), _ptr(cache_len), _ptr(k_cache), _ptr(v_cache),
        _ptr(residual), _ptr(y), _ptr(norm_gain), norm_eps, _ptr(norm_out), _ptr(buf), buf.numel(), st))
    return y


def moe_predictor_workspace_size(pcfg: PredictorConfig, T: int) -> int:
    return int(load_library().moe_predictor_workspace_size(ctypes.byref(pcfg.c()), T))


def predictor_weights_struct(w: Dict) -> moe_predictor_weights:
    """moe_predictor_weights from device tensors: "layers" (dicts with w_qkv, q_norm, k_norm, w_o, in_norm,
    post_norm, gate, up, down), final_norm, c0_embedding, codec_embedding, lm_head.  The layer array is kept
    alive on the returned struct."""
    arr = (moe_predictor_layer * len(w["layers"]))(*[
        moe_predictor_layer(attn_weights_struct(l), _ptr(l["in_norm"]), _ptr(l["post_norm"]), _ptr(l["gate"]),
                            _ptr(l["up"]), _ptr(l["down"])) for l in w["layers"]])
    st = moe_predictor_weights(ctypes.cast(arr, ctypes.POINTER(moe_predictor_layer)), _ptr(w["final_norm"]),
                               _ptr(w["c0_embedding"]), _ptr(w["codec_embedding"]), _ptr(w["lm_head"]))
    st._layers = arr
    return st


def moe_predictor_frame(pcfg: PredictorConfig, weights, h_talker: torch.Tensor, c0: torch.Tensor, codes=None,
                        xn_out=None, ws=None, stream=None):
    """One frame of the depth code predictor.  Returns codes [num_codes, T] int32 (row 0 = c0)."""
    T, dev = h_talker.shape[0], h_talker.device
    codes = codes if codes is not None else torch.empty((pcfg.num_codes, T), dtype=torch.int32, device=dev)
    w = weights if isinstance(weights, moe_predictor_weights) else predictor_weights_struct(weights)
    lib = load_library()
    c = pcfg.c()
    buf = ws if ws is not None else workspace(int(lib.moe_predictor_workspace_size(ctypes.byref(c), T)), dev)
    st = stream if stream is not None else _stream(dev)
    _check("moe_predictor_frame", lib.moe_predictor_frame(ctypes.byref(c), ctypes.byref(w), _ptr(h_talker), _ptr(c0),
                                                          T, _ptr(codes), _ptr(xn_out), _ptr(buf), buf.numel(), st))
    return codes


def moe_talker_decode_workspace_size(cfg: Config, acfg: AttnConfig, T: int, V: int = 0) -> int:
    return int(load_library().moe_talker_decode_workspace_size(ctypes.byref(cfg.c()), ctypes.byref(acfg.c()), T, V))


def talker_layers_struct(layers) -> ctypes.Array:
    """A ctypes array of moe_talker_layer from dicts: "moe" (weight dict or moe_weights), "attn" (attention weight
    dict or moe_attn_weights), "in_norm", "post_norm" (nullable), "k_cache", "v_cache"."""
    mk = lambda w: w if isinstance(w, moe_weights) else weights_struct(w)
    ma = lambda w: w if isinstance(w, moe_attn_weights) else attn_weights_struct(w)
    return (moe_talker_layer * len(layers))(*[
        moe_talker_layer(mk(l["moe"]), ma(l["attn"]), _ptr(l.get("in_norm")), _ptr(l.get("post_norm")),
                         _ptr(l["k_cache"]), _ptr(l["v_cache"])) for l in layers])


def moe_talker_frame_workspace_size(cfg: Config, acfg: AttnConfig, pcfg: PredictorConfig, T: int, V: int) -> int:
    return int(load_library().moe_talker_frame_workspace_size(ctypes.byref(cfg.c()), ctypes.byref(acfg.c()),
                                                              ctypes.byref(pcfg.c()), T, V))


def moe_talker_frame(cfg: Config, acfg: AttnConfig, layers, final_norm, eps: float, codec_head: torch.Tensor,
                     pcfg: PredictorConfig, pweights, cond: torch.Tensor, prev_emb: torch.Tensor, pos: torch.Tensor,
                     cache_len: torch.Tensor, codes=None, h_out=None, xn_out=None, ws=None, stream=None):
    """One frame of the Dual-Track loop (caches, prev_emb, pos and cache_len updated in place).  ``layers``: list
    of dicts (see talker_layers_struct) or a prebuilt array; ``pweights``: predictor weight dict or struct.
    Returns codes [num_codes, T] int32 (row 0 = c_0)."""
    T, dev = cond.shape[0], cond.device
    arr = layers if isinstance(layers, ctypes.Array) else talker_layers_struct(layers)
    pw = pweights if isinstance(pweights, moe_predictor_weights) else predictor_weights_struct(pweights)
    codes = codes if codes is not None else torch.empty((pcfg.num_codes, T), dtype=torch.int32, device=dev)
    V = codec_head.shape[0]
    lib = load_library()
    c, a, p = cfg.c(), acfg.c(), pcfg.c()
    buf = ws if ws is not None else workspace(
        int(lib.moe_talker_frame_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(p), T, V)), dev)
    st = stream if stream is not None else _stream(dev)
    _check("moe_talker_frame", lib.moe_talker_frame(
        ctypes.byref(c), ctypes.byref(a), arr, len(arr), _ptr(final_norm), eps, _ptr(codec_head), V, ctypes.byref(p),
        ctypes.byref(pw), _ptr(cond), T, _ptr(prev_emb), _ptr(pos), _ptr(cache_len), _ptr(codes), _ptr(h_out),
        _ptr(xn_out), _ptr(buf), buf.numel(), st))
    return codes


def moe_talker_decode(cfg: Config, acfg: AttnConfig, layers, x: torch.Tensor, pos: torch.Tensor,
                      cache_len: torch.Tensor, final_norm: Optional[torch.Tensor] = None, eps: float = 1e-6,
                      codec_head: Optional[torch.Tensor] = None, h_out=None, xn_out=None, c0=None,
                      want_c0: bool = True, ws=None, stream=None):
    """One decode step through the layers (caches updated in place).  ``layers``: list of dicts (see
    talker_layers_struct) or a prebuilt array.  Returns (h_out, xn_out or None, c0 or None)."""
    T, dev = x.shape[0], x.device
    arr = layers if isinstance(layers, ctypes.Array) else talker_layers_struct(layers)
    h_out = h_out if h_out is not None else torch.empty_like(x)
    V = 0 if codec_head is None else codec_head.shape[0]
    if c0 is None and want_c0 and codec_head is not None:
        c0 = torch.empty(T, dtype=torch.int32, device=dev)
    lib = load_library()
    c, a = cfg.c(), acfg.c()
    need = int(lib.moe_talker_decode_workspace_size(ctypes.byref(c), ctypes.byref(a), T, V if c0 is not None else 0))
    buf = ws if ws is not None else workspace(need, dev)
    st = stream if stream is not None else _stream(dev)
    _check("moe_talker_decode", lib.moe_talker_decode(
        ctypes.byref(c), ctypes.byref(a), arr, len(arr), _ptr(x), T, _ptr(pos), _ptr(cache_len), _ptr(final_norm),
        eps, _ptr(codec_head), V, _ptr(h_out), _ptr(xn_out), _ptr(c0), _ptr(buf), buf.numel(), st))
    return h_out, xn_out, c0
