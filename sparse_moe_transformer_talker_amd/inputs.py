"""Seeded synthetic inputs for the Talker MoE feed-forward layer.

This module is shared by the CPU oracle tests and the HIP path. It holds none of
the layer's arithmetic: only seeded random draws, the per-expert bias recipe for
the skewed-routing workload, and the fp32 <-> bf16 storage conversion (round to
nearest even), so that both sides see bit-identical inputs.

Shapes follow "3C · Talker MoE (20 lớp, 128 Experts Top-6)" (openarchlab), §1:
hidden 1024, 128 routed experts with intermediate 384, Top-6 renormalised, one
shared expert with intermediate 768, 20 layers, codec_head 1024 -> 3072.  The
lab-scale shape (hidden 6, 6 experts, Top-2) is the size of the NumPy lab on
"Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz Architecture" (openarchlab).

Draw recipe (ours; the pages fix no seeds beyond the lab's seed 30):
  * weights of a layer with seed ``s``: ``numpy.random.default_rng(s)``, drawn in the
    order router [E,H], gate [E,I,H], up [E,I,H], down [E,H,I], shared gate [Is,H],
    shared up [Is,H], shared down [H,Is], each ``standard_normal(float32) * sigma``;
  * activations: ``default_rng(s + 10000)``, ``standard_normal(float32)`` of [T,H];
  * bf16 tensors are the fp32 draw rounded to nearest even;
  * attention ("3C" §1: 16 query / 2 KV heads of 128): ``default_rng(s + 20000)``
    draws w_qkv [(16 + 4) 128, H] then w_o [H, 2048] (sigma 0.02), then the q_norm /
    k_norm gains 1 + N(0, 0.1); caches ``default_rng(s + 30000)``: keys N(0, 1), values
    N(0, 0.64) of [T, n_kv, max_len, 128]; cache lengths ``default_rng(s + 40000)``
    uniform over [0, max_len); speech positions repeat the length on all three
    TM-RoPE axes;
  * code predictor ("用 print(model) 认识 Qwen3-TTS": 5 layers, 16 / 8 heads, SwiGLU
    3072, 15 tables and heads of 2048): ``default_rng(s + 50000)`` draws, per layer,
    the two norm gains, w_qkv, w_o, q/k gains, gate, up, down, then the final gain,
    the c_0 table [3072, H] and the 15 tables (N(0, 1)), then the 15 heads (sigma 0.02).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "LayerShape", "WORKLOADS", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "layer_weights", "activations", "zipf_router_bias", "stack_weights", "AttnShape", "TALKER_ATTN",
    "attention_weights", "kv_cache", "cache_lengths", "speech_positions", "PredictorShape", "PREDICTOR",
    "predictor_weights",
    "bf16_round", "to_f64", "workload_inputs",
]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes of one MoE layer (names as in the pages' configuration fields)."""
    hidden_size: int
    num_experts: int
    num_experts_per_tok: int
    moe_intermediate_size: int
    shared_expert_intermediate_size: int
    norm_topk_prob: bool = True

    @property
    def H(self) -> int:
        return self.hidden_size

    @property
    def E(self) -> int:
        return self.num_experts

    @property
    def k(self) -> int:
        return self.num_experts_per_tok

    @property
    def I(self) -> int:  # noqa: E743
        return self.moe_intermediate_size

    @property
    def Is(self) -> int:
        return self.shared_expert_intermediate_size


TALKER = LayerShape(1024, 128, 6, 384, 768)
LAB = LayerShape(6, 6, 2, 12, 12)

# The workloads: sizes, distributions and seeds.
WORKLOADS: Dict[str, dict] = {
    "lab_f32": dict(shape=LAB, T=4, sigma=0.5, seed=30, dtype="f32"),
    "decode_t64": dict(shape=TALKER, T=64, sigma=0.02, seed=30, dtype="bf16"),
    "prefill_t4096": dict(shape=TALKER, T=4096, sigma=0.02, seed=30, dtype="bf16"),
    "skew_t8192": dict(shape=TALKER, T=8192, sigma=0.02, seed=30, dtype="bf16",
                       zipf_s=1.2, zipf_seed=20030),
    "stack20_t1024": dict(shape=TALKER, T=1024, sigma=0.02, seed=30, dtype="bf16",
                          layers=20, vocab=3072, head_seed=50, eps=1e-6),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> exactly equal fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Value of ``a`` after storage in bf16, as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored tensor (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def layer_weights(shape: LayerShape, seed: int, sigma: float, dtype: str) -> Dict[str, np.ndarray]:
    """Weights of one layer in nn.Linear layout [out, in]; bf16 as uint16 bits, else fp32."""
    rng = np.random.default_rng(seed)
    H, E, I, Is = shape.H, shape.E, shape.I, shape.Is
    out = {}
    for name, shp in (("router", (E, H)), ("gate", (E, I, H)), ("up", (E, I, H)),
                      ("down", (E, H, I)), ("shared_gate", (Is, H)),
                      ("shared_up", (Is, H)), ("shared_down", (H, Is))):
        if name.startswith("shared") and Is == 0:
            out[name] = None
            continue
        out[name] = _store(_normal(rng, shp, sigma), dtype)
    return out


def activations(T: int, H: int, seed: int, dtype: str) -> np.ndarray:
    """Token hidden states [T, H] ~ N(0, 1)."""
    rng = np.random.default_rng(seed + 10000)
    return _store(_normal(rng, (T, H), 1.0), dtype)


def zipf_router_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert logit bias b_e = -s * ln(rank_e) with ranks a seeded permutation of 1..E.

    Adding it to the router logits multiplies each expert's softmax prior by rank^-s,
    i.e. a Zipf(s) popularity over the experts (fp32, length E).
    """
    ranks = np.random.default_rng(seed).permutation(E) + 1
    return (-s * np.log(ranks.astype(np.float64))).astype(np.float32)


def stack_weights(shape: LayerShape, layers: int, seed: int, sigma: float, dtype: str,
                  vocab: int, head_seed: int) -> dict:
    """Weights of an L-layer stack: layer l uses seed+l; codec_head [V,H] uses head_seed."""
    ws = [layer_weights(shape, seed + l, sigma, dtype) for l in range(layers)]
    head = _store(_normal(np.random.default_rng(head_seed), (vocab, shape.H), sigma), dtype)
    return {"layers": ws, "codec_head": head,
            "norm_gain": np.ones(shape.H, dtype=np.float32)}


@dataclasses.dataclass(frozen=True)
class AttnShape:
    """The Talker's attention: hidden size, query heads, key/value heads, head width."""
    H: int = 1024
    n_heads: int = 16
    n_kv_heads: int = 2
    head_dim: int = 128


TALKER_ATTN = AttnShape()


def attention_weights(shape: AttnShape, seed: int, sigma: float = 0.02) -> Dict[str, np.ndarray]:
    """w_qkv [(nq + 2 nkv) d, H] and w_o [H, nq d] (bf16 bits), q_norm / k_norm gains [d] (fp32,
    1 + N(0, 0.1))."""
    rng = np.random.default_rng(seed + 20000)
    d, nq, nkv = shape.head_dim, shape.n_heads, shape.n_kv_heads
    w = {"w_qkv": _store(_normal(rng, ((nq + 2 * nkv) * d, shape.H), sigma), "bf16"),
         "w_o": _store(_normal(rng, (shape.H, nq * d), sigma), "bf16")}
    w["q_norm"] = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    w["k_norm"] = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return w


def kv_cache(T: int, shape: AttnShape, max_len: int, seed: int, v_sigma: float = 0.64) -> Dict[str, np.ndarray]:
    """Random caches [T, nkv, max_len, d] (bf16 bits): keys N(0, 1), values N(0, v_sigma)."""
    rng = np.random.default_rng(seed + 30000)
    shp = (T, shape.n_kv_heads, max_len, shape.head_dim)
    return {"k": _store(_normal(rng, shp, 1.0), "bf16"), "v": _store(_normal(rng, shp, v_sigma), "bf16")}


def cache_lengths(T: int, max_len: int, seed: int, fixed: Optional[int] = None) -> np.ndarray:
    """Cached positions per stream (int32, < max_len): all equal to `fixed`, or uniform over [0, max_len)."""
    if fixed is not None:
        return np.full(T, fixed, dtype=np.int32)
    return np.random.default_rng(seed + 40000).integers(0, max_len, T).astype(np.int32)


def speech_positions(lengths: np.ndarray) -> np.ndarray:
    """(T, H, W) indices [T, 3] int32 of each stream's new token: speech gives all three axes its
    sequence index."""
    p = np.asarray(lengths, np.int32)
    return np.stack([p, p, p], axis=1).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class PredictorShape:
    """The depth code predictor: layers, hidden, heads, MLP width, codes per frame, codebook, c_0 vocabulary."""
    layers: int = 5
    H: int = 1024
    n_heads: int = 16
    n_kv_heads: int = 8
    I: int = 3072  # noqa: E741
    num_codes: int = 16
    codebook: int = 2048
    c0_vocab: int = 3072


PREDICTOR = PredictorShape()


def predictor_weights(shape: PredictorShape, seed: int, sigma: float = 0.02) -> Dict:
    """Weights of the predictor (bf16 bits; gains fp32 1 + N(0, 0.1)); embedding tables N(0, 1)."""
    rng = np.random.default_rng(seed + 50000)
    H, d = shape.H, 128
    gain = lambda n: (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    bf = lambda shp, sg: _store(_normal(rng, shp, sg), "bf16")
    layers = []
    for _ in range(shape.layers):
        layers.append({"in_norm": gain(H), "post_norm": gain(H),
                       "w_qkv": bf(((shape.n_heads + 2 * shape.n_kv_heads) * d, H), sigma),
                       "w_o": bf((H, shape.n_heads * d), sigma), "q_norm": gain(d), "k_norm": gain(d),
                       "gate": bf((shape.I, H), sigma), "up": bf((shape.I, H), sigma),
                       "down": bf((H, shape.I), sigma)})
    return {"layers": layers, "final_norm": gain(H),
            "c0_embedding": bf((shape.c0_vocab, H), 1.0),
            "codec_embedding": bf((shape.num_codes - 1, shape.codebook, H), 1.0),
            "lm_head": bf((shape.num_codes - 1, shape.codebook, H), sigma)}


def workload_inputs(name: str, T: Optional[int] = None) -> dict:
    """Inputs of one named workload (single-layer ones): weights, x and optional bias."""
    cfg = WORKLOADS[name]
    shape: LayerShape = cfg["shape"]
    T = cfg["T"] if T is None else T
    w = layer_weights(shape, cfg["seed"], cfg["sigma"], cfg["dtype"])
    x = activations(T, shape.H, cfg["seed"], cfg["dtype"])
    bias = None
    if "zipf_s" in cfg:
        bias = zipf_router_bias(shape.E, cfg["zipf_s"], cfg["zipf_seed"])
    return {"shape": shape, "dtype": cfg["dtype"], "T": T, "weights": w, "x": x, "bias": bias}
