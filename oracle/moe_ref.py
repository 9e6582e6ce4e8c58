"""Oracle for the Talker MoE feed-forward layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 CPU statement of what the layer computes, used to check the
HIP library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  It shares no code with the HIP path; the only
thing both sides share is the seeded inputs (``inputs.py`` of the package, which
holds none of this arithmetic), and this module does not import it either.

Sources (cited by page title and section):
  [P2] "3C · Talker MoE (20 lớp, 128 Experts Top-6) & Đầu ra mã ngữ nghĩa c_0"
       (openarchlab): §1 "Định nghĩa" (sizes, norm_topk_prob = True, shared
       expert, codec_head 1024 -> 3072) and §3 "Giải pháp" (the routing / combine
       equation: p = softmax(W_r x), S = Top-6, w_i = p_i / sum_{j in S} p_j,
       y = SharedMLP(x) + sum_{i in S} w_i Expert_i(x)).
  [P1] "Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz Architecture" (openarchlab):
       the lab script's [3C] Talker MoE step (pre-RMSNorm, residual add, codec head
       argmax) and its silu / rmsnorm / softmax helpers.
  [P5] "用 print(model) 认识 Qwen3-TTS" (horus-space): the MLP section (SwiGLU is
       down_proj(SiLU(gate_proj(x)) * up_proj(x))), the module print (RMSNorm
       eps = 1e-06, final norm before codec_head) and "Codec Head：语义码预测".

Readings where the pages leave a step open (each listed in the design notes):
  * experts are SwiGLU ([P2] §1 says each expert is a 1024 -> 384 -> 1024 SwiGLU;
    the lab's single-matrix expert is a miniature);
  * the shared expert is added ungated;
  * Top-k is taken on the logits (softmax is strictly increasing), ties go to the
    lower expert index, and the k outputs are listed in descending weight;
  * c_0 is the argmax of the codec_head logits, ties to the lowest code; the
    sampled variant draws by inverse transform from one given uniform per token.

All floating-point work is float64; weights are taken in nn.Linear layout
[out_features, in_features], so a projection is ``x @ W.T``.

Parity pinned by ``tests/test_oracle_pins.py`` (closed forms, brute force over
expert subsets, library routines for SwiGLU / softmax / RMSNorm, invariants).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "silu", "softmax", "router_logits", "topk_select", "topk_weights", "route",
    "swiglu", "moe_layer", "permute", "rmsnorm", "codec_head_logits", "argmax_first", "sample_inverse_cdf",
    "stack_forward", "active_ffn_width",
]


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)  ([P1] lab helper; [P5] act_fn SiLU)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row softmax with the row max subtracted first ([P1] lab helper)."""
    l = np.asarray(logits, dtype=np.float64)
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router scores W_r x for every token ([P2] §3: p = softmax(W_r x)).

    x [T, H], w_router [E, H] (the router linear, [out, in]); optional per-expert
    bias [E] is added to the scores (the skewed-routing workload's Zipf prior).
    """
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per token, largest first, ties -> lower index.

    [P2] §3 picks the Top-6 set S of p; p = softmax(l) is strictly increasing in l,
    so the set and its order are those of l.  A stable sort of -l keeps equal
    scores in ascending index order.
    """
    l = np.asarray(logits, np.float64)
    return np.argsort(-l, axis=-1, kind="stable")[..., :k].astype(np.int64)


def topk_weights(logits: np.ndarray, idx: np.ndarray, norm_topk_prob: bool = True) -> np.ndarray:
    """Gate weights of the selected experts ([P2] §1 norm_topk_prob, §3 equation).

    p = softmax(l); with norm_topk_prob: w_i = p_i / sum_{j in S} p_j, else w_i = p_i.
    """
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(idx, np.int64), axis=-1)
    if norm_topk_prob:
        return sel / sel.sum(axis=-1, keepdims=True)
    return sel


def route(x, w_router, k, bias=None, norm_topk_prob=True) -> Dict[str, np.ndarray]:
    """Router, softmax, Top-k and renormalisation for every token ([P2] §3)."""
    l = router_logits(x, w_router, bias)
    idx = topk_select(l, k)
    return {"logits": l, "probs": softmax(l), "idx": idx,
            "weights": topk_weights(l, idx, norm_topk_prob)}


def swiglu(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One SwiGLU MLP: down(SiLU(gate x) * up x)  ([P5] MLP section; [P2] §1 expert form).

    x [M, H]; w_gate, w_up [I, H]; w_down [H, I].  Returns [M, H].
    """
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(w_gate, np.float64).T
    u = x @ np.asarray(w_up, np.float64).T
    return (silu(g) * u) @ np.asarray(w_down, np.float64).T


def moe_layer(x: np.ndarray, weights: Dict[str, np.ndarray], k: int,
              bias: Optional[np.ndarray] = None, norm_topk_prob: bool = True,
              residual: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One Talker MoE feed-forward layer ([P2] §3 equation).

    y_t = SharedMLP(x_t) + sum_{i in S_t} w_{t,i} * Expert_i(x_t)  (+ residual_t).

    ``weights`` holds router [E,H], gate/up [E,I,H], down [E,H,I] and
    shared_gate/shared_up [Is,H], shared_down [H,Is] (the shared ones may be None).
    Returns y [T,H] plus the routing (idx, weights, probs, logits) and per-expert
    token counts.
    """
    x = np.asarray(x, np.float64)
    T, H = x.shape
    r = route(x, weights["router"], k, bias, norm_topk_prob)
    idx, w = r["idx"], r["weights"]
    E = np.asarray(weights["router"]).shape[0]
    y = np.zeros((T, H), np.float64)
    if weights.get("shared_gate") is not None:
        y += swiglu(x, weights["shared_gate"], weights["shared_up"], weights["shared_down"])
    for e in range(E):
        tok, slot = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        ye = swiglu(x[tok], weights["gate"][e], weights["up"][e], weights["down"][e])
        y[tok] += w[tok, slot][:, None] * ye
    if residual is not None:
        y += np.asarray(residual, np.float64)
    counts = np.bincount(idx.ravel(), minlength=E)
    return dict(r, y=y, counts=counts)


def permute(idx: np.ndarray, num_experts: int) -> Dict[str, np.ndarray]:
    """Grouping of the (token, slot) pairs by expert: a stable counting sort.

    Not a step the pages spell out (the lab loops over each token's experts); this
    is the data-layout view of the same routing.  Pairs are taken in (t, j)
    row-major order and sorted by expert, keeping that order inside an expert.

    counts[e]    = number of pairs routed to e
    offsets      = exclusive prefix sum of counts (length E + 1)
    row_token[r] = token of the pair stored at grouped row r
    row_of[t,j]  = grouped row of pair (t, j)
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.argsort(flat, kind="stable")
    row_token = order // k
    row_of = np.empty(T * k, np.int64)
    row_of[order] = np.arange(T * k)
    return {"counts": counts, "offsets": offsets, "row_token": row_token,
            "row_of": row_of.reshape(T, k)}


def rmsnorm(h: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * gain over the last axis ([P1] lab helper; eps from [P5])."""
    h = np.asarray(h, np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(gain, np.float64)


def codec_head_logits(xf: np.ndarray, w_head: np.ndarray) -> np.ndarray:
    """codec_head: bias-free Linear 1024 -> 3072 ([P2] §1; [P5] "Codec Head")."""
    return np.asarray(xf, np.float64) @ np.asarray(w_head, np.float64).T


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Index of the largest value per row; the lowest index among equal maxima ([P1] lab c_0)."""
    return np.argmax(np.asarray(logits, np.float64), axis=-1).astype(np.int64)


def sample_inverse_cdf(logits: np.ndarray, u: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """c_0 drawn from softmax(logits / temperature), one uniform u per row.

    [P5] "Codec Head" says the 3072 logits go through a softmax and the next
    semantic code is sampled from it (the lab [P1] takes the argmax instead).
    The draw here is inverse transform sampling: the first code v whose
    cumulative probability exceeds u, i.e. sum_{i<=v} e_i > u * sum_i e_i with
    e_i = exp((l_i - max l) / temperature).  u outside [0, 1) clamps to the first
    or the last code.  The pages name no temperature; 1.0 is the plain softmax.
    """
    t = float(temperature)
    if not t > 0:
        raise ValueError("temperature must be positive")
    lg = np.asarray(logits, np.float64)
    e = np.exp((lg - lg.max(axis=-1, keepdims=True)) / t)
    c = np.cumsum(e, axis=-1)
    thr = np.asarray(u, np.float64) * c[..., -1]
    idx = np.sum(c <= thr[..., None], axis=-1)
    return np.minimum(idx, lg.shape[-1] - 1).astype(np.int64)


def stack_forward(x: np.ndarray, layers: Sequence[Dict[str, np.ndarray]], k: int,
                  w_head: np.ndarray, norm_gains: Optional[Sequence[np.ndarray]] = None,
                  final_gain: Optional[np.ndarray] = None, eps: float = 1e-6,
                  norm_topk_prob: bool = True) -> Dict[str, np.ndarray]:
    """Stack of MoE FFN layers with pre-RMSNorm and residuals, then final RMSNorm,
    codec_head and argmax to c_0.

    h <- h + MoE(RMSNorm(h)) per layer ([P1] lab [3C] step: norm, MoE, residual add;
    [P2] §1: 20 layers then codec_head).  The final RMSNorm before codec_head follows
    [P5] ("Codec Head": the backbone output passes the final RMSNorm first).
    Attention sub-layers are not part of this stack.
    """
    h = np.asarray(x, np.float64)
    H = h.shape[1]
    ones = np.ones(H)
    hs = [h]
    for l, w in enumerate(layers):
        g = ones if norm_gains is None else norm_gains[l]
        xn = rmsnorm(h, g, eps)
        h = h + moe_layer(xn, w, k, norm_topk_prob=norm_topk_prob)["y"]
        hs.append(h)
    xf = rmsnorm(h, ones if final_gain is None else final_gain, eps)
    logits = codec_head_logits(xf, w_head)
    return {"hidden": hs, "x_final": xf, "logits": logits, "c0": argmax_first(logits)}


def active_ffn_width(k: int, moe_intermediate_size: int, shared_intermediate_size: int) -> int:
    """FFN width a token activates per layer: k routed experts plus the shared one ([P2] §4)."""
    return k * moe_intermediate_size + shared_intermediate_size
