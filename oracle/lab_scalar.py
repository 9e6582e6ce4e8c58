"""Scalar pure-Python statement of the MoE layer and brute-force Top-k — TEST INFRASTRUCTURE ONLY.

For the lab-scale sizes (hidden 6, 6 experts, Top-2) of "Bài Lab tổng hợp —
Qwen3-Omni & Qwen3-TTS-12Hz Architecture" (openarchlab), where plain loops finish
at once.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use it.

``brute_force_selection`` does not sort: it enumerates every k-subset of experts
and keeps the one whose softmax mass is largest ("3C · Talker MoE (20 lớp, 128
Experts Top-6)", §3: S is the Top-6 set of p), taking the lexicographically
smallest subset among equal masses, which is the lower-index tie rule.  The
layer output is then recomputed for that subset with scalar loops.
"""
from __future__ import annotations

import itertools
import math
from typing import List, Sequence, Tuple

Vector = List[float]
Matrix = List[List[float]]


def _matvec(w: Sequence[Sequence[float]], x: Sequence[float]) -> Vector:
    """w [out][in] times x [in] -> [out] (nn.Linear layout)."""
    out = []
    for row in w:
        acc = 0.0
        for a, b in zip(row, x):
            acc += float(a) * float(b)
        out.append(acc)
    return out


def _silu(z: float) -> float:
    if z >= 0.0:
        return z / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return z * ez / (1.0 + ez)


def swiglu_scalar(x, w_gate, w_up, w_down) -> Vector:
    """down(SiLU(gate x) * up x) for one token ("用 print(model) 认识 Qwen3-TTS", MLP section)."""
    g = _matvec(w_gate, x)
    u = _matvec(w_up, x)
    h = [_silu(a) * b for a, b in zip(g, u)]
    return _matvec(w_down, h)


def softmax_scalar(l: Sequence[float]) -> Vector:
    m = max(l)
    e = [math.exp(v - m) for v in l]
    s = sum(e)
    return [v / s for v in e]


def brute_force_selection(probs: Sequence[float], k: int) -> Tuple[int, ...]:
    """The k-subset with the largest total probability; lexicographically first on ties."""
    best, best_mass = None, -1.0
    for subset in itertools.combinations(range(len(probs)), k):
        mass = math.fsum(probs[i] for i in subset)
        if mass > best_mass:
            best, best_mass = subset, mass
    return best


def moe_token_bruteforce(x, weights, k, bias=None, norm_topk_prob=True):
    """One token through the layer, routing chosen by subset enumeration.

    Returns (y, subset, weights_by_expert) with y = shared(x) + sum_{i in S} w_i E_i(x).
    """
    logits = _matvec(weights["router"], x)
    if bias is not None:
        logits = [a + float(b) for a, b in zip(logits, bias)]
    p = softmax_scalar(logits)
    subset = brute_force_selection(p, k)
    mass = math.fsum(p[i] for i in subset)
    w = {i: (p[i] / mass if norm_topk_prob else p[i]) for i in subset}
    H = len(x)
    y = [0.0] * H
    if weights.get("shared_gate") is not None:
        y = swiglu_scalar(x, weights["shared_gate"], weights["shared_up"], weights["shared_down"])
    for i in subset:
        yi = swiglu_scalar(x, weights["gate"][i], weights["up"][i], weights["down"][i])
        y = [a + w[i] * b for a, b in zip(y, yi)]
    return y, subset, w
