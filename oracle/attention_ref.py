"""Oracle for the Talker's decode-time attention — TEST INFRASTRUCTURE ONLY.

A plain float64 CPU statement of one attention step for a batch of streams,
each with its own key/value cache, used to check the HIP library.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [P2] "3C · Talker MoE (20 lớp, 128 Experts Top-6) & Đầu ra mã ngữ nghĩa c_0"
       (openarchlab) §1: Grouped-Query Attention with 16 query heads sharing
       2 key/value heads of 128 dimensions, hidden size 1024; §4: the KV cache
       is 16 / 2 = 8 times smaller than with one KV head per query head.
  [P4] "1B · Interleaved TM-RoPE 3D (24, 20, 20) & Đồng bộ trục thời gian
       12.5 Hz" (openarchlab) §3: each pair of dimensions (x_2k, x_2k+1) is
       rotated by a 2x2 rotation of angle theta_k; the 64 pairs of a 128-wide
       head split 24 / 20 / 20 over the temporal, height and width axes,
       interleaved (pairs 3j, 3j+1, 3j+2 take T, H, W for j < 20; pairs 60..63
       are temporal); rope_theta = 1,000,000; speech and text tokens give the
       three axes the same index.  §4: the rotation preserves the norm, and
       shifting the query's and the key's temporal index together leaves
       q_rot . k_rot unchanged.
  [P5] "用 print(model) 认识 Qwen3-TTS" (horus-space), the attention module print:
       bias-free q_proj / k_proj / v_proj / o_proj and an RMSNorm over each
       128-wide head of Q and of K (q_norm, k_norm, eps 1e-6).

Readings where the pages leave a step open (each listed in the design notes):
  * the frequency of pair k is rope_theta^(-2k / head_dim) (the usual rotary
    schedule; the pages give rope_theta but not the schedule), and the angle is
    the pair's axis index times it;
  * for other section sizes the interleave generalises as: pair k is H when
    k % 3 == 1 and k < 3 s_H, W when k % 3 == 2 and k < 3 s_W, else T;
  * query head h reads key/value head h // (n_heads / n_kv_heads)
    (consecutive query heads share one KV head);
  * q_norm / k_norm are applied per head before the rotation; values are not
    normalised; scores are scaled by 1 / sqrt(head_dim), no mask beyond the
    cache length (a decode step attends to every cached position and itself).

All arithmetic is float64.  Weights are in nn.Linear layout [out, in].
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

__all__ = ["rope_axis_of_pair", "rope_inv_freq", "tm_rope", "head_rmsnorm", "gqa_attend",
           "attention_decode"]


def rope_axis_of_pair(head_dim: int, sections: Sequence[int]) -> np.ndarray:
    """Axis (0 = T, 1 = H, 2 = W) of each of the head_dim / 2 pairs ([P4] §3 interleave)."""
    n = head_dim // 2
    s_t, s_h, s_w = (int(v) for v in sections)
    if s_t + s_h + s_w != n:
        raise ValueError("sections must add up to head_dim / 2")
    axis = np.zeros(n, dtype=np.int64)
    for k in range(n):
        if k % 3 == 1 and k < 3 * s_h:
            axis[k] = 1
        elif k % 3 == 2 and k < 3 * s_w:
            axis[k] = 2
    return axis


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Frequency of pair k: theta^(-2k / head_dim)."""
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * k / head_dim)


def tm_rope(x: np.ndarray, pos_thw: np.ndarray, theta: float, sections: Sequence[int]) -> np.ndarray:
    """Rotate each adjacent pair (x_2k, x_2k+1) of the last axis by pos[axis(k)] * f_k.

    x: [..., heads, head_dim]; pos_thw: [..., 3] (T, H, W indices of each row).
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    axis = rope_axis_of_pair(d, sections)
    f = rope_inv_freq(d, theta)
    pos = np.asarray(pos_thw, np.float64)
    ang = pos[..., axis] * f                  # [..., d / 2]
    ang = ang[..., None, :]                   # broadcast over heads
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def head_rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over each head's last axis, times the per-dimension gain ([P5] q_norm / k_norm)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, np.float64)


def gqa_attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """One query row per head against L cached positions ([P2] §1 GQA).

    q: [nq, d]; keys, values: [nkv, L, d].  Head h uses KV head h // (nq / nkv).
    softmax(q . k / sqrt(d)) weights the values.
    """
    nq, d = q.shape
    nkv = keys.shape[0]
    group = nq // nkv
    out = np.empty((nq, d))
    for h in range(nq):
        g = h // group
        s = keys[g] @ q[h] / np.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ values[g]
    return out


def attention_decode(x: np.ndarray, w: Dict[str, np.ndarray], pos: np.ndarray, k_cache: np.ndarray,
                     v_cache: np.ndarray, cache_len: np.ndarray, n_heads: int, n_kv_heads: int,
                     theta: float = 1.0e6, sections: Sequence[int] = (24, 20, 20), eps: float = 1e-6,
                     residual: np.ndarray | None = None) -> Dict[str, np.ndarray]:
    """One decode step of the attention block for T streams.

    x [T, H] (the normalised layer input); w: "w_qkv" [(nq + 2 nkv) d, H] (query,
    then key, then value rows), "q_norm" / "k_norm" [d], "w_o" [H, nq d];
    pos [T, 3]; k_cache / v_cache [T, nkv, max_len, d] holding cache_len[t]
    earlier positions of stream t (keys already rotated).  The new key and value
    go to position cache_len[t]; the query attends to positions 0..cache_len[t].
    Returns y = o_proj(attention) (+ residual), the new key / value rows
    [T, nkv, d] and the attention output before o_proj [T, nq, d].
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    d = k_cache.shape[-1]
    nq, nkv = n_heads, n_kv_heads
    qkv = x @ np.asarray(w["w_qkv"], np.float64).T
    q = qkv[:, :nq * d].reshape(T, nq, d)
    k = qkv[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
    v = qkv[:, (nq + nkv) * d:].reshape(T, nkv, d)
    q = tm_rope(head_rmsnorm(q, w["q_norm"], eps), pos, theta, sections)
    k = tm_rope(head_rmsnorm(k, w["k_norm"], eps), pos, theta, sections)
    attn = np.empty((T, nq, d))
    for t in range(T):
        n = int(cache_len[t])
        keys = np.concatenate([np.asarray(k_cache[t, :, :n], np.float64), k[t][:, None, :]], axis=1)
        vals = np.concatenate([np.asarray(v_cache[t, :, :n], np.float64), v[t][:, None, :]], axis=1)
        attn[t] = gqa_attend(q[t], keys, vals)
    y = attn.reshape(T, nq * d) @ np.asarray(w["w_o"], np.float64).T
    if residual is not None:
        y = y + np.asarray(residual, np.float64)
    return {"y": y, "k_new": k, "v_new": v, "attn": attn, "q": q}
