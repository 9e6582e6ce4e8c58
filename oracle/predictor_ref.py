"""Oracle for the depth code predictor's frame — TEST INFRASTRUCTURE ONLY.

A plain float64 CPU statement of how one 80 ms frame's remaining codes c_1 ..
c_15 are produced from the Talker's last hidden state and c_0, used to check
the HIP library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP path.

Sources (cited by page title and section):
  [P1] "Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz Architecture", step [4A]
       of the lab script and the overview table: the predictor is prefilled with
       the pair [h_talker, embed(c_0)] and runs 15 autoregressive steps, step j
       reading head j and appending the embedding of the code it produced from
       that code's own table; the whole frame never re-runs the Talker.
  [P5] "用 print(model) 认识 Qwen3-TTS", the code_predictor print and the "Code
       Predictor" section: 5 decoder layers with the Talker's structure
       (self-attention with q_norm / k_norm, a SwiGLU MLP 1024 -> 3072 -> 1024,
       input_layernorm and post_attention_layernorm, eps 1e-6), a final norm,
       15 codec_embedding tables Embedding(2048, 1024) and 15 lm_head
       Linear(1024 -> 2048); c_0 enters through the Talker's codec_embedding
       (3072 rows); the hidden size equals the Talker's (identity projection).

Readings where the pages leave a step open (each listed in the design notes):
  * the layer is pre-norm: h = x + Attn(RMSNorm(x)); out = h + MLP(RMSNorm(h));
    the frame's positions are 0 .. 15 (three equal TM-RoPE indices);
  * code j (1 <= j <= 15) is the argmax of lm_head[j - 1] applied to the final
    RMSNorm of the output at position j, ties to the lowest code; position
    j + 1's input is codec_embedding[j - 1][c_j];
  * the attention of each layer caches the frame's own positions only.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

from oracle import attention_ref as A
from oracle import moe_ref as R

__all__ = ["decoder_layer", "predictor_frame"]


def decoder_layer(x: np.ndarray, lw: Dict[str, np.ndarray], pos: np.ndarray, k_cache: np.ndarray,
                  v_cache: np.ndarray, cache_len: np.ndarray, n_heads: int, n_kv_heads: int, eps: float,
                  theta: float, sections: Sequence[int], parts=None) -> np.ndarray:
    """One pre-norm decoder layer for one new position per stream; appends its key and
    value to the caches ([T, nkv, max_len, d], in place) at cache_len.  With ``parts``
    (a list), appends (sub-layer output, residual state after it) for the attention
    and then the MLP."""
    xa = R.rmsnorm(x, lw["in_norm"], eps)
    att = A.attention_decode(xa, lw, pos, k_cache, v_cache, cache_len, n_heads, n_kv_heads, theta, sections, eps)
    T = x.shape[0]
    for t in range(T):
        k_cache[t, :, int(cache_len[t])] = att["k_new"][t]
        v_cache[t, :, int(cache_len[t])] = att["v_new"][t]
    h = x + att["y"]
    m = R.swiglu(R.rmsnorm(h, lw["post_norm"], eps), lw["gate"], lw["up"], lw["down"])
    if parts is not None:
        parts += [(att["y"], h), (m, h + m)]
    return h + m


def predictor_frame(h_talker: np.ndarray, c0: np.ndarray, w: Dict, n_heads: int = 16, n_kv_heads: int = 8,
                    num_codes: int = 16, eps: float = 1e-6, theta: float = 1.0e6,
                    sections: Sequence[int] = (24, 20, 20), forced=None, trace: bool = False) -> Dict[str, np.ndarray]:
    """Codes c_0 .. c_{num_codes - 1} [num_codes, T] of one frame for T streams.

    w: "layers" (list of dicts: in_norm, post_norm, w_qkv, q_norm, k_norm, w_o, gate,
    up, down), "final_norm", "c0_embedding" [V0, H], "codec_embedding"
    [num_codes - 1, K, H], "lm_head" [num_codes - 1, K, H].  With ``forced`` [num_codes, T]
    (teacher forcing), position j + 1 embeds forced[j] instead of the code drawn at j;
    the drawn codes are still returned.  With ``trace``, also per position: "sub_ms"
    [num_codes, 2 L, T] the mean square over the hidden of every sub-layer's output
    (attention, MLP, per layer), "resid_ms" [num_codes, 2 L, T] the mean square of
    the residual state after each sub-layer, "resid_sq" [num_codes, T, H] the sum
    over sub-layers of the squared residual state after each, and "h" [num_codes, T,
    H] the state before the final norm.
    """
    h_talker = np.asarray(h_talker, np.float64)
    T, H = h_talker.shape
    d = 128
    L = len(w["layers"])
    kc = [np.zeros((T, n_kv_heads, num_codes, d)) for _ in range(L)]
    vc = [np.zeros((T, n_kv_heads, num_codes, d)) for _ in range(L)]
    codes = np.zeros((num_codes, T), dtype=np.int64)
    codes[0] = np.asarray(c0)
    finals, sub_ms, resid_ms, resid_sq, pre = [], [], [], [], []
    for p in range(num_codes):
        if p == 0:
            x = h_talker
        elif p == 1:
            x = np.asarray(w["c0_embedding"], np.float64)[codes[0]]
        else:
            prev = codes[p - 1] if forced is None else np.asarray(forced[p - 1])
            x = np.asarray(w["codec_embedding"][p - 2], np.float64)[prev]
        pos = np.full((T, 3), p)
        lens = np.full(T, p)
        parts = [] if trace else None
        for li, lw in enumerate(w["layers"]):
            x = decoder_layer(x, lw, pos, kc[li], vc[li], lens, n_heads, n_kv_heads, eps, theta, sections, parts)
        xf = R.rmsnorm(x, w["final_norm"], eps)
        finals.append(xf)
        if trace:
            sub_ms.append(np.stack([np.mean(o * o, axis=1) for o, _ in parts]))
            resid_ms.append(np.stack([np.mean(r * r, axis=1) for _, r in parts]))
            resid_sq.append(sum(r * r for _, r in parts))
            pre.append(x)
        if p >= 1:
            logits = xf @ np.asarray(w["lm_head"][p - 1], np.float64).T
            codes[p] = R.argmax_first(logits)
    out = {"codes": codes, "final": np.stack(finals)}
    if trace:
        out.update(sub_ms=np.stack(sub_ms), resid_ms=np.stack(resid_ms), resid_sq=np.stack(resid_sq),
                   h=np.stack(pre))
    return out
