"""Oracle for the Talker's streaming frame loop — TEST INFRASTRUCTURE ONLY.

A plain float64 CPU statement of consecutive 80 ms frames for T streams: the
frame's Talker input, the Talker decode step through its layers (attention
with the streams' key/value caches, then the MoE FFN), c_0, the depth code
predictor's frame, and the input of the next frame.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [P1] "Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz Architecture", step [3B]
       of the lab script (the Dual-Track loop over 80 ms frames: the previous
       frame's audio embedding plus the frame's text condition is the Talker
       input; the text condition is the frame's trailing text hidden state, or
       the pad embedding once the text has run out; after the depth predictor
       the mean of the frame's code embeddings, one row from each codebook's
       table, becomes the next frame's audio embedding; the first frame starts
       from the codec BOS embedding) and step [4A] (the predictor receives the
       Talker's hidden state and c_0).
  [P2] "3C · Talker MoE (20 lớp, 128 Experts Top-6) & Đầu ra mã ngữ nghĩa c_0"
       (openarchlab) §1-§2: 20 decoder layers (GQA attention, then the MoE
       FFN), codec_head, c_0, and the pair [h_talker, c_0] passed on to the
       code predictor.
  [P5] "用 print(model) 认识 Qwen3-TTS" (horus-space), "Codec Head": the
       backbone output passes the final RMSNorm before codec_head.

Readings where the pages leave a step open (each listed in the design notes):
  * each decoder layer is pre-norm: h = x + Attn(RMSNorm(x)); out = h +
    MoE(RMSNorm(h)); the final RMSNorm gives the state codec_head reads, and
    that final-normed state is the h_talker handed to the predictor;
  * the next frame's audio embedding is the mean over the frame's codes (the
    lab's offset-mean lookup; the flow table of the first page speaks of the
    sum of the codebook vectors, which is 16 times the mean and so a scaling
    of the tables);
  * code c_0 embeds through the c_0 table the predictor reads, code c_j (j >= 1)
    through codebook table j - 1; a code outside its table embeds as a zero row;
  * the text condition of each frame is supplied by the caller per stream (the
    trailing text hidden state or the pad embedding: the caller's choice);
  * each frame appends one position per stream to every layer's cache at
    cache_len and then advances cache_len and the three TM-RoPE indices by one.

All arithmetic is float64.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle import attention_ref as A
from oracle import moe_ref as R
from oracle import predictor_ref as P

__all__ = ["talker_layer", "talker_step", "frame_code_embedding", "frame_loop"]


def talker_layer(h: np.ndarray, lw: Dict, pos: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 cache_len: np.ndarray, k: int, n_heads: int, n_kv_heads: int, eps: float = 1e-6,
                 norm_topk_prob: bool = True) -> np.ndarray:
    """One Talker decoder layer for one new position per stream ([P2] §1-§2).

    lw: "in_norm", "post_norm" [H]; "attn" (w_qkv, w_o, q_norm, k_norm as in
    attention_ref); "moe" (the MoE layer's weights as in moe_ref).  Appends the
    new key and value to the caches ([T, nkv, max_len, d], in place) at cache_len.
    """
    h = np.asarray(h, np.float64)
    xa = R.rmsnorm(h, lw["in_norm"], eps)
    att = A.attention_decode(xa, lw["attn"], pos, k_cache, v_cache, cache_len, n_heads, n_kv_heads, eps=eps,
                             residual=h)
    for t in range(h.shape[0]):
        n = int(cache_len[t])
        if 0 <= n < k_cache.shape[2]:
            k_cache[t, :, n] = att["k_new"][t]
            v_cache[t, :, n] = att["v_new"][t]
    hm = att["y"]
    xm = R.rmsnorm(hm, lw["post_norm"], eps)
    return R.moe_layer(xm, lw["moe"], k, norm_topk_prob=norm_topk_prob, residual=hm)["y"]


def talker_step(x: np.ndarray, layers: Sequence[Dict], pos: np.ndarray, k_caches: Sequence[np.ndarray],
                v_caches: Sequence[np.ndarray], cache_len: np.ndarray, final_norm: np.ndarray,
                w_head: np.ndarray, k: int, n_heads: int, n_kv_heads: int, eps: float = 1e-6) -> Dict:
    """The Talker's decode step: every layer, the final RMSNorm, codec_head and
    c_0 = argmax (ties to the lowest code) ([P2] §1-§2, [P5] Codec Head)."""
    h = np.asarray(x, np.float64)
    for l, lw in enumerate(layers):
        h = talker_layer(h, lw, pos, k_caches[l], v_caches[l], cache_len, k, n_heads, n_kv_heads, eps)
    xn = R.rmsnorm(h, final_norm, eps)
    c0 = R.argmax_first(R.codec_head_logits(xn, w_head))
    return {"h": h, "xn": xn, "c0": c0}


def frame_code_embedding(codes: np.ndarray, c0_table: np.ndarray, tables: np.ndarray) -> np.ndarray:
    """Mean over a frame's codes [Q, T] of their embeddings [T, H] ([P1] [3B]):
    c_0 from c0_table [V0, H], c_j (j >= 1) from tables[j - 1] [K, H]; a code
    outside its table is a zero row."""
    codes = np.asarray(codes)
    Q, T = codes.shape
    H = c0_table.shape[1]
    total = np.zeros((T, H))
    for j in range(Q):
        table = np.asarray(c0_table if j == 0 else tables[j - 1], np.float64)
        for t in range(T):
            c = int(codes[j, t])
            if 0 <= c < table.shape[0]:
                total[t] += table[c]
    return total / Q


def frame_loop(prev0: np.ndarray, conds: np.ndarray, layers: Sequence[Dict], final_norm: np.ndarray,
               w_head: np.ndarray, pred_w: Dict, pos0: np.ndarray, len0: np.ndarray,
               k_caches: List[np.ndarray], v_caches: List[np.ndarray], k: int, n_heads: int = 16,
               n_kv_heads: int = 2, pred_heads: int = 16, pred_kv_heads: int = 8, eps: float = 1e-6,
               forced: Optional[np.ndarray] = None) -> List[Dict]:
    """F consecutive frames for T streams ([P1] [3B] and [4A]).

    prev0 [T, H]: the audio embedding before the first frame (the codec BOS
    embedding in the lab); conds [F, T, H]: each frame's text condition;
    pos0 [T, 3], len0 [T]: the new token's TM-RoPE indices and the cached
    positions at the first frame; k_caches / v_caches: per layer, updated in
    place.  With ``forced`` [F, Q, T] (teacher forcing) frame f's c_0 and codes
    are forced[f] for the predictor and for the next frame's input; the codes
    drawn are still returned.

    Per frame: x = prev + cond; the Talker step gives h, its final-normed state
    xn and c_0; the predictor's frame from (xn, c_0) gives the Q codes; prev for
    the next frame is their mean embedding; cache_len and the positions advance
    by one.
    """
    prev = np.asarray(prev0, np.float64)
    pos = np.asarray(pos0, np.int64).copy()
    lens = np.asarray(len0, np.int64).copy()
    Q = 1 + len(pred_w["codec_embedding"])
    out = []
    for f in range(len(conds)):
        x = prev + np.asarray(conds[f], np.float64)
        step = talker_step(x, layers, pos, k_caches, v_caches, lens, final_norm, w_head, k, n_heads, n_kv_heads,
                           eps)
        c0 = step["c0"] if forced is None else np.asarray(forced[f][0])
        fr = P.predictor_frame(step["xn"], c0, pred_w, n_heads=pred_heads, n_kv_heads=pred_kv_heads, num_codes=Q,
                               eps=eps, forced=None if forced is None else forced[f])
        codes = fr["codes"] if forced is None else np.asarray(forced[f])
        prev = frame_code_embedding(codes, pred_w["c0_embedding"], pred_w["codec_embedding"])
        out.append({"x": x, "h": step["h"], "xn": step["xn"], "c0": step["c0"], "codes": fr["codes"],
                    "pred_final": fr["final"], "prev": prev})
        pos = pos + 1
        lens = lens + 1
    return out
