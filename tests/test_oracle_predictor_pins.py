"""Pins of the code predictor oracle (CPU only).

* The frame's incremental KV cache against recomputing every position from
  scratch with full causal attention over the prefix (torch's
  scaled_dot_product_attention with is_causal, KV heads repeated): the same
  final states and codes.
* With the attention and MLP outputs switched off (o_proj and down_proj zero)
  every layer is the identity, so each code is the argmax of its head on the
  final norm of its own input embedding: a closed form.
* Code j depends only on tables and heads up to j: changing a later table or head
  leaves the earlier codes unchanged.
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import attention_ref as A
from oracle import moe_ref as R
from oracle import predictor_ref as P


def _weights(seed, T=3, H=32, nq=4, nkv=2, I=48, Q=6, K=40, V0=50, L=2, sigma=0.2):
    r = np.random.default_rng(seed)
    d = 128
    layers = []
    for _ in range(L):
        layers.append({"in_norm": 1 + 0.1 * r.normal(size=H), "post_norm": 1 + 0.1 * r.normal(size=H),
                       "w_qkv": r.normal(0, sigma, ((nq + 2 * nkv) * d, H)), "w_o": r.normal(0, sigma, (H, nq * d)),
                       "q_norm": 1 + 0.1 * r.normal(size=d), "k_norm": 1 + 0.1 * r.normal(size=d),
                       "gate": r.normal(0, sigma, (I, H)), "up": r.normal(0, sigma, (I, H)),
                       "down": r.normal(0, sigma, (H, I))})
    w = {"layers": layers, "final_norm": 1 + 0.1 * r.normal(size=H), "c0_embedding": r.normal(size=(V0, H)),
         "codec_embedding": r.normal(size=(Q - 1, K, H)), "lm_head": r.normal(0, sigma, (Q - 1, K, H))}
    return w, r.normal(size=(T, H)), r.integers(0, V0, T)


def _from_scratch(h_talker, c0, w, nq, nkv, Q, eps=1e-6, theta=1.0e6, sections=(24, 20, 20)):
    """Every position recomputed over its whole prefix with causal full attention."""
    T, H = h_talker.shape
    d = 128
    codes = np.zeros((Q, T), dtype=np.int64)
    codes[0] = c0
    inputs = [h_talker]
    finals, subs = [], []
    for p in range(Q):
        if p == 1:
            inputs.append(w["c0_embedding"][codes[0]])
        elif p >= 2:
            inputs.append(w["codec_embedding"][p - 2][codes[p - 1]])
        x = np.stack(inputs, axis=1)                          # [T, p + 1, H]
        n = x.shape[1]
        pos = np.broadcast_to(np.arange(n)[None, :, None], (T, n, 3))
        for lw in w["layers"]:
            xa = R.rmsnorm(x, lw["in_norm"], eps)
            qkv = xa @ lw["w_qkv"].T
            q = qkv[..., :nq * d].reshape(T, n, nq, d)
            k = qkv[..., nq * d:(nq + nkv) * d].reshape(T, n, nkv, d)
            v = qkv[..., (nq + nkv) * d:].reshape(T, n, nkv, d)
            q = A.tm_rope(A.head_rmsnorm(q, lw["q_norm"], eps), pos, theta, sections)
            k = A.tm_rope(A.head_rmsnorm(k, lw["k_norm"], eps), pos, theta, sections)
            tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
            tk = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).repeat_interleave(nq // nkv, dim=1)
            tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3))).repeat_interleave(nq // nkv, dim=1)
            o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy().transpose(0, 2, 1, 3)
            a = o.reshape(T, n, nq * d) @ lw["w_o"].T
            h = x + a
            m = R.swiglu(R.rmsnorm(h, lw["post_norm"], eps), lw["gate"], lw["up"], lw["down"])
            x = h + m
            subs.append((p, a[:, -1], h[:, -1]))
            subs.append((p, m[:, -1], x[:, -1]))
        xf = R.rmsnorm(x[:, -1], w["final_norm"], eps)
        finals.append(xf)
        if p >= 1:
            codes[p] = R.argmax_first(xf @ w["lm_head"][p - 1].T)
    return codes, np.stack(finals), subs


def test_incremental_cache_equals_full_causal_recompute():
    w, h, c0 = _weights(1)
    got = P.predictor_frame(h, c0, w, n_heads=4, n_kv_heads=2, num_codes=6)
    codes, finals, _ = _from_scratch(h, c0, w, 4, 2, 6)
    np.testing.assert_allclose(got["final"], finals, rtol=1e-10, atol=1e-10)
    np.testing.assert_array_equal(got["codes"], codes)


def test_trace_matches_full_causal_recompute():
    # the per-position sub-layer scales the parity bar is built from, against the
    # recompute's own sub-layer outputs and residual states at the last position
    w, h, c0 = _weights(4)
    got = P.predictor_frame(h, c0, w, n_heads=4, n_kv_heads=2, num_codes=6, trace=True)
    plain = P.predictor_frame(h, c0, w, n_heads=4, n_kv_heads=2, num_codes=6)
    np.testing.assert_array_equal(got["final"], plain["final"])
    _, finals, subs = _from_scratch(h, c0, w, 4, 2, 6)
    L = len(w["layers"])
    for p in range(6):
        mine = [s for s in subs if s[0] == p]
        assert len(mine) == 2 * L
        np.testing.assert_allclose(got["sub_ms"][p], np.stack([np.mean(o * o, axis=1) for _, o, _ in mine]),
                                   rtol=1e-9)
        np.testing.assert_allclose(got["resid_ms"][p], np.stack([np.mean(r * r, axis=1) for _, _, r in mine]),
                                   rtol=1e-9)
        np.testing.assert_allclose(got["resid_sq"][p], sum(r * r for _, _, r in mine), rtol=1e-9)
        np.testing.assert_allclose(got["h"][p], mine[-1][2], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(R.rmsnorm(got["h"][p], w["final_norm"]), finals[p], rtol=1e-9, atol=1e-12)


def test_identity_layers_give_closed_form_codes():
    w, h, c0 = _weights(2)
    for lw in w["layers"]:
        lw["w_o"] = np.zeros_like(lw["w_o"])
        lw["down"] = np.zeros_like(lw["down"])
    got = P.predictor_frame(h, c0, w, n_heads=4, n_kv_heads=2, num_codes=6)["codes"]
    want = [np.asarray(c0)]
    emb = w["c0_embedding"][want[0]]
    for j in range(1, 6):
        want.append(np.argmax(R.rmsnorm(emb, w["final_norm"]) @ w["lm_head"][j - 1].T, axis=1))
        emb = w["codec_embedding"][j - 1][want[-1]]
    np.testing.assert_array_equal(got, np.stack(want))


def test_later_tables_and_heads_do_not_change_earlier_codes():
    w, h, c0 = _weights(3)
    base = P.predictor_frame(h, c0, w, n_heads=4, n_kv_heads=2, num_codes=6)["codes"]
    w2 = dict(w, codec_embedding=w["codec_embedding"].copy(), lm_head=w["lm_head"].copy())
    w2["codec_embedding"][3] = np.random.default_rng(9).normal(size=w2["codec_embedding"][3].shape)  # embeds c_4
    w2["lm_head"][4] = np.random.default_rng(8).normal(size=w2["lm_head"][4].shape)                  # gives c_5
    other = P.predictor_frame(h, c0, w2, n_heads=4, n_kv_heads=2, num_codes=6)["codes"]
    np.testing.assert_array_equal(other[:5], base[:5])
