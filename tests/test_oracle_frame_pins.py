"""Pins of the frame-loop oracle (CPU only).

* The frame's code-embedding mean against a closed form: tables whose rows are
  scaled unit vectors, codes outside their table as zero rows.
* With every layer's output switched off (o_proj and the experts' and shared
  expert's down projections zero in the Talker, o_proj and down_proj zero in the
  predictor) each layer is the identity, so the loop reduces to a closed form:
  c_0 = argmax of codec_head on the final norm of the frame input, each later
  code the argmax of its head on the final norm of the previous code's
  embedding, and the next input the codes' mean embedding plus the next text
  condition.
* From empty caches, the Talker's incremental caches over F frames against
  recomputing the last frame with full causal attention (torch's
  scaled_dot_product_attention, KV heads repeated) over the sequence of the
  frames' inputs: the same final state and c_0.
* Teacher forcing with the free-running codes reproduces the free run; cache
  lengths and positions advance by one per frame and the caches gain exactly
  the frames' rows.
* Planted mistakes (the sum instead of the mean, one code's embedding only, the
  pre-norm state handed to the predictor, keys appended at position 0) each
  fail one of these pins.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_ref as A
from oracle import frame_ref as FR
from oracle import moe_ref as R

D = 128


def _talker(seed, H=32, L=2, E=8, k=2, I=16, Is=24, nq=4, nkv=2, V=40, max_len=16, T=3, sigma=0.2):
    r = np.random.default_rng(seed)
    layers = []
    for _ in range(L):
        layers.append({
            "in_norm": 1 + 0.1 * r.normal(size=H), "post_norm": 1 + 0.1 * r.normal(size=H),
            "attn": {"w_qkv": r.normal(0, sigma, ((nq + 2 * nkv) * D, H)), "w_o": r.normal(0, sigma, (H, nq * D)),
                     "q_norm": 1 + 0.1 * r.normal(size=D), "k_norm": 1 + 0.1 * r.normal(size=D)},
            "moe": {"router": r.normal(0, sigma, (E, H)), "gate": r.normal(0, sigma, (E, I, H)),
                    "up": r.normal(0, sigma, (E, I, H)), "down": r.normal(0, sigma, (E, H, I)),
                    "shared_gate": r.normal(0, sigma, (Is, H)), "shared_up": r.normal(0, sigma, (Is, H)),
                    "shared_down": r.normal(0, sigma, (H, Is))}})
    return {"layers": layers, "final_norm": 1 + 0.1 * r.normal(size=H), "head": r.normal(0, 1, (V, H)),
            "k": k, "nq": nq, "nkv": nkv, "H": H, "max_len": max_len, "T": T}


def _predictor(seed, H=32, L=2, nq=4, nkv=2, I=48, Q=4, K=20, V0=40, sigma=0.2):
    r = np.random.default_rng(seed + 1)
    layers = []
    for _ in range(L):
        layers.append({"in_norm": 1 + 0.1 * r.normal(size=H), "post_norm": 1 + 0.1 * r.normal(size=H),
                       "w_qkv": r.normal(0, sigma, ((nq + 2 * nkv) * D, H)), "w_o": r.normal(0, sigma, (H, nq * D)),
                       "q_norm": 1 + 0.1 * r.normal(size=D), "k_norm": 1 + 0.1 * r.normal(size=D),
                       "gate": r.normal(0, sigma, (I, H)), "up": r.normal(0, sigma, (I, H)),
                       "down": r.normal(0, sigma, (H, I))})
    return {"layers": layers, "final_norm": 1 + 0.1 * r.normal(size=H), "c0_embedding": r.normal(size=(V0, H)),
            "codec_embedding": r.normal(size=(Q - 1, K, H)), "lm_head": r.normal(0, 1, (Q - 1, K, H))}


def _caches(tk, L, fill_seed=None, len0=None):
    T, nkv, max_len, H = tk["T"], tk["nkv"], tk["max_len"], tk["H"]
    kc = [np.zeros((T, nkv, max_len, D)) for _ in range(L)]
    vc = [np.zeros((T, nkv, max_len, D)) for _ in range(L)]
    if fill_seed is not None:
        r = np.random.default_rng(fill_seed)
        for l in range(L):
            for t in range(T):
                n = int(len0[t])
                kc[l][t, :, :n] = r.normal(size=(nkv, n, D))
                vc[l][t, :, :n] = r.normal(size=(nkv, n, D))
    return kc, vc


def _run(tk, pw, conds, prev0, len0, forced=None, fill_seed=None):
    L = len(tk["layers"])
    kc, vc = _caches(tk, L, fill_seed, len0)
    pos0 = np.stack([len0, len0, len0], axis=1)
    out = FR.frame_loop(prev0, conds, tk["layers"], tk["final_norm"], tk["head"], pw, pos0, len0, kc, vc, tk["k"],
                        n_heads=tk["nq"], n_kv_heads=tk["nkv"], pred_heads=4, pred_kv_heads=2, forced=forced)
    return out, kc, vc


def test_code_embedding_mean_closed_form():
    H, V0, K, Q = 8, 5, 4, 3
    c0_table = np.zeros((V0, H))
    tables = np.zeros((Q - 1, K, H))
    for i in range(V0):
        c0_table[i, i] = 10.0 * (i + 1)          # row i: 10 (i + 1) e_i
    for j in range(Q - 1):
        for i in range(K):
            tables[j, i, 5 + j] = float(i + 1)   # table j, row i: (i + 1) e_{5 + j}
    codes = np.array([[2, 4, -1], [3, 0, 1], [1, 7, 2]])  # [Q, T]; -1 and 7 lie outside their tables
    got = FR.frame_code_embedding(codes, c0_table, tables)
    want = np.zeros((3, H))
    want[0, 2] = 30.0 / 3; want[0, 5] = 4.0 / 3; want[0, 6] = 2.0 / 3
    want[1, 4] = 50.0 / 3; want[1, 5] = 1.0 / 3
    want[2, 5] = 2.0 / 3; want[2, 6] = 3.0 / 3
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_identity_layers_give_closed_form_loop():
    tk = _talker(1)
    pw = _predictor(1)
    for lw in tk["layers"]:
        lw["attn"]["w_o"] = np.zeros_like(lw["attn"]["w_o"])
        lw["moe"]["down"] = np.zeros_like(lw["moe"]["down"])
        lw["moe"]["shared_down"] = np.zeros_like(lw["moe"]["shared_down"])
    for lw in pw["layers"]:
        lw["w_o"] = np.zeros_like(lw["w_o"])
        lw["down"] = np.zeros_like(lw["down"])
    r = np.random.default_rng(5)
    T, H, Fn = tk["T"], tk["H"], 3
    conds = r.normal(size=(Fn, T, H))
    prev0 = r.normal(size=(T, H))
    out, _, _ = _run(tk, pw, conds, prev0, np.array([0, 3, 7]))
    prev = prev0
    nrm = lambda v, g: v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + 1e-6) * g
    for f in range(Fn):
        x = prev + conds[f]
        c0 = np.argmax(nrm(x, tk["final_norm"]) @ tk["head"].T, axis=1)
        codes = [c0]
        emb = pw["c0_embedding"][c0]
        for j in range(1, 4):
            cj = np.argmax(nrm(emb, pw["final_norm"]) @ pw["lm_head"][j - 1].T, axis=1)
            codes.append(cj)
            emb = pw["codec_embedding"][j - 1][cj]
        codes = np.stack(codes)
        rows = [pw["c0_embedding"][codes[0]]] + [pw["codec_embedding"][j - 1][codes[j]] for j in range(1, 4)]
        prev = sum(rows) / 4.0
        np.testing.assert_array_equal(out[f]["c0"], c0)
        np.testing.assert_array_equal(out[f]["codes"], codes)
        np.testing.assert_allclose(out[f]["x"], x, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out[f]["prev"], prev, rtol=1e-12, atol=1e-12)


def _full_causal_last(tk, xs):
    """The Talker over the sequence xs [n, T, H] with full causal attention;
    the final-normed state of the last position."""
    n, T, H = xs.shape
    nq, nkv = tk["nq"], tk["nkv"]
    h = np.transpose(xs, (1, 0, 2)).copy()  # [T, n, H]
    pos = np.broadcast_to(np.arange(n)[None, :, None], (T, n, 3))
    for lw in tk["layers"]:
        xa = R.rmsnorm(h, lw["in_norm"])
        qkv = xa @ lw["attn"]["w_qkv"].T
        q = qkv[..., :nq * D].reshape(T, n, nq, D)
        k = qkv[..., nq * D:(nq + nkv) * D].reshape(T, n, nkv, D)
        v = qkv[..., (nq + nkv) * D:].reshape(T, n, nkv, D)
        q = A.tm_rope(A.head_rmsnorm(q, lw["attn"]["q_norm"]), pos, 1.0e6, (24, 20, 20))
        k = A.tm_rope(A.head_rmsnorm(k, lw["attn"]["k_norm"]), pos, 1.0e6, (24, 20, 20))
        tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
        tkk = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).repeat_interleave(nq // nkv, dim=1)
        tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3))).repeat_interleave(nq // nkv, dim=1)
        o = F.scaled_dot_product_attention(tq, tkk, tv, is_causal=True).numpy().transpose(0, 2, 1, 3)
        hm = h + o.reshape(T, n, nq * D) @ lw["attn"]["w_o"].T
        y = np.stack([R.moe_layer(R.rmsnorm(hm[:, i], lw["post_norm"]), lw["moe"], tk["k"])["y"] for i in range(n)],
                     axis=1)
        h = hm + y
    return R.rmsnorm(h[:, -1], tk["final_norm"])


def test_incremental_caches_equal_full_causal_recompute():
    tk = _talker(2)
    pw = _predictor(2)
    r = np.random.default_rng(6)
    T, H, Fn = tk["T"], tk["H"], 4
    out, _, _ = _run(tk, pw, r.normal(size=(Fn, T, H)), r.normal(size=(T, H)), np.zeros(T, np.int64))
    xs = np.stack([o["x"] for o in out])
    for f in range(1, Fn + 1):
        xn = _full_causal_last(tk, xs[:f])
        np.testing.assert_allclose(out[f - 1]["xn"], xn, rtol=1e-9, atol=1e-9)
        np.testing.assert_array_equal(out[f - 1]["c0"], R.argmax_first(xn @ tk["head"].T))


def test_forcing_the_free_codes_reproduces_the_free_run_and_advances():
    tk = _talker(3)
    pw = _predictor(3)
    r = np.random.default_rng(7)
    T, H, Fn = tk["T"], tk["H"], 3
    conds, prev0 = r.normal(size=(Fn, T, H)), r.normal(size=(T, H))
    len0 = np.array([2, 5, 0])
    free, kc0, vc0 = _run(tk, pw, conds, prev0, len0, fill_seed=11)
    forced = np.stack([o["codes"] for o in free])
    got, kc1, vc1 = _run(tk, pw, conds, prev0, len0, forced=forced, fill_seed=11)
    for a, b in zip(free, got):
        np.testing.assert_array_equal(a["codes"], b["codes"])
        np.testing.assert_array_equal(a["xn"], b["xn"])
    # the caches: untouched below len0 (the seeded prefix), the frames' rows at
    # len0 .. len0 + F - 1, zero beyond
    kref, _ = _caches(tk, len(tk["layers"]), 11, len0)
    for l in range(len(tk["layers"])):
        for t in range(T):
            n = int(len0[t])
            np.testing.assert_array_equal(kc1[l][t, :, :n], kref[l][t, :, :n])
            assert np.all(np.abs(kc1[l][t, :, n:n + Fn]).sum(axis=-1) > 0)
            assert np.all(kc1[l][t, :, n + Fn:] == 0)
            np.testing.assert_array_equal(kc1[l], kc0[l])
            np.testing.assert_array_equal(vc1[l], vc0[l])


# Planted mistakes in the frame oracle must fail at least one pin above.
_orig_embed = FR.frame_code_embedding
_orig_step = FR.talker_step
_orig_layer = FR.talker_layer


def _sum_not_mean(codes, c0_table, tables):
    return _orig_embed(codes, c0_table, tables) * np.asarray(codes).shape[0]


def _first_code_only(codes, c0_table, tables):
    codes = np.asarray(codes)
    return _orig_embed(codes[:1], c0_table, tables)


def _prenorm_handoff(x, layers, pos, kcs, vcs, lens, final_norm, w_head, k, nq, nkv, eps=1e-6):
    out = _orig_step(x, layers, pos, kcs, vcs, lens, final_norm, w_head, k, nq, nkv, eps)
    return dict(out, xn=out["h"])


def _append_at_zero(h, lw, pos, kc, vc, lens, k, nq, nkv, eps=1e-6, norm_topk_prob=True):
    return _orig_layer(h, lw, pos, kc, vc, np.zeros_like(np.asarray(lens)), k, nq, nkv, eps, norm_topk_prob)


@pytest.mark.parametrize("name,bad", [("frame_code_embedding", _sum_not_mean),
                                      ("frame_code_embedding", _first_code_only),
                                      ("talker_step", _prenorm_handoff),
                                      ("talker_layer", _append_at_zero)],
                         ids=["sum_not_mean", "first_code_only", "prenorm_handoff", "append_at_zero"])
def test_planted_mistake_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(FR, name, bad)
    pins = [test_code_embedding_mean_closed_form, test_identity_layers_give_closed_form_loop,
            test_incremental_caches_equal_full_causal_recompute,
            test_forcing_the_free_codes_reproduces_the_free_run_and_advances]
    failed = []
    for pin in pins:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(pin.__name__)
    assert failed, "planted mistake in frame_ref.%s went unnoticed" % name
