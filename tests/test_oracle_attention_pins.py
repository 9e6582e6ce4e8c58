"""Pins of the attention oracle (CPU only): what the pages and the mathematics fix.

* TM-RoPE ("1B · Interleaved TM-RoPE 3D (24, 20, 20)", §3-§4): the rotation keeps
  every head's norm (the page's bar: below 1e-12); shifting the query's and the
  key's temporal index together keeps q_rot . k_rot; varying one axis moves
  exactly its pairs, 24 / 20 / 20 of them, interleaved T, H, W; one pair's
  rotation in closed form; index 0 is the identity.
* GQA ("3C · Talker MoE" §1: 16 query heads over 2 KV heads): against torch's
  scaled_dot_product_attention with the KV heads repeated; one cached position
  returns its value; equal keys average the values.
* A pure-Python brute force of a whole tiny decode step (loops and math only).
* Planted mistakes in the oracle each fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_ref as A

SECTIONS = (24, 20, 20)


def _rng(s):
    return np.random.default_rng(s)


def test_rope_preserves_norm():
    r = _rng(1)
    x = r.normal(size=(7, 16, 128))
    pos = r.integers(0, 5000, size=(7, 3))
    y = A.tm_rope(x, pos, 1.0e6, SECTIONS)
    err = np.abs(np.linalg.norm(y, axis=-1) - np.linalg.norm(x, axis=-1)).max()
    assert err < 1e-12


def test_rope_temporal_shift_keeps_dot_products():
    r = _rng(2)
    q, k = r.normal(size=(1, 1, 128)), r.normal(size=(1, 1, 128))
    pq, pk = np.array([[37, 5, 9]]), np.array([[12, 3, 40]])
    base = float(np.sum(A.tm_rope(q, pq, 1.0e6, SECTIONS) * A.tm_rope(k, pk, 1.0e6, SECTIONS)))
    for dt in (1, 13, 977):
        sh = np.array([[dt, 0, 0]])
        got = float(np.sum(A.tm_rope(q, pq + sh, 1.0e6, SECTIONS) * A.tm_rope(k, pk + sh, 1.0e6, SECTIONS)))
        assert abs(got - base) < 1e-9 * (1 + abs(base))
    # shifting only the query does change it
    moved = float(np.sum(A.tm_rope(q, pq + np.array([[13, 0, 0]]), 1.0e6, SECTIONS) *
                         A.tm_rope(k, pk, 1.0e6, SECTIONS)))
    assert abs(moved - base) > 1e-3


def test_rope_each_axis_moves_its_interleaved_pairs():
    x = np.ones((1, 1, 128))
    ref = A.tm_rope(x, np.array([[0, 0, 0]]), 1.0e6, SECTIONS)
    moved = []
    for axis in range(3):
        p = np.zeros((1, 3), dtype=np.int64)
        p[0, axis] = 5
        y = A.tm_rope(x, p, 1.0e6, SECTIONS)
        pairs = np.flatnonzero(np.abs(y - ref).reshape(64, 2).max(axis=1) > 1e-15)
        moved.append(set(pairs.tolist()))
    assert [len(m) for m in moved] == [24, 20, 20]
    assert moved[1] == {3 * j + 1 for j in range(20)}
    assert moved[2] == {3 * j + 2 for j in range(20)}
    assert moved[0] == {3 * j for j in range(20)} | {60, 61, 62, 63}


def test_rope_single_pair_closed_form_and_identity():
    # pair 0 turns by the index itself; pair 32 by index * 1e6^(-1/2)
    for k, p, ang in ((0, 1, 1.0), (32, 1000, 1.0), (32, 2000, 2.0), (1, 3, 3 * 1.0e6 ** (-2 / 128))):
        x = np.zeros((1, 1, 128))
        x[0, 0, 2 * k] = 1.0
        y = A.tm_rope(x, np.array([[p, p, p]]), 1.0e6, SECTIONS)[0, 0]
        assert abs(y[2 * k] - math.cos(ang)) < 1e-12 and abs(y[2 * k + 1] - math.sin(ang)) < 1e-12
        assert np.abs(np.delete(y, [2 * k, 2 * k + 1])).max() == 0.0
    x = _rng(3).normal(size=(2, 16, 128))
    np.testing.assert_array_equal(A.tm_rope(x, np.zeros((2, 3)), 1.0e6, SECTIONS), x)


def test_head_rmsnorm_matches_torch():
    r = _rng(4)
    x = r.normal(size=(3, 16, 128))
    g = 1 + 0.1 * r.normal(size=128)
    want = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(A.head_rmsnorm(x, g, 1e-6), want, rtol=1e-12, atol=1e-12)


def test_gqa_matches_torch_sdpa():
    r = _rng(5)
    q = r.normal(size=(16, 128))
    keys, vals = r.normal(size=(2, 37, 128)), r.normal(size=(2, 37, 128))
    got = A.gqa_attend(q, keys, vals)
    tk = torch.from_numpy(keys).repeat_interleave(8, dim=0)      # head h reads KV head h // 8
    tv = torch.from_numpy(vals).repeat_interleave(8, dim=0)
    want = F.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], tk, tv)[:, 0, :].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_gqa_one_position_and_equal_keys():
    r = _rng(6)
    q = r.normal(size=(16, 128))
    keys, vals = r.normal(size=(2, 1, 128)), r.normal(size=(2, 1, 128))
    got = A.gqa_attend(q, keys, vals)
    for h in range(16):
        np.testing.assert_array_equal(got[h], vals[h // 8, 0])
    keys = np.repeat(r.normal(size=(2, 1, 128)), 9, axis=1)
    vals = r.normal(size=(2, 9, 128))
    got = A.gqa_attend(q, keys, vals)
    for h in range(16):
        np.testing.assert_allclose(got[h], vals[h // 8].mean(axis=0), rtol=1e-12, atol=1e-13)


def _brute_step(x, w, pos, kc, vc, lens, nq, nkv, theta, sections, eps):
    """The decode step with Python loops and math only (tiny sizes)."""
    T, H = len(x), len(x[0])
    d = len(kc[0][0][0])
    rows = len(w["w_qkv"])
    qkv = [[sum(x[t][i] * w["w_qkv"][o][i] for i in range(H)) for o in range(rows)] for t in range(T)]
    npair = d // 2
    axis = []
    for k in range(npair):
        if k % 3 == 1 and k < 3 * sections[1]:
            axis.append(1)
        elif k % 3 == 2 and k < 3 * sections[2]:
            axis.append(2)
        else:
            axis.append(0)

    def norm_rot(vec, gain, p):
        ms = sum(v * v for v in vec) / d
        z = [vec[i] / math.sqrt(ms + eps) * gain[i] for i in range(d)]
        out = list(z)
        for k in range(npair):
            a = p[axis[k]] * theta ** (-2.0 * k / d)
            out[2 * k] = z[2 * k] * math.cos(a) - z[2 * k + 1] * math.sin(a)
            out[2 * k + 1] = z[2 * k] * math.sin(a) + z[2 * k + 1] * math.cos(a)
        return out

    ys = []
    for t in range(T):
        q = [norm_rot(qkv[t][h * d:(h + 1) * d], w["q_norm"], pos[t]) for h in range(nq)]
        k = [norm_rot(qkv[t][(nq + g) * d:(nq + g + 1) * d], w["k_norm"], pos[t]) for g in range(nkv)]
        v = [qkv[t][(nq + nkv + g) * d:(nq + nkv + g + 1) * d] for g in range(nkv)]
        o = []
        for h in range(nq):
            g = h // (nq // nkv)
            keys = [list(kc[t][g][i]) for i in range(lens[t])] + [k[g]]
            vals = [list(vc[t][g][i]) for i in range(lens[t])] + [v[g]]
            sc = [sum(q[h][i] * kk[i] for i in range(d)) / math.sqrt(d) for kk in keys]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            o += [sum(e[j] * vals[j][i] for j in range(len(vals))) / z for i in range(d)]
        ys.append([sum(o[i] * w["w_o"][r][i] for i in range(nq * d)) for r in range(len(w["w_o"]))])
    return ys


def test_decode_step_matches_brute_force():
    r = _rng(7)
    T, H, nq, nkv, d, L = 3, 10, 4, 2, 6, 5
    w = {"w_qkv": r.normal(size=((nq + 2 * nkv) * d, H)), "w_o": r.normal(size=(H, nq * d)),
         "q_norm": 1 + 0.1 * r.normal(size=d), "k_norm": 1 + 0.1 * r.normal(size=d)}
    x = r.normal(size=(T, H))
    kc, vc = r.normal(size=(T, nkv, L, d)), r.normal(size=(T, nkv, L, d))
    lens = np.array([0, 2, 4])
    pos = np.array([[0, 0, 0], [2, 7, 1], [4, 1, 9]])
    sec = (1, 1, 1)
    got = A.attention_decode(x, w, pos, kc, vc, lens, nq, nkv, theta=100.0, sections=sec, eps=1e-6)["y"]
    want = _brute_step(x.tolist(), {k: v.tolist() for k, v in w.items()}, pos.tolist(), kc.tolist(), vc.tolist(),
                       lens.tolist(), nq, nkv, 100.0, sec, 1e-6)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-10, atol=1e-10)


# --- planted mistakes -------------------------------------------------------------

_orig = {n: getattr(A, n) for n in ("tm_rope", "rope_axis_of_pair", "rope_inv_freq", "gqa_attend",
                                     "head_rmsnorm", "attention_decode")}


def _rope_backwards(x, pos, theta, sections):
    return _orig["tm_rope"](x, -np.asarray(pos), theta, sections)


def _axes_swapped(head_dim, sections):
    a = _orig["rope_axis_of_pair"](head_dim, sections)
    return np.where(a == 1, 2, np.where(a == 2, 1, a))


def _half_schedule(head_dim, theta):
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -k / head_dim)


def _modulo_heads(q, keys, values):
    nq, d = q.shape
    nkv = keys.shape[0]
    out = np.empty((nq, d))
    for h in range(nq):
        g = h % nkv
        s = keys[g] @ q[h] / np.sqrt(d)
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ values[g]
    return out


def _unscaled(q, keys, values):
    return _orig["gqa_attend"](q * np.sqrt(q.shape[1]), keys, values)


def _eps_outside(x, gain, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * gain


MUTATIONS = [("tm_rope", _rope_backwards), ("rope_axis_of_pair", _axes_swapped),
             ("rope_inv_freq", _half_schedule), ("gqa_attend", _modulo_heads), ("gqa_attend", _unscaled),
             ("head_rmsnorm", _eps_outside)]

PINS = [test_rope_preserves_norm, test_rope_temporal_shift_keeps_dot_products,
        test_rope_each_axis_moves_its_interleaved_pairs, test_rope_single_pair_closed_form_and_identity,
        test_head_rmsnorm_matches_torch, test_gqa_matches_torch_sdpa, test_gqa_one_position_and_equal_keys,
        test_decode_step_matches_brute_force]


def _failures():
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("fn,bad", MUTATIONS, ids=[m[0] + ":" + m[1].__name__ for m in MUTATIONS])
def test_attention_mutation_is_caught(monkeypatch, fn, bad):
    monkeypatch.setattr(A, fn, bad)
    assert _failures(), "planted mistake in attention_ref.%s went unnoticed" % fn
