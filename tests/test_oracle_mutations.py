"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case swaps one oracle function for a plausibly wrong version (a dropped
term, a swapped operand, a wrong tie rule, ...) and checks that at least one pin
of ``test_oracle_pins`` then fails.  The mistakes live here, on the CPU; nothing
in ``oracle/`` changes.
"""
import numpy as np
import pytest

from oracle import moe_ref as R
import tests.test_oracle_pins as P

_orig = {n: getattr(R, n) for n in ("silu", "swiglu", "topk_select", "topk_weights", "rmsnorm",
                                     "permute", "router_logits", "moe_layer", "softmax",
                                     "sample_inverse_cdf")}


def _swapped_gate_up(x, wg, wu, wd):
    x = np.asarray(x, np.float64)
    return (R.silu(x @ np.asarray(wu).T) * (x @ np.asarray(wg).T)) @ np.asarray(wd).T


def _ties_to_higher(l, k):
    l = np.asarray(l, np.float64)
    E = l.shape[-1]
    rev = np.argsort(-l[..., ::-1], axis=-1, kind="stable")[..., :k]
    return (E - 1 - rev).astype(np.int64)


def _no_renorm(l, idx, norm_topk_prob=True):
    return _orig["topk_weights"](l, idx, False)


def _eps_outside(h, gain, eps=1e-6):
    h = np.asarray(h, np.float64)
    return h / (np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) + eps) * gain


def _sigmoid_only(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def _unstable_permute(idx, E):
    p = _orig["permute"](idx, E)
    # reverse the order inside each expert
    rt = p["row_token"].copy()
    for e in range(E):
        a, b = p["offsets"][e], p["offsets"][e + 1]
        rt[a:b] = rt[a:b][::-1]
    return dict(p, row_token=rt)


def _transposed_router(x, w, bias=None):
    w = np.asarray(w, np.float64)
    l = np.asarray(x, np.float64) @ (w.T if w.shape[0] == w.shape[1] else w.T)
    l = l[..., ::-1]
    return l if bias is None else l + bias


def _drop_shared(x, weights, k, bias=None, norm_topk_prob=True, residual=None):
    w = dict(weights, shared_gate=None, shared_up=None, shared_down=None)
    return _orig["moe_layer"](x, w, k, bias, norm_topk_prob, residual)


def _sample_at_or_above(lg, u, temperature=1.0):  # >= instead of > at a boundary
    e = np.exp((lg - lg.max(axis=-1, keepdims=True)) / temperature)
    c = np.cumsum(e, axis=-1)
    return np.minimum(np.sum(c < (u * c[..., -1])[..., None], axis=-1), lg.shape[-1] - 1)


def _sample_times_temperature(lg, u, temperature=1.0):
    return _orig["sample_inverse_cdf"](np.asarray(lg) * temperature * temperature, u, temperature)


def _sample_reversed(lg, u, temperature=1.0):  # cumulated from the last code
    lg = np.asarray(lg)
    return lg.shape[-1] - 1 - _orig["sample_inverse_cdf"](lg[..., ::-1], u, temperature)


MUTATIONS = [
    ("swiglu", _swapped_gate_up),
    ("topk_select", _ties_to_higher),
    ("topk_weights", _no_renorm),
    ("rmsnorm", _eps_outside),
    ("silu", _sigmoid_only),
    ("permute", _unstable_permute),
    ("router_logits", _transposed_router),
    ("moe_layer", _drop_shared),
    ("sample_inverse_cdf", _sample_at_or_above),
    ("sample_inverse_cdf", _sample_times_temperature),
    ("sample_inverse_cdf", _sample_reversed),
]

PINS = [n for n in dir(P) if n.startswith("test_") and not n.startswith("test_bruteforce")
        and n not in ("test_permute_is_a_stable_bucket_sort",)]


def _run_pins(monkeypatch):
    failed = []
    for name in PINS:
        try:
            getattr(P, name)()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(name)
    # parametrised pins, run on a few of their cases
    for args in [(None, 2, True), (1, 3, True), (4, 2, False)]:
        try:
            P.test_bruteforce_subsets(*args)
        except Exception:  # noqa: BLE001
            failed.append("test_bruteforce_subsets%r" % (args,))
    for args in [(37, 16, 4, False), (64, 128, 6, True)]:
        try:
            P.test_permute_is_a_stable_bucket_sort(*args)
        except Exception:  # noqa: BLE001
            failed.append("test_permute%r" % (args,))
    return failed


def test_unmutated_oracle_passes_all(monkeypatch):
    assert _run_pins(monkeypatch) == []


@pytest.mark.parametrize("fn,bad", MUTATIONS, ids=[m[0] + ":" + m[1].__name__ for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, fn, bad):
    monkeypatch.setattr(R, fn, bad)
    failed = _run_pins(monkeypatch)
    assert failed, "planted mistake in oracle.%s went unnoticed" % fn
