"""c_0 sampling through the C ABI against the oracle's inverse transform draw.

The codec head's logits go through a softmax and the next code is drawn (the
Qwen3-TTS module walkthrough, "Codec Head").  The library draws by inverse
transform from caller-supplied fp64 uniforms, so the oracle
(``sample_inverse_cdf`` on fp64 logits of the same bf16 inputs) fixes every draw:
  * random uniforms at T = 64 and a ragged T = 333, temperatures 1 and 0.7, for
    the Talker's head (V = 3072, sigma 0.02) and a sharper one (sigma 0.2, also
    at temperature 0.05): bit-exact;
  * uniforms placed 1e-9 (relative) below and above the oracle's cumulative
    probability at a chosen code of every token: well inside the fp32 scores'
    error, so every token takes the exact fp64 pass; bit-exact;
  * a uniform exactly on a boundary: either neighbouring code (the two fp64
    summation orders may round the boundary apart), and clamped u values;
  * the fp32 lab-scale path (H = 6, V = 10).
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_moe_transformer_talker_amd import api
from sparse_moe_transformer_talker_amd import inputs as INP
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.load_library()


def _head(sigma, seed=50, V=3072):
    shape = INP.TALKER
    return INP.stack_weights(shape, 0, 30, sigma, "bf16", V, seed)["codec_head"]


def _setup(T, sigma, seed=40):
    shape = INP.TALKER
    cfg = G.config(shape, "bf16")
    x_np = INP.activations(T, shape.H, seed, "bf16")
    head_np = _head(sigma)
    logits = R.codec_head_logits(INP.to_f64(x_np, "bf16"), INP.to_f64(head_np, "bf16"))
    return cfg, G.dev(x_np, "bf16"), G.dev(head_np, "bf16"), logits


def _u(a):
    return torch.from_numpy(np.asarray(a, np.float64)).cuda()


@pytest.mark.parametrize("T,sigma,tau", [(64, 0.02, 1.0), (64, 0.02, 0.7), (333, 0.02, 1.0), (333, 0.2, 1.0),
                                         (64, 0.2, 0.05)])
def test_sample_random_uniforms(T, sigma, tau):
    cfg, x, head, logits = _setup(T, sigma)
    u = np.random.default_rng(41 + T).random(T)
    c0, lg = api.moe_codec_head_sample(cfg, x, head, _u(u), tau, want_logits=True)
    torch.cuda.synchronize()
    want = R.sample_inverse_cdf(logits, u, float(np.float32(tau)))
    got = c0.cpu().numpy()
    np.testing.assert_array_equal(got, want)
    err = np.abs(lg.double().cpu().numpy() - logits).max()
    assert err < 1e-4, err  # the fp32 logits the draw was certified from
    print("sample T=%d sigma=%g tau=%g: %d draws equal, %d distinct codes" % (T, sigma, tau, T, len(set(got))),
          flush=True)


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_sample_near_boundaries_takes_exact_pass(tau):
    T = 128
    cfg, x, head, logits = _setup(T, 0.02, seed=42)
    t32 = float(np.float32(tau))
    e = np.exp((logits - logits.max(axis=1, keepdims=True)) / t32)
    c = np.cumsum(e, axis=1)
    cdf = c / c[:, -1:]
    rng = np.random.default_rng(43)
    v = rng.integers(0, logits.shape[1] - 1, T)
    at = cdf[np.arange(T), v]
    for sign, expect in ((-1, v), (1, v + 1)):
        u = at * (1.0 + sign * 1e-9)
        want = R.sample_inverse_cdf(logits, u, t32)
        np.testing.assert_array_equal(want, expect)
        c0, _ = api.moe_codec_head_sample(cfg, x, head, _u(u), tau)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(c0.cpu().numpy(), want)
    # exactly on the boundary: either neighbour is a correct draw
    c0, _ = api.moe_codec_head_sample(cfg, x, head, _u(at), tau)
    torch.cuda.synchronize()
    got = c0.cpu().numpy()
    assert np.all((got == v) | (got == v + 1))
    print("boundary draws tau=%g: %d tokens exact; on-boundary picks v in %d, v+1 in %d" % (
        tau, T, int((got == v).sum()), int((got == v + 1).sum())), flush=True)


def test_sample_clamped_uniforms():
    T = 8
    cfg, x, head, logits = _setup(T, 0.02, seed=44)
    u = np.array([0.0, -0.25, np.nan, 1.0, 7.5, 1.0 - 2.0 ** -53, 2.0 ** -60, 0.5])
    c0, _ = api.moe_codec_head_sample(cfg, x, head, _u(u))
    torch.cuda.synchronize()
    got = c0.cpu().numpy()
    V = logits.shape[1]
    assert list(got[:5]) == [0, 0, 0, V - 1, V - 1]
    np.testing.assert_array_equal(got[5:], R.sample_inverse_cdf(logits[5:], u[5:]))


def test_sample_lab_scale_f32():
    shape = INP.LAB
    cfg = G.config(shape, "f32")
    rng = np.random.default_rng(45)
    T, V = 16, 10
    x_np = rng.normal(0, 1, (T, shape.H)).astype(np.float32)
    w_np = rng.normal(0, 0.5, (V, shape.H)).astype(np.float32)
    u = rng.random(T)
    c0, _ = api.moe_codec_head_sample(cfg, G.dev(x_np, "f32"), G.dev(w_np, "f32"), _u(u), 0.8)
    torch.cuda.synchronize()
    logits = R.codec_head_logits(x_np.astype(np.float64), w_np.astype(np.float64))
    np.testing.assert_array_equal(c0.cpu().numpy(), R.sample_inverse_cdf(logits, u, float(np.float32(0.8))))
