"""Parity of the decode-size layer path (at most 64 tokens, hidden 1024): the
router's score launch (with the shared expert's gate/up) and per-token
selection, the expert kernel over (touched expert, 64-wide slice) items with its
two forms (K-split up to 16 rows, M-split above) and the shared down tiles, and
the partial-row combine.

Bars as everywhere: indices and per-expert counts bit-exact against the fp64
oracle (ties to the lower expert index); outputs within max-abs 2e-2 and
relative L2 1e-2.  Cases: every token count that changes the kernels' form
(1, 2, 15, 16, 17, 37, 63, 64), routed experts crowded past 16 rows and onto
all 64 tokens, exact ties, zero tokens, no shared expert, other slice counts,
a residual, and bitwise reruns.
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


class Layer:
    def __init__(self, shape, seed, sigma=0.02):
        self.shape = shape
        self.w = INP.layer_weights(shape, seed, sigma, "bf16")
        self.wd = G.weights_dev(self.w, "bf16")
        self.w64 = G.weights_f64(self.w, "bf16")
        self.seed = seed


@pytest.fixture(scope="module")
def talker():
    return Layer(INP.TALKER, 30)


def _check(L, x_np, bias=None, residual=None, norm=True, what=""):
    shape = L.shape
    cfg = G.config(shape, "bf16", norm)
    T = x_np.shape[0]
    wd = dict(L.wd)
    if bias is not None:
        wd["router_bias"] = torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    idx = torch.empty((T, shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shape.k), dtype=torch.float32, device="cuda")
    counts = torch.full((shape.E,), -7, dtype=torch.int32, device="cuda")
    res = None if residual is None else G.dev(residual, "bf16")
    y = api.moe_layer_forward(cfg, wd, G.dev(x_np, "bf16"), res, topk_idx=idx, topk_w=wts, counts=counts)
    torch.cuda.synchronize()
    ref = R.moe_layer(INP.to_f64(x_np, "bf16"), L.w64, shape.k, bias, norm,
                      None if residual is None else INP.to_f64(residual, "bf16"))
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    # the weights come from scores certified within 40 2^-23 sum_h |x_h W_eh| of the exact
    # ones (at most 6.2e-5 here), the router bar of the other parity tests
    np.testing.assert_allclose(wts.cpu().numpy(), ref["weights"], atol=1e-4)
    G.assert_close(G.host64(y), ref["y"], "bf16", "%s T=%d" % (what, T))
    return y, ref


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 37, 63, 64])
def test_decode_token_counts(talker, T):
    # T <= 16 runs the shared expert's slices in the K-split form, above in the M-split form
    print("decode layer T=%d" % T, flush=True)
    _check(talker, INP.activations(T, 1024, 40 + T, "bf16"), what="decode")


def test_decode_crowded_experts(talker):
    # a large bias on experts 5 and 77 puts them on every token (64 rows: the
    # M-split form for routed items); a moderate one on expert 9 gives it 33 of
    # the 64 tokens (more than 16: the M-split form with a partial last row block)
    bias = np.zeros(128, np.float32)
    bias[5] = 50.0
    bias[77] = 40.0
    bias[9] = 1.2
    y, ref = _check(talker, INP.activations(64, 1024, 5, "bf16"), bias=bias, what="crowded")
    assert ref["counts"][5] == 64 and ref["counts"][77] == 64 and ref["counts"][9] > 16


def test_decode_zipf_skew(talker):
    c = INP.WORKLOADS["skew_t8192"]
    bias = INP.zipf_router_bias(128, c["zipf_s"], c["zipf_seed"])
    _, ref = _check(talker, INP.activations(64, 1024, 31, "bf16"), bias=bias, what="zipf")
    print("zipf T=64: max count %d, touched %d" % (ref["counts"].max(), (ref["counts"] > 0).sum()), flush=True)


def test_decode_ties_and_zero_tokens(talker):
    # experts 3, 17 and 90 share one router row; tokens 0..3 are zero (every score 0)
    L = Layer.__new__(Layer)
    L.__dict__.update(talker.__dict__)
    r = talker.w["router"].copy()
    r[17] = r[3]
    r[90] = r[3]
    L.w = dict(talker.w, router=r)
    L.wd = dict(talker.wd, router=G.dev(r, "bf16"))
    L.w64 = dict(talker.w64, router=INP.to_f64(r, "bf16"))
    x = INP.activations(64, 1024, 8, "bf16")
    x[:4] = 0
    _, ref = _check(L, x, what="ties")
    assert ref["idx"][0].tolist() == list(range(6))


def test_decode_without_renormalisation(talker):
    _check(talker, INP.activations(33, 1024, 9, "bf16"), norm=False, what="norm_topk_prob=0")


def test_decode_residual_and_determinism(talker):
    x = INP.activations(64, 1024, 10, "bf16")
    res = INP.activations(64, 1024, 11, "bf16")
    y1, _ = _check(talker, x, residual=res, what="residual")
    y2, _ = _check(talker, x, residual=res, what="residual again")
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("dims,T", [
    ((1024, 128, 6, 384, 0), 64),    # no shared expert
    ((1024, 64, 8, 128, 64), 48),    # two slices per expert, one shared slice, k = 8
    ((1024, 16, 2, 192, 256), 20),   # few experts: most items crowded
])
def test_decode_other_shapes(dims, T):
    shape = INP.LayerShape(*dims)
    L = Layer(shape, 12, 0.03)
    _check(L, INP.activations(T, 1024, 13, "bf16"), what=str(dims))
