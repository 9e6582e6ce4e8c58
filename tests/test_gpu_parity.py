"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: expert indices, per-expert counts and the grouping are bit-exact (ties go
to the lower expert index); bf16 outputs within max-abs 2e-2 and relative L2
1e-2; fp32 lab-scale outputs within 1e-5.  Inputs are the seeded synthetic
workloads (decode T=64, prefill T=4096, Zipf-skewed T=8192, lab scale) plus odd
shapes that take the portable kernels, ragged tails and degenerate cases, and a
262144-token batch checked on sampled tokens (the oracle's tokens are
independent).
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
    api.load_library()  # fails loudly when the HIP library is missing


class Layer:
    """One seeded layer: stored weights, device copies and fp64 copies."""

    def __init__(self, shape, seed, sigma, dtype, bias=None):
        self.shape, self.dtype = shape, dtype
        self.w = INP.layer_weights(shape, seed, sigma, dtype)
        self.wd = G.weights_dev(self.w, dtype, bias)
        self.w64 = G.weights_f64(self.w, dtype)
        self.bias = bias
        self.seed = seed

    def x(self, T, seed=None):
        return INP.activations(T, self.shape.H, self.seed if seed is None else seed, self.dtype)


@pytest.fixture(scope="module")
def talker():
    print("building Talker layer inputs (seed 30)", flush=True)
    return Layer(INP.TALKER, 30, 0.02, "bf16")


@pytest.fixture(scope="module")
def zipf_bias():
    c = INP.WORKLOADS["skew_t8192"]
    return INP.zipf_router_bias(128, c["zipf_s"], c["zipf_seed"])


def _route_check(L, x_np, bias=None, norm=True, probs=False, what=""):
    cfg = G.config(L.shape, L.dtype, norm)
    x = G.dev(x_np, L.dtype)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    idx, w, p = api.moe_route(cfg, x, L.wd["router"], b, want_probs=probs)
    torch.cuda.synchronize()
    ref = R.route(INP.to_f64(x_np, L.dtype), L.w64["router"], L.shape.k, bias, norm)
    got_idx = idx.cpu().numpy()
    mism = int((got_idx != ref["idx"]).any(axis=1).sum())
    print("%s route: T=%d tokens with index mismatch=%d" % (what, x_np.shape[0], mism), flush=True)
    np.testing.assert_array_equal(got_idx, ref["idx"])
    np.testing.assert_allclose(w.cpu().numpy(), ref["weights"], atol=1e-4 if L.dtype == "bf16" else 1e-6)
    if probs:
        np.testing.assert_allclose(p.cpu().numpy(), ref["probs"], atol=1e-5 if L.dtype == "bf16" else 1e-6)
    return idx, ref


@pytest.mark.parametrize("T", [64, 4096, 1, 37, 1000])
def test_route_talker(talker, T):
    _route_check(talker, talker.x(T), probs=(T in (64, 37)), what="talker")


def test_route_skewed_bias(talker, zipf_bias):
    idx, ref = _route_check(talker, talker.x(8192), bias=zipf_bias, what="skew")
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=128)
    print("skew counts: touched=%d max=%d" % ((counts > 0).sum(), counts.max()), flush=True)
    assert counts.max() > 4000  # the Zipf prior concentrates the routing


def test_route_plain_weights(talker):
    _route_check(talker, talker.x(256), norm=False, probs=True, what="norm_topk_prob=0")


def test_route_ties_and_zero_tokens(talker):
    # experts 3, 17 and 90 share one router row; tokens 0..3 are zero (all scores 0)
    L = Layer.__new__(Layer)
    L.__dict__.update(talker.__dict__)
    w = dict(talker.w)
    r = w["router"].copy()
    r[17] = r[3]
    r[90] = r[3]
    w["router"] = r
    L.w = w
    L.wd = dict(talker.wd, router=G.dev(r, "bf16"))
    L.w64 = dict(talker.w64, router=INP.to_f64(r, "bf16"))
    x = talker.x(300)
    x[:4] = 0
    idx, ref = _route_check(L, x, what="ties")
    assert ref["idx"][0].tolist() == list(range(6))


def test_permute_exact(talker, zipf_bias):
    cfg = G.config(talker.shape, "bf16")
    for T, bias in ((64, None), (4096, None), (8192, zipf_bias), (3, None)):
        x = G.dev(talker.x(T), "bf16")
        b = None if bias is None else torch.from_numpy(bias).cuda()
        idx, _, _ = api.moe_route(cfg, x, talker.wd["router"], b)
        out = api.moe_permute(cfg, idx, x=x)
        torch.cuda.synchronize()
        ref = R.permute(idx.cpu().numpy(), 128)
        for key in ("counts", "offsets", "row_token", "row_of"):
            np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], err_msg=key)
        xp = out["x_perm"].cpu()
        assert torch.equal(xp.view(torch.int16), x.cpu()[torch.from_numpy(ref["row_token"])].view(torch.int16))
        print("permute T=%d ok" % T, flush=True)


def _expert_rows_ref(x64, row_token, offsets, w64):
    out = np.zeros((row_token.shape[0], x64.shape[1]))
    for e in range(len(offsets) - 1):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            out[a:b] = R.swiglu(x64[row_token[a:b]], w64["gate"][e], w64["up"][e], w64["down"][e])
    return out


@pytest.mark.parametrize("T", [64, 4096])
def test_grouped_shared_combine_entry_points(talker, T):
    cfg = G.config(talker.shape, "bf16")
    x_np = talker.x(T)
    x = G.dev(x_np, "bf16")
    idx, w, _ = api.moe_route(cfg, x, talker.wd["router"])
    perm = api.moe_permute(cfg, idx)
    yp = api.moe_grouped_swiglu(cfg, x, perm["row_token"], perm["offsets"], T, talker.wd["gate"],
                                talker.wd["up"], talker.wd["down"])
    ys = api.moe_shared_swiglu(cfg, x, talker.wd["shared_gate"], talker.wd["shared_up"], talker.wd["shared_down"])
    res_np = INP.activations(T, 1024, 77, "bf16")
    res = G.dev(res_np, "bf16")
    y = api.moe_combine(cfg, yp, perm["row_of"], w, ys, res)
    torch.cuda.synchronize()
    x64 = INP.to_f64(x_np, "bf16")
    rt, off = perm["row_token"].cpu().numpy(), perm["offsets"].cpu().numpy()
    G.assert_close(G.host64(yp), _expert_rows_ref(x64, rt, off, talker.w64), "bf16", "y_perm T=%d" % T)
    G.assert_close(G.host64(ys), R.swiglu(x64, talker.w64["shared_gate"], talker.w64["shared_up"],
                                          talker.w64["shared_down"]), "bf16", "y_shared T=%d" % T)
    # combine from the GPU's own inputs: only the final bf16 rounding remains
    ref = G.host64(ys) + np.einsum("tk,tkh->th", w.cpu().numpy().astype(np.float64),
                                   G.host64(yp)[perm["row_of"].cpu().numpy()]) + INP.to_f64(res_np, "bf16")
    got = G.host64(y)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    # x already grouped (row_token NULL) gives the same expert outputs
    xg = api.moe_permute(cfg, idx, x=x)["x_perm"]
    yp2 = api.moe_grouped_swiglu(cfg, xg, None, perm["offsets"], T, talker.wd["gate"], talker.wd["up"],
                                 talker.wd["down"])
    torch.cuda.synchronize()
    assert torch.equal(yp2.view(torch.int16), yp.view(torch.int16))


def _layer_check(L, x_np, bias=None, residual=None, what="", norm=True):
    cfg = G.config(L.shape, L.dtype, norm)
    T = x_np.shape[0]
    x = G.dev(x_np, L.dtype)
    res = None if residual is None else G.dev(residual, L.dtype)
    wd = dict(L.wd)
    if bias is not None:
        wd["router_bias"] = torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    idx = torch.empty((T, L.shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, L.shape.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(L.shape.E, dtype=torch.int32, device="cuda")
    y = api.moe_layer_forward(cfg, wd, x, res, topk_idx=idx, topk_w=wts, counts=counts)
    torch.cuda.synchronize()
    ref = R.moe_layer(INP.to_f64(x_np, L.dtype), L.w64, L.shape.k, bias, norm,
                      None if residual is None else INP.to_f64(residual, L.dtype))
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    G.assert_close(G.host64(y), ref["y"], L.dtype, "%s layer T=%d" % (what, T))
    return y, ref


@pytest.mark.parametrize("T", [64, 4096, 1, 100, 777])
def test_layer_talker(talker, T):
    _layer_check(talker, talker.x(T), what="talker")


def test_layer_skewed(talker, zipf_bias):
    _layer_check(talker, talker.x(8192), bias=zipf_bias, what="skew")


def test_layer_residual_and_determinism(talker):
    x_np = talker.x(512)
    res = INP.activations(512, 1024, 99, "bf16")
    y1, _ = _layer_check(talker, x_np, residual=res, what="residual")
    y2, _ = _layer_check(talker, x_np, residual=res, what="residual again")
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("T", [64, 300, 4096])
def test_layer_without_renormalisation(talker, T):
    # norm_topk_prob = False: the k softmax probabilities weight the experts as they
    # are (decode path with the router's pair lists, the mid-size grouping, prefill)
    _layer_check(talker, talker.x(T, seed=7), what="norm_topk_prob=0", norm=False)


def test_layer_lab_scale_f32():
    c = INP.WORKLOADS["lab_f32"]
    L = Layer(c["shape"], c["seed"], c["sigma"], "f32")
    _layer_check(L, L.x(c["T"]), what="lab")
    _layer_check(L, L.x(257, seed=5), what="lab ragged")
    _route_check(L, L.x(64, seed=6), probs=True, norm=False, what="lab route")


@pytest.mark.parametrize("dims,T,dtype", [
    ((96, 10, 3, 40, 24), 37, "bf16"),     # portable kernels, ragged everything
    ((256, 32, 4, 64, 128), 300, "bf16"),  # matrix-core tiles, many rows per expert
    ((256, 32, 4, 64, 128), 40, "bf16"),   # matrix-core tiles, few rows per expert
    ((256, 48, 2, 128, 0), 129, "bf16"),   # no shared expert
    ((20, 12, 3, 16, 0), 50, "f32"),
    ((128, 8, 8, 64, 64), 33, "bf16"),     # k == E: every expert on every token
    ((128, 200, 6, 64, 64), 90, "bf16"),   # E > 128: separate scoring and selection kernels
])
def test_layer_other_shapes(dims, T, dtype):
    shape = INP.LayerShape(*dims)
    L = Layer(shape, 11, 0.05, dtype)
    _layer_check(L, L.x(T), what=str(dims))


def test_rmsnorm_and_codec_head(talker):
    cfg = G.config(talker.shape, "bf16")
    T, V = 1024, 3072
    h_np = INP.activations(T, 1024, 3, "bf16")
    gain = torch.ones(1024, dtype=torch.float32, device="cuda")
    xn = api.moe_rmsnorm(cfg, G.dev(h_np, "bf16"), gain, 1e-6)
    head_np = INP.stack_weights(INP.TALKER, 0, 30, 0.02, "bf16", V, 50)["codec_head"]
    head = G.dev(head_np, "bf16")
    c0, logits = api.moe_codec_head_argmax(cfg, xn, head, want_logits=True)
    torch.cuda.synchronize()
    G.assert_close(G.host64(xn), R.rmsnorm(INP.to_f64(h_np, "bf16"), np.ones(1024), 1e-6), "bf16", "rmsnorm")
    ref_logits = R.codec_head_logits(G.host64(xn), INP.to_f64(head_np, "bf16"))
    np.testing.assert_allclose(logits.cpu().numpy(), ref_logits, atol=1e-3)
    np.testing.assert_array_equal(c0.cpu().numpy(), R.argmax_first(ref_logits))
    # duplicated head rows tie exactly: the lower code wins
    hd = head_np.copy()
    top = R.argmax_first(ref_logits)
    hd[3071] = hd[top[0]]
    hd[0] = hd[top[0]]
    c0b, _ = api.moe_codec_head_argmax(cfg, xn, G.dev(hd, "bf16"))
    torch.cuda.synchronize()
    assert int(c0b[0]) == 0
    # decode-sized batch (exact-product scores): the same tie, and parity
    c0c, _ = api.moe_codec_head_argmax(cfg, xn[:64].contiguous(), G.dev(hd, "bf16"))
    c0d, _ = api.moe_codec_head_argmax(cfg, xn[:64].contiguous(), head)
    torch.cuda.synchronize()
    assert int(c0c[0]) == 0
    np.testing.assert_array_equal(c0d.cpu().numpy(), R.argmax_first(ref_logits[:64]))


@pytest.mark.parametrize("V", [4096, 4097, 6000])
def test_codec_head_argmax_row_lengths(talker, V):
    """The exact argmax holds a row of up to 4096 scores in registers and loops
    over longer ones: both forms, at and across the boundary, equal the oracle's
    argmax (ties to the lowest code), including an exact tie placed on the
    boundary's far side and at code 0."""
    cfg = G.config(talker.shape, "bf16")
    T = 64
    xn = G.dev(INP.activations(T, 1024, 11, "bf16"), "bf16")
    head_np = INP.stack_weights(INP.TALKER, 0, 30, 0.02, "bf16", V, 51)["codec_head"]
    ref = R.codec_head_logits(G.host64(xn), INP.to_f64(head_np, "bf16"))
    c0, _ = api.moe_codec_head_argmax(cfg, xn, G.dev(head_np, "bf16"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c0.cpu().numpy(), R.argmax_first(ref))
    hd = head_np.copy()
    top = int(R.argmax_first(ref)[0])
    hd[V - 1] = hd[top]
    c0b, _ = api.moe_codec_head_argmax(cfg, xn, G.dev(hd, "bf16"))
    torch.cuda.synchronize()
    assert int(c0b[0]) == min(top, V - 1)
    hd[0] = hd[top]
    c0c, _ = api.moe_codec_head_argmax(cfg, xn, G.dev(hd, "bf16"))
    torch.cuda.synchronize()
    assert int(c0c[0]) == 0


def test_empty_batch(talker):
    cfg = G.config(talker.shape, "bf16")
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    y = api.moe_layer_forward(cfg, talker.wd, x)
    idx, w, _ = api.moe_route(cfg, x, talker.wd["router"])
    torch.cuda.synchronize()
    assert y.shape == (0, 1024) and idx.shape == (0, 6)


def test_layer_largest_batch_sampled(talker):
    # 262144 tokens (1.57 M token-expert pairs): every token goes through the whole
    # layer; the oracle (tokens are independent) checks routing bit for bit and the
    # outputs within the bars on a sample, and the counts must account for every pair
    T = 262144
    shape = talker.shape
    x_np = talker.x(T, seed=12)
    cfg = G.config(shape, "bf16")
    idx = torch.empty((T, shape.k), dtype=torch.int32, device="cuda")
    counts = torch.empty(shape.E, dtype=torch.int32, device="cuda")
    y = api.moe_layer_forward(cfg, talker.wd, G.dev(x_np, "bf16"), topk_idx=idx, counts=counts)
    torch.cuda.synchronize()
    assert int(counts.sum().item()) == T * shape.k and int(counts.min().item()) >= 0
    sample = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(13).choice(T, 126, replace=False)]))
    ref = R.moe_layer(INP.to_f64(x_np[sample], "bf16"), talker.w64, shape.k)
    np.testing.assert_array_equal(idx.cpu().numpy()[sample], ref["idx"])
    G.assert_close(G.host64(y)[sample], ref["y"], "bf16", "T=%d sampled" % T)
