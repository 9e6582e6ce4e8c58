"""The depth code predictor's frame through the C ABI against its oracle.

One frame for T streams (5 layers, 16 query / 8 KV heads, MLP 3072, 16 codes of
2048, c_0 vocabulary 3072).  The library returns the codes and the final-normed
state at every position.  As for the stack, a code is an argmax over a bf16
state, so the checks are:
  * every code c_j (j >= 1) is the exact argmax (ties to the lowest code) of
    head j - 1 on the library's own state at position j, computed by the oracle;
  * teacher forcing: the oracle's frame fed the library's codes reproduces the
    library's states at every position, per element within six times a sigma
    built from the bf16 roundings on the path (below), and within the common
    relative-L2 bar;
  * the free-running oracle's codes are reported beside the library's.
Cases: 64 streams and a ragged 5; c_0 outside the table (a zero embedding);
the frame captured in a graph and replayed; a smaller predictor (hidden 512,
MLP 1536), whose products take the 16-column skinny forms (the production
shape takes the forms with the token rows in LDS).
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from oracle import predictor_ref as P
from sparse_moe_transformer_talker_amd import api
from sparse_moe_transformer_talker_amd import inputs as INP
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

# Bar for the final-normed states, derived from the bf16 roundings on the path
# (u = 2^-8, bf16's unit roundoff; a rounding of v errs by at most u |v| per
# element, modelled as uniform, variance u^2 v^2 / 3, independent of the others):
#   * inside an attention sub-layer, N_ATTN = 8 roundings at the scale of its
#     output: the normed input (twice: through v, and through q and k into the
#     scores), q and k after their norms, v in the cache, the attention context,
#     and the bf16 q/k/v product of the many-token form;
#   * inside an MLP sub-layer, N_MLP = 3: the normed input (twice: it enters gate
#     and up, whose product is the intermediate) and the intermediate;
#   * a linear map with random weights carries its input's relative mean-square
#     error to its output, so the residual stream's accumulated error entering a
#     sub-layer through its norm adds its relative mean square to that
#     sub-layer's output;
#   * each stored residual state rounds at the element's own magnitude, and so
#     does the final norm's output.
# Summing the variances along the path gives a per-element sigma (row terms from
# the oracle's own sub-layer scales, the trace of its forced run); the bar is
# Z = 6 sigma per element (a Gaussian tail of 2e-9 per element, about 1e6
# elements per test), beside the common rel-L2 bar.
U = 2.0 ** -8
N_ATTN, N_MLP = 8, 3
Z = 6.0


def _sigma(tr, p, gain, eps=1e-6):
    """Per-element sigma [T, H] of the final state at position p from the trace."""
    sub_ms, resid_ms = tr["sub_ms"][p], tr["resid_ms"][p]   # [2L, T]
    q = U * U / 3.0
    W = np.zeros(sub_ms.shape[1])  # propagated error variance (row mean)
    R = np.zeros(sub_ms.shape[1])  # residual-rounding variance (row mean)
    for s in range(sub_ms.shape[0]):
        rel_in = (W + R) / resid_ms[s - 1] if s > 0 else 0.0
        W = W + sub_ms[s] * ((N_ATTN if s % 2 == 0 else N_MLP) * q + rel_in)
        R = R + q * resid_ms[s]
    h = tr["h"][p]
    scale = gain[None, :] / np.sqrt(np.mean(h * h, axis=1) + eps)[:, None]
    xn = tr["final"][p]
    return np.sqrt(scale ** 2 * (W[:, None] + q * tr["resid_sq"][p]) + q * xn * xn)


def _close(got, tr, p, gain, what):
    ref = tr["final"][p]
    max_abs, rel = G.errors(got, ref)
    z = float(np.max(np.abs(got - ref) / _sigma(tr, p, gain)))
    print("%s: max_abs=%.3e rel_l2=%.3e worst |err| / sigma %.2f" % (what, max_abs, rel, z), flush=True)
    assert z <= Z and rel <= G.BF16_REL_L2, (what, max_abs, rel, z)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.load_library()


@pytest.fixture(scope="module")
def pred():
    shape = INP.PREDICTOR
    w = INP.predictor_weights(shape, 80)
    dev = lambda a: G.dev(a, "bf16") if a.dtype == np.uint16 else torch.from_numpy(a).cuda()
    wd = {k: dev(v) for k, v in w.items() if k != "layers"}
    wd["layers"] = [{k: dev(v) for k, v in lw.items()} for lw in w["layers"]]
    f64 = lambda a: INP.to_f64(a, "bf16") if a.dtype == np.uint16 else a.astype(np.float64)
    w64 = {k: f64(v) for k, v in w.items() if k != "layers"}
    w64["layers"] = [{k: f64(v) for k, v in lw.items()} for lw in w["layers"]]
    return shape, wd, w64


def _run(shape, wd, T, seed, c0=None):
    h = INP.activations(T, shape.H, seed, "bf16")
    if c0 is None:
        c0 = np.random.default_rng(seed).integers(0, shape.c0_vocab, T).astype(np.int32)
    xn = torch.empty((shape.num_codes, T, shape.H), dtype=torch.bfloat16, device="cuda")
    codes = api.moe_predictor_frame(api.PredictorConfig(), wd, G.dev(h, "bf16"), torch.from_numpy(c0).cuda(),
                                    xn_out=xn)
    torch.cuda.synchronize()
    return h, c0, codes.cpu().numpy().astype(np.int64), G.host64(xn.reshape(-1, shape.H)).reshape(
        shape.num_codes, T, shape.H)


@pytest.mark.parametrize("T", [64, 5])
def test_predictor_frame(pred, T):
    shape, wd, w64 = pred
    h, c0, codes, xn = _run(shape, wd, T, 81 + T)
    np.testing.assert_array_equal(codes[0], c0)
    for j in range(1, shape.num_codes):
        np.testing.assert_array_equal(codes[j], R.argmax_first(xn[j] @ w64["lm_head"][j - 1].T), err_msg="code %d" % j)
    forced = P.predictor_frame(INP.to_f64(h, "bf16"), c0, w64, forced=codes, trace=True)
    for j in range(shape.num_codes):
        _close(xn[j], forced, j, w64["final_norm"], "T=%d position %d" % (T, j))
    free = P.predictor_frame(INP.to_f64(h, "bf16"), c0, w64)["codes"]
    agree = float(np.mean(free[1:] == codes[1:]))
    print("predictor T=%d: codes exact on the library's states; free-running oracle agreement %.3f" % (T, agree),
          flush=True)


def test_predictor_c0_outside_the_table(pred):
    shape, wd, w64 = pred
    c0 = np.array([-1, shape.c0_vocab, 7], np.int32)
    h, _, codes, xn = _run(shape, wd, 3, 90, c0=c0)
    np.testing.assert_array_equal(codes[0], c0)
    for j in range(1, shape.num_codes):
        np.testing.assert_array_equal(codes[j], R.argmax_first(xn[j] @ w64["lm_head"][j - 1].T))
    # position 1 of streams 0 and 1 saw a zero embedding: the oracle with a zero row agrees
    w0 = dict(w64, c0_embedding=np.vstack([w64["c0_embedding"], np.zeros((1, shape.H))]))
    forced = P.predictor_frame(INP.to_f64(h, "bf16"), np.array([shape.c0_vocab, shape.c0_vocab, 7]), w0,
                               forced=codes, trace=True)
    for j in range(shape.num_codes):
        _close(xn[j], forced, j, w64["final_norm"], "outside position %d" % j)


def test_predictor_graph_replay(pred):
    shape, wd, _ = pred
    T = 16
    dev = torch.device("cuda", 0)
    pc = api.PredictorConfig()
    h = G.dev(INP.activations(T, shape.H, 95, "bf16"), "bf16")
    c0 = torch.from_numpy(np.random.default_rng(95).integers(0, shape.c0_vocab, T).astype(np.int32)).cuda()
    ws = api.workspace(api.moe_predictor_workspace_size(pc, T), dev)
    wst = api.predictor_weights_struct(wd)
    codes_e = api.moe_predictor_frame(pc, wst, h, c0, ws=ws).clone()
    torch.cuda.synchronize()
    codes_g = torch.empty_like(codes_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_predictor_frame(pc, wst, h, c0, codes=codes_g, ws=ws)
    h2 = G.dev(INP.activations(T, shape.H, 96, "bf16"), "bf16")
    for rep in range(3):
        api.moe_predictor_frame(pc, wst, h2, c0)  # eager work between replays
        torch.cuda.synchronize()
        codes_g.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes_g, codes_e), "replay %d differs" % rep


def test_predictor_frame_small_shape():
    """Hidden 512, 8 query / 4 KV heads, MLP 1536, 2 layers, 4 codes of 256: the
    SwiGLU product's K (512) and the other products' sizes select the 16-column
    skinny kernels."""
    shape = INP.PredictorShape(layers=2, H=512, n_heads=8, n_kv_heads=4, I=1536, num_codes=4, codebook=256,
                               c0_vocab=300)
    pc = api.PredictorConfig(num_layers=2, hidden_size=512, num_heads=8, num_kv_heads=4, intermediate_size=1536,
                             num_codes=4, codebook_size=256, c0_vocab=300)
    w = INP.predictor_weights(shape, 83)
    dev = lambda a: G.dev(a, "bf16") if a.dtype == np.uint16 else torch.from_numpy(a).cuda()
    wd = {k: dev(v) for k, v in w.items() if k != "layers"}
    wd["layers"] = [{k: dev(v) for k, v in lw.items()} for lw in w["layers"]]
    f64 = lambda a: INP.to_f64(a, "bf16") if a.dtype == np.uint16 else a.astype(np.float64)
    w64 = {k: f64(v) for k, v in w.items() if k != "layers"}
    w64["layers"] = [{k: f64(v) for k, v in lw.items()} for lw in w["layers"]]
    T = 23
    h = INP.activations(T, shape.H, 84, "bf16")
    c0 = np.random.default_rng(84).integers(0, shape.c0_vocab, T).astype(np.int32)
    xn = torch.empty((shape.num_codes, T, shape.H), dtype=torch.bfloat16, device="cuda")
    codes = api.moe_predictor_frame(pc, wd, G.dev(h, "bf16"), torch.from_numpy(c0).cuda(), xn_out=xn)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy().astype(np.int64)
    xn = G.host64(xn.reshape(-1, shape.H)).reshape(shape.num_codes, T, shape.H)
    np.testing.assert_array_equal(codes[0], c0)
    for j in range(1, shape.num_codes):
        np.testing.assert_array_equal(codes[j], R.argmax_first(xn[j] @ w64["lm_head"][j - 1].T), err_msg="code %d" % j)
    forced = P.predictor_frame(INP.to_f64(h, "bf16"), c0, w64, n_heads=8, n_kv_heads=4, num_codes=4,
                               forced=codes, trace=True)
    for j in range(shape.num_codes):
        _close(xn[j], forced, j, w64["final_norm"], "small shape position %d" % j)
