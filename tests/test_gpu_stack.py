"""Parity of the stacked layer and of the graph-replayed layer (through the C ABI).

* The 20-layer stack with pre-RMSNorm and residual adds, then the final RMSNorm,
  codec_head and argmax to c_0 (T=1024, bf16, seeds 30+l, head seed 50).  Each
  layer is checked on the GPU's own bf16 input (teacher forcing): the RMSNorm
  output and the layer output within the bf16 bars, routing indices bit-exact;
  c_0 bit-exact against the oracle's argmax of the GPU's final normalised state.
  The free-running fp64 stack is run beside it; its c_0 agreement and final
  relative L2 are reported, not asserted (bf16 rounding differences compound
  over 20 layers).
* The layer captured in a HIP graph, replayed several times with other eager
  layer calls in between (the launch configuration the benchmark times): every
  replay equals the eager result bit for bit.
* The stack entry point (each layer's combine, residual add and the next
  RMSNorm in one launch; T = 64, 333 and 4096, three layers, non-unit gains)
  against moe_rmsnorm + moe_layer_forward called layer by layer: bit for bit,
  in place too; those calls against the oracle step by step (teacher forced,
  with the same non-unit gains: every normalised input, every layer output and
  its routing, the final norm); c_0 exact against the oracle's argmax of its
  final state; and the whole stack with its head captured in one graph and
  replayed.
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


@pytest.mark.timeout(900)
def test_stack20_teacher_forced():
    c = INP.WORKLOADS["stack20_t1024"]
    shape, T, L = c["shape"], c["T"], c["layers"]
    cfg = G.config(shape, "bf16")
    eps = c["eps"]
    ones = np.ones(shape.H)
    gain = torch.ones(shape.H, dtype=torch.float32, device="cuda")
    x_np = INP.activations(T, shape.H, c["seed"], "bf16")
    h = G.dev(x_np, "bf16")
    h_free = INP.to_f64(x_np, "bf16")  # free-running fp64 stack
    idx = torch.empty((T, shape.k), dtype=torch.int32, device="cuda")
    worst = 0.0
    for layer in range(L):
        w = INP.layer_weights(shape, c["seed"] + layer, c["sigma"], "bf16")
        wd = G.weights_dev(w, "bf16")
        xn = api.moe_rmsnorm(cfg, h, gain, eps)
        y = api.moe_layer_forward(cfg, wd, xn, h, topk_idx=idx)
        torch.cuda.synchronize()
        h64, xn64 = G.host64(h), G.host64(xn)
        w64 = G.weights_f64(w, "bf16")
        G.assert_close(xn64, R.rmsnorm(h64, ones, eps), "bf16", "stack layer %d rmsnorm" % layer)
        ref = R.moe_layer(xn64, w64, shape.k, residual=h64)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"], err_msg="layer %d routing" % layer)
        got = G.host64(y)
        G.assert_close(got, ref["y"], "bf16", "stack layer %d" % layer)
        worst = max(worst, float(np.abs(got - ref["y"]).max()))
        h_free = h_free + R.moe_layer(R.rmsnorm(h_free, ones, eps), w64, shape.k)["y"]
        h = y
        del wd, w, w64
    head_np = INP.stack_weights(shape, 0, c["seed"], c["sigma"], "bf16", c["vocab"], c["head_seed"])["codec_head"]
    head = G.dev(head_np, "bf16")
    xf = api.moe_rmsnorm(cfg, h, gain, eps)
    c0, _ = api.moe_codec_head_argmax(cfg, xf, head)
    torch.cuda.synchronize()
    head64 = INP.to_f64(head_np, "bf16")
    xf64 = G.host64(xf)
    G.assert_close(xf64, R.rmsnorm(G.host64(h), ones, eps), "bf16", "stack final rmsnorm")
    np.testing.assert_array_equal(c0.cpu().numpy(), R.argmax_first(R.codec_head_logits(xf64, head64)))
    c0_free = R.argmax_first(R.codec_head_logits(R.rmsnorm(h_free, ones, eps), head64))
    agree = float(np.mean(c0.cpu().numpy() == c0_free))
    rel = float(np.linalg.norm(G.host64(h) - h_free) / np.linalg.norm(h_free))
    print("stack: %d layers, T=%d; worst per-layer max_abs %.3e; free-running c0 agreement %.3f, "
          "final hidden rel_l2 %.3e" % (L, T, worst, agree, rel), flush=True)


@pytest.mark.parametrize("T", [64, 4096])
def test_layer_graph_replay(T):
    shape = INP.TALKER
    cfg = G.config(shape, "bf16")
    wd = G.weights_dev(INP.layer_weights(shape, 30, 0.02, "bf16"), "bf16")
    other = G.weights_dev(INP.layer_weights(shape, 31, 0.02, "bf16"), "bf16")
    x = G.dev(INP.activations(T, shape.H, 30, "bf16"), "bf16")
    x2 = G.dev(INP.activations(T, shape.H, 31, "bf16"), "bf16")
    dev = torch.device("cuda", 0)
    ws = api.workspace(api.moe_workspace_size(cfg, T), dev)
    ws2 = api.workspace(api.moe_workspace_size(cfg, T), dev)
    y_eager = api.moe_layer_forward(cfg, wd, x, ws=ws)
    torch.cuda.synchronize()
    y_g = torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_layer_forward(cfg, wd, x, y=y_g, ws=ws)
    for rep in range(3):
        y_other = api.moe_layer_forward(cfg, other, x2, ws=ws2)  # eager work between replays
        torch.cuda.synchronize()
        y_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_eager.view(torch.int16)), "replay %d differs" % rep
        assert not torch.equal(y_other.view(torch.int16), y_eager.view(torch.int16))
    print("graph replay T=%d: 3 replays equal to eager" % T, flush=True)


def _stack_inputs(T, L, dev, with_np=False):
    shape = INP.TALKER
    layers_np = [INP.layer_weights(shape, 30 + l, 0.02, "bf16") for l in range(L)]
    layers = [G.weights_dev(w, "bf16") for w in layers_np]
    head_np = INP.stack_weights(shape, 0, 30, 0.02, "bf16", 3072, 50)["codec_head"]
    rng = np.random.default_rng(70)
    gains = torch.from_numpy((1.0 + 0.1 * rng.standard_normal((L + 1, shape.H))).astype(np.float32)).to(dev)
    x = G.dev(INP.activations(T, shape.H, 30, "bf16"), "bf16")
    if with_np:
        return shape, layers, G.dev(head_np, "bf16"), head_np, gains, x, layers_np
    return shape, layers, G.dev(head_np, "bf16"), head_np, gains, x


def _layer_by_layer(cfg, layers, x, gains, eps, head, layers_np=None, what=""):
    """The stack as separate moe_rmsnorm + moe_layer_forward calls.  With layers_np,
    every step is also checked against the oracle on the GPU's own input
    (teacher forced): each normalised input with its non-unit gain, each layer's
    output and routing."""
    h = x
    k = cfg.num_experts_per_tok
    T = x.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    for l, wd in enumerate(layers):
        xn = api.moe_rmsnorm(cfg, h, gains[l], eps)
        h_next = api.moe_layer_forward(cfg, wd, xn, h, topk_idx=idx)
        if layers_np is not None:
            torch.cuda.synchronize()
            h64, xn64, g64 = G.host64(h), G.host64(xn), gains[l].double().cpu().numpy()
            G.assert_close(xn64, R.rmsnorm(h64, g64, eps), "bf16", "%s layer %d input norm" % (what, l))
            ref = R.moe_layer(xn64, G.weights_f64(layers_np[l], "bf16"), k, residual=h64)
            np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"], err_msg="%s layer %d routing" % (what, l))
            G.assert_close(G.host64(h_next), ref["y"], "bf16", "%s layer %d output" % (what, l))
        h = h_next
    xf = api.moe_rmsnorm(cfg, h, gains[len(layers)], eps)
    c0, _ = api.moe_codec_head_argmax(cfg, xf, head)
    if layers_np is not None:
        torch.cuda.synchronize()
        G.assert_close(G.host64(xf), R.rmsnorm(G.host64(h), gains[len(layers)].double().cpu().numpy(), eps),
                       "bf16", "%s final norm" % what)
    return h, xf, c0


@pytest.mark.parametrize("T", [64, 333, 4096])
def test_stack_entry_point_matches_layer_by_layer(T):
    """moe_stack_forward (combine, residual and the next RMSNorm fused) equals
    moe_rmsnorm + moe_layer_forward called layer by layer, bit for bit, and those
    calls match the oracle step by step with the stack's non-unit gains (so the
    fused path does too); its c_0 is the exact argmax of the oracle's codec_head
    logits of its own final state."""
    dev = torch.device("cuda", 0)
    L, eps = 3, 1e-6
    shape, layers, head, head_np, gains, x, layers_np = _stack_inputs(T, L, dev, with_np=True)
    cfg = G.config(shape, "bf16")
    h_ref, xf_ref, c0_ref = _layer_by_layer(cfg, layers, x, gains, eps, head, layers_np, "stack T=%d" % T)
    xn = torch.empty_like(x)
    h, _, c0 = api.moe_stack_forward(cfg, layers, x, gains, eps, head, xn_out=xn)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
    assert torch.equal(xn.view(torch.int16), xf_ref.view(torch.int16))
    assert torch.equal(c0, c0_ref)
    want = R.argmax_first(R.codec_head_logits(G.host64(xn), INP.to_f64(head_np, "bf16")))
    np.testing.assert_array_equal(c0.cpu().numpy(), want)
    # h_out may alias x (the stack updates the hidden state in place)
    h_in = x.clone()
    api.moe_stack_forward(cfg, layers, h_in, gains, eps, head, h_out=h_in, want_c0=False)
    torch.cuda.synchronize()
    assert torch.equal(h_in.view(torch.int16), h_ref.view(torch.int16))
    # no gains (all 1.0), no head
    ones = torch.ones((L + 1, shape.H), dtype=torch.float32, device=dev)
    h1_ref, xf1_ref, _ = _layer_by_layer(cfg, layers, x, ones, eps, head)
    xn1 = torch.empty_like(x)
    h1, _, none = api.moe_stack_forward(cfg, layers, x, None, eps, None, xn_out=xn1)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(h1.view(torch.int16), h1_ref.view(torch.int16))
    assert torch.equal(xn1.view(torch.int16), xf1_ref.view(torch.int16))
    print("stack entry point T=%d L=%d: equal to layer-by-layer; c0 exact" % (T, L), flush=True)


def test_stack_graph_replay():
    """The stack with its head captured in one HIP graph: every replay, with other
    eager stack calls in between, equals the eager result."""
    dev = torch.device("cuda", 0)
    T, L, eps = 64, 4, 1e-6
    shape, layers, head, _, gains, x = _stack_inputs(T, L, dev)
    cfg = G.config(shape, "bf16")
    ws = api.workspace(api.moe_stack_workspace_size(cfg, T, 3072), dev)
    h_e, _, c0_e = api.moe_stack_forward(cfg, layers, x, gains, eps, head, ws=ws)
    torch.cuda.synchronize()
    h_g, c0_g = torch.empty_like(x), torch.empty(T, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_stack_forward(cfg, layers, x, gains, eps, head, h_out=h_g, c0=c0_g, ws=ws)
    x2 = G.dev(INP.activations(T, shape.H, 31, "bf16"), "bf16")
    for rep in range(3):
        h_o, _, _ = api.moe_stack_forward(cfg, layers[::-1], x2, gains, eps, head)
        torch.cuda.synchronize()
        h_g.zero_()
        c0_g.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h_g.view(torch.int16), h_e.view(torch.int16)), "replay %d differs" % rep
        assert torch.equal(c0_g, c0_e), "replay %d c0 differs" % rep
        assert not torch.equal(h_o.view(torch.int16), h_e.view(torch.int16))
    print("stack graph replay T=%d L=%d: 3 replays equal to eager" % (T, L), flush=True)
