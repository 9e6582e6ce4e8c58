"""The allocation-free entry point (moe_layer_forward_static): the layer on the
library's static per-GPU scratch must give the same results as
moe_layer_forward with a caller workspace, on two calls in a row (the second
with fewer tokens, so stale contents of the shared scratch would show), and
stay within the oracle bars."""
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


def test_static_scratch_matches_workspace_entry_point():
    shape = INP.TALKER
    w = INP.layer_weights(shape, 30, 0.02, "bf16")
    wd = G.weights_dev(w, "bf16")
    w64 = G.weights_f64(w, "bf16")
    cfg = G.config(shape, "bf16")
    for T, seed in ((64, 21), (37, 22)):
        print("static scratch: T=%d" % T, flush=True)
        x_np = INP.activations(T, shape.H, seed, "bf16")
        res_np = INP.activations(T, shape.H, seed + 100, "bf16")
        x, res = G.dev(x_np, "bf16"), G.dev(res_np, "bf16")
        outs = []
        for static in (True, False):
            idx = torch.full((T, shape.k), -1, dtype=torch.int32, device="cuda")
            wts = torch.zeros((T, shape.k), dtype=torch.float32, device="cuda")
            counts = torch.full((shape.E,), -1, dtype=torch.int32, device="cuda")
            if static:
                y = api.moe_layer_forward_static(cfg, wd, x, res, topk_idx=idx, topk_w=wts, counts=counts)
            else:
                y = api.moe_layer_forward(cfg, wd, x, res, topk_idx=idx, topk_w=wts, counts=counts)
            torch.cuda.synchronize()
            outs.append((y, idx, wts, counts))
        (ys, idxs, wss, cs), (yw, idxw, wsw, cw) = outs
        assert torch.equal(ys.view(torch.int16), yw.view(torch.int16))
        assert torch.equal(idxs, idxw) and torch.equal(wss, wsw) and torch.equal(cs, cw)
        ref = R.moe_layer(INP.to_f64(x_np, "bf16"), w64, shape.k, residual=INP.to_f64(res_np, "bf16"))
        np.testing.assert_array_equal(idxs.cpu().numpy(), ref["idx"])
        np.testing.assert_array_equal(cs.cpu().numpy(), ref["counts"])
        G.assert_close(G.host64(ys), ref["y"], "bf16", "static scratch T=%d" % T)


def test_static_scratch_rejects_oversize():
    # 4096 tokens need far more than the static array: refused before any launch
    shape = INP.TALKER
    cfg = G.config(shape, "bf16")
    wd = G.weights_dev(INP.layer_weights(shape, 30, 0.02, "bf16"), "bf16")
    x = torch.zeros((4096, shape.H), dtype=torch.bfloat16, device="cuda")
    assert api.moe_layer_forward_static(cfg, wd, x, check=False) == api.MOE_ERR_SCRATCH
