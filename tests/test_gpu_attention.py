"""Decode-time attention through the C ABI against the attention oracle.

One step of the Talker's attention block for T streams with their own caches
(16 query heads over 2 KV heads of 128, q/k RMSNorm, interleaved TM-RoPE 24/20/20,
rope_theta 1e6): the output y = residual + o_proj(attention) and the cache rows
written at each stream's length are compared with the float64 oracle under the
bf16 bars; every other cache entry must be unchanged bit for bit.  The value
cache is transposed in the library ([T, nkv, head_dim, max_len]).  Cases: random
lengths up to 1024 (T = 64); ragged 128-position chunks with lengths 0 / 1 /
126..129 / max_len - 1 (T = 37, max_len = 256: two chunks, the merge runs);
512-position chunks with lengths 510..513 / 1022 / 1023 (max_len 1024); the chunk
merge in both of its forms (four chunks at 2048 positions, five at 2560); 3D
positions with distinct T/H/W indices; long caches (max_len 4096 and 32768); the
16/8 head split at 256 positions, and 16/8 and 8/2 at 1024 (the 16-wave chunk
with 2 and 4 query heads per KV head); hidden 512 (the 16-column skinny
products); hidden 2048 and 3072 with the fused norm (its register and memory
forms); the fused RMSNorm of y; a batch of 96 streams (the grouped GEMM path
for the projections); streams whose length is out of range; and a captured graph
replayed.
"""
import numpy as np
import pytest
import torch

from oracle import attention_ref as A
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


def _vt(v):
    """The value cache in the library's layout: [T, nkv, head_dim, max_len]."""
    return np.ascontiguousarray(np.swapaxes(v, 2, 3))


def _case(T, max_len, lens, pos=None, shape=INP.TALKER_ATTN, seed=60):
    w = INP.attention_weights(shape, seed)
    kv = INP.kv_cache(T, shape, max_len, seed + 1)
    x = INP.activations(T, shape.H, seed + 2, "bf16")
    res = INP.activations(T, shape.H, seed + 3, "bf16")
    lens = np.asarray(lens, np.int32)
    pos = INP.speech_positions(lens) if pos is None else np.asarray(pos, np.int32)
    return w, kv, x, res, lens, pos


def _run(shape, max_len, w, kv, x, res, lens, pos, norm=False):
    acfg = api.AttnConfig(max_len=max_len, hidden_size=shape.H, num_heads=shape.n_heads,
                          num_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim)
    wd = {"w_qkv": G.dev(w["w_qkv"], "bf16"), "w_o": G.dev(w["w_o"], "bf16"),
          "q_norm": torch.from_numpy(w["q_norm"]).cuda(), "k_norm": torch.from_numpy(w["k_norm"]).cuda()}
    kc, vc = G.dev(kv["k"], "bf16"), G.dev(_vt(kv["v"]), "bf16")
    xd, rd = G.dev(x, "bf16"), G.dev(res, "bf16")
    ld = torch.from_numpy(lens).cuda()
    pd = torch.from_numpy(np.ascontiguousarray(pos)).cuda()
    nout = torch.empty_like(xd) if norm else None
    y = api.moe_attention_decode(acfg, wd, xd, pd, ld, kc, vc, residual=rd, norm_out=nout)
    torch.cuda.synchronize()
    return y, kc, vc, nout


def _check(shape, max_len, w, kv, x, res, lens, pos, what, norm=False):
    y, kc, vc, nout = _run(shape, max_len, w, kv, x, res, lens, pos, norm)
    T = x.shape[0]
    w64 = {"w_qkv": INP.to_f64(w["w_qkv"], "bf16"), "w_o": INP.to_f64(w["w_o"], "bf16"),
           "q_norm": w["q_norm"].astype(np.float64), "k_norm": w["k_norm"].astype(np.float64)}
    kc64, vc64 = INP.to_f64(kv["k"], "bf16"), INP.to_f64(kv["v"], "bf16")
    ref = A.attention_decode(INP.to_f64(x, "bf16"), w64, pos, kc64, vc64, lens, shape.n_heads, shape.n_kv_heads,
                             residual=INP.to_f64(res, "bf16"))
    G.assert_close(G.host64(y), ref["y"], "bf16", what + " y")
    kg = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    vg = np.swapaxes(vc.view(torch.int16).cpu().numpy().view(np.uint16), 2, 3)
    tt = np.arange(T)
    knew = INP.to_f64(kg[tt, :, lens], "bf16")   # [T, nkv, d]
    vnew = INP.to_f64(vg[tt, :, lens], "bf16")
    G.assert_close(knew, ref["k_new"], "bf16", what + " new keys")
    G.assert_close(vnew, ref["v_new"], "bf16", what + " new values")
    mask = np.ones(kg.shape[:3], bool)
    mask[tt, :, lens] = False
    np.testing.assert_array_equal(kg[mask], kv["k"][mask])
    np.testing.assert_array_equal(vg[mask], kv["v"][mask])
    if norm:
        G.assert_close(G.host64(nout), R.rmsnorm(G.host64(y), np.ones(shape.H), 1e-6), "bf16", what + " norm")
    return y


def test_attention_decode_random_lengths():
    T, L = 64, 1024
    w, kv, x, res, lens, pos = _case(T, L, INP.cache_lengths(T, L, 64))
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "T=64 L<=1024")


def test_attention_decode_ragged_chunks_and_edges():
    # max_len 256: 128-position chunks (4 waves), two per stream, so lengths
    # around 128 cross a chunk boundary and the chunk merge runs
    T, L = 37, 256
    lens = INP.cache_lengths(T, L, 65)
    lens[:8] = [0, 1, 126, 127, 128, 129, 254, L - 1]
    w, kv, x, res, lens, pos = _case(T, L, lens)
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "ragged", norm=True)


def test_attention_decode_long_chunk_boundaries():
    # max_len 1024: 512-position chunks (16 waves); lengths around the chunk
    # boundary and the cache's end
    T, L = 9, 1024
    lens = np.array([510, 511, 512, 513, 1022, 1023, 0, 255, 767], np.int32)
    w, kv, x, res, lens, pos = _case(T, L, lens)
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "chunk boundaries")


@pytest.mark.parametrize("L", [2048, 2560])
def test_attention_decode_merge_forms(L):
    # the chunk merge requests every chunk at once up to four chunks (2048
    # positions) and loops above (2560: five chunks); streams holding 1 .. all
    # of the chunks, lengths on the chunk boundaries and at the cache's end
    lens = np.array([0, 1, 511, 512, 513, 1023, 1024, 1535, 1536, 2047, L - 2, L - 1], np.int32)
    T = len(lens)
    w, kv, x, res, lens, pos = _case(T, L, lens)
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "merge, %d positions" % L)


@pytest.mark.parametrize("heads", [(16, 8), (8, 2)])
def test_attention_decode_other_groups_long_cache(heads):
    # 2 and 4 query heads per KV head on the 16-wave (512-position chunk) kernel
    shape = INP.AttnShape(1024, heads[0], heads[1], 128)
    T, L = 12, 1024
    lens = INP.cache_lengths(T, L, 70)
    lens[:4] = [511, 512, 513, 1023]
    w, kv, x, res, lens, pos = _case(T, L, lens, shape=shape)
    _check(shape, L, w, kv, x, res, lens, pos, "%dq/%dkv L=1024" % heads)


def test_attention_decode_3d_positions():
    T, L = 16, 512
    lens = INP.cache_lengths(T, L, 66)
    pos = np.stack([lens, (lens * 7) % 23, (lens * 5) % 31], axis=1).astype(np.int32)
    w, kv, x, res, lens, pos = _case(T, L, lens, pos=pos)
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "3d positions")


def test_attention_decode_long_cache():
    T, L = 8, 4096
    lens = np.array([4095, 4000, 3000, 2049, 2048, 1000, 17, 0], np.int32)
    w, kv, x, res, lens, pos = _case(T, L, lens)
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "long")


def test_attention_decode_small_hidden():
    """Hidden 512, 8 query / 2 KV heads: the QKV (1536 x 512) and O (512 x 1024)
    products take the 16-column skinny kernel."""
    shape = INP.AttnShape(512, 8, 2, 128)
    T, L = 20, 256
    w, kv, x, res, lens, pos = _case(T, L, INP.cache_lengths(T, L, 68), shape=shape)
    _check(shape, L, w, kv, x, res, lens, pos, "hidden 512", norm=True)


@pytest.mark.parametrize("H", [2048, 3072])
def test_attention_decode_wide_hidden_norm(H):
    """Hidden 2048 and 3072 with the fused RMSNorm of y: the output reduction
    keeps its first two 1024-wide passes in registers and reads any further
    pass back from memory (3072), so both forms of its norm run."""
    shape = INP.AttnShape(H, 16, 2, 128)
    T, L = 24, 256
    w, kv, x, res, lens, pos = _case(T, L, INP.cache_lengths(T, L, 69), shape=shape)
    _check(shape, L, w, kv, x, res, lens, pos, "hidden %d" % H, norm=True)


def test_attention_decode_16q_8kv():
    shape = INP.AttnShape(1024, 16, 8, 128)
    T, L = 24, 256
    w, kv, x, res, lens, pos = _case(T, L, INP.cache_lengths(T, L, 67), shape=shape)
    _check(shape, L, w, kv, x, res, lens, pos, "16q/8kv")


def test_attention_decode_out_of_range_length():
    T, L = 4, 128
    lens = np.array([5, -1, L, 0], np.int32)
    w, kv, x, res, _, pos = _case(T, L, np.array([5, 0, 0, 0], np.int32))
    y, kc, vc, _ = _run(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos)
    kg = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    # streams 1 and 2 wrote nothing; their attention output is zero, so y = residual
    np.testing.assert_array_equal(kg[1:3], kv["k"][1:3])
    np.testing.assert_array_equal(G.host64(y)[1:3], INP.to_f64(res, "bf16")[1:3])


def test_attention_decode_graph_replay():
    shape, T, L = INP.TALKER_ATTN, 64, 512
    w, kv, x, res, lens, pos = _case(T, L, INP.cache_lengths(T, L, 68))
    acfg = api.AttnConfig(max_len=L)
    wd = {"w_qkv": G.dev(w["w_qkv"], "bf16"), "w_o": G.dev(w["w_o"], "bf16"),
          "q_norm": torch.from_numpy(w["q_norm"]).cuda(), "k_norm": torch.from_numpy(w["k_norm"]).cuda()}
    kc, vc = G.dev(kv["k"], "bf16"), G.dev(_vt(kv["v"]), "bf16")
    xd, rd = G.dev(x, "bf16"), G.dev(res, "bf16")
    ld, pd = torch.from_numpy(lens).cuda(), torch.from_numpy(pos).cuda()
    dev = torch.device("cuda", 0)
    ws = api.workspace(api.moe_attention_workspace_size(acfg, T), dev)
    y_e = api.moe_attention_decode(acfg, wd, xd, pd, ld, kc, vc, residual=rd, ws=ws)
    torch.cuda.synchronize()
    y_g = torch.empty_like(xd)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_attention_decode(acfg, wd, xd, pd, ld, kc, vc, residual=rd, y=y_g, ws=ws)
    x2 = G.dev(INP.activations(T, shape.H, 99, "bf16"), "bf16")
    kc2, vc2 = kc.clone(), vc.clone()
    for rep in range(3):
        api.moe_attention_decode(acfg, wd, x2, pd, ld, kc2, vc2, residual=rd)  # eager work between replays
        torch.cuda.synchronize()
        y_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), "replay %d differs" % rep


def test_attention_decode_batch_above_64():
    # more streams than the skinny products take: the grouped GEMM tile path
    T, L = 96, 256
    w, kv, x, res, lens, pos = _case(T, L, INP.cache_lengths(T, L, 69))
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "T=96", norm=True)


def test_attention_decode_very_long_cache():
    # 32768-position caches (256 chunks per stream and KV head)
    T, L = 3, 32768
    lens = np.array([L - 1, 20000, 129], np.int32)
    w, kv, x, res, lens, pos = _case(T, L, lens)
    _check(INP.TALKER_ATTN, L, w, kv, x, res, lens, pos, "32k cache")
