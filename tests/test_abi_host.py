"""The C ABI on the host (no GPU): the library loads, exports every function the
header declares, and validates arguments before anything reaches HIP."""
import ctypes
import os
import re

import pytest

from sparse_moe_transformer_talker_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "talker_moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(api.LIB_PATH), reason="library not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


def _cfg(**kw):
    base = dict(hidden_size=1024, num_experts=128, num_experts_per_tok=6, moe_intermediate_size=384,
                shared_expert_intermediate_size=768, norm_topk_prob=1, dtype=api.MOE_BF16)
    base.update(kw)
    return api.moe_config(**base)


def test_header_declares_the_six_layer_entry_points():
    names = _declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_swiglu", "moe_shared_swiglu", "moe_combine",
              "moe_layer_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(api.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(api.EXPORTS)
    api.load_library()


def test_status_strings():
    assert api.status_string(0) == "ok"
    assert api.status_string(-1) == "invalid argument"
    assert api.status_string(-3) == "workspace too small"
    assert api.status_string(99) == "unknown status"


@pytest.mark.parametrize("kw,expect", [
    ({}, 0),
    ({"num_experts_per_tok": 129}, -1),          # k > E
    ({"num_experts_per_tok": 0}, -1),
    ({"hidden_size": 0}, -1),
    ({"shared_expert_intermediate_size": -1}, -1),
    ({"norm_topk_prob": 2}, -1),
    ({"dtype": 7}, -1),
    ({"num_experts": 2048, "num_experts_per_tok": 6}, -2),   # beyond the supported sizes
    ({"num_experts_per_tok": 33}, -2),
    ({"shared_expert_intermediate_size": 0}, 0),
    ({"dtype": api.MOE_F32, "hidden_size": 6, "num_experts": 6, "num_experts_per_tok": 2,
      "moe_intermediate_size": 12, "shared_expert_intermediate_size": 12}, 0),
])
def test_check_config(kw, expect):
    lib = api.load_library()
    assert lib.moe_check_config(ctypes.byref(_cfg(**kw))) == expect


def test_workspace_size_grows_with_T_and_is_zero_on_bad_config():
    lib = api.load_library()
    c = _cfg()
    s64 = lib.moe_workspace_size(ctypes.byref(c), 64)
    s4096 = lib.moe_workspace_size(ctypes.byref(c), 4096)
    assert 0 < s64 < s4096
    assert s64 % 256 == 0
    # the layer needs at least its expert-output slots: T * (k + 1) * H bf16
    assert s4096 >= 4096 * 7 * 1024 * 2
    assert lib.moe_workspace_size(ctypes.byref(_cfg(num_experts_per_tok=200)), 64) == 0
    assert lib.moe_workspace_size(ctypes.byref(c), -1) == 0


FAKE = 0x7F0000000000  # never dereferenced: every call below fails its checks first


def _p(off=0):
    return ctypes.c_void_p(FAKE + off)


def test_route_argument_errors():
    lib = api.load_library()
    c = _cfg()
    ws = lib.moe_workspace_size(ctypes.byref(c), 16)
    ok = lambda **kw: lib.moe_route(ctypes.byref(kw.get("cfg", c)), kw.get("x", _p()), kw.get("r", _p()), None,
                                     kw.get("T", 16), kw.get("idx", _p()), kw.get("w", _p()), None, _p(), ws, None)
    assert ok(x=None) == -1
    assert ok(idx=None) == -1
    assert ok(w=None) == -1
    assert ok(x=_p(2)) == -1            # not 16-byte aligned
    assert ok(T=-3) == -1
    assert ok(T=0) == 0                 # empty batch: nothing to do
    assert ok(T=1 << 22) == -2          # T * k beyond 2^22
    assert ok(cfg=_cfg(num_experts_per_tok=130)) == -1
    # the portable router needs score scratch: a too-small workspace is reported
    f32 = _cfg(dtype=api.MOE_F32, hidden_size=6, num_experts=6, num_experts_per_tok=2, moe_intermediate_size=12,
               shared_expert_intermediate_size=12)
    assert lib.moe_route(ctypes.byref(f32), _p(), _p(), None, 4, _p(), _p(), None, _p(), 0, None) == -3


def test_layer_and_helper_argument_errors():
    lib = api.load_library()
    c = _cfg()
    w = api.moe_weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = lib.moe_workspace_size(ctypes.byref(c), 64)
    call = lambda **kw: lib.moe_layer_forward(
        ctypes.byref(c), kw.get("w", ctypes.byref(w)), kw.get("x", _p()), None, 64, kw.get("y", _p(4096)), None,
        None, None, _p(), kw.get("ws", need), None)
    assert call(x=None) == -1
    assert call(y=_p()) == -1          # y may not alias x
    assert call(w=None) == -1
    assert call(ws=need - 256) == -3
    w_noshared = api.moe_weights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    assert call(w=ctypes.byref(w_noshared)) == -1   # Is > 0 needs the shared expert
    assert lib.moe_shared_swiglu(ctypes.byref(_cfg(shared_expert_intermediate_size=0)), _p(), 8, _p(), _p(), _p(),
                                 _p(), _p(), 1 << 20, None) == -1
    assert lib.moe_combine(ctypes.byref(c), _p(), None, _p(), None, None, 8, _p(), None) == -1
    assert lib.moe_rmsnorm(ctypes.byref(c), _p(), _p(), ctypes.c_float(-1.0), 8, _p(), None) == -1
    assert lib.moe_codec_head_argmax(ctypes.byref(c), _p(), _p(), 0, 8, None, _p(), _p(), 1 << 30, None) == -1
    assert lib.moe_codec_head_workspace_size(ctypes.byref(c), 3072, 1024) >= 2 * 3072 * 1024 * 4
    assert lib.moe_permute(ctypes.byref(c), _p(), 8, _p(), _p(), _p(), _p(), _p(), None, _p(), 1 << 20,
                           None) == -1          # x without x_perm
    assert lib.moe_grouped_swiglu(ctypes.byref(c), _p(), None, None, 8, _p(), _p(), _p(), _p(), _p(), 1 << 30,
                                  None) == -1   # offsets required


def test_static_scratch_entry_point_errors():
    # moe_layer_forward_static checks everything on the host before its first HIP
    # call: bad arguments, and workspaces beyond MOE_STATIC_SCRATCH_BYTES
    lib = api.load_library()
    c = _cfg()
    w = api.moe_weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    call = lambda T, **kw: lib.moe_layer_forward_static(
        ctypes.byref(c), kw.get("w", ctypes.byref(w)), kw.get("x", _p()), None, T, kw.get("y", _p(4096)), None,
        None, None, None)
    assert call(64, x=None) == -1
    assert call(64, y=_p()) == -1
    assert call(-1) == -1
    assert call(0) == 0
    assert lib.moe_workspace_size(ctypes.byref(c), 64) <= api.STATIC_SCRATCH_BYTES  # the decode size fits
    assert lib.moe_workspace_size(ctypes.byref(c), 4096) > api.STATIC_SCRATCH_BYTES
    assert call(4096) == api.MOE_ERR_SCRATCH
    assert api.status_string(api.MOE_ERR_SCRATCH) == "the call needs more than the static scratch"


def test_stack_argument_errors():
    lib = api.load_library()
    c = _cfg()
    w = api.moe_weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    arr = (api.moe_weights * 3)(w, w, w)
    T, V = 64, 3072
    need = lib.moe_stack_workspace_size(ctypes.byref(c), T, V)
    need0 = lib.moe_stack_workspace_size(ctypes.byref(c), T, 0)
    # the stack needs one layer's workspace, the normalised input and the head's scores
    assert need0 >= lib.moe_workspace_size(ctypes.byref(c), T) + T * 1024 * 2
    assert need >= need0 + lib.moe_codec_head_workspace_size(ctypes.byref(c), V, T)
    assert lib.moe_stack_workspace_size(ctypes.byref(c), T, -1) == 0

    def call(**kw):
        return lib.moe_stack_forward(
            ctypes.byref(c), kw.get("layers", arr), kw.get("L", 3), kw.get("x", _p()), kw.get("T", T),
            kw.get("gains", None), ctypes.c_float(kw.get("eps", 1e-6)), kw.get("head", _p(1 << 24)),
            kw.get("V", V), kw.get("h", _p(1 << 26)), kw.get("xn", None), kw.get("c0", _p(1 << 28)), _p(1 << 30),
            kw.get("ws", need), None)

    assert call(L=0) == -1
    assert call(layers=None) == -1
    assert call(eps=-1.0) == -1
    assert call(x=None) == -1
    assert call(h=None) == -1
    assert call(head=None) == -1                 # c0 needs the head
    assert call(V=0) == -1
    assert call(xn=_p()) == -1                   # xn_out may not alias x
    assert call(xn=_p(1 << 26)) == -1            # ... nor h_out
    assert call(ws=need - 256) == -3
    assert call(T=0) == 0
    w_bad = api.moe_weights(FAKE, None, FAKE, FAKE, None, FAKE, FAKE, FAKE)
    assert call(layers=(api.moe_weights * 3)(w, w, w_bad)) == -1   # every layer checked before launching


def test_codec_head_sample_argument_errors():
    lib = api.load_library()
    c = _cfg()
    need = lib.moe_codec_head_workspace_size(ctypes.byref(c), 3072, 64)

    def call(**kw):
        return lib.moe_codec_head_sample(ctypes.byref(c), _p(), _p(1 << 24), kw.get("V", 3072), kw.get("T", 64),
                                         ctypes.c_float(kw.get("temp", 1.0)), kw.get("u", _p(1 << 26)), None,
                                         _p(1 << 27), _p(1 << 28), kw.get("ws", need), None)

    assert call(temp=0.0) == -1
    assert call(temp=-1.0) == -1
    assert call(temp=float("nan")) == -1
    assert call(temp=float("inf")) == -1
    assert call(u=None) == -1
    assert call(V=0) == -1
    assert call(V=8193) == -2          # the exact pass keeps one token's logits in LDS
    assert call(ws=need - 256) == -3
    assert call(T=0) == 0


def test_attention_config_and_argument_errors():
    lib = api.load_library()
    good = api.AttnConfig(max_len=1024)
    c = good.c()
    n = lib.moe_attention_workspace_size(ctypes.byref(c), 64)
    assert n > 64 * 1024 * 2 * 3
    bad = [dict(num_kv_heads=3), dict(rope_sections=(24, 20, 21)), dict(rope_theta=0.5), dict(max_len=0),
           dict(eps=-1.0)]
    for kw in bad:
        assert lib.moe_attention_workspace_size(ctypes.byref(api.AttnConfig(**dict(dict(max_len=1024), **kw)).c()),
                                                64) == 0, kw
    w = api.moe_attn_weights(FAKE, FAKE, FAKE, FAKE)

    def call(cfg=c, **kw):
        return lib.moe_attention_decode(ctypes.byref(cfg), kw.get("w", ctypes.byref(w)), kw.get("x", _p()),
                                        kw.get("T", 64), _p(1 << 20), _p(1 << 21), _p(1 << 24), _p(1 << 26), None,
                                        kw.get("y", _p(1 << 28)), None, ctypes.c_float(1e-6), kw.get("no", None),
                                        _p(1 << 30), kw.get("ws", n), None)

    assert call(w=None) == -1
    assert call(x=None) == -1
    assert call(ws=n - 256) == -3
    assert call(T=0) == 0
    assert call(T=70000) == -2
    assert call(no=_p(1 << 28)) == -1            # norm_out may not alias y
    for kw, want in ((dict(head_dim=64, rope_sections=(12, 10, 10)), -2), (dict(num_heads=48, num_kv_heads=2), -2),
                     (dict(num_heads=16, num_kv_heads=3), -1)):
        assert call(cfg=api.AttnConfig(**dict(dict(max_len=1024), **kw)).c()) == want, kw


def test_predictor_config_and_argument_errors():
    lib = api.load_library()
    c = api.PredictorConfig().c()
    n = lib.moe_predictor_workspace_size(ctypes.byref(c), 64)
    assert n > 5 * 2 * 64 * 8 * 32 * 128 * 2     # the layers' frame caches live in the workspace
    assert lib.moe_predictor_workspace_size(ctypes.byref(c), 65) == 0   # the skinny products take up to 64
    assert lib.moe_predictor_workspace_size(ctypes.byref(api.PredictorConfig(intermediate_size=3080).c()), 8) == 0
    assert lib.moe_predictor_workspace_size(ctypes.byref(api.PredictorConfig(num_codes=1).c()), 8) == 0
    layer = api.moe_predictor_layer(api.moe_attn_weights(FAKE, FAKE, FAKE, FAKE), FAKE, FAKE, FAKE, FAKE, FAKE)
    arr = (api.moe_predictor_layer * 5)(*([layer] * 5))
    w = api.moe_predictor_weights(ctypes.cast(arr, ctypes.POINTER(api.moe_predictor_layer)), FAKE, FAKE, FAKE, FAKE)

    def call(**kw):
        return lib.moe_predictor_frame(ctypes.byref(c), kw.get("w", ctypes.byref(w)), kw.get("h", _p()),
                                       _p(1 << 20), kw.get("T", 64), _p(1 << 24), None, _p(1 << 26), kw.get("ws", n),
                                       None)

    assert call(w=None) == -1
    assert call(h=None) == -1
    assert call(ws=n - 256) == -3
    assert call(T=0) == 0
    assert call(T=100) == -2
    arr[3].down = None
    assert call() == -1                          # every layer checked before launching


def test_talker_decode_argument_errors():
    lib = api.load_library()
    c = _cfg()
    a = api.AttnConfig(max_len=1024).c()
    n = lib.moe_talker_decode_workspace_size(ctypes.byref(c), ctypes.byref(a), 64, 3072)
    assert n > lib.moe_workspace_size(ctypes.byref(c), 64) + lib.moe_attention_workspace_size(ctypes.byref(a), 64)
    bad = api.AttnConfig(max_len=1024, hidden_size=2048).c()
    assert lib.moe_talker_decode_workspace_size(ctypes.byref(c), ctypes.byref(bad), 64, 0) == 0  # hidden sizes differ
    lay = api.moe_talker_layer(api.moe_weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE),
                               api.moe_attn_weights(FAKE, FAKE, FAKE, FAKE), None, None, FAKE, FAKE)
    arr = (api.moe_talker_layer * 2)(lay, lay)

    def call(**kw):
        return lib.moe_talker_decode(ctypes.byref(c), ctypes.byref(a), kw.get("layers", arr), kw.get("L", 2),
                                     kw.get("x", _p()), kw.get("T", 64), _p(1 << 20), _p(1 << 21), None,
                                     ctypes.c_float(1e-6), kw.get("head", _p(1 << 22)), 3072, _p(1 << 24),
                                     kw.get("xn", None), _p(1 << 26), _p(1 << 28), kw.get("ws", n), None)

    assert call(L=0) == -1
    assert call(layers=None) == -1
    assert call(x=None) == -1
    assert call(head=None) == -1          # c0 needs the head
    assert call(xn=_p(1 << 24)) == -1     # xn_out may not alias h_out
    assert call(ws=n - 256) == -3
    assert call(T=0) == 0
    arr[1].v_cache = None
    assert call() == -1                   # every layer checked before launching


def test_talker_frame_argument_errors():
    lib = api.load_library()
    c = _cfg()
    a = api.AttnConfig(max_len=1024).c()
    p = api.PredictorConfig().c()
    n = lib.moe_talker_frame_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(p), 64, 3072)
    assert n > (lib.moe_talker_decode_workspace_size(ctypes.byref(c), ctypes.byref(a), 64, 3072) +
                lib.moe_predictor_workspace_size(ctypes.byref(p), 64))
    assert lib.moe_talker_frame_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(p), 65, 3072) == 0
    assert lib.moe_talker_frame_workspace_size(ctypes.byref(c), ctypes.byref(a), ctypes.byref(p), 64, 0) == 0
    lay = api.moe_talker_layer(api.moe_weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE),
                               api.moe_attn_weights(FAKE, FAKE, FAKE, FAKE), None, None, FAKE, FAKE)
    arr = (api.moe_talker_layer * 2)(lay, lay)
    player = api.moe_predictor_layer(api.moe_attn_weights(FAKE, FAKE, FAKE, FAKE), FAKE, FAKE, FAKE, FAKE, FAKE)
    parr = (api.moe_predictor_layer * 5)(*([player] * 5))
    pw = api.moe_predictor_weights(ctypes.cast(parr, ctypes.POINTER(api.moe_predictor_layer)), FAKE, FAKE, FAKE, FAKE)

    def call(**kw):
        return lib.moe_talker_frame(ctypes.byref(c), ctypes.byref(a), arr, 2, None, ctypes.c_float(1e-6),
                                    kw.get("head", _p(1 << 22)), 3072, ctypes.byref(p), kw.get("pw", ctypes.byref(pw)),
                                    kw.get("cond", _p()), kw.get("T", 64), _p(1 << 20), _p(1 << 21), _p(1 << 23),
                                    _p(1 << 24), kw.get("h", None), kw.get("xn", None), _p(1 << 26), kw.get("ws", n),
                                    None)

    assert call(head=None) == -1
    assert call(pw=None) == -1
    assert call(cond=None) == -1
    assert call(h=_p(1 << 25), xn=_p(1 << 25)) == -1   # h_out and xn_out may not alias
    assert call(ws=n - 256) == -3
    assert call(T=0) == 0
    assert call(T=65) == -2                             # the predictor takes up to 64 streams
    parr[2].gate = None
    assert call() == -1                                 # the predictor's layers are checked before any launch
