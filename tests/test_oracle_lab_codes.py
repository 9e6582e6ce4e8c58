"""Pin of the oracle's routing and c_0 to the codes the lab page prints (no GPU).

"Bài Lab tổng hợp — Qwen3-Omni & Qwen3-TTS-12Hz Architecture" states, in its
introduction and in the reading guide to steps [3A]-[4A], that frame 0 of its
NumPy lab yields the codes [4, 1, 6, 4]: c_0 from the Talker MoE step [3C],
then c_1..c_3 from its depth predictor [4A].  That lab is a miniature (hidden
6, six routed experts with Top-2, single-matrix SiLU experts, one shared
expert, no final norm before codec_head), so it does not exercise the SwiGLU
workload; what it does exercise is the routing of the production oracle:
router scores, Top-k with renormalisation (norm_topk_prob), the weighted sum
of the chosen experts plus the shared one, and the argmax that picks c_0.

This test restates the lab's input recipe (its generator, seeded 30, and the
order, shapes and spreads of its draws, as the page's script lists them) and
its frame-0 arithmetic, with the oracle's own functions for RMSNorm, the router
scores, Top-k, the renormalised weights, SiLU and the argmax.  The depth codes
come from a restatement of the lab's toy predictor (not the production
predictor the oracle implements); matching them shows the draw recipe is
aligned, so the c_0 match cannot come from a shifted random stream.
"""
import numpy as np

from oracle import moe_ref as R

# Lab miniature sizes ([1A]-[6B] configuration block of the lab script).
THINKER_DIM, TALKER_DIM = 8, 6
MEL_BINS, MEL_FRAMES = 8, 16
NUM_EXPERTS, TOP_K = 6, 2
NUM_QUANTIZERS, CODEBOOK_SIZE = 4, 8


def _lab_draws():
    """Every draw the lab makes before its frame loop, in the script's order
    (name, spread, shape); unused draws are taken to keep the stream aligned."""
    rng = np.random.default_rng(30)
    spec = [
        ("mel", 0.8, (MEL_BINS, MEL_FRAMES)),
        ("aut_proj", 0.35, (1, THINKER_DIM)),
        ("aut_q", 0.35, (THINKER_DIM, THINKER_DIM)),
        ("aut_k", 0.35, (THINKER_DIM, THINKER_DIM)),
        ("aut_v", 0.35, (THINKER_DIM, THINKER_DIM)),
        ("thinker_l12", 0.3, (THINKER_DIM, THINKER_DIM)),
        ("thinker_l24", 0.3, (THINKER_DIM, THINKER_DIM)),
        ("thinker_top", 0.3, (THINKER_DIM, THINKER_DIM)),
        ("text_emb", 0.5, (2, THINKER_DIM)),
        ("txt_w1", 0.35, (THINKER_DIM, THINKER_DIM)),
        ("txt_b1", 0.05, (THINKER_DIM,)),
        ("txt_w2", 0.35, (THINKER_DIM, TALKER_DIM)),
        ("txt_b2", 0.05, (TALKER_DIM,)),
        ("hid_w1", 0.35, (THINKER_DIM, THINKER_DIM)),
        ("hid_b1", 0.05, (THINKER_DIM,)),
        ("hid_w2", 0.35, (THINKER_DIM, TALKER_DIM)),
        ("hid_b2", 0.05, (TALKER_DIM,)),
        ("speaker_2301", 0.4, (TALKER_DIM,)),
        ("speaker_2302", 0.4, (TALKER_DIM,)),
        ("speaker_2303", 0.4, (TALKER_DIM,)),
        ("tts_pad", 0.25, (TALKER_DIM,)),
        ("codec_bos", 0.25, (TALKER_DIM,)),
        ("router", 0.4, (TALKER_DIM, NUM_EXPERTS)),
        ("experts", 0.3, (NUM_EXPERTS, TALKER_DIM, TALKER_DIM)),
        ("shared", 0.3, (TALKER_DIM, TALKER_DIM)),
        ("codec_head", 0.4, (TALKER_DIM, CODEBOOK_SIZE)),
        ("rvq_table", 0.45, (NUM_QUANTIZERS * CODEBOOK_SIZE, TALKER_DIM)),
        ("depth_attn", 0.3, (TALKER_DIM, TALKER_DIM)),
        ("depth_mlp", 0.3, (TALKER_DIM, TALKER_DIM)),
    ] + [("depth_head_%d" % j, 0.4, (TALKER_DIM, CODEBOOK_SIZE)) for j in range(NUM_QUANTIZERS - 1)]
    return {name: rng.normal(0.0, sd, size=shape) for name, sd, shape in spec}


def _frame0_text_condition(d):
    """[2A] the layer-24 hand-off, then [3A] the hidden-state ResizeMLP; frame 0
    reads the first trailing text state ([3B])."""
    h12 = np.tanh(d["text_emb"] @ d["thinker_l12"])
    h24 = h12 + R.silu(h12 @ d["thinker_l24"])
    hid = R.silu(h24 @ d["hid_w1"] + d["hid_b1"]) @ d["hid_w2"] + d["hid_b2"]
    return hid[0]


def _lab_talker_step(dual_in, speaker, d):
    """[3C] of the lab: pre-norm on the speaker-conditioned input, Top-2 of 6
    renormalised, single-matrix SiLU experts plus the shared one, residual on
    the frame input, codec_head, argmax.  The routing goes through the oracle."""
    x = R.rmsnorm((dual_in + 0.25 * speaker)[None, :], np.ones(TALKER_DIM))
    logits = R.router_logits(x, d["router"].T)  # the lab's router is [hidden, experts]
    idx = R.topk_select(logits, TOP_K)
    w = R.topk_weights(logits, idx, norm_topk_prob=True)
    routed = sum(w[0, j] * R.silu(x[0] @ d["experts"][int(idx[0, j])]) for j in range(TOP_K))
    shared = R.silu(x[0] @ d["shared"])
    h = dual_in + routed + shared
    c0 = int(R.argmax_first((h @ d["codec_head"])[None, :])[0])
    return h, c0, idx[0], w[0]


def _lab_depth_codes(h, c0, d):
    """[4A] of the lab's toy predictor: one attention-like mix over the growing
    sequence [h, embed(c_0), ...] and a SiLU MLP per step, a head per code; the
    embedding of code j is row j * codebook + c of the unified table ([6A])."""
    seq = [h, d["rvq_table"][int(c0)]]
    codes = [int(c0)]
    for step in range(NUM_QUANTIZERS - 1):
        mat = np.stack(seq)
        scores = (mat[-1] @ mat.T) / np.sqrt(TALKER_DIM)
        ctx = R.softmax(scores[None, :])[0] @ (mat @ d["depth_attn"])
        hd = mat[-1] + ctx + R.silu((mat[-1] + ctx) @ d["depth_mlp"])
        ck = int(R.argmax_first((hd @ d["depth_head_%d" % step])[None, :])[0])
        codes.append(ck)
        seq.append(d["rvq_table"][(step + 1) * CODEBOOK_SIZE + ck])
    return codes


def test_lab_frame0_codes_match_the_page():
    d = _lab_draws()
    dual_in = d["codec_bos"] + _frame0_text_condition(d)  # [3B]: first frame starts from the BOS embedding
    h, c0, idx, w = _lab_talker_step(dual_in, d["speaker_2302"], d)
    assert abs(float(w.sum()) - 1.0) < 1e-12  # the page's own check on the Top-k weights
    assert c0 == 4  # the page's frame-0 c_0
    assert _lab_depth_codes(h, c0, d) == [4, 1, 6, 4]  # the page's frame-0 codes


def test_lab_codes_catch_a_dropped_second_expert():
    """How much the printed codes pin: the miniature's codes are coarse (an
    8-way argmax), so most routing mistakes leave them unchanged (plain softmax
    weights, the wrong experts, no shared expert: checked by hand, all still
    give [4, 1, 6, 4]).  Dropping the second chosen expert (Top-1 weight only)
    does change c_0, and the pin catches that."""
    d = _lab_draws()
    dual_in = d["codec_bos"] + _frame0_text_condition(d)
    x = R.rmsnorm((dual_in + 0.25 * d["speaker_2302"])[None, :], np.ones(TALKER_DIM))
    logits = R.router_logits(x, d["router"].T)
    idx = R.topk_select(logits, TOP_K)
    h = dual_in + R.silu(x[0] @ d["experts"][int(idx[0, 0])]) + R.silu(x[0] @ d["shared"])
    assert int(R.argmax_first((h @ d["codec_head"])[None, :])[0]) != 4
