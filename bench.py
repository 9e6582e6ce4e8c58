#!/usr/bin/env python3
"""Benchmark of the Talker MoE feed-forward layer on one MI355X.

One step = one whole layer (route, group, routed + shared SwiGLU experts,
combine) over one batch of synthetic tokens already resident in HBM.  The
headline line is the decode workload (T=64 tokens: 64 streams x one 80 ms
frame); the prefill workload (T=4096) is reported alongside.  Weights rotate
over several independently seeded layers so that timed reads come from HBM and
not from the 256 MB Infinity Cache.

    python bench.py [--steps K] [--warmup W] [--rotate R] [--no-cpu-baseline]

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
METRIC = "Talker MoE layer tokens/s (T=64 decode, T=4096 prefill); % HBM/MFMA peak"


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def decode_path(shape, T):
    """Whether the library runs the decode-size layer (router scores and per-token
    selection, one expert launch over (expert, 64-wide slice) items and the shared
    expert's slices, partial-row combine): at most 64
    tokens, hidden 1024, E <= 128, k <= 8, I and I_s multiples of 64."""
    return (1 <= T <= 64 and shape.H == 1024 and shape.E <= 128 and shape.k <= 8 and shape.I % 64 == 0
            and shape.Is % 64 == 0)


def layer_costs(shape, T, touched):
    """Algorithmic bytes and flops of one layer step and of its dominant kernel.

    Weight bytes count each touched expert once (bf16); activations count the
    token rows read and written once; routing outputs 8 bytes per (token, slot).
    At decode sizes the dominant kernel is the expert launch: every touched
    expert's weights, the shared expert's down weights and its gate/up output,
    and the token rows it reads (its partial output rows are design traffic, not
    counted).  Otherwise it is the grouped gate/up pass.
    """
    H, E, k, I, Is = shape.H, shape.E, shape.k, shape.I, shape.Is
    expert_b = 3 * I * H * 2
    shared_b = 3 * Is * H * 2
    router_b = E * H * 2
    layer_bytes = touched * expert_b + shared_b + router_b + 2 * T * H * 2 + T * k * 8
    layer_flops = T * (2 * H * E + 6 * H * I * k + 6 * H * Is)
    if decode_path(shape, T):
        # the expert launch: routed experts' weights, the shared expert's down
        # weights and gate/up output, the token rows (the shared gate/up runs in
        # the router's launch)
        return (layer_bytes, layer_flops, touched * expert_b + Is * H * 2 + T * Is * 2 + T * H * 2,
                T * (6 * H * I * k + 2 * H * Is))
    gu_bytes = touched * 2 * I * H * 2 + 2 * Is * H * 2 + T * H * 2 + T * k * I * 2 + T * Is * 2
    gu_flops = T * (4 * H * I * k + 4 * H * Is)
    return layer_bytes, layer_flops, gu_bytes, gu_flops


# Sources whose change invalidates the recorded HBM counters of the decode expert kernel.
TRAFFIC_SOURCES = ("decode.hip", "common.hpp", "kernels.hpp", "api.hip")


def measured_traffic():
    """HBM bytes per launch of the decode expert kernel from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summary in profiles/ (scaled by the copy-kernel
    calibration stated there), with where they come from; (None, reason) when
    the summary is missing or any source that shapes the kernel has changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_bytes_pmc.md")
    try:
        text = open(path).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None, "no counter record"
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "sparse_moe_transformer_talker_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None, "the kernel's sources changed since the counters were taken"
    return float(rec["traffic_bytes_per_launch"]), ("rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel source "
                                                    "(profiles/hbm_bytes_pmc.md), not measured in this run")


def pct(a, q):
    return float(np.percentile(np.asarray(a), q)) if len(a) else None


def measure(api, torch, INP, shape, T, weight_sets, steps, warmup, bias=None):
    cfg = api.Config(shape.H, shape.E, shape.k, shape.I, shape.Is, True, torch.bfloat16)
    dev = torch.device("cuda", 0)
    if bias is not None:
        b = torch.from_numpy(np.asarray(bias, np.float32)).to(dev)
        weight_sets = [dict(w, router_bias=b) for w in weight_sets]
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    xs = [to_dev(INP.activations(T, shape.H, 30 + i, "bf16")) for i in range(len(weight_sets))]
    ys = [torch.empty_like(x) for x in xs]
    ws = api.workspace(api.moe_workspace_size(cfg, T), dev)
    structs = [api.weights_struct(w) for w in weight_sets]
    R = len(weight_sets)

    # routing of each weight set: number of experts that receive tokens
    touched, max_rows = [], []
    counts = torch.empty(shape.E, dtype=torch.int32, device=dev)
    for i in range(R):
        api.moe_layer_forward(cfg, structs[i], xs[i], y=ys[i], counts=counts, ws=ws)
        touched.append(int((counts > 0).sum().item()))
        max_rows.append(int(counts.max().item()))
    torch.cuda.synchronize()

    for i in range(warmup):
        api.moe_layer_forward(cfg, structs[i % R], xs[i % R], y=ys[i % R], ws=ws)
    torch.cuda.synchronize()

    # HIP graphs: the R layers (one per weight set) back to back in one graph, as
    # consecutive layers of the stack run, and each layer alone for a remainder
    chain = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chain):
        for i in range(R):
            api.moe_layer_forward(cfg, structs[i], xs[i], y=ys[i], ws=ws)
    graphs = []
    for i in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            api.moe_layer_forward(cfg, structs[i], xs[i], y=ys[i], ws=ws)
        graphs.append(g)
    for i in range(max(1, warmup // R)):
        chain.replay()
    torch.cuda.synchronize()

    def timed(fn):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            fn(i)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop), time.perf_counter() - t0

    def replay(n):  # exactly n layer steps
        for _ in range(n // R):
            chain.replay()
        for i in range(n % R):
            graphs[i].replay()

    # timed region: exactly `steps` layer steps (graph replay), then the same eagerly
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    replay(steps)
    stop.record()
    torch.cuda.synchronize()
    gpu_ms, wall = start.elapsed_time(stop), time.perf_counter() - t0
    eager_ms, _ = timed(lambda i: api.moe_layer_forward(cfg, structs[i % R], xs[i % R], y=ys[i % R], ws=ws))

    # per-step times on the graph path: each layer's own graph replayed with an
    # event recorded on the stream between consecutive replays
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    pev[0].record()
    for i in range(steps):
        graphs[i % R].replay()
        pev[i + 1].record()
    torch.cuda.synchronize()
    graph_step_us = [pev[i].elapsed_time(pev[i + 1]) * 1e3 for i in range(steps)]

    # the same steps with HIP events at every stage boundary, on the library's stream
    # (events 6 and 7 are timestamped by the dominant kernel's own launch: the
    # decode expert kernel, or the gate/up pass at larger sizes)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(steps)]
    for row in evs:  # torch creates the HIP event on first record; the library re-records it
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        api.moe_layer_forward(cfg, structs[i % R], xs[i % R], y=ys[i % R], ws=ws, stage_events=evs[i])
    torch.cuda.synchronize()
    names = ["route", "permute", "experts" if decode_path(shape, T) else "gate_up",
             "down" if not decode_path(shape, T) else "(none)", "combine"]
    stages = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) * 1e3 for i in range(steps)] for j, n in enumerate(names)}
    step_us = [evs[i][0].elapsed_time(evs[i][5]) * 1e3 for i in range(steps)]
    gu_kernel_us = [evs[i][6].elapsed_time(evs[i][7]) * 1e3 for i in range(steps)]

    mean_touched = float(np.mean([touched[i % R] for i in range(steps)]))
    lb, lf, gb, gf = layer_costs(shape, T, mean_touched)
    s = gpu_ms / 1e3 / steps
    gu_s = float(np.mean(gu_kernel_us)) * 1e-6
    return {
        "T": T, "steps": steps, "warmup": warmup, "weight_sets": R,
        "ms_per_step": gpu_ms / steps, "wall_ms_per_step": wall * 1e3 / steps,
        "eager_ms_per_step": eager_ms / steps,
        "tokens_per_s": T / s, "touched_experts": touched, "max_rows_per_expert": max_rows,
        "layer_bytes": lb, "layer_flops": lf, "layer_hbm_frac": lb / s / (HBM_PEAK_GBS * 1e9),
        "layer_mfma_frac": lf / s / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "step_us": {"p50": pct(graph_step_us, 50), "p95": pct(graph_step_us, 95), "p99": pct(graph_step_us, 99),
                    "mean": float(np.mean(graph_step_us)),
                    "timing": "per-replay events between single-layer graph replays (same rotation)"},
        "eager_step_us": {"p50": pct(step_us, 50), "p95": pct(step_us, 95), "p99": pct(step_us, 99)},
        "stages_us_mean": {n: float(np.mean(v)) for n, v in stages.items() if n != "(none)"},
        "kernel": {"bytes": gb, "flops": gf, "mean_us": gu_s * 1e6,
                    "p50_us": pct(gu_kernel_us, 50), "p99_us": pct(gu_kernel_us, 99),
                    "timing": "kernel start/end timestamps of its own launch (hipExtLaunchKernel events)",
                    "gbs": gb / gu_s / 1e9, "tflops": gf / gu_s / 1e12},
    }


def measure_stack(api, torch, INP, shape, T, weight_sets, L, frames, vocab=3072):
    """The L-layer stack and the codec head (moe_stack_forward) as one HIP graph:
    layer l uses weight set l % len(weight_sets); per frame, T tokens through all
    L layers, the final RMSNorm and the c_0 argmax."""
    cfg = api.Config(shape.H, shape.E, shape.k, shape.I, shape.Is, True, torch.bfloat16)
    dev = torch.device("cuda", 0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    structs = [api.weights_struct(weight_sets[l % len(weight_sets)]) for l in range(L)]
    head = to_dev(INP.stack_weights(shape, 0, 30, 0.02, "bf16", vocab, 50)["codec_head"])
    gains = torch.ones((L + 1, shape.H), dtype=torch.float32, device=dev)
    x = to_dev(INP.activations(T, shape.H, 30, "bf16"))
    h = torch.empty_like(x)
    c0 = torch.empty(T, dtype=torch.int32, device=dev)
    ws = api.workspace(api.moe_stack_workspace_size(cfg, T, vocab), dev)
    run = lambda: api.moe_stack_forward(cfg, structs, x, gains, 1e-6, head, h_out=h, c0=c0, ws=ws)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(frames):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    frame_ms = start.elapsed_time(stop) / frames
    start.record()
    for _ in range(frames):
        run()
    stop.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / frames
    # the head alone on the final state: exact argmax against the sampled draw
    xn = torch.empty_like(x)
    api.moe_stack_forward(cfg, structs[:1], x, gains[:2], 1e-6, None, xn_out=xn, ws=ws)
    u = torch.rand(T, dtype=torch.float64, device=dev)
    c0s = torch.empty_like(c0)
    hws = api.workspace(api.moe_stack_workspace_size(cfg, T, vocab), dev)
    head_us = {}
    for name, fn in (("argmax", lambda: api.moe_codec_head_argmax(cfg, xn, head, c0=c0s, ws=hws)),
                     ("sample", lambda: api.moe_codec_head_sample(cfg, xn, head, u, 1.0, c0=c0s, ws=hws))):
        fn()
        torch.cuda.synchronize()
        hg = torch.cuda.CUDAGraph()  # 20 calls in one graph: device time, not launch overhead
        with torch.cuda.graph(hg):
            for _ in range(20):
                fn()
        hg.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(5):
            hg.replay()
        stop.record()
        torch.cuda.synchronize()
        head_us[name] = start.elapsed_time(stop) * 1e3 / 100
    return {"workload": "talker_moe_stack%d_codec_head_T%d" % (L, T), "layers": L, "tokens": T, "vocab": vocab,
            "weight_sets_rotated": len(weight_sets), "frames": frames,
            "frame_us": frame_ms * 1e3, "per_layer_us": frame_ms * 1e3 / L, "eager_frame_us": eager_ms * 1e3,
            "codec_head_us": head_us,
            "tokens_per_s": T / (frame_ms / 1e3),
            "timing": "one HIP graph per frame: RMSNorm, L layers (combine + residual + next RMSNorm fused), "
                      "codec_head argmax"}


def measure_attention(api, torch, INP, T, L, steps, R=4):
    """One decode step of the attention block for T streams with L cached positions
    each (the new token makes L + 1), R layers' weights and caches rotated in one
    graph so that reads come from HBM."""
    shape = INP.TALKER_ATTN
    dev = torch.device("cuda", 0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    acfg = api.AttnConfig(max_len=L + 1)
    layers = []
    for r in range(R):
        w = INP.attention_weights(shape, 60 + r)
        wd = {"w_qkv": to_dev(w["w_qkv"]), "w_o": to_dev(w["w_o"]),
              "q_norm": torch.from_numpy(w["q_norm"]).to(dev), "k_norm": torch.from_numpy(w["k_norm"]).to(dev)}
        kv = INP.kv_cache(T, shape, L + 1, 61 + r)
        layers.append((api.attn_weights_struct(wd), wd, to_dev(kv["k"]),
                       to_dev(np.ascontiguousarray(np.swapaxes(kv["v"], 2, 3)))))
    lens = torch.full((T,), L, dtype=torch.int32, device=dev)
    pos = torch.from_numpy(INP.speech_positions(np.full(T, L, np.int32))).to(dev)
    x = to_dev(INP.activations(T, shape.H, 62, "bf16"))
    res = to_dev(INP.activations(T, shape.H, 63, "bf16"))
    y = torch.empty_like(x)
    ws = api.workspace(api.moe_attention_workspace_size(acfg, T), dev)
    run = lambda i: api.moe_attention_decode(acfg, layers[i][0], x, pos, lens, layers[i][2], layers[i][3],
                                             residual=res, y=y, ws=ws)
    for i in range(R):
        run(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            run(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // R)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / (reps * R)
    d, nq, nkv, H = shape.head_dim, shape.n_heads, shape.n_kv_heads, shape.H
    kv_bytes = T * nkv * (L + 1) * d * 2 * 2
    w_bytes = ((nq + 2 * nkv) * d * H + H * nq * d) * 2
    act_bytes = T * H * 2 * 3 + T * (nq + 2 * nkv) * d * 2 * 2 + T * nq * d * 2 * 2
    total = kv_bytes + w_bytes + act_bytes
    return {"workload": "talker_attention_decode_T%d_ctx%d" % (T, L + 1), "streams": T, "positions": L + 1,
            "layers_rotated": R, "us_per_step": us, "tokens_per_s": T / (us * 1e-6),
            "bytes_per_step": total, "kv_bytes": kv_bytes, "weight_bytes": w_bytes,
            "hbm_frac": total / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "timing": "HIP graph of %d layers' attention steps back to back" % R}


def measure_talker_frame(api, torch, INP, shape, T, ctx, weight_sets, L, frames, vocab=3072):
    """Consecutive Dual-Track frames (moe_talker_frame): the frame input (previous frame's code-embedding mean +
    text condition), the Talker's decode step through L whole layers (attention over the cached positions, then
    the MoE) and the codec head, the depth predictor's frame and the frame's end (next input, positions and cache
    lengths advanced on the device).  One frame is captured as a HIP graph and replayed `frames` times, the next
    text condition copied in before each replay; the caches start at ctx positions and grow by one per frame.
    Layer l uses MoE weight set l % R and attention weight set l % R; every layer has its own caches (filled on
    the device with seeded normal values)."""
    dev = torch.device("cuda", 0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    ashape, pshape = INP.TALKER_ATTN, INP.PREDICTOR
    R = len(weight_sets)
    attn_w = []
    for r in range(R):
        w = INP.attention_weights(ashape, 60 + r)
        attn_w.append({"w_qkv": to_dev(w["w_qkv"]), "w_o": to_dev(w["w_o"]),
                       "q_norm": torch.from_numpy(w["q_norm"]).to(dev), "k_norm": torch.from_numpy(w["k_norm"]).to(dev)})
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    max_len = (ctx + frames + 2 + 31) // 32 * 32
    layers = []
    for l in range(L):
        kc = torch.randn((T, ashape.n_kv_heads, max_len, ashape.head_dim), generator=gen, device=dev,
                         dtype=torch.float32).to(torch.bfloat16)
        vc = (0.64 * torch.randn((T, ashape.n_kv_heads, ashape.head_dim, max_len), generator=gen, device=dev,
                                 dtype=torch.float32)).to(torch.bfloat16)
        layers.append({"moe": api.weights_struct(weight_sets[l % R]), "attn": attn_w[l % R], "k_cache": kc,
                       "v_cache": vc})
    arr = api.talker_layers_struct(layers)
    cfg = api.Config(shape.H, shape.E, shape.k, shape.I, shape.Is, True, torch.bfloat16)
    acfg = api.AttnConfig(max_len=max_len)
    head = to_dev(INP.stack_weights(shape, 0, 30, 0.02, "bf16", vocab, 50)["codec_head"])
    pw = INP.predictor_weights(pshape, 80)
    pdev = lambda a: to_dev(a) if a.dtype == np.uint16 else torch.from_numpy(a).to(dev)
    pwd = {k: pdev(v) for k, v in pw.items() if k != "layers"}
    pwd["layers"] = [{k: pdev(v) for k, v in lw.items()} for lw in pw["layers"]]
    pst = api.predictor_weights_struct(pwd)
    pc = api.PredictorConfig()
    conds = torch.stack([to_dev(INP.activations(T, shape.H, 200 + f, "bf16")) for f in range(frames + 2)])
    prev = to_dev(INP.activations(T, shape.H, 199, "bf16"))  # the codec BOS embedding
    lens = torch.full((T,), ctx, dtype=torch.int32, device=dev)
    pos = torch.from_numpy(INP.speech_positions(np.full(T, ctx, np.int32))).to(dev)
    cond = torch.empty((T, shape.H), dtype=torch.bfloat16, device=dev)
    codes = torch.empty((pc.num_codes, T), dtype=torch.int32, device=dev)
    ws = api.workspace(api.moe_talker_frame_workspace_size(cfg, acfg, pc, T, vocab), dev)
    run = lambda: api.moe_talker_frame(cfg, acfg, arr, None, 1e-6, head, pc, pst, cond, prev, pos, lens,
                                       codes=codes, ws=ws)
    cond.copy_(conds[0])
    run()  # frame 0, eager
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    cond.copy_(conds[1])
    g.replay()  # frame 1
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for f in range(frames):
        cond.copy_(conds[2 + f])
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / frames
    assert int(lens[0].item()) == ctx + frames + 2, "positions advanced on the device"
    touched = 124  # experts a T=64 batch touches (the decode measurement's count for these weight sets)
    moe_b = touched * 3 * shape.I * shape.H * 2 + 3 * shape.Is * shape.H * 2 + shape.E * shape.H * 2
    mid = ctx + 2 + frames // 2  # mean cached positions over the timed frames
    attn_b = T * ashape.n_kv_heads * (mid + 1) * ashape.head_dim * 4 + (
        (ashape.n_heads + 2 * ashape.n_kv_heads) * ashape.head_dim * shape.H + shape.H * ashape.n_heads *
        ashape.head_dim) * 2
    p_layer = sum(v.numel() * v.element_size() for lw in pwd["layers"] for v in lw.values())
    pred_b = pshape.num_codes * p_layer + 2 * (pshape.num_codes - 1) * pshape.codebook * shape.H * 2
    alg = L * (moe_b + attn_b) + vocab * shape.H * 2 + pred_b
    return {"workload": "talker_frame_%dlayers_predictor_T%d_ctx%d" % (L, T, ctx), "layers": L, "streams": T,
            "frames_timed": frames, "bytes_per_frame": alg, "hbm_frac": alg / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "bytes_note": "touched experts, shared expert and router per layer; keys and values of the cached "
                          "positions and the attention weights per layer; codec head; the predictor's layer "
                          "weights once per position, its 15 heads and 15 tables once",
            "positions_start": ctx, "frame_us": us, "per_layer_us": us / L, "tokens_per_s": T / (us * 1e-6),
            "timing": "one HIP graph per frame (frame input, %d Talker layers, codec head, predictor frame, next "
                      "input and positions on the device), replayed for consecutive frames with the next text "
                      "condition copied in before each replay" % L}


def measure_predictor(api, torch, INP, T, frames):
    """One frame of the depth code predictor (16 positions x 5 layers + 15 heads) for T streams, as one graph."""
    shape = INP.PREDICTOR
    dev = torch.device("cuda", 0)
    w = INP.predictor_weights(shape, 80)
    todev = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
                       if a.dtype == np.uint16 else torch.from_numpy(a).to(dev))
    wd = {k: todev(v) for k, v in w.items() if k != "layers"}
    wd["layers"] = [{k: todev(v) for k, v in lw.items()} for lw in w["layers"]]
    pc = api.PredictorConfig()
    wst = api.predictor_weights_struct(wd)
    h = todev(INP.activations(T, shape.H, 81, "bf16"))
    c0 = torch.from_numpy(np.random.default_rng(81).integers(0, shape.c0_vocab, T).astype(np.int32)).to(dev)
    codes = torch.empty((shape.num_codes, T), dtype=torch.int32, device=dev)
    ws = api.workspace(api.moe_predictor_workspace_size(pc, T), dev)
    api.moe_predictor_frame(pc, wst, h, c0, codes=codes, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_predictor_frame(pc, wst, h, c0, codes=codes, ws=ws)
    g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(frames):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / frames
    layer_bytes = sum(v.numel() * v.element_size() for lw in wd["layers"] for v in lw.values())
    head_bytes = (shape.num_codes - 1) * shape.codebook * shape.H * 2
    alg = shape.num_codes * layer_bytes + head_bytes + shape.num_codes * T * shape.H * 2
    return {"workload": "depth_code_predictor_frame_T%d" % T, "streams": T, "positions": shape.num_codes,
            "bytes_per_frame": alg, "hbm_frac": alg / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "bytes_note": "every position reads every layer's weights once (the steps are sequential), each head once",
            "layers": shape.layers, "frame_us": us, "position_us": us / shape.num_codes,
            "codes_per_s": T * (shape.num_codes - 1) / (us * 1e-6), "layer_weight_bytes": layer_bytes,
            "timing": "one HIP graph per frame: 16 positions x 5 layers (attention + SwiGLU) and 15 heads"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        return 1


def oracle_rate(fn, units, unit, seconds, sample):
    """Oracle baseline: fn() repeated for about `seconds` (the first call untimed); units per call."""
    fn()
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": units * n / el, "unit": unit, "cores": blas_threads(), "kind": "oracle",
            "sample": "%s; %d calls in %.1f s" % (sample, n, el)}


def oracle_baselines(INP, shape, seconds):
    """Bounded oracle timings beside the attention step, the Talker frame, the predictor and sampling."""
    from oracle import attention_ref as A
    from oracle import moe_ref as R
    from oracle import predictor_ref as P
    out = {}
    ash = INP.TALKER_ATTN
    aw = INP.attention_weights(ash, 60)
    aw64 = {k: (INP.to_f64(v, "bf16") if v.dtype == np.uint16 else v.astype(np.float64)) for k, v in aw.items()}

    def attn_inputs(T, ctx):
        kv = INP.kv_cache(T, ash, ctx + 1, 61)
        lens = np.full(T, ctx, np.int32)
        return (INP.to_f64(INP.activations(T, ash.H, 62, "bf16"), "bf16"), INP.speech_positions(lens),
                INP.to_f64(kv["k"], "bf16"), INP.to_f64(kv["v"], "bf16"), lens)

    x, pos, kc, vc, lens = attn_inputs(64, 1023)
    out["attention"] = oracle_rate(lambda: A.attention_decode(x, aw64, pos, kc, vc, lens, ash.n_heads, ash.n_kv_heads),
                                   64, "tokens/s", seconds, "fp64 numpy oracle, one attention step, 64 streams x "
                                   "1024 positions")
    x8, pos8, kc8, vc8, lens8 = attn_inputs(8, 1023)
    w = INP.layer_weights(shape, 30, 0.02, "bf16")
    w64 = {k: INP.to_f64(v, "bf16") for k, v in w.items()}

    def talker_layer():
        a = A.attention_decode(R.rmsnorm(x8, np.ones(shape.H)), aw64, pos8, kc8, vc8, lens8,
                               ash.n_heads, ash.n_kv_heads)["y"] + x8
        return a + R.moe_layer(R.rmsnorm(a, np.ones(shape.H)), w64, shape.k)["y"]

    out["talker_frame"] = oracle_rate(talker_layer, 8, "tokens x layers/s", seconds,
                                      "fp64 numpy oracle, one Talker decoder layer (attention over 1024 positions, "
                                      "then the MoE), 8 streams")
    ps = INP.PREDICTOR
    pw = INP.predictor_weights(ps, 80)
    f64 = lambda a: INP.to_f64(a, "bf16") if a.dtype == np.uint16 else a.astype(np.float64)
    pw64 = {k: f64(v) for k, v in pw.items() if k != "layers"}
    pw64["layers"] = [{k: f64(v) for k, v in lw.items()} for lw in pw["layers"]]
    h4 = INP.to_f64(INP.activations(4, ps.H, 81, "bf16"), "bf16")
    c04 = np.arange(4) * 7
    out["predictor"] = oracle_rate(lambda: P.predictor_frame(h4, c04, pw64), 4 * (ps.num_codes - 1), "codes/s",
                                   seconds, "fp64 numpy oracle, one predictor frame, 4 streams")
    head = INP.to_f64(INP.stack_weights(shape, 0, 30, 0.02, "bf16", 3072, 50)["codec_head"], "bf16")
    xs = INP.to_f64(INP.activations(64, shape.H, 40, "bf16"), "bf16")
    u = np.random.default_rng(41).random(64)
    out["sampling"] = oracle_rate(lambda: R.sample_inverse_cdf(R.codec_head_logits(xs, head), u), 64, "tokens/s",
                                  seconds, "fp64 numpy oracle, codec head + inverse-transform draw, 64 tokens")
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_conditions(torch, steps, warmup, rotate):
    """The conditions of the run: the GPU (name, architecture, compute units,
    memory), its shader and memory clock levels as the driver's sysfs reports
    them under a matrix-product load after the timed loops (None where they
    cannot be read), the HIP and torch versions, the host CPU, the seeds of the
    synthetic inputs and the counts of the timed loop.  Reads files only: no
    tool is started."""
    import glob
    p = torch.cuda.get_device_properties(0)
    cond = {"gpu": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "hbm_gib": round(p.total_memory / 2 ** 30, 1),
            "sclk_dpm_level": None, "mclk_dpm_level": None, "hip": torch.version.hip, "torch": torch.__version__,
            "host_cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "seeds": {"weights": [30 + i for i in range(rotate)], "activations": "weight seed + 10000",
                      "zipf_ranks": 20030},
            "timed_steps": steps, "warmup_steps": warmup}
    dev_dir = None
    bus = getattr(p, "pci_bus_id", None)
    if bus is not None:
        cand = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0) or 0, bus,
                                                         getattr(p, "pci_device_id", 0) or 0)
        dev_dir = cand if os.path.exists(os.path.join(cand, "pp_dpm_sclk")) else None
    if dev_dir is None:
        found = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
        dev_dir = os.path.dirname(found[0]) if len(found) == 1 else None
    if dev_dir is not None:
        # the levels read while a stream of large bf16 products keeps the GPU
        # busy (the DPM level drops once it idles)
        a = torch.ones(8192, 8192, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        for _ in range(40):
            b = a @ a
        time.sleep(0.005)
        for key, fname in (("sclk_dpm_level", "pp_dpm_sclk"), ("mclk_dpm_level", "pp_dpm_mclk")):
            try:
                for line in open(os.path.join(dev_dir, fname)):
                    if line.rstrip().endswith("*"):  # the current level
                        cond[key] = line.split(":", 1)[-1].strip(" *\n")
            except OSError:
                pass
        torch.cuda.synchronize()
        del a, b
        cond["clocks_read"] = ("the DPM level sysfs marks current during 40 back-to-back 8192^3 bf16 products, "
                               "after the timed loops: a coarse indicator, not a measured clock")
    return cond


def cpu_baseline(INP, shape, T, seconds, threads=None):
    """The oracle (fp64 numpy, never tuned) timed for about `seconds` on one
    Talker layer at T tokens; threads=1 limits BLAS to one thread."""
    from oracle import moe_ref as R
    w = INP.layer_weights(shape, 30, 0.02, "bf16")
    w64 = {k: INP.to_f64(v, "bf16") for k, v in w.items()}
    x64 = INP.to_f64(INP.activations(T, shape.H, 30, "bf16"), "bf16")

    def run():
        R.moe_layer(x64, w64, shape.k)  # first call outside the clock
        n, t0 = 0, time.perf_counter()
        while True:
            R.moe_layer(x64, w64, shape.k)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return n, el, blas_threads()

    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads, user_api="blas"):
            n, el, used = run()
    else:
        n, el, used = run()
    return {"value": T * n / el, "unit": "tokens/s", "cores": used, "kind": "oracle", "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "sample": "fp64 numpy oracle, one Talker MoE layer at T=%d (seed 30), %d calls in %.1f s with %d BLAS "
                      "threads" % (T, n, el, used)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=4, help="independently seeded weight sets cycled per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--stack-layers", type=int, default=20)
    ap.add_argument("--stack-frames", type=int, default=20)
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-predictor", action="store_true")
    ap.add_argument("--no-talker-frame", action="store_true")
    ap.add_argument("--no-reports", action="store_true",
                    help="skip the report-only workloads (Zipf-skewed T=8192 layer, 20-layer stack at T=1024)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB once (a plain copy kernel of known size, "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_moe_transformer_talker_amd import api
    from sparse_moe_transformer_talker_amd import inputs as INP

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    api.load_library()
    shape = INP.TALKER
    dev = torch.device("cuda", 0)
    log("generating %d seeded weight sets" % args.rotate)
    sets = []
    for i in range(args.rotate):
        w = INP.layer_weights(shape, 30 + i, 0.02, "bf16")
        sets.append({k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
                     for k, v in w.items()})
        sets[-1]["router_bias"] = None
    dec = None
    if not args.no_decode:
        log("decode T=64")
        dec = measure(api, torch, INP, shape, 64, sets, args.steps, args.warmup)
        log("decode: %.2f us/step, %.3f M tok/s, expert kernel %.1f us" % (
            dec["ms_per_step"] * 1e3, dec["tokens_per_s"] / 1e6, dec["kernel"]["mean_us"]))
    pre = None
    if not args.no_prefill:
        log("prefill T=4096")
        pre = measure(api, torch, INP, shape, 4096, sets, args.steps, args.warmup)
        log("prefill: %.2f us/step, %.2f M tok/s" % (pre["ms_per_step"] * 1e3, pre["tokens_per_s"] / 1e6))
    stack = None
    if not args.no_stack and not args.no_decode:
        log("stack: %d layers + codec head, T=64" % args.stack_layers)
        stack = measure_stack(api, torch, INP, shape, 64, sets, args.stack_layers, args.stack_frames)
        log("stack: %.1f us/frame, %.2f us/layer" % (stack["frame_us"], stack["per_layer_us"]))
    attn = None
    if not args.no_attention and not args.no_decode:
        log("attention decode: 64 streams x 1024 cached positions")
        attn = measure_attention(api, torch, INP, 64, 1023, args.steps)
        log("attention: %.2f us/step, %.1f%% of HBM peak" % (attn["us_per_step"], 100 * attn["hbm_frac"]))
    tframe = None
    if not args.no_talker_frame and not args.no_decode:
        log("talker frames: input + 20 layers (attention + MoE) + codec head + predictor, 64 streams x ~1024 "
            "positions, consecutive frames")
        tframe = measure_talker_frame(api, torch, INP, shape, 64, 1000, sets, 20, max(5, args.stack_frames // 2))
        log("talker frame: %.1f us/frame" % tframe["frame_us"])
    pred = None
    if not args.no_predictor and not args.no_decode:
        log("depth code predictor frame: 64 streams")
        pred = measure_predictor(api, torch, INP, 64, max(5, args.stack_frames // 2))
        log("predictor: %.1f us/frame, %.1f us/position" % (pred["frame_us"], pred["position_us"]))
    reports = None
    if not args.no_reports and not args.no_decode and not args.no_prefill:
        c = INP.WORKLOADS["skew_t8192"]
        log("report: Zipf-skewed layer T=8192")
        sk = measure(api, torch, INP, shape, 8192, sets, max(10, args.steps // 4), max(2, args.warmup // 4),
                     bias=INP.zipf_router_bias(shape.E, c["zipf_s"], c["zipf_seed"]))
        log("report: stack of 20 layers + codec head, T=1024")
        st1k = measure_stack(api, torch, INP, shape, 1024, sets, 20, max(5, args.stack_frames // 4))
        reports = {
            "skew": {"workload": "talker_moe_layer_zipf%.1f_T8192" % c["zipf_s"], "tokens_per_s": sk["tokens_per_s"],
                     "ms_per_step": sk["ms_per_step"], "mfma_frac": sk["layer_mfma_frac"],
                     "hbm_frac": sk["layer_hbm_frac"], "touched_experts": sk["touched_experts"],
                     "max_rows_per_expert": sk["max_rows_per_expert"], "stages_us_mean": sk["stages_us_mean"]},
            "stack_T1024": st1k,
        }
        log("skew: %.1f us/step; stack T=1024: %.1f us/frame" % (sk["ms_per_step"] * 1e3, st1k["frame_us"]))
    if args.copy_calibration_mb:
        # one device-to-device copy of n bytes from a source evicted from the
        # caches (a 2 GiB sweep after it was written), so the counters of that
        # dispatch read n bytes from HBM and write n bytes
        n = args.copy_calibration_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        sweep = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        sweep.fill_(1)
        torch.cuda.synchronize()
        del sweep
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy of %d MiB done" % args.copy_calibration_mb)
    if dec is None:
        print(json.dumps({"prefill": pre}), flush=True)
        return
    cpu = cpu_extra = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle): decode T=64 and prefill T=4096, all threads and one thread (~%.0f s)"
            % (2 * args.cpu_seconds))
        cpu = cpu_baseline(INP, shape, 64, args.cpu_seconds / 2)
        cpu_extra = {"decode_T64_1thread": cpu_baseline(INP, shape, 64, args.cpu_seconds / 4, threads=1),
                     "prefill_T4096": cpu_baseline(INP, shape, 4096, args.cpu_seconds / 2),
                     "prefill_T4096_1thread": cpu_baseline(INP, shape, 4096, args.cpu_seconds / 4, threads=1)}

    extra_cpu = None
    if not args.no_cpu_baseline and (attn or tframe or pred):
        log("oracle baselines for attention, the Talker frame, the predictor and sampling (~%.0f s each)"
            % (args.cpu_seconds / 3))
        extra_cpu = oracle_baselines(INP, shape, args.cpu_seconds / 3)

    g = dec["kernel"]
    traffic, traffic_source = measured_traffic()
    layer_gbs = dec["layer_bytes"] / (dec["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": dec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "talker_moe_layer_decode_T64", "tokens": 64, "hidden": shape.H,
                   "experts": shape.E, "top_k": shape.k, "expert_intermediate": shape.I,
                   "shared_intermediate": shape.Is, "weight_sets_rotated": args.rotate},
        "roofline": {"bound": "hbm",
                     "kernel": "decode expert kernel: every (expert, 64-wide slice) item of the touched routed "
                               "experts (gate/up + SwiGLU + partial down) and the shared expert's down tiles, "
                               "in one launch",
                     "achieved": g["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": g["gbs"] / HBM_PEAK_GBS, "traffic": traffic, "traffic_source": traffic_source,
                     "bytes_per_launch": g["bytes"], "mean_us": g["mean_us"],
                     "timing": g["timing"],
                     "layer": {"achieved": layer_gbs, "frac": layer_gbs / HBM_PEAK_GBS,
                               "bytes_per_step": dec["layer_bytes"], "us_per_step": dec["ms_per_step"] * 1e3,
                               "timing": "the whole layer (route, experts, combine) per graph-timed step"}},
        "layer": {"hbm_frac": dec["layer_hbm_frac"], "mfma_frac": dec["layer_mfma_frac"],
                  "bytes_per_step": dec["layer_bytes"],
                  "timing": "HIP graph replay (the rotated layers back to back in one graph); "
                            "eager_ms_per_step without graphs",
                  "eager_ms_per_step": dec["eager_ms_per_step"],
                  "step_us": dec["step_us"], "eager_step_us": dec["eager_step_us"],
                  "stages_us_mean": dec["stages_us_mean"],
                  "touched_experts": dec["touched_experts"]},
        "cpu_baseline": cpu,
        "conditions": run_conditions(torch, args.steps, args.warmup, args.rotate),
    }
    if cpu_extra is not None:
        line["cpu_baseline_more"] = cpu_extra
    if stack is not None:
        line["stack"] = stack
    if reports is not None:
        line["reports"] = reports
    if attn is not None:
        line["attention"] = attn
    if pred is not None:
        line["predictor"] = pred
    if tframe is not None:
        line["talker_frame"] = tframe
    if extra_cpu is not None:
        for key in ("attention", "predictor", "talker_frame"):
            if key in line:
                line[key]["cpu_baseline"] = extra_cpu[key]
        line.setdefault("stack", {})["sampling_cpu_baseline"] = extra_cpu["sampling"]
    if pre is not None:
        gp = pre["kernel"]
        line["prefill"] = {"workload": "talker_moe_layer_prefill_T4096", "tokens_per_s": pre["tokens_per_s"],
                           "ms_per_step": pre["ms_per_step"], "eager_ms_per_step": pre["eager_ms_per_step"],
                           "mfma_frac": pre["layer_mfma_frac"],
                           "hbm_frac": pre["layer_hbm_frac"], "step_us": pre["step_us"],
                           "stages_us_mean": pre["stages_us_mean"],
                           "gate_up": {"mean_us": gp["mean_us"], "tflops": gp["tflops"],
                                       "mfma_frac": gp["tflops"] / MFMA_BF16_PEAK_TFLOPS, "gbs": gp["gbs"]}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
