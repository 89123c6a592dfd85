#!/usr/bin/env python3
"""Scan tokens/s of liblinscan on one MI355X at the 720p minute-scale shapes.

One step is one pass of the whole hot path over one batch of synthetic input:
  1. SANA-Video 720p minute-scale block-autoregressive rollout, ReLU linear
     attention: B1 H70 D32, 45x80 = 3600 tokens per frame, 241 latent frames
     in 25 calls (24 x 10 + 1) chained by ls_state_carry;
  2. SANA-WM 720p 60 s frame-wise Gated DeltaNet: B1 H24 D128, 23x40 = 920
     tokens per frame, 181 latent frames in one call.
Inputs are drawn once on the GPU (seeded, N(0,1) bf16, L2-normalised GDN
keys) and stay resident in HBM; the timed region holds only library calls.

Prints one JSON line: the throughput (tokens = B*F*N summed over both parts,
all heads of a token counted once), the roofline object of the dominant
kernel, and the fp64 CPU oracle timed on a sample of the same workload.

The headline pass times K steps with one event pair per step.  Per-kernel
durations come from a second pass over the same K steps in which the library
records an event pair around each of its launches, on the stream it launches
on; those per-launch events cost about 8% of a step, so they stay out of the
headline pass.

The roofline's `traffic` (HBM bytes per launch) comes from the hardware
counter summary in profiles/hbm_traffic_720p_minute.md, and only while the
kernel's sources still hash to the ones that summary was taken from.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan tokens/sec (1 GPU) at 720p minute-scale; % of MFMA/HBM roofline"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_720p_minute.md")
# sources each fused kernel is built from: counters taken on other sources are stale
KERNEL_SOURCES = {
    "relu_fused": ["device_common.h", "sync.h", "relu_items.h", "relu_mfma.hip"],
    "gdn_fused": ["device_common.h", "sync.h", "gdn_items.h", "gdn_mfma.hip"],
    "gdn_phased": ["device_common.h", "sync.h", "gdn_items.h", "gdn_mfma.hip"],
    "gdn_step": ["device_common.h", "sync.h", "gdn_items.h", "gdn_mfma.hip"],
    "relu_wide_fused": ["device_common.h", "sync.h", "relu_wide_items.h", "relu_wide_mfma.hip"],
}


def kernel_sources_sha(name):
    """sha256 over a kernel's HIP sources and the build flags."""
    pkg = os.path.join(ROOT, "block_causal_linear_attn_amd")
    h = hashlib.sha256()
    for f in [os.path.join(pkg, "csrc", x) for x in KERNEL_SOURCES[name]] + [os.path.join(pkg, "build.py")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) or None if absent or stale."""
    if name not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("traffic-json:"):
                rec = json.loads(line.split(":", 1)[1]).get(name)
                if rec is None:
                    return None, "kernel not in counter summary"
                if rec["sources_sha256"] != kernel_sources_sha(name):
                    return None, "kernel changed since the counters were taken"
                return rec["fetch_bytes"] + rec["write_bytes"], "FETCH_SIZE %.0f + WRITE_SIZE %.0f bytes" % (
                    rec["fetch_bytes"], rec["write_bytes"])
    return None, "no traffic line in counter summary"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the per-launch timing pass (no roofline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads per part in the oracle sample (default: 2 per oracle thread for "
                         "the ReLU part, all for the GDN part)")
    ap.add_argument("--no-head-dim-112", action="store_true",
                    help="skip the side measurement of both workloads at head dim 112")
    ap.add_argument("--no-token-gate", action="store_true",
                    help="skip the side measurement of the GDN part with per-token update gates")
    ap.add_argument("--no-reversed", action="store_true",
                    help="skip the side measurement of the reversed GDN scan (chunks of 8 frames)")
    ap.add_argument("--no-temporal-conv", action="store_true",
                    help="skip the side measurement of the block-causal temporal convolution")
    ap.add_argument("--no-strided", action="store_true",
                    help="skip the side measurement of the strided [B][F][N][H][D] layout")
    ap.add_argument("--no-480p", action="store_true",
                    help="skip the side measurement of the 480p 5 s ReLU call")
    ap.add_argument("--no-prologue", action="store_true",
                    help="skip the side measurement of the fused per-token prologue")
    ap.add_argument("--no-chunk-step", action="store_true",
                    help="skip the side measurement of the single-frame GDN call latency")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--only", choices=sorted(ONLY_CONFIGS),
                    help="run only this workload's library calls, --steps passes after one warm-up pass, "
                         "untimed, and print its algorithmic bytes per pass (for hardware counter runs)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: liblinscan has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from block_causal_linear_attn_amd import binding as ls
    from block_causal_linear_attn_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch, for
        # scaling hardware byte counters
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        run_only(args, torch, ls, inputs)
        return
    wv = inputs.WORKLOADS["sana_video_720p_minute"]
    wg = inputs.WORKLOADS["sana_wm_720p_60s"]

    # ---- resident inputs and outputs
    calls = [inputs.workload_call_inputs(wv, i, device=dev) for i in range(len(wv.calls))]
    outs = [torch.empty_like(c["q"]) for c in calls]
    cache = torch.zeros((wv.B, wv.H, wv.D, wv.D), device=dev)
    ncache = torch.zeros((wv.B, wv.H, wv.D), device=dev)
    S_blk = torch.empty_like(cache)
    z_blk = torch.empty_like(ncache)
    g = inputs.workload_call_inputs(wg, 0, device=dev)
    g_out = torch.empty_like(g["q"])
    g_state = torch.empty((wg.B, wg.H, wg.D, wg.D), device=dev)
    torch.cuda.synchronize()

    def part_video():
        for i, c in enumerate(calls):
            first = i == 0  # each pass starts the rollout from the zero state
            ls.ls_relu_block_forward(c["q"], c["k"], c["v"], None if first else cache,
                                     None if first else ncache, out=outs[i], state_out=S_blk,
                                     norm_out=z_blk)
            ls.ls_state_carry(S_blk, cache, z_blk, ncache)

    def part_wm():
        ls.ls_gdn_frame_forward(g["q"], g["k"], g["v"], g["alpha"], g["beta"], None, out=g_out,
                                state_out=g_state)

    # the workspaces' fault words (set when a bounded wait of a single-launch
    # call gives up, which would make that call's results invalid) start at
    # zero and are read once every measurement is done: the word is sticky
    ls.ls_clear_fault_word(dev)
    for _ in range(args.warmup):
        part_video()
        part_wm()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        part_video()
        e1.record()
        part_wm()
        e2.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # second pass over the same steps: the library records an event pair
    # around each of its launches, on the stream it launches on
    kstats = {}
    if not args.no_kernel_events:
        ls.ls_profile_begin()
        for _ in range(args.steps):
            part_video()
            part_wm()
        torch.cuda.synchronize()
        kstats = ls.ls_profile_end()
    ms_video = sorted(a.elapsed_time(b) for a, b, _ in ev)
    ms_wm = sorted(b.elapsed_time(c) for _, b, c in ev)
    ms_step = sorted(a.elapsed_time(c) for a, _, c in ev)
    gpu_total_s = sum(ms_step) / 1e3
    print("timed %d steps: wall %.3f s, events %.3f s" % (args.steps, wall, gpu_total_s),
          file=sys.stderr, flush=True)

    tok_video = wv.B * wv.F * wv.N
    tok_wm = wg.B * wg.F * wg.N
    tokens = tok_video + tok_wm
    elt = 2  # bf16 bytes
    bytes_video = 4 * wv.B * wv.H * wv.F * wv.N * wv.D * elt
    bytes_wm = 4 * wg.B * wg.H * wg.F * wg.N * wg.D * elt
    value = tokens * args.steps / gpu_total_s
    med = lambda xs: xs[len(xs) // 2]

    # ---- per-kernel timing over the timed steps
    # algorithmic HBM bytes per launch: the token tensors each kernel must move
    half_video = 2 * wv.B * wv.H * wv.F * wv.N * wv.D * elt  # two of q, k, v, o over all calls
    half_wm = 2 * wg.B * wg.H * wg.F * wg.N * wg.D * elt
    n_calls = len(wv.calls)
    alg = {
        "relu_fused": 2 * half_video / n_calls,  # q, k, v in, o out (per call, averaged over the calls)
        "relu_summary": half_video / n_calls,    # k, v in
        "relu_output": half_video / n_calls,     # q in, o out
        "gdn_fused": 2 * half_wm,                # q, k, v in, o out
        "gdn_gram": half_wm,                     # k, v in
        "gdn_output": half_wm,                   # q in, o out
    }
    # algorithmic MFMA work per launch (for information): ReLU 4 H D^2 flop per
    # token (v phi(k)^T and S phi(q)), GDN 6 H D^2 per token (G, U and S q) plus
    # 2 H D^3 per frame (the state times beta G)
    flops = {
        "relu_fused": 4 * wv.B * wv.H * wv.F * wv.N * wv.D ** 2 / n_calls,
        "gdn_fused": 6 * wg.B * wg.H * wg.F * wg.N * wg.D ** 2 + 2 * wg.B * wg.H * wg.F * wg.D ** 3,
    }
    copy_gbs = device_copy_gbs(torch)
    # the ReLU call's own mix (three tensors read, one written, the sizes of a
    # 10-frame call's tensors) as a second ceiling beside the device copy
    mix_gbs = stream_mix_gbs(torch, wv.B * wv.H * wv.N * wv.D * 10)
    kernels = {}
    for name, (launches, total_ms) in kstats.items():
        avg_us = 1e3 * total_ms / max(1, launches)
        k = {"launches_per_step": launches / args.steps, "avg_us": round(avg_us, 2),
             "ms_per_step": round(total_ms / args.steps, 4)}
        if name in alg:
            gbs = alg[name] / (avg_us * 1e-6) / 1e9
            k["alg_bytes_per_launch"] = int(alg[name])
            k["achieved_GBs"] = round(gbs, 1)
            k["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
            k["copy_frac"] = round(gbs / copy_gbs, 4)
        if name in flops:
            k["mfma_frac"] = round(flops[name] / (avg_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        kernels[name] = k
    roofline = None
    if kernels:
        dom = max((n for n in kernels if n in alg), key=lambda n: kernels[n]["ms_per_step"])
        traffic, note = measured_traffic(dom)
        roofline = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["achieved_GBs"],
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["hbm_frac"],
                    "traffic": None if traffic is None else int(traffic),
                    "alg_bytes": kernels[dom]["alg_bytes_per_launch"], "traffic_note": note,
                    "copy_GBs": round(copy_gbs, 1), "frac_of_copy": kernels[dom]["copy_frac"],
                    "read3_write1_GBs": round(mix_gbs, 1),
                    "frac_of_read3_write1": round(kernels[dom]["achieved_GBs"] / mix_gbs, 4),
                    "mfma_frac": kernels[dom].get("mfma_frac")}

    chunk_step = None if args.no_chunk_step else time_chunk_step(torch, ls, inputs)
    v480 = None if args.no_480p else time_480p(torch, ls, inputs)
    # GDN side measurements run each timed call right after the rollout, as in
    # the step: back to back, GDN calls hold the shader clock lower
    d112 = None if args.no_head_dim_112 else time_head_dim_112(torch, ls, inputs, part_video)
    tgate = None if args.no_token_gate else time_token_gate(torch, ls, inputs, g, wg, part_video)
    rev = None if args.no_reversed else time_reversed(torch, ls, g, wg, part_video)
    conv = None if args.no_temporal_conv else time_temporal_conv(torch, ls)
    strided = None if args.no_strided else time_strided(torch, ls, calls[0], g, part_video)
    pro = None if args.no_prologue else time_prologue(torch, ls, inputs, calls[0], g, part_video, copy_gbs)

    # ---- CPU baseline: the fp64 oracle on a sample of the same workload
    fault = ls.ls_fault_word(dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, inputs, wv, wg, tokens)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_total_s * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "720p minute-scale scan: SANA-Video ReLU block-AR rollout (B1 H70 D32 N3600, "
                        "241 frames in 24x10+1 calls with state carry) + SANA-WM frame-wise GDN "
                        "(B1 H24 D128 N920 F181)",
            "global_batch": 1,
            "tokens_per_step": tokens,
            "parallelism": "none (1 GPU)",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parts": {
            "sana_video_720p_minute": {"ms_median": round(med(ms_video), 4), "tokens": tok_video,
                                       "tokens_per_s": round(tok_video / (med(ms_video) / 1e3), 1),
                                       "hbm_frac": round(bytes_video / (med(ms_video) / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
            "sana_wm_720p_60s": {"ms_median": round(med(ms_wm), 4), "tokens": tok_wm,
                                 "tokens_per_s": round(tok_wm / (med(ms_wm) / 1e3), 1),
                                 "hbm_frac": round(bytes_wm / (med(ms_wm) / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
            "step_ms_p10_p50_p90": [round(ms_step[int(0.1 * (len(ms_step) - 1))], 4), round(med(ms_step), 4),
                                    round(ms_step[int(0.9 * (len(ms_step) - 1))], 4)],
            "step_hbm_frac": round((bytes_video + bytes_wm) / (med(ms_step) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "side": {"sana_wm_chunk_step": chunk_step, "sana_video_480p_5s": v480, "head_dim_112": d112, "sana_wm_720p_60s_token_gate": tgate,
                 "sana_wm_720p_60s_reversed_c8": rev, "causal_mix_ffn_temporal_conv": conv,
                 "bshd_layout": strided, "fused_prologue": pro},
        "kernels": kernels,
        "fault_word": fault,
    }
    print(json.dumps(line), flush=True)
    if fault != 0:
        print("a bounded wait gave up (workspace fault word %#x): results of this run are invalid" % fault,
              file=sys.stderr, flush=True)
        sys.exit(3)


def time_480p(torch, ls, inputs, reps=5):
    """The SANA-Video 480p 5 s ReLU call (B1 H70 D32 F21 N1560, one call of
    21 frames, frame-causal), two input sets alternating; median of `reps`
    calls after one warm-up call each."""
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["sana_video_480p_5s"]
    xs = [inputs.relu_inputs(w.B, w.H, w.F, w.N, w.D, "bf16", seed=w.seed, part=p, device=dev) for p in (0, 1)]
    outs = [torch.empty_like(x["q"]) for x in xs]
    for i in range(2):
        ls.ls_relu_block_forward(xs[i]["q"], xs[i]["k"], xs[i]["v"], out=outs[i])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for j, (a, b) in enumerate(ev):
        x = xs[j % 2]
        a.record()
        ls.ls_relu_block_forward(x["q"], x["k"], x["v"], out=outs[j % 2])
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    tokens = w.B * w.F * w.N
    nbytes = 4 * w.B * w.H * w.F * w.N * w.D * 2
    del xs, outs
    return {"ms_median": round(ms, 4), "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "workload": w.note}


def device_copy_gbs(torch, nbytes=1 << 30, reps=5):
    """Bandwidth of a plain device-to-device copy (bytes read + written per
    second, median of `reps` copies of 1 GiB), the practical ceiling the
    roofline's second line divides by."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9


def stream_mix_gbs(torch, n, reps=5):
    """Bytes per second of torch.addcmul over bf16 tensors of n elements
    (three read, one written: the ReLU call's mix of q, k, v in and o out),
    median of `reps` calls."""
    dev = torch.device("cuda:0")
    a, b, c = (torch.ones(n, dtype=torch.bfloat16, device=dev) for _ in range(3))
    d = torch.empty_like(a)
    torch.addcmul(a, b, c, out=d)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        torch.addcmul(a, b, c, out=d)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    del a, b, c, d
    return 4 * n * 2 / (ms / 1e3) / 1e9


def time_head_dim_112(torch, ls, inputs, prelude, reps=3):
    """Both parts of the step at head dim 112 (not part of the step).

    The ReLU rollout (B1 H20 D112 N3600, 25 calls with state carry) and the
    GDN call (B1 H28 D112 N920 F181), each timed over `reps` passes after one
    warm-up pass; tokens/s and the HBM fraction of the token tensors' bytes.
    """
    dev = torch.device("cuda:0")
    res = {}
    wv = inputs.WORKLOADS["sana_video_720p_minute_d112"]
    calls = [inputs.workload_call_inputs(wv, i, device=dev) for i in range(len(wv.calls))]
    outs = [torch.empty_like(c["q"]) for c in calls]
    cache = torch.zeros((wv.B, wv.H, wv.D, wv.D), device=dev)
    ncache = torch.zeros((wv.B, wv.H, wv.D), device=dev)
    S_blk, z_blk = torch.empty_like(cache), torch.empty_like(ncache)

    def video():
        for i, c in enumerate(calls):
            ls.ls_relu_block_forward(c["q"], c["k"], c["v"], None if i == 0 else cache,
                                     None if i == 0 else ncache, out=outs[i], state_out=S_blk, norm_out=z_blk)
            ls.ls_state_carry(S_blk, cache, z_blk, ncache)

    wg = inputs.WORKLOADS["sana_wm_720p_60s_d112"]
    g = inputs.workload_call_inputs(wg, 0, device=dev)
    g_out = torch.empty_like(g["q"])
    g_state = torch.empty((wg.B, wg.H, wg.D, wg.D), device=dev)

    def wm():
        ls.ls_gdn_frame_forward(g["q"], g["k"], g["v"], g["alpha"], g["beta"], None, out=g_out, state_out=g_state)

    for name, w, fn in (("sana_video_720p_minute_d112", wv, video), ("sana_wm_720p_60s_d112", wg, wm)):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            if fn is wm:
                prelude()  # the GDN call after a rollout, as in the step
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        tokens = w.B * w.F * w.N
        nbytes = 4 * w.B * w.H * w.F * w.N * w.D * 2
        res[name] = {"ms_median": round(ms, 4), "tokens_per_s": round(tokens / (ms / 1e3), 1),
                     "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "workload": w.note}
    del calls, outs, g, g_out
    return res


def time_token_gate(torch, ls, inputs, g, wg, prelude, reps=3):
    """The GDN part with one update gate per token (same inputs, gates drawn
    per token), timed over `reps` calls after one warm-up call, each after
    `prelude` (untimed), as in the step."""
    dev = torch.device("cuda:0")
    bt = inputs.token_gates(wg.B, wg.H, wg.F, wg.N, seed=wg.seed, device=dev)
    out = torch.empty_like(g["q"])
    st = torch.empty((wg.B, wg.H, wg.D, wg.D), device=dev)

    def call():
        ls.ls_gdn_frame_forward_token_gate(g["q"], g["k"], g["v"], g["alpha"], bt, None, out=out, state_out=st)

    call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        prelude()
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    tokens = wg.B * wg.F * wg.N
    nbytes = 4 * wg.B * wg.H * wg.F * wg.N * wg.D * 2 + wg.B * wg.H * wg.F * wg.N * 4  # + the gates
    return {"ms_median": round(ms, 4), "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "B1 H24 D128 F181 N920 bf16, one update gate per token"}


def time_reversed(torch, ls, g, wg, prelude, chunk=8, reps=3):
    """The GDN part through the reversed scan that resets every `chunk` frames,
    timed over `reps` calls after one warm-up call, each after `prelude`."""
    out = torch.empty_like(g["q"])

    def call():
        ls.ls_gdn_frame_forward_reversed(g["q"], g["k"], g["v"], g["alpha"], g["beta"], chunk, out=out)

    call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        prelude()
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    tokens = wg.B * wg.F * wg.N
    nbytes = 4 * wg.B * wg.H * wg.F * wg.N * wg.D * 2
    return {"ms_median": round(ms, 4), "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "B1 H24 D128 F181 N920 bf16, reversed scan reset every %d frames" % chunk}


def time_temporal_conv(torch, ls, reps=5):
    """The Causal Mix-FFN's temporal convolution over one 10-frame block of
    720p tokens at the hidden width (B1 F10 N3600, 2240 channels, bf16), with
    a carried frame; two input sets alternate.  Mean kernel time over `reps` calls."""
    dev = torch.device("cuda:0")
    F, N, C = 10, 3600, 2240
    g = torch.Generator(device=dev)
    g.manual_seed(777)
    xs = [torch.randn((1, 1, F, N, C), generator=g, device=dev).to(torch.bfloat16) for _ in range(2)]
    w = 0.5 * torch.randn((1, C, 3), generator=g, device=dev)
    b = 0.1 * torch.randn((1, C), generator=g, device=dev)
    carry = torch.zeros((1, 1, N, C), dtype=torch.bfloat16, device=dev)
    ys = [torch.empty_like(x) for x in xs]
    co = torch.empty_like(carry)

    def call(i):
        ls.ls_temporal_conv3(xs[i % 2], w, b, carry, block_frames=F, out=ys[i % 2], carry_out=co)

    call(0)
    call(1)
    torch.cuda.synchronize()
    # a call is ~0.1 ms, close to the binding's host time per call: the library's
    # per-launch events time the kernel itself
    ls.ls_profile_begin()
    for i in range(reps):
        call(i)
    torch.cuda.synchronize()
    launches, total_ms = ls.ls_profile_end()["temporal_conv3"]
    us = 1e3 * total_ms / launches
    nbytes = 2 * F * N * C * 2 + 2 * N * C * 2  # x read, y written, carry in and out
    return {"us_mean": round(us, 2), "alg_bytes": nbytes,
            "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "B1 F10 N3600 C2240 bf16, one block of 10 frames with a carried frame"}


def kernel_us(torch, ls, fn, name, reps, prelude=None):
    """Mean duration of kernel `name` over `reps` calls of fn (after one
    warm-up call), from the library's per-launch events; with a prelude,
    each call follows it (untimed), as the GDN call follows the rollout in
    the step: back-to-back GDN calls run at a lower shader clock."""
    fn()
    torch.cuda.synchronize()
    ls.ls_profile_begin()
    for _ in range(reps):
        if prelude is not None:
            prelude()
        fn()
    torch.cuda.synchronize()
    n, ms = ls.ls_profile_end()[name]
    return round(1e3 * ms / n, 2)


def time_strided(torch, ls, relu_call, g, prelude, reps=4):
    """One 10-frame ReLU call of the rollout and the GDN call (after the
    rollout, as in the step) with q, k, v, o stored [B][F][N][H][D] (heads
    interleaved in every token row), against the same calls on the packed
    layout; mean kernel time from the library's per-launch events."""
    def bshd(x):
        return x.permute(0, 2, 3, 1, 4).contiguous().permute(0, 3, 1, 2, 4)

    res = {}
    r = relu_call
    rs = {n: bshd(r[n]) for n in ("q", "k", "v")}
    res["relu_h70_d32_10_frames_us"] = {
        "packed": kernel_us(torch, ls, lambda: ls.ls_relu_block_forward(r["q"], r["k"], r["v"]), "relu_fused", reps),
        "bshd": kernel_us(torch, ls, lambda: ls.ls_relu_block_forward_strided(rs["q"], rs["k"], rs["v"]),
                          "relu_fused", reps)}
    del rs
    gs = {n: bshd(g[n]) for n in ("q", "k", "v")}
    res["gdn_h24_d128_181_frames_us"] = {
        "packed": kernel_us(torch, ls, lambda: ls.ls_gdn_frame_forward(g["q"], g["k"], g["v"], g["alpha"], g["beta"]),
                            "gdn_fused", reps, prelude),
        "bshd": kernel_us(torch, ls, lambda: ls.ls_gdn_frame_forward_strided(gs["q"], gs["k"], gs["v"], g["alpha"],
                                                                             g["beta"]), "gdn_fused", reps, prelude)}
    del gs
    return res


def time_prologue(torch, ls, inputs, relu_call, g, prelude, copy_gbs, reps=4):
    """The per-token prologue fused into the load stage: one 10-frame ReLU call
    of the rollout with RMSNorm (weights) on q and k, and the GDN call with
    RMSNorm on q and k, ReLU and L2 keys (each once more with a 3D rotary
    embedding), against the same calls without a prologue (mean kernel time
    from the library's per-launch events), and the GDN call after the same
    prologue as separate torch ops (wall time of both, CUDA events), which
    reads and writes q and k once more; separate_pass_bound_us is what the
    bytes of such a pass (q and k read and written) take at the device-copy
    rate copy_gbs, the least any separate pass could cost."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)

    res = {}
    r = relu_call
    H, D = r["q"].shape[1], r["q"].shape[-1]
    wq, wk = (1.0 + 0.1 * torch.randn((H, D), generator=gen, device=dev) for _ in range(2))
    # 3D rotary embedding: 4 pairs by frame, 12 by the 45 x 80 latent grid
    fr, tr = inputs.rope_tables(r["q"].shape[2], r["q"].shape[3], 80, D, 4, device=dev)
    res["relu_h70_d32_10_frames_rmsnorm_qk_us"] = {
        "plain": kernel_us(torch, ls, lambda: ls.ls_relu_block_forward(r["q"], r["k"], r["v"]), "relu_fused", reps),
        "fused_prologue": kernel_us(torch, ls, lambda: ls.ls_relu_block_forward_prologue(
            r["q"], r["k"], r["v"], wq, wk, norm_eps=1e-6), "relu_fused", reps),
        "fused_prologue_with_3d_rope": kernel_us(torch, ls, lambda: ls.ls_relu_block_forward_prologue(
            r["q"], r["k"], r["v"], wq, wk, norm_eps=1e-6, rope=(fr, tr, 4, 0)), "relu_fused", reps)}
    del fr, tr
    H, D = g["q"].shape[1], g["q"].shape[-1]
    wq, wk = (1.0 + 0.1 * torch.randn((H, D), generator=gen, device=dev) for _ in range(2))
    out = torch.empty_like(g["q"])

    def fused():
        ls.ls_gdn_frame_forward_prologue(g["q"], g["k"], g["v"], g["alpha"], g["beta"], wq, wk, norm_eps=1e-6,
                                         relu=True, l2_keys=True, out=out)

    def torch_prologue(x, w, l2):
        y = x.float()
        y = y * torch.rsqrt(y.pow(2).mean(-1, keepdim=True) + 1e-6) * w[None, :, None, None, :]
        y = torch.relu(y)
        if l2:
            y = y / y.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        return y.to(torch.bfloat16)

    def unfused():
        q2, k2 = torch_prologue(g["q"], wq, False), torch_prologue(g["k"], wk, True)
        ls.ls_gdn_frame_forward(q2, k2, g["v"], g["alpha"], g["beta"], out=out)

    # 3D rotary embedding at synthetic positions: 16 pairs by frame, 48 by the
    # 23 x 40 latent grid's rows and columns
    fcs, tcs = inputs.rope_tables(g["q"].shape[2], g["q"].shape[3], 40, D, 16, device=dev)

    def fused_rope():
        ls.ls_gdn_frame_forward_prologue(g["q"], g["k"], g["v"], g["alpha"], g["beta"], wq, wk, norm_eps=1e-6,
                                         relu=True, l2_keys=True, out=out, rope=(fcs, tcs, 16, 0))

    gdn = {"plain": kernel_us(torch, ls, lambda: ls.ls_gdn_frame_forward(g["q"], g["k"], g["v"], g["alpha"],
                                                                         g["beta"], out=out),
                              "gdn_fused", reps, prelude),
           "fused_prologue": kernel_us(torch, ls, fused, "gdn_fused", reps, prelude),
           "fused_prologue_with_3d_rope": kernel_us(torch, ls, fused_rope, "gdn_fused", reps, prelude)}
    # the torch variant last: its fp32 temporaries come and go after the library's timings
    unfused()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        prelude()
        a.record()
        unfused()
        b.record()
    torch.cuda.synchronize()
    ms_unfused = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    gdn["torch_prologue_then_plain_wall"] = round(1e3 * ms_unfused, 2)
    # what a separate bf16 prologue pass would cost at best: q and k read and
    # written once more, at the device-copy rate measured in this run
    for key, t in (("relu", r), ("gdn", g)):
        sep_bytes = 4 * t["q"].numel() * t["q"].element_size()
        (res["relu_h70_d32_10_frames_rmsnorm_qk_us"] if key == "relu" else gdn)["separate_pass_bound_us"] = round(
            sep_bytes / (copy_gbs * 1e9) * 1e6, 2)
    res["gdn_h24_d128_181_frames_rmsnorm_relu_l2_us"] = gdn
    del fcs, tcs
    return res


def time_chunk_step(torch, ls, inputs):
    """Latency of single-frame GDN calls (B4 H24 D128 N920) re-reading one carried state.

    Not part of the step: the 50 denoising-step calls of the chunk-causal
    workload, each on its own resident input set, timed one by one after a
    warm-up pass over all of them.
    """
    w = inputs.WORKLOADS["sana_wm_chunk_step"]
    dev = torch.device("cuda:0")
    calls = [inputs.workload_call_inputs(w, i, device=dev) for i in range(w.steps)]
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    state = 0.05 * torch.randn((w.B, w.H, w.D, w.D), generator=g, device=dev)  # any carried state
    outs = [torch.empty_like(c["q"]) for c in calls]
    s_out = torch.empty_like(state)

    def call(i):
        c = calls[i]
        ls.ls_gdn_frame_forward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], state, out=outs[i],
                                state_out=s_out)

    for i in range(w.steps):
        call(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    us = sorted(1e3 * a.elapsed_time(b) for a, b in ev)
    med_us = us[len(us) // 2]
    tokens = w.B * w.N
    alg = 4 * w.B * w.H * w.N * w.D * 2 + 2 * w.B * w.H * w.D * w.D * 4  # q, k, v, o + state in/out
    del calls, outs
    return {"calls": w.steps, "us_median": round(med_us, 2), "us_p10": round(us[len(us) // 10], 2),
            "us_p90": round(us[(9 * len(us)) // 10], 2), "tokens_per_s": round(tokens / (med_us * 1e-6), 1),
            "hbm_frac": round(alg / (med_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "B4 H24 D128 N920, F=1 per call, 50 distinct input sets, one carried state"}


def _only_rollout(torch, ls, inputs, name):
    w = inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    calls = [inputs.workload_call_inputs(w, i, device=dev) for i in range(len(w.calls))]
    outs = [torch.empty_like(c["q"]) for c in calls]
    cache = torch.zeros((w.B, w.H, w.D, w.D), device=dev)
    ncache = torch.zeros((w.B, w.H, w.D), device=dev)
    S_blk, z_blk = torch.empty_like(cache), torch.empty_like(ncache)

    def run():
        for i, c in enumerate(calls):
            ls.ls_relu_block_forward(c["q"], c["k"], c["v"], None if i == 0 else cache, None if i == 0 else ncache,
                                     out=outs[i], state_out=S_blk, norm_out=z_blk)
            ls.ls_state_carry(S_blk, cache, z_blk, ncache)
    # q, k, v in and o out for every call, the carried state read and the new one written
    return run, 4 * w.B * w.H * w.F * w.N * w.D * 2 + (len(w.calls) - 1) * 2 * w.B * w.H * (w.D * w.D + w.D) * 4


def _only_gdn(torch, ls, inputs, name, variant):
    w = inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    g = inputs.workload_call_inputs(w, 0, device=dev)
    out = torch.empty_like(g["q"])
    st = torch.empty((w.B, w.H, w.D, w.D), device=dev)
    tok = 4 * w.B * w.H * w.F * w.N * w.D * 2
    if variant == "plain":
        return (lambda: ls.ls_gdn_frame_forward(g["q"], g["k"], g["v"], g["alpha"], g["beta"], out=out,
                                                state_out=st)), tok
    if variant == "token_gate":
        bt = inputs.token_gates(w.B, w.H, w.F, w.N, seed=w.seed, device=dev)
        return (lambda: ls.ls_gdn_frame_forward_token_gate(g["q"], g["k"], g["v"], g["alpha"], bt, out=out,
                                                           state_out=st)), tok + w.B * w.H * w.F * w.N * 4
    if variant == "reversed_c8":
        return (lambda: ls.ls_gdn_frame_forward_reversed(g["q"], g["k"], g["v"], g["alpha"], g["beta"], 8,
                                                         out=out)), tok
    if variant == "bshd":
        gs = {n: g[n].permute(0, 2, 3, 1, 4).contiguous().permute(0, 3, 1, 2, 4) for n in ("q", "k", "v")}
        return (lambda: ls.ls_gdn_frame_forward_strided(gs["q"], gs["k"], gs["v"], g["alpha"], g["beta"])), tok
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    wq, wk = (1.0 + 0.1 * torch.randn((w.H, w.D), generator=gen, device=dev) for _ in range(2))
    rope = None
    if variant == "prologue_rope":
        rope = inputs.rope_tables(w.F, w.N, 40, w.D, 16, device=dev) + (16, 0)
    return (lambda: ls.ls_gdn_frame_forward_prologue(g["q"], g["k"], g["v"], g["alpha"], g["beta"], wq, wk,
                                                     norm_eps=1e-6, relu=True, l2_keys=True, out=out,
                                                     rope=rope)), tok


def _only_relu_call(torch, ls, inputs, variant):
    """The first 10-frame call of the 720p minute-scale rollout (B1 H70 D32 N3600)."""
    w = inputs.WORKLOADS["sana_video_720p_minute"]
    dev = torch.device("cuda:0")
    r = inputs.workload_call_inputs(w, 0, device=dev)
    out = torch.empty_like(r["q"])
    tok = 4 * r["q"].numel() * 2
    if variant == "bshd":
        rs = {n: r[n].permute(0, 2, 3, 1, 4).contiguous().permute(0, 3, 1, 2, 4) for n in ("q", "k", "v")}
        return (lambda: ls.ls_relu_block_forward_strided(rs["q"], rs["k"], rs["v"])), tok
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    H, D = r["q"].shape[1], r["q"].shape[-1]
    wq, wk = (1.0 + 0.1 * torch.randn((H, D), generator=gen, device=dev) for _ in range(2))
    rope = None
    if variant == "prologue_rope":
        rope = inputs.rope_tables(r["q"].shape[2], r["q"].shape[3], 80, D, 4, device=dev) + (4, 0)
    return (lambda: ls.ls_relu_block_forward_prologue(r["q"], r["k"], r["v"], wq, wk, norm_eps=1e-6, out=out,
                                                      rope=rope)), tok


def _only_480p(torch, ls, inputs):
    w = inputs.WORKLOADS["sana_video_480p_5s"]
    x = inputs.relu_inputs(w.B, w.H, w.F, w.N, w.D, "bf16", seed=w.seed, device=torch.device("cuda:0"))
    out = torch.empty_like(x["q"])
    return (lambda: ls.ls_relu_block_forward(x["q"], x["k"], x["v"], out=out)), 4 * x["q"].numel() * 2


def _only_chunk_step(torch, ls, inputs):
    w = inputs.WORKLOADS["sana_wm_chunk_step"]
    dev = torch.device("cuda:0")
    calls = [inputs.workload_call_inputs(w, i, device=dev) for i in range(w.steps)]
    state = torch.zeros((w.B, w.H, w.D, w.D), device=dev)
    outs = [torch.empty_like(c["q"]) for c in calls]
    s_out = torch.empty_like(state)

    def run():
        for c, o in zip(calls, outs):
            ls.ls_gdn_frame_forward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], state, out=o, state_out=s_out)
    return run, w.steps * (4 * w.B * w.H * w.N * w.D * 2 + 2 * w.B * w.H * w.D * w.D * 4)


def _only_temporal_conv(torch, ls, inputs):
    dev = torch.device("cuda:0")
    F, N, C = 10, 3600, 2240
    g = torch.Generator(device=dev)
    g.manual_seed(777)
    x = torch.randn((1, 1, F, N, C), generator=g, device=dev).to(torch.bfloat16)
    w = 0.5 * torch.randn((1, C, 3), generator=g, device=dev)
    b = 0.1 * torch.randn((1, C), generator=g, device=dev)
    carry = torch.zeros((1, 1, N, C), dtype=torch.bfloat16, device=dev)
    y, co = torch.empty_like(x), torch.empty_like(carry)
    return (lambda: ls.ls_temporal_conv3(x, w, b, carry, block_frames=F, out=y, carry_out=co)), \
        2 * F * N * C * 2 + 2 * N * C * 2


# workloads of --only: name -> f(torch, ls, inputs) -> (one pass, algorithmic HBM bytes per pass)
ONLY_CONFIGS = {
    "video_720p_minute": lambda t, l, i: _only_rollout(t, l, i, "sana_video_720p_minute"),
    "video_720p_minute_d112": lambda t, l, i: _only_rollout(t, l, i, "sana_video_720p_minute_d112"),
    "video_480p_5s": _only_480p,
    "video_call_bshd": lambda t, l, i: _only_relu_call(t, l, i, "bshd"),
    "video_call_prologue": lambda t, l, i: _only_relu_call(t, l, i, "prologue"),
    "video_call_prologue_rope": lambda t, l, i: _only_relu_call(t, l, i, "prologue_rope"),
    "wm_720p_60s": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s", "plain"),
    "wm_720p_60s_d112": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s_d112", "plain"),
    "wm_token_gate": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s", "token_gate"),
    "wm_reversed_c8": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s", "reversed_c8"),
    "wm_bshd": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s", "bshd"),
    "wm_prologue": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s", "prologue"),
    "wm_prologue_rope": lambda t, l, i: _only_gdn(t, l, i, "sana_wm_720p_60s", "prologue_rope"),
    "wm_chunk_step": _only_chunk_step,
    "temporal_conv": _only_temporal_conv,
}


def run_only(args, torch, ls, inputs):
    """One workload alone: a warm-up pass, then --steps passes (no timing)."""
    run, alg = ONLY_CONFIGS[args.only](torch, ls, inputs)
    ls.ls_clear_fault_word()
    run()
    torch.cuda.synchronize()
    ls.ls_profile_begin()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    launches = {k: v[0] // args.steps for k, v in ls.ls_profile_end().items()}
    fault = ls.ls_fault_word()
    print(json.dumps({"only": args.only, "passes": args.steps + 1, "alg_bytes_per_pass": int(alg),
                      "launches_per_pass": launches, "fault_word": fault}), flush=True)
    if fault:
        sys.exit(3)


def cpu_baseline(args, inputs, wv, wg, tokens):
    """Time the fp64 oracle on Hs heads of each part (all frames), scaled to the step."""
    import oracle
    threads = oracle.max_threads()
    # about 10 s of oracle work on a 16-core host: two heads per thread for
    # the ReLU rollout, every head of the GDN scan
    hv = min(args.cpu_heads or 2 * threads, wv.H)
    hg = min(args.cpu_heads or wg.H, wg.H)
    xv = inputs.relu_inputs(1, hv, wv.F, wv.N, wv.D, "bf16", seed=wv.seed, part=999)
    xv = {k: t.float().numpy() for k, t in xv.items()}
    t0 = time.perf_counter()
    oracle.relu_block(xv["q"], xv["k"], xv["v"], nthreads=threads)
    tv = time.perf_counter() - t0
    del xv
    xg = inputs.gdn_inputs(1, hg, wg.F, wg.N, wg.D, "bf16", seed=wg.seed, part=999, l2_keys=True)
    xg = {k: t.float().numpy() for k, t in xg.items()}
    t0 = time.perf_counter()
    oracle.gdn_frame(xg["q"], xg["k"], xg["v"], xg["alpha"], xg["beta"], nthreads=threads)
    tg = time.perf_counter() - t0
    step_s = tv * wv.H / hv + tg * wg.H / hg
    # the same on one thread, one head of each part (about 3 s)
    x1 = inputs.relu_inputs(1, 1, wv.F, wv.N, wv.D, "bf16", seed=wv.seed, part=998)
    x1 = {k: t.float().numpy() for k, t in x1.items()}
    t0 = time.perf_counter()
    oracle.relu_block(x1["q"], x1["k"], x1["v"], nthreads=1)
    tv1 = time.perf_counter() - t0
    x1 = inputs.gdn_inputs(1, 1, wg.F, wg.N, wg.D, "bf16", seed=wg.seed, part=998, l2_keys=True)
    x1 = {k: t.float().numpy() for k, t in x1.items()}
    t0 = time.perf_counter()
    oracle.gdn_frame(x1["q"], x1["k"], x1["v"], x1["alpha"], x1["beta"], nthreads=1)
    tg1 = time.perf_counter() - t0
    del x1
    step_1 = tv1 * wv.H + tg1 * wg.H
    print("oracle: %d+%d heads in %.2f+%.2f s on %d threads; one head each on one thread %.2f+%.2f s"
          % (hv, hg, tv, tg, threads, tv1, tg1), file=sys.stderr, flush=True)
    return {"value": round(tokens / step_s, 1), "unit": "tokens/s", "cores": min(threads, max(hv, hg)),
            "kind": "oracle",
            "sample": "%d of %d heads of the ReLU rollout (all 241 frames) and %d of %d heads of the GDN "
                      "scan (all 181 frames), same shapes and distributions, timed %.1f s + %.1f s and "
                      "scaled by the head ratio" % (hv, wv.H, hg, wg.H, tv, tg),
            "value_1thread": round(tokens / step_1, 1),
            "sample_1thread": "one head of each part on one thread, %.2f s + %.2f s, scaled by the head "
                              "counts" % (tv1, tg1)}


if __name__ == "__main__":
    main()
