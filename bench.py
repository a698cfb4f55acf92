#!/usr/bin/env python3
"""Decode throughput of the LeapQuant per-window int8 state path on one MI355X.

Workload (default): Gated DeltaNet decode at batch 256 x 32 heads with four
stacked layers' states resident (32,768 states, 8,192 per layer, dk = dv =
128), window p = 16, r = 4 compensator rows, 1,024 tokens.  One step is the
whole decode of that batch: quantize the initial states, then 64 windows of
16 tokens x 4 per-layer launches.  With --close fused (default) the last
token of a window is decoded and the layer's window closed in one launch
(leapquant_decode_close); with --close separate all 16 tokens are decode
steps and one window close covers all four layers' states.  Inputs are
synthetic (seeded generators) and resident in HBM before timing starts.

Prints one JSON line (see the fields below).  --gpus > 1 is refused: this
path runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode head-tokens/s (dk=dv=128, int8 state, p=16) + % of HBM BW roofline"
UNIT = "head-tokens/s"
HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def _comp_read(dk, dv, r, dense):
    """Compensator bytes a kernel reads per state: rows and indices, or
    dense tokens (values and keys; the starting rows are not read)."""
    return r * (4 * dv + 4 * dk) if dense else r * (4 * dv + 4)


def _boundary_rw(dk, dv, r, dense):
    """Boundary-state bytes a close reads and writes per state (dense
    tokens: keys and values read; keys, values and starting rows written)."""
    base = dk * dv + 4 * (dk + dv)
    if dense:
        return 2 * base + r * (4 * dv + 4 * dk) + r * (4 * dv + 4 * dk + 4)
    return 2 * (base + r * (4 * dv + 4))


def step_bytes(t, dk, dv, r, kda, dense=False):
    """Algorithmic HBM bytes of one decode step at window position t (t
    records already buffered) for one state: int8 codes, row and column
    scales, compensators, t buffered records, the token's inputs, its
    output and the record it appends."""
    G = dk if kda else 1
    R = G + dk + dv
    return (dk * dv + 4 * (dk + dv) + _comp_read(dk, dv, r, dense) + 4 * t * R
            + 4 * (2 * dk + dv + 1 + G) + 4 * dv + 4 * R)


def close_bytes(p, dk, dv, r, kda, dense=False):
    """Algorithmic HBM bytes of one window close for one state: read and
    write the boundary state, read the p buffered records."""
    G = dk if kda else 1
    R = G + dk + dv
    return _boundary_rw(dk, dv, r, dense) + 4 * p * R


def fused_bytes(t, dk, dv, r, kda, dense=False):
    """Algorithmic HBM bytes of one fused last-token decode and window close
    for one state: read and write the boundary state, read the t buffered
    records and the token's inputs, write its output."""
    G = dk if kda else 1
    R = G + dk + dv
    return _boundary_rw(dk, dv, r, dense) + 4 * t * R + 4 * (2 * dk + dv + 1 + G) + 4 * dv


def bytes_per_head_token(p, dk, dv, r, kda, fused=False, dense=False):
    """Algorithmic bytes per state and token, the window's work spread over
    its p tokens: p decode steps and a window close, or p - 1 decode steps
    and the fused last-token decode and close."""
    if fused:
        dec = sum(step_bytes(t, dk, dv, r, kda, dense) for t in range(p - 1))
        return (dec + fused_bytes(p - 1, dk, dv, r, kda, dense)) / p
    dec = sum(step_bytes(t, dk, dv, r, kda, dense) for t in range(p)) / p
    return dec + close_bytes(p, dk, dv, r, kda, dense) / p


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gdn_b256_4layers.txt")
KERNEL_SRCS = [os.path.join(ROOT, "recurrent_state_quant_amd", "csrc", f)
               for f in ("lq_device.h", "lq_decode_one.h", "lq_decode_body.inc", "lq_close16_body.inc",
                         "lq_decode.hip", "lq_close.hip", "lq_baselines.hip")]


def kernel_source_sha256():
    """sha256 of the kernel sources, concatenated in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(cfg):
    """HBM bytes per state {decode, close, fused} from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary; empty when the counters were
    taken on another workload or on kernel source that has changed since."""
    from workloads.configs import HEADLINE
    if cfg.name != HEADLINE or not os.path.exists(TRAFFIC_FILE):
        return {}
    doc = json.load(open(TRAFFIC_FILE))
    if doc.get("source_sha256") != kernel_source_sha256():
        return {}
    names = {"decode_fused": "decode_step_kernel<GDN> (fused schedule)",
             "decode_separate": "decode_step_kernel<GDN> (separate schedule)",
             "close": "close16_kernel<GDN, window close>", "fused": "close16_kernel<GDN, fused decode_close>"}
    return {key: doc["kernels"][nm]["traffic_bytes_per_state"]
            for key, nm in names.items() if nm in doc["kernels"]}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="gdn_b256_h32_4layers",
                    choices=("gdn_single_head_b1", "gdn_layer_h32_b64", "gdn_b256_h32_4layers",
                             "kda_h32_b128", "gdn_long64k_h16_b8"),
                    help="workload (default: the batch-256 x 32-head x 4-layer GDN decode)")
    ap.add_argument("--tokens", type=int, default=0, help="tokens per step (default: the workload's)")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--close", choices=("fused", "separate"), default="fused",
                    help="fused: last token decoded and window closed per layer in one launch; "
                         "separate: p decode steps, then one window close over all layers")
    ap.add_argument("--comp", choices=("rows", "dense"), default="rows",
                    help="compensator form: rows of largest norm (default) or dense tokens "
                         "(LQ_DENSE_COMP, keys by subspace iteration)")
    ap.add_argument("--comp-iters", type=int, default=2, help="subspace iterations with --comp dense")
    ap.add_argument("--ablations", action="store_true",
                    help="instead of the headline line, print one line with the kernel-throughput "
                         "analogues of the pages' Table 2 (per-step fp32 / bf16 / int8 baselines, "
                         "per-window, compensators) and Table 3 (window length p, compensator count r) on this workload")
    ap.add_argument("--ablation-tokens", type=int, default=64)
    ap.add_argument("--ablation-set", choices=("all", "continuous_batching"), default="all",
                    help="with --ablations: every table, or only the continuous-batching one")
    ap.add_argument("--stream-lab", action="store_true",
                    help="instead of the headline line, print one line with the stream reference at the "
                         "decode step's launch shape: the rate against an idle phase per wave after its "
                         "loads, and against waves per launch")
    ap.add_argument("--size-sweep", action="store_true",
                    help="instead of the headline line, print one line with the decode step's and the fused "
                         "close's launch time against states per launch (the workload's gate, p and r; four "
                         "layers cycled; 64 tokens; graph launches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the short separate-close and KDA-workload runs reported beside the headline")
    ap.add_argument("--cpu-sample-states", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=6.0)
    return ap.parse_args()


def run_schedule(cfg, S_init, tok, T, fused, mode, steps, warmup, dev, comp_flags=0, comp_iters=2):
    """Time one decode schedule of workload `cfg` over the first T tokens of
    `tok` (inputs resident in HBM): per step, quantize the initial states,
    then T / p windows of p tokens x L per-layer launches (fused: p - 1 decode
    steps and one decode_close per layer; separate: p decode steps per layer
    and one window close over the whole slab).  HIP events on the launch
    stream bracket every window's decode launches and its closing launches.
    Returns the wall time per step and the average launch times."""
    import torch

    import recurrent_state_quant_amd as lq

    L, nl, n = cfg.layers, cfg.states_per_layer, cfg.n_states
    windows = T // cfg.p
    # the layers' states live in one slab: decoded layer by layer through
    # views, quantized and window-closed together in one launch each
    slab = lq.LeapQuantState(n, cfg.p, cfg.r, cfg.gate, dev, comp_flags, comp_iters=comp_iters)
    slabs = [slab.view(l * nl, nl) for l in range(L)]
    outs = [torch.empty((nl, cfg.dv), device=dev) for _ in range(L)]

    def sl(x, t, l):
        return x[t, l * nl:(l + 1) * nl]

    def quantize_phase():
        lq.leapquant_quantize_state(slab, S_init)

    n_steps = cfg.p - 1 if fused else cfg.p  # decode-step launches per layer and window

    def token_args(t, l):
        return (sl(tok["q"], t, l), sl(tok["k"], t, l), sl(tok["v"], t, l), sl(tok["beta"], t, l),
                sl(tok["alpha"], t, l), outs[l])

    def decode_phase(w):
        for j in range(n_steps):
            t = w * cfg.p + j
            for l in range(L):
                lq.leapquant_decode_step(slabs[l], j, *token_args(t, l))

    def close_phase(w):
        if fused:
            t = w * cfg.p + cfg.p - 1
            for l in range(L):
                lq.leapquant_decode_close(slabs[l], cfg.p - 1, *token_args(t, l))
        else:
            lq.leapquant_window_close(slab, cfg.p)

    if mode == "graph":
        stream = torch.cuda.Stream(device=dev)
        # one warm eager pass on the capture stream before capturing
        with torch.cuda.stream(stream):
            quantize_phase(); decode_phase(0); close_phase(0)
        torch.cuda.synchronize()
        gq = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gq, stream=stream):
            quantize_phase()
        gd, gc = [], []
        for w in range(windows):
            gw = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw, stream=stream):
                decode_phase(w)
            gd.append(gw)
            if fused or w == 0:
                gw = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gw, stream=stream):
                    close_phase(w)
                gc.append(gw)
        torch.cuda.synchronize()
        run_q, run_d = gq.replay, (lambda w: gd[w].replay())
        run_c = (lambda w: gc[w].replay()) if fused else (lambda w: gc[0].replay())
    else:
        stream = torch.cuda.current_stream(dev)
        run_q, run_d, run_c = quantize_phase, decode_phase, close_phase

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(windows)]

    def one_step(record):
        run_q()
        for w in range(windows):
            if record:
                ev[w][0].record(stream)
            run_d(w)
            if record:
                ev[w][1].record(stream)
            run_c(w)
            if record:
                ev[w][2].record(stream)

    with torch.cuda.stream(stream):
        for _ in range(warmup):
            one_step(False)
        torch.cuda.synchronize()
        dec_ms = close_ms = 0.0
        t0 = time.perf_counter()
        for _ in range(steps):
            one_step(True)
            torch.cuda.synchronize()   # events are reused per step: read them now
            dec_ms += sum(e[0].elapsed_time(e[1]) for e in ev)
            close_ms += sum(e[1].elapsed_time(e[2]) for e in ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    close_launches = L if fused else 1
    return {"wall_per_step": wall / steps, "value": n * T / (wall / steps),
            "dec_avg_ms": dec_ms / (steps * windows * n_steps * L),
            "close_avg_ms": close_ms / (steps * windows * close_launches), "n_steps": n_steps,
            "close_launches": close_launches}


def context_runs(dev, tokens=256, steps=2, warmup=1):
    """Short measurements beside the headline (about 10-20 s in all): the
    headline workload in the separate-close schedule, and the KDA workload
    (per-channel gates, r = 8) in the fused schedule, each over its first
    `tokens` tokens.  Reported as head-tokens/s and % of 8 TB/s under each
    schedule's own byte model."""
    import torch

    from workloads import generators as G
    from workloads.configs import WORKLOADS

    out = {}
    for key, name, fused in (("separate_close", "gdn_b256_h32_4layers", False),
                             ("kda_h32_b128", "kda_h32_b128", True)):
        cfg = WORKLOADS[name]
        kda = cfg.gate == "kda"
        g = G.make_generator(cfg.seed, dev)
        S_init = G.initial_state(cfg, cfg.n_states, g, dev)
        tok = G.token_inputs(cfg, cfg.n_states, tokens, g, dev)
        r = run_schedule(cfg, S_init, tok, tokens, fused, "graph", steps, warmup, dev)
        bpht = bytes_per_head_token(cfg.p, cfg.dk, cfg.dv, cfg.r, kda, fused)
        out[key] = {"workload": name, "close": "fused" if fused else "separate", "states": cfg.n_states,
                    "r": cfg.r, "tokens": tokens, "value": round(r["value"], 1), "unit": UNIT,
                    "frac": round(r["value"] * bpht / 1e9 / HBM_PEAK_GBS, 4),
                    "bytes_per_head_token": round(bpht, 1),
                    "decode_avg_launch_us": round(r["dec_avg_ms"] * 1e3, 2),
                    "close_avg_launch_us": round(r["close_avg_ms"] * 1e3, 2)}
        del S_init, tok
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this decode path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the states shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch

    import recurrent_state_quant_amd as lq
    from workloads import generators as G
    from workloads.configs import WORKLOADS

    cfg = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.ablations:
        print(json.dumps(ablations(args, cfg, dev)), flush=True)
        return
    if args.stream_lab:
        print(json.dumps(stream_lab(cfg, dev)), flush=True)
        return
    if args.size_sweep:
        print(json.dumps(size_sweep(cfg, dev)), flush=True)
        return
    kda = cfg.gate == "kda"
    T = args.tokens or cfg.steps
    assert T % cfg.p == 0
    L, nl = cfg.layers, cfg.states_per_layer
    n = cfg.n_states

    # ---- inputs, resident in HBM (untimed)
    t_gen = time.time()
    g = G.make_generator(cfg.seed, dev)
    S_init = G.initial_state(cfg, n, g, dev)
    tok = G.token_inputs(cfg, n, T, g, dev)
    torch.cuda.synchronize()
    print(f"[bench] generated {n} states x {T} tokens in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    dense = args.comp == "dense" and cfg.r > 0
    comp_flags = lq.LQ_DENSE_COMP if dense else 0
    fused = args.close == "fused"
    copy_gbs = copy_calibration(dev)
    run = run_schedule(cfg, S_init, tok, T, fused, args.mode, args.steps, args.warmup, dev, comp_flags,
                       args.comp_iters)
    n_steps = run["n_steps"]
    ms_per_step = 1e3 * run["wall_per_step"]
    value = run["value"]
    bpht = bytes_per_head_token(cfg.p, cfg.dk, cfg.dv, cfg.r, kda, fused, dense)
    bpht_unfused = bytes_per_head_token(cfg.p, cfg.dk, cfg.dv, cfg.r, kda, dense=dense)
    dec_avg_ms = run["dec_avg_ms"]
    dec_bytes = nl * sum(step_bytes(t, cfg.dk, cfg.dv, cfg.r, kda, dense) for t in range(n_steps)) / n_steps
    dec_gbs = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    close_states = nl if fused else n           # per launch
    close_state_bytes = (fused_bytes(cfg.p - 1, cfg.dk, cfg.dv, cfg.r, kda, dense) if fused
                         else close_bytes(cfg.p, cfg.dk, cfg.dv, cfg.r, kda, dense))
    close_avg_ms = run["close_avg_ms"]
    close_gbs = close_states * close_state_bytes / (close_avg_ms * 1e-3) / 1e9
    # matrix-path work of the rebuild as issued: windows of up to 16 records
    # (row compensators, r <= 8) run three bf16 16x16x32 steps per 16 x 16
    # output tile (the six cross products of a three-part split); other
    # shapes run fp32 16x16x4 steps over the records padded to a multiple
    # of 4 (dense tokens add r records)
    slots = (cfg.p - 1 if fused else cfg.p) + (cfg.r if dense else 0)
    bf16_path = not dense and cfg.p <= 16 and cfg.r <= 8
    if bf16_path:
        close_flops = close_states * 64 * 3 * 2 * 16 * 16 * 32
        mfma_peak, mfma_dtype = MFMA_BF16_PEAK_TFLOPS, "bf16 (three-part split of fp32 operands)"
    else:
        close_flops = close_states * 2 * cfg.dk * cfg.dv * ((slots + 3) // 4 * 4)
        mfma_peak, mfma_dtype = MFMA_FP32_PEAK_TFLOPS, "fp32"
    close_mfma_util = close_flops / (close_avg_ms * 1e-3) / (mfma_peak * 1e12)
    # a plain stream with the decode step's mean bytes per state, one wave
    # per state and as many waves as one decode launch: the rows it writes
    # (record t, o_t, u_t) at the end of the wave, the rest read (to the
    # nearest KiB)
    wr = 512 * (3 + (1 if kda else 0))
    stream_ref = stream_reference(dev, max(1, round((dec_bytes / nl - wr) / 1024)) * 1024, wr, nl)
    stream_ref["decode_frac_of_stream"] = round(dec_gbs / stream_ref["GBs"], 4)
    # the same plain stream with the close's bytes per state, one wave per
    # state and as many waves as one close launch: the boundary state it
    # writes (and o_t when fused) at the end of the wave, the rest read.  A
    # third of the close's bytes are writes, which the device moves more
    # slowly than reads; this is the rate of that mix with no arithmetic.
    # Part of the context (skipped with --no-context, as in the profiled
    # runs, whose stream-reference dispatches then all have the decode's
    # shape).
    if not dense and not args.no_context:
        cw = _boundary_rw(cfg.dk, cfg.dv, cfg.r, False) // 2 + (4 * cfg.dv if fused else 0)
        cwr = max(512, round(cw / 512) * 512)
        crd = max(1024, round((close_state_bytes - cw) / 1024) * 1024)
        close_mix = stream_reference(dev, crd, cwr, close_states)
        close_mix["close_frac_of_stream"] = round(close_gbs / close_mix["GBs"], 4)
        stream_ref["close_mix"] = close_mix
    whole_gbs = value * bpht / 1e9
    traffic = {} if dense else measured_traffic(cfg)
    dkey = "decode_fused" if fused else "decode_separate"
    dec_traffic = round(traffic[dkey] * nl) if dkey in traffic else None
    ckey = "fused" if fused else "close"
    close_traffic = round(traffic[ckey] * close_states) if ckey in traffic else None

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "gate": cfg.gate, "batch": cfg.batch, "heads": cfg.heads,
                   "layers": L, "states": n, "dk": cfg.dk, "dv": cfg.dv, "p": cfg.p, "r": cfg.r,
                   "tokens": T, "state_storage": "int8 codes + fp32 scales, fp32 compensators",
                   "launch": args.mode, "close": args.close},
        "whole_step": {"algorithmic_GBs": round(whole_gbs, 1), "frac": round(whole_gbs / HBM_PEAK_GBS, 4),
                       "bytes_per_head_token": round(bpht, 1),
                       "unfused_bytes_per_head_token": round(bpht_unfused, 1),
                       "frac_of_unfused_model": round(value * bpht_unfused / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "decode_step", "achieved": round(dec_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": dec_traffic, "bytes_per_launch": round(dec_bytes),
                     "avg_launch_us": round(dec_avg_ms * 1e3, 2)},
        "window_close": {"kernel": "decode_close (fused)" if fused else "window_close",
                         "avg_launch_us": round(close_avg_ms * 1e3, 2), "achieved_GBs": round(close_gbs, 1),
                         "frac": round(close_gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": close_states * close_state_bytes,
                         "states_per_launch": close_states, "launches_per_window": run["close_launches"],
                         "traffic": close_traffic, "mfma_dtype": mfma_dtype,
                         "mfma_flops_per_launch": close_flops, "mfma_util": round(close_mfma_util, 4)},
        "hbm_copy_GBs": round(copy_gbs, 1),
        "stream_reference": stream_ref,
    }

    if dense:
        result["config"]["compensators"] = f"dense tokens, {args.comp_iters} subspace iterations"
    if not args.no_context and args.workload == "gdn_b256_h32_4layers" and not dense and T == cfg.steps:
        t_ctx = time.perf_counter()
        result["context"] = context_runs(dev)
        result["context"]["wall_s"] = round(time.perf_counter() - t_ctx, 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, cfg, S_init, tok, comp_flags, args.comp_iters)
    print(json.dumps(result), flush=True)


def dense_bytes(dk, dv, kda, elem):
    """Algorithmic bytes of one dense-state token for one state: read and
    write the state, read the token's inputs, write its output."""
    G = dk if kda else 1
    return 2 * elem * dk * dv + 4 * (2 * dk + dv + 1 + G) + 4 * dv


def bf16w_bytes(p, dk, dv, kda):
    """Algorithmic bytes per state and token of the "BF16 + per-window" row:
    p decode steps (read the bf16 boundary state and the buffered records,
    read the token's inputs, write its output and record) and one window
    close (read and write the bf16 state, read the p records), spread over
    the window's p tokens."""
    G = dk if kda else 1
    R = G + dk + dv
    dec = sum(2 * dk * dv + 4 * t * R + 4 * (2 * dk + dv + 1 + G) + 4 * dv + 4 * R for t in range(p)) / p
    return dec + (4 * dk * dv + 4 * p * R) / p


def ablations(args, cfg, dev, reps=3):
    """Kernel-level analogues of the pages' Table 2 and Table 3 on this
    workload's shape: head-tokens/s of each variant (all layers' states
    resident, one launch per layer and token, launches replayed from one
    graph per variant), and the ratio to the fp32 per-step baseline."""
    import torch
    import recurrent_state_quant_amd as lq
    from workloads import generators as G
    T = args.ablation_tokens
    L, nl, n = cfg.layers, cfg.states_per_layer, cfg.n_states
    kda = cfg.gate == "kda"
    g = G.make_generator(cfg.seed, dev)
    S_init = G.initial_state(cfg, n, g, dev)
    tok = G.token_inputs(cfg, n, T, g, dev)
    outs = [torch.empty((nl, cfg.dv), device=dev) for _ in range(L)]

    def targs(t, l):
        sl = slice(l * nl, (l + 1) * nl)
        return (tok["q"][t, sl], tok["k"][t, sl], tok["v"][t, sl], tok["beta"][t, sl],
                tok["alpha"][t, sl], outs[l])

    def timed(run):
        stream = torch.cuda.Stream(device=dev)
        with torch.cuda.stream(stream):
            run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        return n * T * reps / (time.perf_counter() - t0)

    def dense(dtype):
        S = S_init.clone() if dtype == torch.float32 else S_init.to(dtype)
        views = [S[l * nl:(l + 1) * nl] for l in range(L)]

        def run():
            for t in range(T):
                for l in range(L):
                    lq.leapquant_dense_step(views[l], cfg.gate, *targs(t, l))
        value = timed(run)
        del S, views
        return value, dense_bytes(cfg.dk, cfg.dv, kda, 4 if dtype == torch.float32 else 2)

    def bf16win(p):
        B = S_init.to(torch.bfloat16)
        slab = lq.LeapQuantState(n, p, 0, cfg.gate, dev)
        views = [(slab.view(l * nl, nl), B[l * nl:(l + 1) * nl]) for l in range(L)]

        def run():
            for t in range(T):
                j = t % p
                for l in range(L):
                    lq.leapquant_bf16w_decode_step(views[l][0], views[l][1], j, *targs(t, l))
                if j == p - 1:
                    for l in range(L):
                        lq.leapquant_bf16w_window_close(views[l][0], views[l][1], p)
        value = timed(run)
        del B, slab, views
        return value, bf16w_bytes(p, cfg.dk, cfg.dv, kda)

    def windowed(p, r, flags, iters=0):
        slab = lq.LeapQuantState(n, p, r, cfg.gate, dev, flags, comp_iters=iters)
        lq.leapquant_quantize_state(slab, S_init)
        views = [slab.view(l * nl, nl) for l in range(L)]

        def run():
            for t in range(T):
                j = t % p
                for l in range(L):
                    if j == p - 1:
                        lq.leapquant_decode_close(views[l], j, *targs(t, l))
                    else:
                        lq.leapquant_decode_step(views[l], j, *targs(t, l))
        value = timed(run)
        del slab, views
        return value, bytes_per_head_token(p, cfg.dk, cfg.dv, r, kda, fused=True,
                                           dense=bool(flags & lq.LQ_DENSE_COMP) and r > 0)

    def slots(p, r, compact=False, mixed=False, grouped=False, concurrent=False):
        # continuous batching: every slot has its own window phase (seeded,
        # uniform), so about 1/p of the slots close at every token; the
        # positions live on the device.  (Phases strided by a multiple of 8
        # in slot order would put every closing workgroup on one XCD: the
        # dispatcher deals workgroups to the 8 XCDs round-robin.)
        slab = lq.LeapQuantState(n, p, r, cfg.gate, dev)
        lq.leapquant_quantize_state(slab, S_init)
        views = [slab.view(l * nl, nl) for l in range(L)]
        gp = torch.Generator(device=dev).manual_seed(cfg.seed + 1)
        if grouped:
            # four consecutive slots share a phase (a decode workgroup's four
            # waves then decode at one window position)
            phase = torch.randint(0, p, ((nl + 3) // 4,), generator=gp, device=dev,
                                  dtype=torch.int32).repeat_interleave(4)[:nl]
        else:
            phase = torch.randint(0, p, (nl,), generator=gp, device=dev, dtype=torch.int32)
        pos = [(phase + t) % p for t in range(T)]
        step_pos = [torch.where(x == p - 1, -1, x).to(torch.int32) for x in pos]
        close_pos = [torch.where(x == p - 1, x, -1).to(torch.int32) for x in pos]
        # compact: the ids of the slots that close at token t, one workgroup each
        close_list = [torch.nonzero(x == p - 1).flatten().to(torch.int32) for x in pos]
        # concurrent: the closing slots' closes on a second stream (default
        # priority) beside the other slots' decode step; the next token's
        # step of a layer waits for that layer's closes
        side = torch.cuda.Stream(device=dev) if concurrent else None

        def run():
            main = torch.cuda.current_stream(dev)
            joins = [None] * L
            for t in range(T):
                for l in range(L):
                    if concurrent:
                        if joins[l] is not None:
                            main.wait_event(joins[l])
                        fork = torch.cuda.Event()
                        fork.record(main)
                        side.wait_event(fork)
                        with torch.cuda.stream(side):
                            lq.leapquant_decode_close_list(views[l], pos[t], close_list[t], *targs(t, l))
                        joins[l] = torch.cuda.Event()
                        joins[l].record(side)
                        lq.leapquant_decode_step_slots(views[l], step_pos[t], *targs(t, l))
                        continue
                    if mixed:
                        lq.leapquant_decode_step_close_list(views[l], pos[t], close_list[t], *targs(t, l))
                        continue
                    lq.leapquant_decode_step_slots(views[l], step_pos[t], *targs(t, l))
                    if compact:
                        lq.leapquant_decode_close_list(views[l], pos[t], close_list[t], *targs(t, l))
                    else:
                        lq.leapquant_decode_close_slots(views[l], close_pos[t], *targs(t, l))
            for e in joins:
                if e is not None:
                    main.wait_event(e)
        value = timed(run)
        del slab, views
        return value, bytes_per_head_token(p, cfg.dk, cfg.dv, r, kda, fused=True)

    rows2 = [("FP32 per-step", lambda: dense(torch.float32)),
             ("BF16 per-step", lambda: dense(torch.bfloat16)),
             ("BF16 + per-window (p = 16, separate close)", lambda: bf16win(16)),
             ("INT8 per-step", lambda: windowed(1, 0, 1)),
             ("+ Per-window (p = 16)", lambda: windowed(16, 0, 1)),
             ("+ Comp. Tokens (r = 4) and smoothing", lambda: windowed(16, cfg.r, 0))]
    rows3 = [(f"p = {p}", (lambda p=p: windowed(p, cfg.r, 0))) for p in (4, 8, 16, 32)]
    rows3r = [(f"r = {r}", (lambda r=r: windowed(cfg.p, r, 0))) for r in (0, 2, 4, 8, 16)]

    def table(rows, ref):
        out = []
        for name, fn in rows:
            value, bpht = fn()
            out.append({"row": name, "head_tokens_per_s": round(value, 1),
                        "kernel_speedup": round(value / ref, 3) if ref else 1.0,
                        "bytes_per_head_token": round(bpht, 1),
                        "hbm_frac": round(value * bpht / 1e9 / HBM_PEAK_GBS, 4)})
            if ref is None:
                ref = value
        return out, ref

    rows_cb = [("lockstep windows (all slots at the same position)", lambda: windowed(cfg.p, cfg.r, 0)),
               ("continuous batching (slot phases spread over the window)", lambda: slots(cfg.p, cfg.r)),
               ("continuous batching, closes launched for the closing slots only (slot list)",
                lambda: slots(cfg.p, cfg.r, compact=True)),
               ("continuous batching, one launch per token (closing slots' workgroups spread among the decode steps)",
                lambda: slots(cfg.p, cfg.r, mixed=True)),
               ("continuous batching, one launch per token, four consecutive slots sharing a phase",
                lambda: slots(cfg.p, cfg.r, mixed=True, grouped=True)),
               ("continuous batching, the closing slots' closes on a second stream beside the decode steps",
                lambda: slots(cfg.p, cfg.r, concurrent=True))]
    DC = lq.LQ_DENSE_COMP
    rows_dc = [("row compensators", lambda: windowed(cfg.p, cfg.r, 0))] + \
        [(f"dense tokens, {i} subspace iteration{'s' if i != 1 else ''}", (lambda i=i: windowed(cfg.p, cfg.r, DC, i)))
         for i in (0, 1, 2)]
    if args.ablation_set == "continuous_batching":
        tcb, _ = table(rows_cb, None)
        return {"metric": "continuous batching throughput (head-tokens/s; ratio to lockstep windows)",
                "workload": cfg.name, "tokens": T, "reps": reps, "launch": "graph", "continuous_batching": tcb}
    t2, ref = table(rows2, None)
    t3, _ = table(rows3, ref)
    t3r, _ = table(rows3r, ref)
    tcb, _ = table(rows_cb, ref)
    tdc, _ = table(rows_dc, ref)
    lat = latency(dev)
    return {"metric": "kernel throughput ablations (head-tokens/s; speedup over fp32 per-step)",
            "workload": cfg.name, "tokens": T, "reps": reps, "launch": "graph",
            "schedule": "one launch per layer and token; last token of each window fused with its close",
            "table2": t2, "table3_r": cfg.r, "table3": t3, "table3_p": cfg.p, "table3_r_sweep": t3r,
            "continuous_batching": tcb,
            "compensator_forms": tdc,
            "latency_single_state": lat}


def latency(dev, windows=8, reps=20):
    """Per-token latency of the single-head, batch-1 workload (one state, one
    layer): a window of decode steps with the fused last token, replayed from
    a graph; reported as microseconds per token (window time / p)."""
    import torch
    import recurrent_state_quant_amd as lq
    from workloads import generators as G
    from workloads.configs import WORKLOADS
    cfg = WORKLOADS["gdn_single_head_b1"]
    T = windows * cfg.p
    g = G.make_generator(cfg.seed, dev)
    S_init = G.initial_state(cfg, 1, g, dev)
    tok = G.token_inputs(cfg, 1, T, g, dev)
    out = torch.empty((1, cfg.dv), device=dev)
    res = {}
    for sched in ("fused", "separate"):
        st = lq.LeapQuantState(1, cfg.p, cfg.r, cfg.gate, dev)
        lq.leapquant_quantize_state(st, S_init)

        def run():
            for t in range(T):
                j = t % cfg.p
                args = (tok["q"][t], tok["k"][t], tok["v"][t], tok["beta"][t], tok["alpha"][t], out)
                if j == cfg.p - 1 and sched == "fused":
                    lq.leapquant_decode_close(st, j, *args)
                else:
                    lq.leapquant_decode_step(st, j, *args)
                    if j == cfg.p - 1:
                        lq.leapquant_window_close(st, cfg.p)
        stream = torch.cuda.Stream(device=dev)
        with torch.cuda.stream(stream):
            run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        res[sched + "_us_per_token"] = round((time.perf_counter() - t0) / (reps * T) * 1e6, 2)
    res["workload"] = cfg.name
    return res


def copy_calibration(dev, nbytes=1 << 31, reps=5):
    """Measured device-to-device copy rate (read + write bytes per second) of
    a plain copy of nbytes, as a reference ceiling for the HBM figures."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def stream_reference(dev, read_bytes, write_bytes, waves, slabs=4, reps=24, idle=0):
    """Rate of a plain stream in the decode step's launch shape: waves waves
    per launch, each reading its own read_bytes bytes and then writing
    write_bytes bytes (leapquant_stream_reference), over `slabs` buffers
    cycled like layers so that no launch finds its bytes in a cache.  HIP
    events on the launch stream bracket the timed launches."""
    import torch
    import recurrent_state_quant_amd as lq
    stream = torch.cuda.Stream(device=dev)
    srcs = [torch.empty(read_bytes * waves, dtype=torch.uint8, device=dev) for _ in range(slabs)]
    dsts = [torch.empty(write_bytes * waves, dtype=torch.uint8, device=dev) if write_bytes else None
            for _ in range(slabs)]
    out = torch.empty((waves, 64), dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for x, y in zip(srcs, dsts):
            x.fill_(1)
            lq.leapquant_stream_reference(x, read_bytes, y, write_bytes, out, stream, idle)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            lq.leapquant_stream_reference(srcs[i % slabs], read_bytes, dsts[i % slabs], write_bytes, out, stream,
                                          idle)
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del srcs, dsts, out
    return {"read_bytes_per_wave": read_bytes, "write_bytes_per_wave": write_bytes, "waves": waves,
            "avg_launch_us": round(us, 2), "GBs": round((read_bytes + write_bytes) * waves / (us * 1e-6) / 1e9, 1)}


def size_sweep(cfg, dev, sizes=(1, 64, 256, 1024, 2048, 4096, 8192, 16384, 32768), T=64):
    """Launch time of the decode step and of the fused last-token close
    against states per launch: the workload's gate, p and r with `size`
    states per layer, four layers cycled (so that no launch finds its state
    in a cache), the fused schedule over T tokens replayed from graphs
    (run_schedule).  Rates use the algorithmic bytes of step_bytes and
    fused_bytes."""
    import dataclasses
    import torch
    from workloads import generators as G
    kda = cfg.gate == "kda"
    rows = []
    for nl in sizes:
        c = dataclasses.replace(cfg, batch=nl, heads=1, layers=4, steps=T)
        g = G.make_generator(c.seed, dev)
        S_init = G.initial_state(c, c.n_states, g, dev)
        tok = G.token_inputs(c, c.n_states, T, g, dev)
        run = run_schedule(c, S_init, tok, T, True, "graph", 2, 1, dev)
        dec_b = nl * sum(step_bytes(t, c.dk, c.dv, c.r, kda) for t in range(c.p - 1)) / (c.p - 1)
        fb = nl * fused_bytes(c.p - 1, c.dk, c.dv, c.r, kda)
        d_us, c_us = run["dec_avg_ms"] * 1e3, run["close_avg_ms"] * 1e3
        rows.append({"states_per_launch": nl, "decode_us": round(d_us, 2), "decode_TBs": round(dec_b / d_us / 1e6, 3),
                     "fused_close_us": round(c_us, 2), "fused_close_TBs": round(fb / c_us / 1e6, 3)})
        del S_init, tok
        torch.cuda.empty_cache()
    return {"metric": "launch time against states per launch (us; TB/s of algorithmic bytes)",
            "workload": cfg.name, "gate": cfg.gate, "p": cfg.p, "r": cfg.r, "tokens": T, "rows": rows}


def stream_lab(cfg, dev):
    """The stream reference at the decode step's shape on `cfg` (mean bytes
    per state read and the rows written, one wave per state): the rate with
    an idle phase of 0 .. 32 x 512 cycles per wave between its loads and its
    stores (a stand-in for the work a decode wave does once its loads have
    returned), and the rate for 1/2 .. 4x the waves of one launch."""
    kda = cfg.gate == "kda"
    nl = cfg.states_per_layer
    dec = sum(step_bytes(t, cfg.dk, cfg.dv, cfg.r, kda) for t in range(cfg.p - 1)) / (cfg.p - 1)
    wr = 512 * (3 + (1 if kda else 0))
    rd = max(1, round((dec - wr) / 1024)) * 1024
    idle = []
    for k in (0, 4, 8, 16, 32):
        r = stream_reference(dev, rd, wr, nl, idle=k)
        idle.append({"idle_cycles_per_wave": 512 * k, "avg_launch_us": r["avg_launch_us"], "GBs": r["GBs"]})
    waves = []
    for m in (0.5, 1, 2, 4):
        r = stream_reference(dev, rd, wr, int(nl * m))
        waves.append({"waves": int(nl * m), "avg_launch_us": r["avg_launch_us"], "GBs": r["GBs"]})
    return {"metric": "stream reference at the decode step's launch shape (GB/s, read + write)",
            "workload": cfg.name, "read_bytes_per_wave": rd, "write_bytes_per_wave": wr,
            "idle_phase": idle, "waves_per_launch": waves}


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_group(job):
    """One worker's share of the all-core oracle run: free-running decode of
    its group of states over all tokens (inputs memory-mapped from a .npz
    written by the parent).  Returns (head-tokens, seconds of compute)."""
    path, g, p, r, gate, flags, iters, barrier_path = job
    import numpy as np

    from oracle import leapquant_oracle as O
    d = np.load(path, mmap_mode="r")
    S0 = np.array(d[f"S{g}"])
    tk = {k: np.array(d[f"{k}{g}"]).astype(np.float64) for k in ("q", "k", "v", "beta", "alpha")}
    # start together: wait until every worker has loaded its inputs
    open(f"{barrier_path}.{g}", "w").close()
    while len([f for f in os.listdir(os.path.dirname(barrier_path))
               if f.startswith(os.path.basename(barrier_path) + ".")]) < int(d["workers"]):
        time.sleep(0.005)
    t0 = time.perf_counter()
    b = O.quantize(S0, r, flags, iters)
    T = tk["q"].shape[0]
    for t in range(0, T, p):
        _, _, _, b = O.window(b, tk, t, p, gate, r, flags, iters=iters)
    return S0.shape[0] * T, time.perf_counter() - t0


def cpu_baseline(args, cfg, S_init, tok, comp_flags=0, iters=0):
    """The CPU oracle, free-running on bounded samples of the same inputs.

    All cores: one worker process per host core (at most 16, the host's
    share for one GPU), each decoding its own group of `cpu_sample_states` states
    of layer 0 over all tokens; the rate is the groups' head-tokens over the
    wall time from the common start to the last worker's end.  One process:
    groups decoded one after another until about `cpu_seconds` have passed.
    Inputs are copied to the host before either timed region."""
    import multiprocessing as mp
    import tempfile

    import numpy as np
    import torch

    from oracle import leapquant_oracle as O

    ns = min(args.cpu_sample_states, cfg.states_per_layer)
    T = tok["q"].shape[0]
    gate = O.GATE_GDN if cfg.gate == "gdn" else O.GATE_KDA
    flags = O.DENSE_COMP if comp_flags else 0

    def group(gi):
        idx = torch.arange(gi * ns, (gi + 1) * ns, device=S_init.device)
        S0 = S_init.index_select(0, idx).cpu().numpy()
        tk = {k: v.index_select(1, idx).cpu().numpy() for k, v in tok.items()}
        return S0, tk

    # ---- one process
    t0 = time.perf_counter()
    head_tokens, groups, busy = 0, 0, 0.0
    while busy < args.cpu_seconds and (groups + 1) * ns <= cfg.states_per_layer:
        S0, tk = group(groups)
        tk = {k: v.astype(np.float64) for k, v in tk.items()}
        c0 = time.perf_counter()
        b = O.quantize(S0, cfg.r, flags, iters)
        for t_ in range(0, T, cfg.p):
            _, _, _, b = O.window(b, tk, t_, cfg.p, gate, cfg.r, flags, iters=iters)
        busy += time.perf_counter() - c0
        head_tokens += ns * T
        groups += 1
    single = head_tokens / busy

    # ---- all cores: one group per worker, started together
    workers = max(1, min(16, os.cpu_count() or 1, cfg.states_per_layer // ns))
    with tempfile.TemporaryDirectory(dir="/dev/shm" if os.path.isdir("/dev/shm") else None) as tmp:
        path = os.path.join(tmp, "inputs.npz")
        arrays = {"workers": np.array(workers)}
        for gi in range(workers):
            S0, tk = group(gi)
            arrays[f"S{gi}"] = S0
            for k, v in tk.items():
                arrays[f"{k}{gi}"] = v
        np.savez(path, **arrays)
        del arrays
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"  # one thread per worker process
        try:
            jobs = [(path, gi, cfg.p, cfg.r, gate, flags, iters, os.path.join(tmp, "ready"))
                    for gi in range(workers)]
            ctx = mp.get_context("spawn")
            w0 = time.perf_counter()
            with ctx.Pool(workers) as pool:
                res = pool.map(_oracle_group, jobs)
            wall_pool = time.perf_counter() - w0
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    total = sum(h for h, _ in res)
    # every worker started at the common barrier: the slowest one's compute
    # time is the parallel run's wall time
    wall = max(sec for _, sec in res)
    return {"value": round(total / wall, 1), "unit": UNIT, "cores": workers, "kind": "oracle",
            "sample": f"{workers} groups of {ns} states of layer 0 x {T} tokens, one group per worker process, "
                      "free-running, fp64 numpy; inputs copied to the host before timing",
            "wall_s": round(wall, 2),
            "single_process": {"value": round(single, 1), "unit": UNIT, "cores": 1,
                               "sample": f"{groups} groups of {ns} states x {T} tokens", "busy_s": round(busy, 2)},
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
            "total_s": round(time.perf_counter() - t0, 2), "pool_s": round(wall_pool, 2)}


if __name__ == "__main__":
    main()
