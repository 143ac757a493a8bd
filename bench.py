"""Benchmark of the MoE layer forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
tokens already resident in HBM: router + KeepTopK + softmax, grouping by
expert, expert up projection + activation, down projection, gate-weighted
combine, and the side statistics (counts, Importance, CV^2, load-balance
loss).  The step issues the same kernels as moe_forward, through the stage
entry points, so that the dominant kernel (the expert up projection) can
be bracketed with HIP events on the stream it runs on.

Prints one JSON line.  Default workload: the Mixtral-8x7B-shape layer
(T=4096, d=4096, h=14336, 8 experts, top-2, SwiGLU, bf16); the default line
also carries the gpt-oss-20b-shape decode layer (T=64, d=h=2880, 32
experts, top-4, SwiGLU, bf16) under "decode", timed in the same process.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
IMPORTANCE_LOSS_WEIGHT = 0.01   # training step: w * CV^2(Importance)
LOAD_LOSS_WEIGHT = 0.01         # training step with the noisy gate: w * CV^2(smooth Load)
METRIC = "MoE layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak); decode HBM GB/s"


GATES = {"topk-softmax": 0, "bias-selects": 1, "softmax-all": 2}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", default="mixtral-8x7b")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--gate", choices=list(GATES), default="topk-softmax",
                   help="gate mode: softmax over the kept k, bias that selects only, "
                        "or softmax over all experts")
    p.add_argument("--noisy", action="store_true",
                   help="training-time noisy top-k gate (moe_route_noisy) in the step")
    p.add_argument("--backward", action="store_true",
                   help="training step: the forward stages, then moe_backward")
    p.add_argument("--weight-copies", type=int, default=0,
                   help="copies of the layer (weights and x) that the steps rotate through, "
                        "so that no step finds its weights in the memory-side cache; "
                        "0: enough copies for 1 GiB when the layer is smaller (at most 32)")
    p.add_argument("--capacity-factor", type=float, default=0.0,
                   help="per-expert capacity ceil(f*T*k/E) with drops (0: none)")
    p.add_argument("--overflow", choices=["drop", "next-choice"], default="drop",
                   help="beyond the capacity: drop, or hand the slot on once to the "
                        "token's next choice")
    p.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.txt"),
                   help="measured HBM bytes of the dominant kernel per workload (JSON text)")
    p.add_argument("--grouped-copy", action="store_true",
                   help="the dispatch writes the grouped copy x_perm and the up projection "
                        "reads it (default: the up projection reads the rows of x in place)")
    p.add_argument("--no-decode", action="store_true",
                   help="default workload only: skip the decode-shape layer that the line "
                        "also reports")
    p.add_argument("--weight-layout", choices=["tiled", "row-major"], default=None,
                   help="order of the expert matrices in HBM (default for bf16 forward "
                        "steps: tiled, rewritten once by moe_tile_weights before timing, "
                        "as at weight loading; otherwise row-major, the only order the "
                        "backward pass and fp32 layers read)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first copy 1 GiB device to device three times, so that a PMC "
                        "run sees a plain copy of known size beside the layer's kernels")
    return p.parse_args()


def source_digest() -> str:
    """sha256 over the sources of the grouped-GEMM kernels: measured traffic
    is reported only while they are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_bf16.hip", "common.h"):
        with open(os.path.join(ROOT, "sparse_mixture_experts_07_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def run_one(args):
    """Time args.steps steps of args.workload; the result object (the JSON
    line's fields)."""
    import numpy as np
    import torch

    import synthetic
    from sparse_mixture_experts_07_amd import binding as B
    from sparse_mixture_experts_07_amd.device import DeviceLayer, Forward

    cfg = synthetic.BY_NAME[args.workload].with_(gate=GATES[args.gate])
    if args.noisy and cfg.gate != 0:
        sys.exit("--noisy takes the default gate only")
    t_gen = time.time()
    L = synthetic.make_inputs(cfg)
    if args.noisy:
        L.w_noise, noise_np = synthetic.make_noisy_gate(cfg)
    cap = 0
    if args.capacity_factor > 0:
        cap = B.moe_expert_capacity(cfg.T, cfg.k, cfg.E, args.capacity_factor)
    overflow = B.MOE_OVERFLOW_NEXT_CHOICE if args.overflow == "next-choice" else 0
    if overflow and not cap:
        sys.exit("--overflow next-choice needs --capacity-factor")
    if overflow and args.noisy:
        # the next choices are ranked by moe_route's scores; the noisy gate
        # selects on H = s + n * Softplus(...), which no call outputs
        sys.exit("--noisy does not combine with --overflow next-choice")
    dl = DeviceLayer.upload(L, capacity=cap, overflow=overflow)
    # Steps rotate through copies of the layer: a layer whose weights fit in
    # the 256 MB memory-side cache would otherwise be read back from it,
    # which a model (other layers' weights between two calls) never sees.
    # Measured: at the Mixtral, DeepSeek-V3 and decode shapes rotation changes
    # nothing (their weights exceed the cache several times); at the GPT-2
    # shape (57 MB of weights) one copy runs 5 % faster.
    layer_bytes = sum(a.nbytes for a in (L.x, L.w_up, L.w_down, L.w_up_shared, L.w_down_shared)
                      if a is not None)
    ncopy = args.weight_copies or min(32, max(1, -(-(1 << 30) // layer_bytes)))
    copies = [dl] + [DeviceLayer.upload(L, capacity=cap, overflow=overflow)
                     for _ in range(ncopy - 1)]
    layout = args.weight_layout or ("tiled" if cfg.dtype == synthetic.BF16 and not args.backward
                                    else "row-major")
    if layout == "tiled":
        if args.backward or cfg.dtype != synthetic.BF16:
            sys.exit("--weight-layout tiled: bf16 forward steps only")
        copies = [cp.tiled() for cp in copies]
        dl = copies[0]
        torch.cuda.synchronize()
    copy_w = [cp.weights() for cp in copies]
    turn = [0]
    gen_s = time.time() - t_gen
    c, W = dl.cfg, dl.weights()
    T, k, E, d, h = cfg.T, cfg.k, cfg.E, cfg.d, cfg.h
    dev = dl.x.device
    dt = dl.act_dtype
    R = B.moe_grouped_rows(c)

    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    imp = torch.empty(E, dtype=torch.float32, device=dev)
    stats = torch.empty(3, dtype=torch.float64, device=dev)
    gathers = T * d * (2 if dt == torch.bfloat16 else 4) < 2 ** 31 and not args.grouped_copy
    x_perm = torch.empty((T * k, d), dtype=dt, device=dev)
    hidden = torch.empty((R, h), dtype=dt, device=dev)
    y_perm = torch.empty((R, d), dtype=dt, device=dev)
    y = torch.empty((T, d), dtype=dt, device=dev)
    ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    # the softmax-all gate's backward and next-choice re-routing read the
    # forward's router scores
    logits = (torch.empty((T, E), dtype=torch.float32, device=dev)
              if (args.backward and cfg.gate == synthetic.GATE_SOFTMAX_ALL) or overflow
              else None)
    if args.noisy:
        from sparse_mixture_experts_07_amd.device import to_device
        w_noise, noise = to_device(L.w_noise, dev), to_device(noise_np, dev)
        clean = torch.empty((T, E), dtype=torch.float32, device=dev)
        nscale = torch.empty((T, E), dtype=torch.float32, device=dev)
        nimp = torch.empty(E, dtype=torch.float32, device=dev)
        nload = torch.empty(E, dtype=torch.float32, device=dev)
        ncv2 = torch.empty(2, dtype=torch.float64, device=dev)

    def route(dl):
        if args.noisy:
            B.moe_route_noisy(c, dl.x, dl.w_gate, dl.b_gate, w_noise, noise, clean, nscale,
                              idx, tw, counts, nimp, nload, ncv2, ws)
        else:
            # counts come from the grouping, as in moe_forward
            B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, tw, None, logits)

    if args.backward:
        if cfg.dtype != synthetic.BF16:
            sys.exit("--backward: bf16 layers only")
        f32 = dict(dtype=torch.float32, device=dev)
        n_up = cfg.n_up
        b16 = dict(dtype=dt, device=dev)   # gradients of bf16 parameters
        g_t = dict(dx=torch.empty((T, d), **b16),
                   w_gate=torch.empty((E, d), **f32), w_up=torch.empty((E, n_up, d), **b16),
                   w_down=torch.empty((E, d, h), **b16),
                   b_gate=torch.empty(E, **f32) if L.b_gate is not None else None,
                   w_up_shared=torch.empty((1, n_up, d), **b16) if cfg.S else None,
                   w_down_shared=torch.empty((1, d, h), **b16) if cfg.S else None)
        grads = B.grads(g_t["dx"], g_t["w_gate"], g_t["w_up"], g_t["w_down"], g_t["b_gate"],
                        dw_up_shared=g_t["w_up_shared"], dw_down_shared=g_t["w_down_shared"])
        ws_b = torch.empty(B.moe_backward_workspace_bytes(c), dtype=torch.uint8, device=dev)
        dy = torch.randn((T, d), generator=torch.Generator(device="cpu").manual_seed(1)).to(
            device=dev, dtype=dt)
        preact = torch.empty((R, cfg.n_up), dtype=dt, device=dev)
        bwd_evs = []
        nz = None
        if args.noisy:   # the noisy gate's share: W_noise and the smooth-Load loss
            g_t["w_noise"] = torch.empty((E, d), **f32)
            nz = B.noisy_grad(w_noise, noise, clean, nscale, g_t["w_noise"], nload,
                              LOAD_LOSS_WEIGHT)

    def step(ev=None):
        # this step's copy of the layer (x and weights)
        dl, W = copies[turn[0] % ncopy], copy_w[turn[0] % ncopy]
        turn[0] += 1
        route(dl)
        # the up projection reads the token rows of x in place (as moe_forward
        # does); the training step keeps the grouped copy for the backward
        xp = x_perm if args.backward or not gathers else None
        B.moe_permute(c, idx, tw, dl.x, offsets, perm_src, pos, imp, stats, xp, ws,
                      logits=logits, counts=None if args.noisy else counts)
        if ev is not None:
            ev[0].record()
        if args.backward:   # the training forward keeps the pre-activations
            B.moe_expert_up_train(c, W, x_perm, dl.x, offsets, hidden, preact)
        else:
            B.moe_expert_up(c, W, xp, dl.x, offsets, hidden, perm_src=perm_src)
        if ev is not None:
            ev[1].record()
        B.moe_expert_down(c, W, hidden, offsets, y_perm)
        B.moe_combine(c, y_perm, pos, tw, y)
        if args.backward:
            if ev is not None:
                bwd_evs.append((torch.cuda.Event(enable_timing=True),
                                torch.cuda.Event(enable_timing=True)))
                bwd_evs[-1][0].record()
            B.moe_backward(c, W, dl.x, dy, idx, tw, offsets, pos, x_perm, y_perm, imp,
                           IMPORTANCE_LOSS_WEIGHT, grads, ws_b, hidden=hidden, preact=preact,
                           logits=logits, noisy=nz)
            if ev is not None:
                bwd_evs[-1][1].record()

    # the stage sequence is the moe_forward sequence: check once, bitwise
    # (the noisy gate routes differently from moe_forward: not compared)
    same = None
    if not args.noisy:
        fw = Forward(dl)
        fw()
        step()
        torch.cuda.synchronize()
        same = torch.equal(fw.y.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           y.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        del fw

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    loop0 = torch.cuda.Event(enable_timing=True)
    loop1 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]   # step ends
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop0.record()
    for i in range(args.steps):
        step(evs[i])
        marks[i].record()
    loop1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = loop0.elapsed_time(loop1) / args.steps
    step_ms = [(loop0 if i == 0 else marks[i - 1]).elapsed_time(marks[i])
               for i in range(args.steps)]
    up_ms = [a.elapsed_time(b) for a, b in evs]
    up_avg = float(np.mean(up_ms))

    cnt = counts.cpu().numpy()
    kept_cnt = np.diff(offsets.cpu().numpy())
    kept = int(kept_cnt.sum())
    touched = int((kept_cnt > 0).sum())
    n_up = cfg.n_up
    rows = kept + cfg.S * T
    up_flops = 2.0 * rows * d * n_up
    layer_flops = float(cfg.expert_flops()) * rows / (T * k + cfg.S * T)
    es = 2 if cfg.dtype == synthetic.BF16 else 4
    up_w_bytes = (touched + cfg.S) * n_up * d * es
    down_w_bytes = (touched + cfg.S) * d * h * es
    up_bytes = up_w_bytes + rows * (d + h) * es   # weights + A read + H write
    decode = (T * k) / E < 32

    tokens_per_s = T / (ms_step / 1e3)
    if decode:
        roof = {"bound": "hbm", "achieved": up_bytes / (up_avg / 1e3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": up_flops / (up_avg / 1e3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "expert up projection + activation (moe_expert_up: gemm_dma_kernel / gemm_pp_kernel / gemm_bf16_kernel by group size and K)"
    roof["avg_ms"] = up_avg
    roof["algorithmic_bytes"] = up_bytes   # per step: W_up of touched experts + A read + H write
    # HBM bytes per launch of the dominant kernel from the FETCH_SIZE and
    # WRITE_SIZE counters, scaled by the counters of a plain 1 GiB copy;
    # null when not measured for these kernel sources
    roof["traffic"] = None
    # measured for the default step of each workload (no capacity, default
    # gate, clean gate, inference up projection)
    default_step = not (cap or cfg.gate or args.noisy or args.backward)
    if default_step and args.traffic and os.path.exists(args.traffic):
        rec = json.load(open(args.traffic)).get(args.workload)
        if rec and rec.get("gemm_source_sha256") == source_digest():
            roof["traffic"] = rec["traffic_bytes"]
            roof["traffic_over_algorithmic_bytes"] = rec["traffic_bytes"] / up_bytes

    cpu = None
    # the oracle's token loop has no noisy gate: no CPU baseline for --noisy
    if not args.no_cpu_baseline and not args.noisy:
        import oracle
        nthr = oracle.max_threads()
        probe = list(range(min(T, max(2, nthr))))
        t1 = time.perf_counter()
        oracle.forward_tokens(L, probe)
        per_tok = (time.perf_counter() - t1) / len(probe)
        n = int(min(T, max(len(probe), args.cpu_seconds / max(per_tok, 1e-9))))
        sample = np.linspace(0, T - 1, n).astype(np.int64)
        keep = assign = None
        if cap:   # the capacity decision is over the whole batch (not timed)
            ridx, _, rsc = oracle.route(L, want_scores=overflow != 0)
            if overflow:
                assign = oracle.capacity_reroute(cfg, ridx, rsc, cap)
            else:
                keep = oracle.capacity_keep(cfg, ridx, cap)
        t1 = time.perf_counter()
        oracle.forward_tokens(L, sample, keep=keep, assign=assign)
        el = time.perf_counter() - t1
        model = "unknown CPU"
        try:
            with open("/proc/cpuinfo") as fh:
                model = next((l.split(":", 1)[1].strip() for l in fh
                              if l.startswith("model name")), model)
        except OSError:
            pass
        cpu = {"value": n / el, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
               "sample": f"{n} of {T} tokens (evenly spaced), full routing + "
                         f"expert FFNs + combine per token, {el:.1f} s on {nthr} "
                         f"OpenMP threads of {model} ({os.cpu_count()} logical CPUs)"}

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms": {"median": float(np.median(step_ms)), "min": float(np.min(step_ms)),
                    "p90": float(np.percentile(step_ms, 90))},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == synthetic.BF16 else "f32",
        "data": "synthetic (seeded numpy PCG64, seed 0; random-init weights)",
        "config": {"workload": cfg.name, "T": T, "d_model": d, "d_hidden": h,
                   "experts": E, "top_k": k, "shared": cfg.S,
                   "act": "swiglu" if cfg.act == synthetic.SWIGLU else "gelu",
                   "router_bias": cfg.router_bias,
                   **({"gate": args.gate} if cfg.gate else {}),
                   **({"noisy_gate": True} if args.noisy else {}),
                   **({"capacity_factor": args.capacity_factor, "capacity": cap,
                       "overflow": args.overflow} if cap else {}),
                   "weight_copies": ncopy, "weight_layout": layout},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer_tflops": layer_flops / (ms_step / 1e3) / 1e12,
        "layer_frac_mfma_peak": layer_flops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "expert_weight_gbs": (up_w_bytes + down_w_bytes) / (ms_step / 1e3) / 1e9,
        "experts_touched": touched,
        "dropped_fraction": 1.0 - kept / (T * k) if T else 0.0,
        "wall_s_timed": wall,
        "input_gen_upload_s": gen_s,
        "stage_sequence_equals_moe_forward": same,
    }
    if roof["traffic"] is not None:
        roof["traffic_source"] = ("rocprofv3 FETCH_SIZE and WRITE_SIZE of this kernel at this "
                                  "workload, committed in " + os.path.relpath(args.traffic, ROOT) +
                                  " for the same kernel sources (not measured in this run)")
    if args.backward:
        bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in bwd_evs]))
        # algorithmic backward work: dX and dW of both projections, twice
        # the forward's expert FLOPs (the pre-activation recomputation and
        # the transposes are overhead, not counted)
        bflops = 2.0 * layer_flops
        out["config"]["training_step"] = True
        out["backward"] = {"ms": bwd_ms, "tflops": bflops / (bwd_ms / 1e3) / 1e12,
                           "frac_mfma_peak": bflops / (bwd_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                           "importance_loss_weight": IMPORTANCE_LOSS_WEIGHT,
                           **({"load_loss_weight": LOAD_LOSS_WEIGHT} if args.noisy else {})}
    del copies, copy_w, dl, L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


DEFAULT_WORKLOAD = "mixtral-8x7b"
DECODE_WORKLOAD = "gpt-oss-20b-decode"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(expert parallelism is a design note, not code)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out = run_one(args)
    # The default line also times the decode-shape layer (the metric's
    # "decode HBM GB/s"), in the same process, after the headline workload.
    plain = not (args.capacity_factor or args.noisy or args.backward or args.gate != "topk-softmax")
    if args.workload == DEFAULT_WORKLOAD and plain and not args.no_decode:
        dargs = argparse.Namespace(**vars(args))
        dargs.workload = DECODE_WORKLOAD
        dargs.no_cpu_baseline = True
        dargs.steps = max(args.steps, 50)
        dargs.warmup = max(args.warmup, 20)
        dec = run_one(dargs)
        out["decode"] = {
            "workload": DECODE_WORKLOAD, "config": dec["config"],
            "steps": dargs.steps, "warmup": dargs.warmup,
            "decode_ms_per_step": dec["ms_per_step"], "step_ms": dec["step_ms"],
            "tokens_per_s": dec["value"],
            "expert_weight_gbs": dec["expert_weight_gbs"],
            "frac_hbm_peak": dec["expert_weight_gbs"] / PEAK_HBM_GBS,
            "experts_touched": dec["experts_touched"],
            "roofline": dec["roofline"],
            "stage_sequence_equals_moe_forward": dec["stage_sequence_equals_moe_forward"],
        }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
