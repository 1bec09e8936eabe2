"""Throughput of the MoE expert layer (forward + backward) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fwdbwd_1t]

A step is one pass of the whole hot path over one batch: router logits,
top-k routing, counting + permutation, the gate/up and down grouped GEMMs,
the weighted combine, and the backward of each (combine, dH, dX, dW, route,
router, unpermute).  Inputs are seeded synthetic tensors already resident in
HBM when the timed region starts.  Every entry point is bracketed by HIP
events on the stream it is launched on; the dominant kernel's average
duration gives the roofline fraction.  Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwdbwd_1t_hbm_traffic.txt")


def _kernel_source_sha():
    """Digest of the HIP sources the GEMM and data-movement kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _measured_traffic(row):
    """HBM bytes per launch of `row` from the committed counter summary, or None.

    The summary holds FETCH_SIZE + WRITE_SIZE per launch (scaled by a copy
    kernel's reading, see the file) and the digest of the sources it was
    measured on; a different digest means the kernel changed since, and the
    figure no longer applies.
    """
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    sha = _kernel_source_sha()
    for ln in lines:
        f = ln.split()
        if len(f) >= 5 and f[0] == "traffic" and f[1] == row and f[2] == f"sha={sha}":
            kv = dict(x.split("=", 1) for x in f[3:])
            return int(float(kv["fetch"]) + float(kv["write"]))
    return None


def _copy_calibration(nbytes):
    """A plain device copy of nbytes, for scaling the HBM byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)


def _cpu_baseline(cfg, inp, sample_tokens, n_groups=1):
    """The oracle, as it stands, on the first `sample_tokens` tokens of the workload."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    Ts = sample_tokens
    dt = cfg.dtype
    x = synth.as_f32(inp["x"][:Ts], dt).astype(np.float64)
    dy = synth.as_f32(inp["dy"][:Ts], dt).astype(np.float64)
    wr = synth.as_f32(inp["wr"], dt)
    w1 = synth.as_f32(inp["w1"], dt)
    w3 = synth.as_f32(inp["w3"], dt)
    w2 = synth.as_f32(inp["w2"], dt)
    t0 = time.perf_counter()
    fwd = oracle.layer_forward(x, wr, w1, w3, w2, cfg.k, cfg.expert_begin, cfg.num_local, cfg.renormalize,
                               n_groups=n_groups)
    if cfg.backward:
        oracle.layer_backward(fwd, x, wr, w1, w3, w2, dy, cfg.renormalize)
    dt_s = time.perf_counter() - t0
    return {"value": Ts / dt_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {Ts} of {cfg.T} tokens of {cfg.name}, all {cfg.num_local} local experts' "
                      f"weights, {'forward+backward' if cfg.backward else 'forward'}, float64 numpy; "
                      f"{dt_s:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwdbwd_1t")
    ap.add_argument("--n-groups", type=int, default=1,
                    help="group-limited routing: take k/n_groups experts from each of n_groups expert groups")
    ap.add_argument("--schedule", choices=["static", "dynamic"], default="static",
                    help="tile order of the grouped GEMMs")
    ap.add_argument("--hold-cus", type=int, default=0,
                    help="before each grouped GEMM, occupy this many CUs with another kernel (contention)")
    ap.add_argument("--hold-us", type=int, default=2000, help="how long each --hold-cus kernel runs")
    ap.add_argument("--gather", action="store_true",
                    help="gather fused into gate/up and dW1|dW3: no x_perm (A4 is index generation only)")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="expert weights held as blockwise-128 E4M3 codes + scales, dequantised to bf16 each step")
    ap.add_argument("--fp8-gemm", action="store_true",
                    help="with --fp8-weights: the forward expert GEMMs read the FP8 weights directly")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        _copy_calibration(args.copy_calibration)
        return

    import torch

    import mixture_experts_layer_02_amd as moe
    import synth

    cfg = synth.CONFIGS[args.workload]

    def note(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    t_gen = time.perf_counter()
    inp = synth.make_inputs(cfg)
    gen_s = time.perf_counter() - t_gen
    note(f"inputs of {cfg.name} drawn in {gen_s:.1f} s")
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    g = {n: up(inp[n]) for n in ("x", "wr", "w1", "w3", "w2", "dy")}
    bias = up(inp["bias"]) if "bias" in inp else None
    routing = (up(inp["idx"]), up(inp["w"])) if cfg.routing == "roundrobin" else None
    counters = moe.new_tile_counters(dev) if args.schedule == "dynamic" else None
    D = moe.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype,
                      cfg.renormalize, tile_counters=counters)
    b = moe.Buffers(D, backward=cfg.backward, gather=args.gather)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=dev)
    gemm_rows = {"A5_gate_up", "A6_down", "B2_dh", "B3_dx", "B4_dw"}

    fp8 = {}
    if args.fp8_weights:
        for n in ("w1", "w3", "w2"):
            q = torch.empty(g[n].numel(), dtype=torch.uint8, device=dev)
            sc = torch.empty(g[n].numel() // 128, dtype=torch.float32, device=dev)
            moe.fp8_quantize(g[n], q, sc)
            fp8[n] = (q, sc)
        torch.cuda.synchronize()
        qs, qe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        qs.record()
        for n in ("w1", "w3", "w2"):
            moe.fp8_quantize(g[n], fp8[n][0], fp8[n][1])
        qe.record()
        torch.cuda.synchronize()
        fp8_quant_ms = qs.elapsed_time(qe)
    rows = ["A1_router_logits", "A2_route", "A34_permute", "A5_gate_up", "A6_down", "A7_combine"]
    if args.fp8_gemm and not args.fp8_weights:
        raise SystemExit("--fp8-gemm needs --fp8-weights")
    if args.fp8_weights and not (args.fp8_gemm and not cfg.backward):
        rows = ["A0_fp8_dequant"] + rows      # bf16 weights for the GEMMs (or for the backward)
    if cfg.backward:
        rows += ["B1_combine_bwd", "B2_dh", "B3_dx", "B4_dw", "B5_route_bwd", "B5_unpermute", "B5_router_bwd"]
    ev = {r: [] for r in rows}

    def timed(name, fn, rec):
        if args.hold_cus and name in gemm_rows:
            # Another kernel takes hold_cus CUs as the product starts (the main
            # stream waits 20 us so that the holder's workgroups are resident).
            side.wait_stream(stream)
            moe.hold_cus(args.hold_cus, args.hold_us, stream=side)
            moe.hold_cus(1, 20, lds_bytes=64, stream=stream)
        if rec:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            ev[name].append((s, e))
        else:
            fn()

    def dequant_all():
        for n in ("w1", "w3", "w2"):
            moe.fp8_dequantize(fp8[n][0], fp8[n][1], g[n])

    def step(rec):
        if args.fp8_weights and "A0_fp8_dequant" in rows:
            timed("A0_fp8_dequant", dequant_all, rec)
        if routing is None:
            timed("A1_router_logits", lambda: moe.router_logits(D, g["x"], g["wr"], bias, b.logits, b.ws_router), rec)
            if args.n_groups > 1:
                timed("A2_route", lambda: moe.route_grouped(D, b.logits, args.n_groups, b.topk_idx, b.topk_w), rec)
            else:
                timed("A2_route", lambda: moe.route(D, b.logits, b.topk_idx, b.topk_w), rec)
            idx, w = b.topk_idx, b.topk_w
        else:
            idx, w = routing
        if args.fp8_gemm:
            if args.gather:
                timed("A34_permute", lambda: moe.permute(D, idx, None, b.counts, b.offsets, b.row_token,
                                                         b.slot_row, None, b.ws_permute), rec)
            else:
                timed("A34_permute", lambda: moe.permute(D, idx, g["x"], b.counts, b.offsets, b.row_token,
                                                         b.slot_row, b.x_perm, b.ws_permute), rec)
            timed("A5_gate_up", lambda: moe.expert_gate_up_fp8(
                D, b.offsets, b.row_token if args.gather else None, g["x"] if args.gather else b.x_perm,
                fp8["w1"][0], fp8["w1"][1], fp8["w3"][0], fp8["w3"][1], b.gu, b.h), rec)
        elif args.gather:
            timed("A34_permute", lambda: moe.permute(D, idx, None, b.counts, b.offsets, b.row_token, b.slot_row,
                                                     None, b.ws_permute), rec)
            timed("A5_gate_up", lambda: moe.expert_gate_up_gather(D, b.offsets, b.row_token, g["x"], g["w1"],
                                                                  g["w3"], b.gu, b.h), rec)
        else:
            timed("A34_permute", lambda: moe.permute(D, idx, g["x"], b.counts, b.offsets, b.row_token,
                                                     b.slot_row, b.x_perm, b.ws_permute), rec)
            timed("A5_gate_up", lambda: moe.expert_gate_up(D, b.offsets, b.x_perm, g["w1"], g["w3"], b.gu, b.h),
                  rec)
        if args.fp8_gemm:
            timed("A6_down", lambda: moe.expert_down_fp8(D, b.offsets, b.h, fp8["w2"][0], fp8["w2"][1], b.y_perm),
                  rec)
        else:
            timed("A6_down", lambda: moe.expert_down(D, b.offsets, b.h, g["w2"], b.y_perm), rec)
        timed("A7_combine", lambda: moe.combine(D, b.slot_row, w, b.y_perm, b.y), rec)
        if not cfg.backward:
            return
        timed("B1_combine_bwd", lambda: moe.combine_bwd(D, b.slot_row, w, b.y_perm, g["dy"], b.dy_perm,
                                                        b.dtopk_w), rec)
        timed("B2_dh", lambda: moe.expert_bwd_dh(D, b.offsets, g["w2"], b.gu, b.dy_perm, b.dgu), rec)
        timed("B3_dx", lambda: moe.expert_bwd_dx(D, b.offsets, g["w1"], g["w3"], b.dgu, b.dx_perm), rec)
        if args.gather:
            timed("B4_dw", lambda: moe.grouped_ffn_bwd_dw_gather(D, b.offsets, b.row_token, g["x"], b.h, b.dgu,
                                                                 b.dy_perm, b.dW1, b.dW3, b.dW2), rec)
        else:
            timed("B4_dw", lambda: moe.grouped_ffn_bwd_dw(D, b.offsets, b.x_perm, b.h, b.dgu, b.dy_perm, b.dW1,
                                                          b.dW3, b.dW2), rec)
        timed("B5_route_bwd", lambda: moe.route_bwd(D, b.logits, idx, w, b.dtopk_w, b.dlogits), rec)
        timed("B5_unpermute", lambda: moe.unpermute_bwd(D, b.slot_row, b.dx_perm, None, b.dx), rec)
        timed("B5_router_bwd", lambda: moe.router_bwd_acc(D, g["x"], g["wr"], b.dlogits, b.dx, b.dWr,
                                                          b.ws_router_bwd), rec)

    note("inputs resident in HBM; warming up")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    note(f"{args.warmup} warmup steps done; timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    peak_mem = torch.cuda.max_memory_allocated()
    R = int(b.offsets[-1].item())
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    bb = 2 if cfg.dtype == "bf16" else 4
    avg_ms = {r: float(np.mean([s.elapsed_time(e) for s, e in ev[r]])) for r in rows if ev[r]}
    flops = {"A1_router_logits": 2.0 * T * d * E, "A5_gate_up": 4.0 * R * d * f, "A6_down": 2.0 * R * d * f,
             "B2_dh": 2.0 * R * d * f, "B3_dx": 4.0 * R * d * f, "B4_dw": 6.0 * R * d * f,
             "B5_router_bwd": 4.0 * T * d * E}
    ntok_local = int((b.slot_row >= 0).any(dim=1).sum().item())
    nw = 3 * cfg.num_local * d * f
    hbm_bytes = {"A0_fp8_dequant": nw * (1 + 2) + nw // 128 * 4,
                 "A2_route": T * E * 4 + T * cfg.k * 8,
                 "A34_permute": (0 if args.gather else ntok_local * d * bb + R * d * bb) + T * cfg.k * 12 + R * 4,
                 "A7_combine": R * d * bb + T * d * bb + T * cfg.k * 8,
                 "B1_combine_bwd": T * d * bb + 2 * R * d * bb + T * cfg.k * 12,
                 "B5_route_bwd": T * E * 4 + T * cfg.k * 12,
                 "B5_unpermute": R * d * bb + T * d * bb + T * cfg.k * 4}
    # GEMM rows: each operand read once and each output written once (weights in the stored type)
    wb = 1 if args.fp8_gemm else bb
    NL = cfg.num_local
    gemm_bytes = {"A1_router_logits": T * d * bb + E * d * bb + T * E * 4,
                  "A5_gate_up": R * d * bb + 2 * NL * f * d * wb + R * f * bb + (R * 2 * f * bb if cfg.backward else 0),
                  "A6_down": R * f * bb + NL * f * d * wb + R * d * bb,
                  "B2_dh": R * d * bb + NL * f * d * bb + 2 * R * 2 * f * bb,
                  "B3_dx": R * 2 * f * bb + 2 * NL * f * d * bb + R * d * bb,
                  "B4_dw": 2 * R * d * bb + R * 3 * f * bb + 3 * NL * f * d * 4}
    per_row = {}
    for r, ms in avg_ms.items():
        ent = {"ms": round(ms, 4)}
        if r in flops:
            ent["TFLOP/s"] = round(flops[r] / ms / 1e9, 1)
            ent["frac_mfma"] = round(flops[r] / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
        if r in hbm_bytes or r in gemm_bytes:
            nbytes = hbm_bytes.get(r, gemm_bytes.get(r))
            ent["GB/s"] = round(nbytes / ms / 1e6, 1)
            ent["frac_hbm"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)
        per_row[r] = ent
    gemm_rows = [r for r in ("A5_gate_up", "A6_down", "B2_dh", "B3_dx", "B4_dw") if r in avg_ms]
    gemm_tflops = sum(flops[r] for r in gemm_rows) / sum(avg_ms[r] for r in gemm_rows) / 1e9
    # dominant single-kernel row: the largest time among rows that launch one kernel
    single = [r for r in ("A1_router_logits", "A2_route", "A5_gate_up", "A6_down", "A7_combine", "B1_combine_bwd",
                          "B2_dh", "B3_dx", "B5_route_bwd", "B5_unpermute") if r in avg_ms]
    dom = max(single, key=lambda r: avg_ms[r])
    # the committed traffic figures were measured on the default fwdbwd_1t step only
    default_run = (cfg.name == "fwdbwd_1t" and not (args.gather or args.fp8_weights or args.fp8_gemm or
                   args.hold_cus or args.n_groups > 1 or args.schedule != "static"))
    traffic = _measured_traffic(dom) if default_run else None
    # a GEMM whose arithmetic intensity is under the ridge (peak flops / peak bytes) is bound by HBM
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if dom in flops and flops[dom] / gemm_bytes[dom] >= ridge:
        ach = flops[dom] / avg_ms[dom] / 1e9
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    else:
        nbytes = gemm_bytes[dom] if dom in gemm_bytes else hbm_bytes[dom]
        ach = nbytes / avg_ms[dom] / 1e6
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}

    note(f"timed region: {ms_step:.3f} ms/step")
    cpu = None
    if not args.no_cpu_baseline:
        note(f"cpu baseline: oracle on {min(args.cpu_sample_tokens, cfg.T)} tokens")
        del g, b
        torch.cuda.empty_cache()
        cpu = _cpu_baseline(cfg, inp, min(args.cpu_sample_tokens, cfg.T), args.n_groups)

    out = {
        "metric": METRIC, "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} d={d} E={E} ({cfg.num_local} local from {cfg.expert_begin}) "
                               f"top-{cfg.k} f={f} {'fwd+bwd' if cfg.backward else 'fwd'}",
                   "routed_rows": R, "global_batch": T, "parallelism": "single GPU",
                   "routing": f"group-limited, {args.n_groups} groups" if args.n_groups > 1 else "top-k",
                   "tile_schedule": args.schedule,
                   "gather_fused": bool(args.gather),
                   "expert_weights": ("bf16" if not args.fp8_weights else
                                      "fp8 e4m3 blocks of 128, read by the forward GEMMs" if args.fp8_gemm else
                                      "fp8 e4m3 blocks of 128, dequantised each step"),
                   "contention": (f"{args.hold_cus} CUs held for {args.hold_us} us at each grouped GEMM"
                                  if args.hold_cus else None)},
        "device_mem_peak_gb": round(peak_mem / 1e9, 2),
        "fp8_quantize": ({"ms": round(fp8_quant_ms, 4),
                          "GB/s": round((nw * (2 + 1) + nw // 128 * 4) / fp8_quant_ms / 1e6, 1)}
                         if args.fp8_weights else None),
        "grouped_gemm_tflops": round(gemm_tflops, 1),
        "grouped_gemm_frac_mfma": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "rows": per_row,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
