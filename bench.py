"""Throughput of the MoE expert layer (forward + backward) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fwdbwd_1t]

A step is one pass of the whole hot path over one batch: router logits,
top-k routing, counting + index generation + the permuted copy of x, the
gate/up and down grouped GEMMs, the weighted combine, and the backward of
each (combine, dH, dX, dW1|dW3, dW2, route, unpermute, router), with dH and
dW2 reading dy in place through row_token (no permuted copy of dy).  Inputs are seeded synthetic tensors already
resident in HBM.  Before each timed step a 1 GiB buffer is rewritten by a
fill kernel, outside the timed events, so that every step starts with the
L2 and infinity caches holding none of its data.  Every entry point is
bracketed by HIP events on the stream it is launched on; the step time is
the span from the first to the last event of the step.

The longest single kernel launch of the step is graded against its roofline:
its algorithmic flops (or bytes) per launch over its average event duration.

After the main workload, the forward-only 1T-shape workloads (the one-GPU
expert-parallel share, and the Zipf-skewed and forced-uniform routings of the
96 local experts) are timed the same way and reported in a nested object.
Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
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
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop/B where the two roofs meet
FLUSH_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwdbwd_1t_hbm_traffic.txt")
GEMM_ROWS = ("A5_gate_up", "A6_down", "B2_dh", "B3_dx", "B4_dw13", "B4_dw2")
EXTRA_WORKLOADS = ("fwdbwd_1t_wgrad_f32", "share_1t", "share_1t_fp8mm", "zipf_1t", "uniform_1t")


@dataclasses.dataclass
class Row:
    """One timed entry point of the step: its launches, algorithmic flops and bytes."""
    name: str
    fn: object
    launches: int
    flops: float = 0.0
    nbytes: float = 0.0
    peak_tflops: float = PEAK_BF16_TFLOPS   # the matrix-core peak of the row's operand type


def pick_dominant(avg_ms, launches):
    """The row holding the longest single kernel launch.

    Rows that make one launch are compared by their average duration.  A row
    of several launches is timed as a whole, so its longest launch is not
    known; it can only be ruled out, by its whole time being shorter than the
    chosen single launch.  If it is not, the choice is ambiguous and this
    raises, rather than grade the wrong kernel."""
    single = [r for r in avg_ms if launches[r] == 1]
    if not single:
        raise ValueError("no single-launch row to grade")
    dom = max(single, key=lambda r: avg_ms[r])
    for r in avg_ms:
        if launches[r] > 1 and avg_ms[r] >= avg_ms[dom]:
            raise ValueError(f"row {r} ({launches[r]} launches, {avg_ms[r]:.3f} ms) may hold a launch longer "
                             f"than {dom} ({avg_ms[dom]:.3f} ms); time its launches separately")
    return dom


def grade(row, ms):
    """Roofline of one launch: MFMA when its arithmetic intensity (algorithmic
    flops per algorithmic byte) is at or above the ridge of its operand
    type's matrix-core peak and the HBM peak, else HBM."""
    if row.flops and row.flops / row.nbytes >= row.peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9):
        ach = row.flops / ms / 1e9
        return {"kernel": row.name, "bound": "mfma", "achieved": round(ach, 1), "peak": row.peak_tflops,
                "unit": "TFLOP/s", "frac": round(ach / row.peak_tflops, 4)}
    ach = row.nbytes / ms / 1e6
    return {"kernel": row.name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}


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


def _vendor_gemm(torch, dev, NL, R, d, f, ours):
    """The vendor's bf16 GEMM (torch.bmm, hipBLASLt) on the products of the grouped GEMM rows, with
    equal segments of R / NL rows per expert, for comparison with the grouped kernels' own times.
    Every operand is a contiguous tensor; outputs are bf16 (the weight gradients here as --wgrad-dtype)."""
    m = max(1, round(R / NL))
    g = torch.Generator(device=dev).manual_seed(5)

    def rnd(*shape):
        return torch.randn(*shape, device=dev, dtype=torch.bfloat16, generator=g)

    shapes = {"A5_gate_up": (m, d, 2 * f), "A6_down": (m, f, d), "B2_dh": (m, d, f), "B3_dx": (m, 2 * f, d),
              "B4_dw13": (2 * f, m, d), "B4_dw2": (d, m, f)}
    out = {}
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for row, (a0, k0, n0) in shapes.items():
        a, b = rnd(NL, a0, k0), rnd(NL, k0, n0)
        for _ in range(3):
            torch.bmm(a, b)
        torch.cuda.synchronize()
        st.record()
        for _ in range(5):
            torch.bmm(a, b)
        en.record()
        torch.cuda.synchronize()
        ms = st.elapsed_time(en) / 5
        fl = 2.0 * NL * a0 * k0 * n0
        out[row] = {"bmm": f"{NL} x [{a0} x {k0}] . [{k0} x {n0}]", "vendor_ms": round(ms, 4),
                    "vendor_tflops": round(fl / ms / 1e9, 1),
                    "ours_ms": round(ours[row]["ms"], 4) if row in ours else None}
        del a, b
    torch.cuda.empty_cache()
    return {"what": f"torch.bmm bf16 (hipBLASLt) on the same products, {NL} equal segments of {m} rows",
            "rows": out}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(cfg, inp, sample_tokens, n_groups, extra_inputs):
    """The oracle, as it stands, on the first `sample_tokens` tokens of the
    workload (every host core this process may use), plus single-thread
    forward times on small samples of the tiny, small and 1T-share configs."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))

    def f64(a, dt):
        return synth.as_f32(a, dt).astype(np.float64)

    def forward_backward(c, data, Ts, threads, groups=1):
        dt = c.dtype
        x = f64(data["x"][:Ts], dt)
        w = {n: synth.as_f32(data[n], dt) for n in ("wr", "w1", "w3", "w2")}
        with threadpool_limits(threads):
            t0 = time.perf_counter()
            fwd = oracle.layer_forward(x, w["wr"], w["w1"], w["w3"], w["w2"], c.k, c.expert_begin, c.num_local,
                                       c.renormalize, bias=data.get("bias"), n_groups=groups)
            if c.backward:
                oracle.layer_backward(fwd, x, w["wr"], w["w1"], w["w3"], w["w2"], f64(data["dy"][:Ts], dt),
                                      c.renormalize)
            return time.perf_counter() - t0

    Ts = sample_tokens
    wall = forward_backward(cfg, inp, Ts, cores, n_groups)
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    single = {}
    for name, n in (("tiny_f32", 256), ("small_bf16", 256), ("share_1t", 64)):
        c = dataclasses.replace(synth.CONFIGS[name], backward=False)
        data = extra_inputs.get(name) or synth.make_inputs(c, want=("x", "wr", "w1", "w3", "w2"))
        s = forward_backward(c, data, n, 1)
        single[name] = {"tokens": n, "forward_s": round(s, 3), "tokens/s": round(n / s, 1)}
    return {"value": Ts / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {Ts} of {cfg.T} tokens of {cfg.name}, all {cfg.num_local} local experts' "
                      f"weights, {'forward+backward' if cfg.backward else 'forward'}, float64 numpy with the "
                      f"BLAS pool limited to the {cores} cores of the process's affinity mask; {wall:.1f} s wall",
            "cpu_model": _cpu_model(), "blas_threads_max": int(blas),
            "single_thread_forward": single}


class Workload:
    """Device tensors and the ordered rows of one workload's step."""

    def __init__(self, moe, torch, cfg, inp, args, dev, fp8mm=False, wgrad=None):
        """fp8mm: gate/up and down on the FP8 matrix cores (forward only): W1,
        W3 and W2 held as E4M3 codes with power-of-two block scales, x and h
        quantised each step.  wgrad: the expert weight gradients' type, "bf16"
        or "f32" (default --wgrad-dtype; fp32 layers always write fp32)."""
        self.cfg = cfg
        T, d, f, E, k, NL = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.num_local

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        names = ("x", "wr", "w1", "w3", "w2") + (("dy",) if cfg.backward else ())
        g = self.g = {n: up(inp[n]) for n in names}
        bias = up(inp["bias"]) if "bias" in inp else None
        routing = (up(inp["idx"]), up(inp["w"])) if cfg.routing == "roundrobin" else None
        counters = moe.new_tile_counters(dev) if args.schedule == "dynamic" else None
        wgrad = (wgrad or args.wgrad_dtype) if cfg.dtype == "bf16" else "f32"
        self.wgrad = wgrad
        wb = 2 if wgrad == "bf16" else 4   # bytes per weight-gradient element written
        D = self.D = moe.make_desc(T, d, f, E, k, cfg.expert_begin, NL, cfg.dtype, cfg.renormalize,
                                   tile_counters=counters, wgrad_dtype=wgrad)
        gather = args.x_path == "gather" or fp8mm
        gdy = args.dy_path == "gather" and cfg.dtype == "bf16"
        fuse_rdx = args.router_dx == "fused" and bool(cfg.renormalize)
        b = self.b = moe.Buffers(D, backward=cfg.backward, gather=gather, gather_dy=gdy)
        bb = 2 if cfg.dtype == "bf16" else 4
        fp8 = self.fp8 = {}
        if args.fp8_weights:
            for n in ("w1", "w3", "w2"):
                q = torch.empty(g[n].numel(), dtype=torch.uint8, device=dev)
                sc = torch.empty(g[n].numel() // 128, dtype=torch.float32, device=dev)
                moe.fp8_quantize(g[n], q, sc)
                fp8[n] = (q, sc)
        self.routing = routing
        self.gather = gather
        R_est = T * min(k, NL)       # replaced by the measured R after the run
        self.R = R_est
        wb = 1 if args.fp8_gemm else bb
        idx, w = (b.topk_idx, b.topk_w) if routing is None else routing
        rows = []

        def add(name, fn, launches, flops=lambda R: 0.0, nbytes=lambda R: 0.0, peak=PEAK_BF16_TFLOPS):
            rows.append((name, fn, launches, flops, nbytes, peak))

        nw = 3 * NL * d * f
        if args.fp8_weights and not (args.fp8_gemm and not cfg.backward):
            def dequant():
                for n in ("w1", "w3", "w2"):
                    moe.fp8_dequantize(fp8[n][0], fp8[n][1], g[n])
            add("A0_fp8_dequant", dequant, 3, nbytes=lambda R: nw * 3 + nw // 128 * 4)
        if routing is None:
            add("A1_router_logits", lambda: moe.router_logits(D, g["x"], g["wr"], bias, b.logits, b.ws_router),
                1 + (moe.workspace_size(D, moe.OP_ROUTER_LOGITS) > 0),
                lambda R: 2.0 * T * d * E, lambda R: T * d * bb + E * d * bb + T * E * 4)
            if args.n_groups > 1:
                add("A2_route", lambda: moe.route_grouped(D, b.logits, args.n_groups, b.topk_idx, b.topk_w), 1,
                    nbytes=lambda R: T * E * 4 + T * k * 8)
            else:
                add("A2_route", lambda: moe.route(D, b.logits, b.topk_idx, b.topk_w), 1,
                    nbytes=lambda R: T * E * 4 + T * k * 8)
        # counting (2 kernels), the expert offsets, placement, and the gather when x_perm is built
        self.ntok_local = None
        add("A34_permute", lambda: moe.permute(D, idx, None if gather else g["x"], b.counts, b.offsets,
                                               b.row_token, b.slot_row, None if gather else b.x_perm,
                                               b.ws_permute),
            4 if gather else 5,
            nbytes=lambda R: (0 if gather else self.ntok_local * d * bb + R * d * bb) + T * k * 12 + R * 4)
        gu_bytes = (lambda R: R * 2 * f * bb) if cfg.backward else (lambda R: 0)
        if fp8mm:
            assert not cfg.backward and cfg.dtype == "bf16"
            q8 = {}
            for n in ("w1", "w3"):
                qq = torch.empty(g[n].numel(), dtype=torch.uint8, device=dev)
                ee = torch.empty(g[n].numel() // 128, dtype=torch.uint8, device=dev)
                moe.fp8_quantize_pow2(g[n], qq, ee)
                q8[n] = (qq, ee)
            xq = torch.empty(T * d, dtype=torch.uint8, device=dev)
            xe = torch.empty(T * d // 128, dtype=torch.uint8, device=dev)
            add("A4_quant_x", lambda: moe.fp8_quantize_pow2(g["x"], xq, xe), 1,
                nbytes=lambda R: T * d * (bb + 1) + T * d // 128)
            add("A5_gate_up", lambda: moe.expert_gate_up_fp8mm(D, b.offsets, b.row_token, xq, xe, q8["w1"][0],
                                                               q8["w1"][1], q8["w3"][0], q8["w3"][1], None, b.h), 1,
                lambda R: 4.0 * R * d * f,
                lambda R: R * d + R * d // 128 + 2 * NL * f * d + 2 * NL * f * d // 128 + R * f * bb,
                peak=PEAK_FP8_TFLOPS)
            # down on the FP8 matrix cores too: W2 quantised once by rows of f, h each step
            S8 = moe.fp8_scale_row_bytes(f)
            w2q = torch.empty(NL * d, f, dtype=torch.uint8, device=dev)
            w2e = torch.empty(NL * d, S8, dtype=torch.uint8, device=dev)
            moe.fp8_quantize_pow2_rows(g["w2"].view(NL * d, f), w2q, w2e)
            Rc = D.R_cap
            hq = torch.empty(Rc, f, dtype=torch.uint8, device=dev)
            he = torch.empty(Rc, S8, dtype=torch.uint8, device=dev)
            add("A6_quant_h", lambda: moe.fp8_quantize_pow2_rows(b.h, hq, he, b.offsets[NL:]), 1,
                nbytes=lambda R: R * f * (bb + 1) + R * S8)
            add("A6_down", lambda: moe.expert_down_fp8mm(D, b.offsets, hq, he, w2q, w2e, b.y_perm), 1,
                lambda R: 2.0 * R * d * f, lambda R: R * f + R * S8 + NL * f * d + NL * d * S8 + R * d * bb,
                peak=PEAK_FP8_TFLOPS)
        elif args.fp8_gemm:
            add("A5_gate_up", lambda: moe.expert_gate_up_fp8(
                D, b.offsets, b.row_token if gather else None, g["x"] if gather else b.x_perm,
                fp8["w1"][0], fp8["w1"][1], fp8["w3"][0], fp8["w3"][1], b.gu, b.h), 1,
                lambda R: 4.0 * R * d * f, lambda R: R * d * bb + 2 * NL * f * d * wb + R * f * bb + gu_bytes(R))
            add("A6_down", lambda: moe.expert_down_fp8(D, b.offsets, b.h, fp8["w2"][0], fp8["w2"][1], b.y_perm), 1,
                lambda R: 2.0 * R * d * f, lambda R: R * f * bb + NL * f * d * wb + R * d * bb)
        else:
            if gather:
                fn = lambda: moe.expert_gate_up_gather(D, b.offsets, b.row_token, g["x"], g["w1"], g["w3"], b.gu, b.h)
            else:
                fn = lambda: moe.expert_gate_up(D, b.offsets, b.x_perm, g["w1"], g["w3"], b.gu, b.h)
            add("A5_gate_up", fn, 1,
                lambda R: 4.0 * R * d * f, lambda R: R * d * bb + 2 * NL * f * d * bb + R * f * bb + gu_bytes(R))
            add("A6_down", lambda: moe.expert_down(D, b.offsets, b.h, g["w2"], b.y_perm), 1,
                lambda R: 2.0 * R * d * f, lambda R: R * f * bb + NL * f * d * bb + R * d * bb)
        add("A7_combine", lambda: moe.combine(D, b.slot_row, w, b.y_perm, b.y), 1,
            nbytes=lambda R: R * d * bb + T * d * bb + T * k * 8)
        NP = moe.dtopk_parts(D)
        parts = cfg.backward and gdy and args.dtopk == "parts"
        if cfg.backward and gdy and parts:
            # dy read in place: no dy_perm; the routing weight of each row is
            # applied inside dH, which also writes hw = w silu(G) U for dW2 and
            # the rows' partial sums of <dy W2, h> = <dy, y_perm> (dtopk_w)
            add("B1_row_weights", lambda: moe.row_weights(D, b.slot_row, w, b.row_w), 1,
                nbytes=lambda R: T * k * 8 + R * 4)
            add("B2_dh", lambda: moe.expert_bwd_dh_gather(D, b.offsets, b.row_token, b.row_w, g["dy"], g["w2"],
                                                          b.gu, b.dgu, b.hw, b.dtopk_part), 1,
                lambda R: 2.0 * R * d * f,
                lambda R: R * d * bb + NL * f * d * bb + 2 * R * 2 * f * bb + R * f * bb + R * 4 + R * NP * 4)
        elif cfg.backward and gdy:
            # dy read in place, dtopk_w by dot products over dy and y_perm
            add("B1_combine_bwd", lambda: moe.combine_bwd_gather(D, b.slot_row, w, b.y_perm, g["dy"], b.row_w,
                                                                 b.dtopk_w), 1,
                nbytes=lambda R: T * d * bb + R * d * bb + T * k * 8 + R * 4)
            add("B2_dh", lambda: moe.expert_bwd_dh_gather(D, b.offsets, b.row_token, b.row_w, g["dy"], g["w2"],
                                                          b.gu, b.dgu, b.hw), 1,
                lambda R: 2.0 * R * d * f,
                lambda R: R * d * bb + NL * f * d * bb + 2 * R * 2 * f * bb + R * f * bb + R * 4)
        elif cfg.backward:
            add("B1_combine_bwd", lambda: moe.combine_bwd(D, b.slot_row, w, b.y_perm, g["dy"], b.dy_perm,
                                                          b.dtopk_w), 1,
                nbytes=lambda R: T * d * bb + 2 * R * d * bb + T * k * 12)
            add("B2_dh", lambda: moe.expert_bwd_dh(D, b.offsets, g["w2"], b.gu, b.dy_perm, b.dgu), 1,
                lambda R: 2.0 * R * d * f, lambda R: R * d * bb + NL * f * d * bb + 2 * R * 2 * f * bb)
        if cfg.backward:
            add("B3_dx", lambda: moe.expert_bwd_dx(D, b.offsets, g["w1"], g["w3"], b.dgu, b.dx_perm), 1,
                lambda R: 4.0 * R * d * f, lambda R: R * 2 * f * bb + 2 * NL * f * d * bb + R * d * bb)
            add("B4_dw13", lambda: moe.expert_bwd_dw_gate_up(D, b.offsets, b.row_token if gather else None,
                                                             g["x"] if gather else b.x_perm, b.dgu, b.dW1,
                                                             b.dW3), 1,
                lambda R: 4.0 * R * d * f, lambda R: R * d * bb + R * 2 * f * bb + 2 * NL * f * d * wb)
            if gdy:
                add("B4_dw2", lambda: moe.expert_bwd_dw_down_gather(D, b.offsets, b.row_token, g["dy"], b.hw,
                                                                    b.dW2), 1,
                    lambda R: 2.0 * R * d * f, lambda R: R * d * bb + R * f * bb + NL * f * d * wb)
            else:
                add("B4_dw2", lambda: moe.expert_bwd_dw_down(D, b.offsets, b.dy_perm, b.h, b.dW2), 1,
                    lambda R: 2.0 * R * d * f, lambda R: R * d * bb + R * f * bb + NL * f * d * wb)
            if parts:
                add("B5_dtopk_w", lambda: moe.dtopk_w_from_parts(D, b.slot_row, b.dtopk_part, b.dtopk_w), 1,
                    nbytes=lambda R: T * k * 8 + R * NP * 4)
            if routing is None:
                add("B5_route_bwd", lambda: moe.route_bwd(D, b.logits, idx, w, b.dtopk_w, b.dlogits), 1,
                    nbytes=lambda R: T * E * 4 + T * k * 12)
            if routing is None and fuse_rdx:
                # dx = the unpermute sum + the k selected rows of Wr times dlogits, in one pass
                add("B5_unpermute", lambda: moe.unpermute_router_bwd(D, b.slot_row, b.dx_perm, idx, b.dlogits,
                                                                     g["wr"], b.dx), 1,
                    nbytes=lambda R: R * d * bb + T * d * bb + T * k * 12 + E * d * bb)
                # dlogits to bf16, dWr split-K partials, their sum
                add("B5_router_bwd", lambda: moe.router_bwd_acc(D, g["x"], g["wr"], b.dlogits, None, b.dWr,
                                                                b.ws_router_bwd), 3,
                    lambda R: 2.0 * T * d * E, lambda R: T * d * bb + T * E * 4 + E * d * 4)
            else:
                add("B5_unpermute", lambda: moe.unpermute_bwd(D, b.slot_row, b.dx_perm, None, b.dx), 1,
                    nbytes=lambda R: R * d * bb + T * d * bb + T * k * 4)
            if routing is None and not fuse_rdx:
                # dlogits to bf16, dx += dlogits Wr, dWr split-K partials, their sum
                add("B5_router_bwd", lambda: moe.router_bwd_acc(D, g["x"], g["wr"], b.dlogits, b.dx, b.dWr,
                                                                b.ws_router_bwd), 4,
                    lambda R: 4.0 * T * d * E, lambda R: 2 * T * d * bb + 2 * E * d * bb + T * E * 4 + E * d * 4)
        self._rows = rows

    def steps(self):
        """(name, entry-point call) of each row, in step order."""
        return [(n, fn) for n, fn, _, _, _, _ in self._rows]

    def rows(self):
        """Every row with its algorithmic flops and bytes at the measured R."""
        R = self.R
        return [Row(n, fn, l, fl(R), nb(R), pk) for n, fn, l, fl, nb, pk in self._rows]


def run(moe, torch, wl, args, steps, warmup, flush, note):
    """Warm-up, then `steps` timed steps (each after a cache flush); per-row
    and per-step event times in ms, and the timed loop's wall time."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=stream.device)
    calls = wl.steps()
    ev = {n: [] for n, _ in calls}
    spans = []

    def step(rec):
        first = last = None
        for name, fn in calls:
            if args.hold_cus and name in GEMM_ROWS:
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
                first = first or s
                last = e
            else:
                fn()
        if rec:
            spans.append((first, last))

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    note(f"{wl.cfg.name}: {warmup} warmup steps done; timing {steps} steps")
    t0 = time.perf_counter()
    for i in range(steps):
        flush.fill_(i & 0xFF)          # outside the step's events
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = {r: float(np.mean([s.elapsed_time(e) for s, e in ev[r]])) for r in ev if ev[r]}
    step_ms = [s.elapsed_time(e) for s, e in spans]
    return avg, step_ms, wall


def summarize(wl, avg, step_ms, wall, steps, default_run):
    """Per-row figures, the grouped-GEMM aggregate and the roofline of the longest launch."""
    cfg, b = wl.cfg, wl.b
    R = int(b.offsets[-1].item())
    wl.R = R
    wl.ntok_local = int((b.slot_row >= 0).any(dim=1).sum().item())
    rows = {r.name: r for r in wl.rows()}
    launches = {n: rows[n].launches for n in avg}
    per_row = {}
    for n, ms in avg.items():
        r = rows[n]
        ent = {"ms": round(ms, 4), "launches": r.launches}
        if r.flops:
            ent["TFLOP/s"] = round(r.flops / ms / 1e9, 1)
            ent["frac_mfma"] = round(r.flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
        if r.nbytes:
            ent["GB/s"] = round(r.nbytes / ms / 1e6, 1)
            ent["frac_hbm"] = round(r.nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)
        per_row[n] = ent
    gemm = [n for n in GEMM_ROWS if n in avg]
    gemm_tflops = sum(rows[n].flops for n in gemm) / sum(avg[n] for n in gemm) / 1e9
    dom = pick_dominant(avg, launches)
    roof = grade(rows[dom], avg[dom])
    roof["traffic"] = _measured_traffic(dom) if default_run else None
    ms_step = float(np.mean(step_ms))
    return {"ms_per_step": ms_step, "R": R, "rows": per_row, "gemm_tflops": gemm_tflops, "roofline": roof,
            "step_ms_min": float(np.min(step_ms)), "step_ms_max": float(np.max(step_ms)),
            "wall_ms_per_step_incl_flush": wall * 1e3 / steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwdbwd_1t")
    ap.add_argument("--extra-workloads", default=",".join(EXTRA_WORKLOADS),
                    help="forward-only workloads timed after the main one (comma list, or 'none')")
    ap.add_argument("--extra-steps", type=int, default=10)
    ap.add_argument("--n-groups", type=int, default=1,
                    help="group-limited routing: take k/n_groups experts from each of n_groups expert groups")
    ap.add_argument("--schedule", choices=["static", "dynamic"], default="static",
                    help="tile order of the grouped GEMMs")
    ap.add_argument("--hold-cus", type=int, default=0,
                    help="before each grouped GEMM, occupy this many CUs with another kernel (contention)")
    ap.add_argument("--hold-us", type=int, default=2000, help="how long each --hold-cus kernel runs")
    ap.add_argument("--x-path", choices=["perm", "gather"], default="perm",
                    help="perm: the permute step copies x into x_perm for gate/up and dW1|dW3; gather: they read "
                         "x through row_token (no x_perm)")
    ap.add_argument("--dy-path", choices=["perm", "gather"], default="gather",
                    help="gather: dH and dW2 read dy through row_token with the routing weight applied inside "
                         "(no dy_perm); perm: the combine backward writes dy_perm")
    ap.add_argument("--dtopk", choices=["parts", "dot"], default="parts",
                    help="dtopk_w with dy read in place: parts, partial sums of <dy W2, h> from the dH product "
                         "(y_perm is not read); dot, dot products of dy and y_perm in the combine backward")
    ap.add_argument("--router-dx", choices=["fused", "gemm"], default="fused",
                    help="the router's share of dx: fused, k rows of Wr added in the unpermute pass (renormalised "
                         "weights: dlogits is zero outside the selection); gemm, dx += dlogits Wr as a product")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="expert weights held as blockwise-128 E4M3 codes + scales, dequantised to bf16 each step")
    ap.add_argument("--fp8-gemm", action="store_true",
                    help="with --fp8-weights: the forward expert GEMMs read the FP8 weights directly")
    ap.add_argument("--wgrad-dtype", choices=["bf16", "f32"], default="bf16",
                    help="type of the expert weight gradients dW1, dW3, dW2: bf16 (float32 sums rounded once at "
                         "the store; gradients computed in bf16 and reduced in fp32, as on the pages) or f32")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip timing the vendor bf16 GEMM (torch.bmm) on the grouped GEMMs' products")
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
    if args.fp8_gemm and not args.fp8_weights:
        raise SystemExit("--fp8-gemm needs --fp8-weights")

    import torch

    import mixture_experts_layer_02_amd as moe
    import synth

    def note(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.workload]
    t_gen = time.perf_counter()
    inp = synth.make_inputs(cfg)
    gen_s = time.perf_counter() - t_gen
    note(f"inputs of {cfg.name} drawn in {gen_s:.1f} s")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    wl = Workload(moe, torch, cfg, inp, args, dev)
    torch.cuda.synchronize()
    note("inputs resident in HBM; warming up")
    avg, step_ms, wall = run(moe, torch, wl, args, args.steps, args.warmup, flush, note)
    peak_mem = torch.cuda.max_memory_allocated()
    default_run = (cfg.name == "fwdbwd_1t" and args.x_path == "perm" and args.dy_path == "gather"
                   and args.router_dx == "fused" and args.dtopk == "parts" and args.wgrad_dtype == "bf16" and not (
        args.fp8_weights or args.fp8_gemm or args.hold_cus or args.n_groups > 1 or args.schedule != "static"))
    main_sum = summarize(wl, avg, step_ms, wall, args.steps, default_run)
    ms_step = main_sum["ms_per_step"]
    note(f"timed region: {ms_step:.3f} ms/step")
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    del wl
    torch.cuda.empty_cache()

    # the other 1T workloads after the main one: the same step with fp32 weight
    # gradients (on the main step's inputs), then forward-only ones
    extras, extra_inputs = {}, {}
    names = [] if args.extra_workloads == "none" else [n for n in args.extra_workloads.split(",") if n]
    for name in names:
        fp8mm = name.endswith("_fp8mm")
        wf32 = name.endswith("_wgrad_f32")
        base = name[:-len("_fp8mm")] if fp8mm else name[:-len("_wgrad_f32")] if wf32 else name
        c = synth.CONFIGS[base]
        if wf32 and (base != cfg.name or args.wgrad_dtype == "f32" or c.dtype != "bf16"):
            continue                       # only beside a bf16-gradient run of the same workload
        data = inp if base == cfg.name else extra_inputs.get(base) or synth.make_inputs(c)
        if base == "share_1t":             # reused by the fp8 variant and the CPU baseline's sample
            extra_inputs[base] = data
        w2 = Workload(moe, torch, c, data, args, dev, fp8mm=fp8mm, wgrad="f32" if wf32 else None)
        torch.cuda.synchronize()
        a2, s2, wall2 = run(moe, torch, w2, args, args.extra_steps, args.warmup, flush, note)
        sm = summarize(w2, a2, s2, wall2, args.extra_steps, False)
        extras[name] = {
            "workload": f"{base}: T={c.T} d={c.d} E={c.E} ({c.num_local} local) top-{c.k} f={c.f} "
                        f"{'fwd+bwd' if c.backward else 'fwd'}, routing {c.routing}"
                        + (", gate/up and down on the fp8 matrix cores (e4m3 x, h and W1/W3/W2 with "
                           "power-of-two block-128 scales)" if fp8mm else "")
                        + (", weight gradients dW1, dW3, dW2 in fp32" if wf32 else ""),
            "steps": args.extra_steps, "ms_per_step": round(sm["ms_per_step"], 4),
            "tokens/s": round(c.T / sm["ms_per_step"] * 1e3, 1), "routed_rows": sm["R"],
            "grouped_gemm_tflops": round(sm["gemm_tflops"], 1),
            "grouped_gemm_frac_mfma": round(sm["gemm_tflops"] / PEAK_BF16_TFLOPS, 4),
            "roofline": sm["roofline"], "rows": sm["rows"]}
        note(f"{name}: {sm['ms_per_step']:.3f} ms/step")
        del w2
        torch.cuda.empty_cache()

    vendor = None
    if not args.no_vendor_gemm and cfg.backward:
        vendor = _vendor_gemm(torch, dev, cfg.num_local, main_sum["R"], d, f, main_sum["rows"])
        note("vendor gemm: " + ", ".join(f"{k} {v['vendor_ms']:.3f} ms" for k, v in vendor["rows"].items()))

    cpu = None
    if not args.no_cpu_baseline:
        note(f"cpu baseline: oracle on {min(args.cpu_sample_tokens, cfg.T)} tokens")
        del flush
        torch.cuda.empty_cache()
        cpu = _cpu_baseline(cfg, inp, min(args.cpu_sample_tokens, cfg.T), args.n_groups, extra_inputs)

    out = {
        "metric": METRIC, "value": round(T / ms_step * 1e3, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} d={d} E={E} ({cfg.num_local} local from {cfg.expert_begin}) "
                               f"top-{cfg.k} f={f} {'fwd+bwd' if cfg.backward else 'fwd'}",
                   "routed_rows": main_sum["R"], "global_batch": T, "parallelism": "single GPU",
                   "routing": f"group-limited, {args.n_groups} groups" if args.n_groups > 1 else "top-k",
                   "tile_schedule": args.schedule,
                   "x_path": ("x_perm copy" if args.x_path == "perm" else "x read through row_token"),
                   "dy_path": ("dy read through row_token, no dy_perm" if args.dy_path == "gather"
                               else "dy_perm copy"),
                   "router_dx": ("k rows of Wr added in the unpermute pass" if args.router_dx == "fused"
                                 and cfg.renormalize else "dx += dlogits Wr product"),
                   "dtopk_w": ("partial sums of <dy W2, h> in the dH product" if args.dtopk == "parts"
                               else "dot products of dy and y_perm"),
                   "weight_grads": ("bf16: float32 sums rounded once at the store (the pages compute "
                                    "gradients in bf16 and reduce them in fp32); the same step with fp32 "
                                    "weight gradients is workloads.fwdbwd_1t_wgrad_f32"
                                    if args.wgrad_dtype == "bf16" and cfg.dtype == "bf16" else "fp32"),
                   "expert_weights": ("bf16" if not args.fp8_weights else
                                      "fp8 e4m3 blocks of 128, read by the forward GEMMs" if args.fp8_gemm else
                                      "fp8 e4m3 blocks of 128, dequantised each step"),
                   "contention": (f"{args.hold_cus} CUs held for {args.hold_us} us at each grouped GEMM"
                                  if args.hold_cus else None),
                   "timing": "per-step span of HIP events after a 1 GiB cache flush outside the events"},
        "step_ms_min_max": [round(main_sum["step_ms_min"], 3), round(main_sum["step_ms_max"], 3)],
        "wall_ms_per_step_incl_flush": round(main_sum["wall_ms_per_step_incl_flush"], 3),
        "device_mem_peak_gb": round(peak_mem / 1e9, 2),
        "grouped_gemm_tflops": round(main_sum["gemm_tflops"], 1),
        "grouped_gemm_frac_mfma": round(main_sum["gemm_tflops"] / PEAK_BF16_TFLOPS, 4),
        "roofline": main_sum["roofline"],
        "cpu_baseline": cpu,
        "rows": main_sum["rows"],
        "workloads": extras,
        "vendor_gemm": vendor,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
