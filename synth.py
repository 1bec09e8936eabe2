"""Seeded synthetic inputs for the MoE expert layer (shared by tests, bench and smoke).

This module holds the input recipes only: shapes, seeds, value distributions
and routing patterns that are *inputs* to the layer.  It computes nothing the
layer itself computes (no logits, no top-k, no counting, no GEMM).

Recipe (stated once, used everywhere):

* Every tensor is drawn i.i.d. N(0, sigma) in float32 with numpy's PCG64.
  A tensor of n elements is cut into chunks of ``CHUNK`` elements; chunk c of
  the tensor with draw-order index i in a config with seed s is drawn by
  ``Generator(PCG64(SeedSequence([s, i, c]))).standard_normal``.  The chunks
  are independent streams, so the values do not depend on how many threads
  fill them.
* Draw order (the index i): W_r, W1, W3, W2, x, dy, then the Zipf permutation.
* bf16 configs round each float32 draw to bfloat16 with round-to-nearest-even;
  bf16 tensors are returned as uint16 bit patterns.
* Weight layouts are those of a linear layer (out x in), concatenated over the
  experts held on this GPU, as the Aurora FastSparseMoE page (section 3.1,
  stage 4) concatenates every expert's gate_proj / up_proj / down_proj weight:
  W_r [E][d], W1 = gate [NL][f][d], W3 = up [NL][f][d], W2 = down [NL][d][f].
* Zipf-skewed routing adds a per-expert bias to the router logits:
  q_e = (pi_e + 1)^-1.2 for a seeded permutation pi of the experts and
  bias_e = beta * ln(q_e / max q).  beta is fixed per config (calibrated so
  that the busiest expert receives about 10x the mean load; the calibration
  script sits in tests/golden/).
* Forced-uniform ("round-robin") routing: idx[t][j] = (t*k + j) mod E with
  weight 1/k on every slot (the forced uniform routing ablation of the Aurora
  page, section 2.3 of its evaluation).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    T: int
    d: int
    E: int
    k: int
    f: int
    expert_begin: int
    num_local: int
    dtype: str            # "f32" or "bf16"
    x_std: float
    routing: str          # "router", "zipf" or "roundrobin"
    backward: bool
    zipf_beta: float = 0.0
    w_std: float = 0.02
    renormalize: int = 1

    @property
    def R_cap(self) -> int:
        return self.T * min(self.k, self.num_local)


CONFIGS = {
    # fp32 tiny layer: forward + backward, tolerance 1e-5
    "tiny_f32": Config("tiny_f32", 1, 256, 128, 8, 2, 64, 0, 8, "f32", 0.02, "router", True),
    # small bf16 layer, forward
    "small_bf16": Config("small_bf16", 2, 4096, 2048, 64, 8, 1024, 0, 64, "bf16", 1.0, "router", False),
    # 1T shape, one GPU's expert-parallel share: 96 of 384 experts local
    "share_1t": Config("share_1t", 3, 8192, 6144, 384, 8, 1792, 0, 96, "bf16", 1.0, "router", False),
    # 1T shape, 96 local experts, Zipf-skewed router bias
    "zipf_1t": Config("zipf_1t", 4, 16384, 6144, 96, 8, 1792, 0, 96, "bf16", 1.0, "zipf", False,
                      zipf_beta=0.96875),
    # 1T shape, 96 local experts, forced-uniform round-robin routing
    "uniform_1t": Config("uniform_1t", 4, 16384, 6144, 96, 8, 1792, 0, 96, "bf16", 1.0, "roundrobin", False),
    # 1T shape, one 65,536-token sequence, forward + backward
    "fwdbwd_1t": Config("fwdbwd_1t", 5, 65536, 6144, 384, 8, 1792, 0, 96, "bf16", 1.0, "router", True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, index: int, shape, std: float) -> np.ndarray:
    """N(0, std) float32 tensor, chunked PCG64 streams (see module docstring)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index, c])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= np.float32(std)

    if nchunks == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Uses torch's float32 -> bfloat16 conversion (round-to-nearest-even) for
    speed; tests check it against the bit-level definition."""
    import torch
    a = np.ascontiguousarray(a, np.float32)
    t = torch.from_numpy(a).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_to_bf16_bits_reference(a: np.ndarray) -> np.ndarray:
    """Bit-level round-to-nearest-even float32 -> bfloat16 (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _tensor(cfg: Config, index: int, shape, std: float) -> np.ndarray:
    a = normal_f32(cfg.seed, index, shape, std)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(a)
    return a


def zipf_bias(cfg: Config) -> np.ndarray:
    """Per-expert router-logit bias of the Zipf-skewed workload (float32 [E])."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 6, 0])))
    pi = g.permutation(cfg.E)
    q = (pi.astype(np.float64) + 1.0) ** -1.2
    return (cfg.zipf_beta * np.log(q / q.max())).astype(np.float32)


def roundrobin_routing(T: int, E: int, k: int):
    """Forced-uniform routing: idx[t][j] = (t*k + j) mod E, weight 1/k."""
    t = np.arange(T, dtype=np.int64)[:, None]
    j = np.arange(k, dtype=np.int64)[None, :]
    idx = ((t * k + j) % E).astype(np.int32)
    w = np.full((T, k), 1.0 / k, np.float32)
    return idx, w


def make_inputs(cfg: Config, want=("wr", "w1", "w3", "w2", "x", "dy")) -> dict:
    """Draw the inputs of one config.  bf16 tensors come back as uint16 bits.

    Tensors not in ``want`` are skipped (their streams are independent, so
    skipping one does not change the others)."""
    NL, d, f, E, T = cfg.num_local, cfg.d, cfg.f, cfg.E, cfg.T
    shapes = {
        "wr": (0, (E, d), cfg.w_std),
        "w1": (1, (NL, f, d), cfg.w_std),
        "w3": (2, (NL, f, d), cfg.w_std),
        "w2": (3, (NL, d, f), cfg.w_std),
        "x": (4, (T, d), cfg.x_std),
        "dy": (5, (T, d), 1.0),
    }
    out = {}
    for name in want:
        idx, shape, std = shapes[name]
        out[name] = _tensor(cfg, idx, shape, std)
    if cfg.routing == "zipf":
        out["bias"] = zipf_bias(cfg)
    if cfg.routing == "roundrobin":
        out["idx"], out["w"] = roundrobin_routing(T, E, cfg.k)
    return out


def scaled(cfg: Config, **changes) -> Config:
    """A copy of ``cfg`` with some fields replaced (for reduced test shapes)."""
    return dataclasses.replace(cfg, **changes)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Float32 view of an input as the layer sees it (bf16 bits widened)."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)
