"""FP8 (E4M3) blockwise-128 expert weights on the GPU against the oracle
(Domyn page, section "FP8 expert weight all-gather").

Codes and scales are integer/byte and float32 decisions taken in float32 on
both sides, so they must match the oracle bit for bit; the dequantised bf16
weights too (decode * scale in float32, rounded to nearest even).  At the 1T
expert shape the codes of sampled blocks are recomputed by the oracle one
block at a time, and the page's error bound (at most 1/16 of the block
maximum) is checked on every value.  The layer run on dequantised weights is
checked against the oracle layer on the oracle's dequantised weights, and
the GEMMs that read the FP8 codes directly against the oracle's expert MLP on
those weights.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_02_amd as moe
import oracle
import synth
from gpu_util import f64, to_dev, to_host
from layer_checks import TOL, _desc, random_routing
from metrics import max_row_rel_err

pytestmark = pytest.mark.gpu


def _special_blocks(rng, nblk):
    w = rng.normal(0, 0.02, (nblk, 128)).astype(np.float32)
    w[0] = 0.0
    w[1] = -0.0                                             # zeros with the sign bit
    w[2] = 0.0
    w[2, 5] = -0.25                                         # a single value
    w[3] *= 1e-30                                           # tiny (subnormal codes after scaling)
    grid = oracle.fp8_e4m3_decode(np.arange(127))
    mids = ((grid[1:] + grid[:-1]) / 2)[:126]
    w[4, :126] = mids * 2.0 ** -10                          # exact ties after scaling by 2^10
    w[4, 126] = 448 * 2.0 ** -10
    w[4, 127] = -mids[50] * 2.0 ** -10
    w[5, ::2] = -0.0                                        # negative zeros in a live block
    return w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nblk", [1, 7, 1000, 40961])
def test_quantize_and_dequantize_match_the_oracle(gpu, dtype, nblk):
    rng = np.random.default_rng(nblk)
    w = _special_blocks(rng, max(nblk, 8))[:nblk].reshape(-1) if nblk >= 8 else \
        rng.normal(0, 1, nblk * 128).astype(np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(w)
        w = synth.bf16_bits_to_f32(bits)                   # the values the GPU sees
        wd = to_dev(bits)
    else:
        wd = to_dev(w)
    q = torch.empty(w.size, dtype=torch.uint8, device=gpu)
    s = torch.empty(nblk, dtype=torch.float32, device=gpu)
    moe.fp8_quantize(wd, q, s)
    codes, scales = oracle.fp8_quantize_blocks(w)
    np.testing.assert_array_equal(q.cpu().numpy(), codes)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), scales.view(np.uint32))
    out = torch.empty(w.size, dtype=torch.bfloat16, device=gpu)
    moe.fp8_dequantize(q, s, out)
    want = oracle.fp8_dequantize_blocks(codes, scales)
    np.testing.assert_array_equal(to_host(out).view(np.uint32), want.view(np.uint32))


def test_expert_weights_at_full_size(gpu):
    # W1 of the 1T expert-parallel share: 96 experts x 1792 x 6144 bf16.
    cfg = synth.CONFIGS["fwdbwd_1t"]
    w = synth.make_inputs(cfg, want=("w1",))["w1"].reshape(-1)
    n = w.size
    wd = to_dev(w)
    q = torch.empty(n, dtype=torch.uint8, device=gpu)
    s = torch.empty(n // 128, dtype=torch.float32, device=gpu)
    moe.fp8_quantize(wd, q, s)
    out = torch.empty(n, dtype=torch.bfloat16, device=gpu)
    moe.fp8_dequantize(q, s, out)
    torch.cuda.synchronize()
    # the page's bound on every value, on the device
    wf = wd.float().view(-1, 128)
    amax = wf.abs().amax(dim=1, keepdim=True)
    err = (out.float().view(-1, 128) - wf).abs()
    # 1/16 of the block max from the E4M3 rounding, plus the final bf16 rounding (2^-8 relative)
    assert bool((err <= amax / 16 + wf.abs() * 2.0 ** -8 + 1e-30).all())
    del wf, err
    # sampled blocks, bit-exact
    rng = np.random.default_rng(7)
    blocks = np.unique(np.concatenate([[0, n // 128 - 1], rng.choice(n // 128, 500, replace=False)]))
    qs, ss = q.view(-1, 128).cpu().numpy(), s.cpu().numpy()
    wf32 = synth.as_f32(w, "bf16").reshape(-1, 128)
    for b in blocks:
        c, sc = oracle.fp8_quantize_blocks(wf32[b])
        assert np.array_equal(qs[b], c), b
        assert ss[b].view(np.uint32) == sc[0].view(np.uint32), b


def test_layer_on_fp8_weights(gpu):
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], T=512, d=256, f=128, E=32, num_local=8, expert_begin=8)
    inp = synth.make_inputs(cfg)
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2")}
    deq, ref_w = {}, {}
    for n in ("w1", "w3", "w2"):
        q = torch.empty(dev[n].numel(), dtype=torch.uint8, device=gpu)
        s = torch.empty(dev[n].numel() // 128, dtype=torch.float32, device=gpu)
        moe.fp8_quantize(dev[n], q, s)
        deq[n] = torch.empty_like(dev[n])
        moe.fp8_dequantize(q, s, deq[n])
        c, sc = oracle.fp8_quantize_blocks(synth.as_f32(inp[n], "bf16"))
        ref_w[n] = oracle.fp8_dequantize_blocks(c, sc).reshape(inp[n].shape).astype(np.float64)
    D = _desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    b = moe.Buffers(D)
    moe.forward(b, dev["x"], dev["wr"], deq["w1"], deq["w3"], deq["w2"])
    torch.cuda.synchronize()
    for n in ("w1", "w3", "w2"):
        np.testing.assert_array_equal(to_host(deq[n]), ref_w[n].astype(np.float32))
    x, wr = f64(inp["x"], "bf16"), f64(inp["wr"], "bf16")
    ref = oracle.layer_forward(x, wr, ref_w["w1"], ref_w["w3"], ref_w["w2"], cfg.k, cfg.expert_begin,
                               cfg.num_local, cfg.renormalize)
    assert (to_host(b.topk_idx) == ref["idx"]).all()
    assert max_row_rel_err(to_host(b.y), ref["y"]) <= TOL["bf16"]


@pytest.mark.parametrize("gather,dyn", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("scale", [
    dict(T=2048, d=512, f=256, E=32, num_local=16, expert_begin=8),
    dict(T=1500, d=384, f=256, E=64, num_local=24, expert_begin=40, k=6),    # ragged, empty experts
    dict(T=300, d=128, f=128, E=8, num_local=8, expert_begin=0, k=2),        # K of 2 k-tiles
])
def test_fp8_gemms_equal_bf16_on_dequantised_weights(gpu, scale, gather, dyn):
    # The FP8-weight GEMMs decode the codes in the kernel exactly as
    # moe_fp8_dequantize does, so they must equal the bf16 GEMMs run on the
    # dequantised weights bit for bit.
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[fp8 gemm] {scale} gather={gather} dynamic={dyn}", flush=True)
    inp = synth.make_inputs(cfg, want=("x", "wr", "w1", "w3", "w2"))
    dev = {n: to_dev(inp[n]) for n in ("x", "wr", "w1", "w3", "w2")}
    q, deq = {}, {}
    for n in ("w1", "w3", "w2"):
        c = torch.empty(dev[n].numel(), dtype=torch.uint8, device=gpu)
        sc = torch.empty(dev[n].numel() // 128, dtype=torch.float32, device=gpu)
        moe.fp8_quantize(dev[n], c, sc)
        q[n] = (c, sc)
        deq[n] = torch.empty_like(dev[n])
        moe.fp8_dequantize(c, sc, deq[n])
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local, cfg.dtype, cfg.renormalize)
    D = moe.make_desc(*args, tile_counters=moe.new_tile_counters(gpu) if dyn else None)
    b = moe.Buffers(D, backward=True)
    moe.forward(b, dev["x"], dev["wr"], deq["w1"], deq["w3"], deq["w2"])     # reference: bf16 on dequantised
    R = int(b.offsets[-1].item())
    gu8 = torch.empty_like(b.gu)
    h8 = torch.empty_like(b.h)
    y8 = torch.empty_like(b.y_perm)
    a = dev["x"] if gather else b.x_perm
    moe.expert_gate_up_fp8(D, b.offsets, b.row_token if gather else None, a, q["w1"][0], q["w1"][1],
                           q["w3"][0], q["w3"][1], gu8, h8)
    moe.expert_down_fp8(D, b.offsets, h8, q["w2"][0], q["w2"][1], y8)
    torch.cuda.synchronize()
    for name, got, ref in (("gu", gu8, b.gu), ("h", h8, b.h), ("y_perm", y8, b.y_perm)):
        assert torch.equal(got[:R].view(torch.int16), ref[:R].view(torch.int16)), name


def test_fp8_gemms_reject_unsupported_shapes(gpu):
    D = _desc(64, 192, 128, 8, 2, 0, 8, "bf16")                 # d not a multiple of 128
    z = torch.zeros(1 << 16, dtype=torch.float32, device=gpu)
    with pytest.raises(moe.MoeError):
        moe.expert_gate_up_fp8(D, z, None, z, z, z, z, z, z, z)
    with pytest.raises(moe.MoeError):
        moe.expert_down_fp8(D, z, z, z, z, z)


@pytest.mark.parametrize("gather,dyn", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("scale", [
    dict(T=1024, d=512, f=256, E=32, num_local=16, expert_begin=8, k=4),
    dict(T=700, d=384, f=256, E=64, num_local=24, expert_begin=40, k=6),     # ragged, empty experts
])
def test_fp8_gemms_match_the_oracle(gpu, scale, gather, dyn):
    # gate/up + SwiGLU and down reading E4M3 codes and block scales, against
    # the oracle's expert MLP on the oracle's own dequantised weights.
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[fp8 gemm vs oracle] {scale} gather={gather} dynamic={dyn}", flush=True)
    T, d, f, E, k, e0, NL = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local
    inp = synth.make_inputs(cfg, want=("x", "w1", "w3", "w2"))
    idx = random_routing(np.random.default_rng(T + d), T, E, k, skew=1.0)
    D = moe.make_desc(T, d, f, E, k, e0, NL, "bf16", 1, tile_counters=moe.new_tile_counters(gpu) if dyn else None)
    b = moe.Buffers(D, backward=True, gather=gather)
    x = to_dev(inp["x"])
    moe.permute(D, to_dev(idx), None if gather else x, b.counts, b.offsets, b.row_token, b.slot_row,
                None if gather else b.x_perm, b.ws_permute)
    q, ref_w = {}, {}
    for n in ("w1", "w3", "w2"):
        wd = to_dev(inp[n])
        c = torch.empty(wd.numel(), dtype=torch.uint8, device=gpu)
        sc = torch.empty(wd.numel() // 128, dtype=torch.float32, device=gpu)
        moe.fp8_quantize(wd, c, sc)
        q[n] = (c, sc)
        codes, scales = oracle.fp8_quantize_blocks(synth.as_f32(inp[n], "bf16"))
        ref_w[n] = oracle.fp8_dequantize_blocks(codes, scales).reshape(inp[n].shape).astype(np.float64)
    moe.expert_gate_up_fp8(D, b.offsets, b.row_token if gather else None, x if gather else b.x_perm,
                           q["w1"][0], q["w1"][1], q["w3"][0], q["w3"][1], b.gu, b.h)
    moe.expert_down_fp8(D, b.offsets, b.h, q["w2"][0], q["w2"][1], b.y_perm)
    torch.cuda.synchronize()
    _, off = oracle.count_tokens(idx, E, e0, NL)
    rows, _ = oracle.generate_indices(idx, e0, NL, off)
    np.testing.assert_array_equal(to_host(b.offsets), off)
    R = int(off[-1])
    xp = oracle.permute(f64(inp["x"], "bf16"), rows)
    G, U, H, Y = oracle.expert_ffn(xp, off, ref_w["w1"], ref_w["w3"], ref_w["w2"])
    tol = TOL["bf16"]
    gu = to_host(b.gu)[:R]
    assert max_row_rel_err(gu[:, :f], G) <= tol
    assert max_row_rel_err(gu[:, f:], U) <= tol
    assert max_row_rel_err(to_host(b.h)[:R], H) <= tol
    assert max_row_rel_err(to_host(b.y_perm)[:R], Y) <= tol


# ---------------------------------------------------------------------------
# Power-of-two block scales and the gate/up GEMM on the FP8 matrix cores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nblk", [1, 7, 1000, 40961])
def test_quantize_pow2_matches_the_oracle(gpu, dtype, nblk):
    rng = np.random.default_rng(100 + nblk)
    w = _special_blocks(rng, max(nblk, 8))[:nblk].reshape(-1) if nblk >= 8 else \
        (rng.normal(0, 1, nblk * 128) * 10.0 ** rng.uniform(-8, 6)).astype(np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(w)
        w = synth.bf16_bits_to_f32(bits)
        wd = to_dev(bits)
    else:
        wd = to_dev(w)
    q = torch.empty(w.size, dtype=torch.uint8, device=gpu)
    e8 = torch.empty(nblk, dtype=torch.uint8, device=gpu)
    moe.fp8_quantize_pow2(wd, q, e8)
    codes, e8_o = oracle.fp8_quantize_blocks_pow2(w)
    np.testing.assert_array_equal(q.cpu().numpy(), codes)
    np.testing.assert_array_equal(e8.cpu().numpy(), e8_o)


def _quant_pow2(t, gpu):
    q = torch.empty(t.numel(), dtype=torch.uint8, device=gpu)
    e8 = torch.empty(t.numel() // 128, dtype=torch.uint8, device=gpu)
    moe.fp8_quantize_pow2(t, q, e8)
    return q, e8


@pytest.mark.parametrize("dyn", [False, True])
@pytest.mark.parametrize("scale", [
    dict(T=1024, d=512, f=256, E=32, num_local=16, expert_begin=8, k=4),
    dict(T=700, d=1024, f=384, E=64, num_local=24, expert_begin=40, k=6),    # ragged, empty experts, 3 n-tiles
    dict(T=300, d=512, f=128, E=8, num_local=8, expert_begin=0, k=2),        # K of 4 k-tiles: no hand-over
])
def test_fp8mm_gate_up_matches_the_oracle(gpu, scale, dyn):
    # x and W1/W3 quantised to E4M3 with power-of-two block scales; G, U and
    # h against the oracle's expert MLP on the oracle's own dequantised x
    # rows and weights (the codes and scales are first checked bit-exact).
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[fp8mm] {scale} dynamic={dyn}", flush=True)
    T, d, f, E, k, e0, NL = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local
    inp = synth.make_inputs(cfg, want=("x", "w1", "w3"))
    idx = random_routing(np.random.default_rng(T + d), T, E, k, skew=1.0)
    D = moe.make_desc(T, d, f, E, k, e0, NL, "bf16", 1, tile_counters=moe.new_tile_counters(gpu) if dyn else None)
    b = moe.Buffers(D, gather=True, backward=True)
    moe.permute(D, to_dev(idx), None, b.counts, b.offsets, b.row_token, b.slot_row, None, b.ws_permute)
    xq, xs = _quant_pow2(to_dev(inp["x"]), gpu)
    wq = {n: _quant_pow2(to_dev(inp[n]), gpu) for n in ("w1", "w3")}
    moe.expert_gate_up_fp8mm(D, b.offsets, b.row_token, xq, xs, wq["w1"][0], wq["w1"][1], wq["w3"][0],
                             wq["w3"][1], b.gu, b.h)
    torch.cuda.synchronize()
    deq = {}
    for n, a in (("x", inp["x"]), ("w1", inp["w1"]), ("w3", inp["w3"])):
        c, e = oracle.fp8_quantize_blocks_pow2(synth.as_f32(a, "bf16"))
        got = (xq, xs) if n == "x" else wq[n]
        np.testing.assert_array_equal(got[0].cpu().numpy(), c)
        np.testing.assert_array_equal(got[1].cpu().numpy(), e)
        deq[n] = oracle.fp8_dequantize_blocks_pow2(c, e).reshape(a.shape)
    _, off = oracle.count_tokens(idx, E, e0, NL)
    rows, _ = oracle.generate_indices(idx, e0, NL, off)
    np.testing.assert_array_equal(to_host(b.offsets), off)
    R = int(off[-1])
    xp = oracle.permute(deq["x"], rows)
    G, U, H, _ = oracle.expert_ffn(xp, off, deq["w1"], deq["w3"], np.zeros((NL, d, f)))
    tol = TOL["bf16"]
    gu = to_host(b.gu)[:R]
    assert max_row_rel_err(gu[:, :f], G) <= tol
    assert max_row_rel_err(gu[:, f:], U) <= tol
    assert max_row_rel_err(to_host(b.h)[:R], H) <= tol


def test_fp8mm_rejects_unsupported_shapes(gpu):
    z = torch.zeros(1 << 16, dtype=torch.float32, device=gpu)
    D = _desc(64, 256, 128, 8, 2, 0, 8, "bf16")                 # d not a multiple of 512
    with pytest.raises(moe.MoeError):
        moe.expert_gate_up_fp8mm(D, z, z, z, z, z, z, z, z, z, z)
    D = _desc(64, 512, 128, 8, 2, 0, 8, "f32")
    with pytest.raises(moe.MoeError):
        moe.expert_gate_up_fp8mm(D, z, z, z, z, z, z, z, z, z, z)


def test_fp8mm_gate_up_at_full_size_sampled(gpu):
    # The 1T expert-parallel share (T = 8192, d = 6144, 96 of 384 experts,
    # f = 1792) in the benchmark's launch configuration; the oracle quantises
    # and multiplies only what the sampled tokens' rows need (their x rows
    # and their experts' W1 / W3).
    cfg = synth.CONFIGS["share_1t"]
    T, d, f, E, k, e0, NL = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local
    print(f"[fp8mm full size] T={T} d={d} f={f} E={E} NL={NL}", flush=True)
    inp = synth.make_inputs(cfg, want=("x", "w1", "w3"))
    idx = random_routing(np.random.default_rng(3), T, E, k)
    D = _desc(T, d, f, E, k, e0, NL, "bf16")
    b = moe.Buffers(D, gather=True)
    moe.permute(D, to_dev(idx), None, b.counts, b.offsets, b.row_token, b.slot_row, None, b.ws_permute)
    xq, xs = _quant_pow2(to_dev(inp["x"]), gpu)
    wq = {n: _quant_pow2(to_dev(inp[n]), gpu) for n in ("w1", "w3")}
    moe.expert_gate_up_fp8mm(D, b.offsets, b.row_token, xq, xs, wq["w1"][0], wq["w1"][1], wq["w3"][0],
                             wq["w3"][1], None, b.h)
    torch.cuda.synchronize()
    _, off = oracle.count_tokens(idx, E, e0, NL)
    rows, slot = oracle.generate_indices(idx, e0, NL, off)
    np.testing.assert_array_equal(to_host(b.offsets), off)
    np.testing.assert_array_equal(to_host(b.slot_row), slot)
    # sampled tokens (the first and the last among them) with at least one local slot
    has = (slot >= 0).any(axis=1)
    cand = np.nonzero(has)[0]
    toks = np.unique(np.concatenate([cand[[0, -1]], np.random.default_rng(5).choice(cand, 3, replace=False)]))
    x32 = synth.as_f32(inp["x"], "bf16")
    deq_w = {}
    hg = to_host(b.h[torch.as_tensor(slot[toks][slot[toks] >= 0].astype(np.int64), device=b.h.device)])
    want = []
    for t in toks:
        c, e = oracle.fp8_quantize_blocks_pow2(x32[t])
        xr = oracle.fp8_dequantize_blocks_pow2(c, e)
        for j in range(k):
            if slot[t, j] < 0:
                continue
            n = int(idx[t, j]) - e0
            if n not in deq_w:
                deq_w[n] = [oracle.fp8_dequantize_blocks_pow2(*oracle.fp8_quantize_blocks_pow2(
                    synth.as_f32(inp[w][n], "bf16"))).reshape(f, d) for w in ("w1", "w3")]
            G, U, H, _ = oracle.expert_ffn_rows(xr[None, :], deq_w[n][0], deq_w[n][1], np.zeros((d, f)))
            want.append(H[0])
    assert max_row_rel_err(hg, np.array(want)) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# A6 on the FP8 matrix cores: h and W2 quantised by rows, scales in rows of
# fp8_scale_row_bytes(f) bytes (f/128 rounded up to a multiple of 4).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,ld,nrows", [(1, 128, 4, None), (37, 1792, 16, 20), (300, 640, 5, None),
                                                (64, 6144, 48, 64), (50, 256, 17, 0), (129, 384, 3, 129)])
def test_quantize_pow2_rows_matches_the_oracle(gpu, dtype, rows, cols, ld, nrows):
    rng = np.random.default_rng(rows + cols)
    w = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-4, 2, (rows, 1))).astype(np.float32)
    w[0, :128] = 0.0                                         # a zero block
    w = synth.as_f32(synth.f32_to_bf16_bits(w), "bf16") if dtype == "bf16" else w
    wd = to_dev(w, dtype)
    q = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device=gpu)
    e8 = torch.full((rows, ld), 0xCD, dtype=torch.uint8, device=gpu)
    nr = None if nrows is None else torch.tensor([nrows], dtype=torch.int32, device=gpu)
    moe.fp8_quantize_pow2_rows(wd, q, e8, nr)
    torch.cuda.synchronize()
    lim = rows if nrows is None else min(rows, nrows)
    c, e = oracle.fp8_quantize_blocks_pow2(w[:lim])
    qh, eh = q.cpu().numpy(), e8.cpu().numpy()
    cb = cols // 128
    np.testing.assert_array_equal(qh[:lim].reshape(-1), c)
    np.testing.assert_array_equal(eh[:lim, :cb].reshape(-1), e)
    assert (eh[:lim, cb:] == 0).all()                        # the padding
    assert (qh[lim:] == 0xAB).all() and (eh[lim:] == 0xCD).all()   # rows past nrows untouched


def test_quantize_pow2_rows_rejects_bad_pitches(gpu):
    w = torch.zeros(4, 256, dtype=torch.bfloat16, device=gpu)
    q = torch.empty(4, 256, dtype=torch.uint8, device=gpu)
    for ld in (1, 18):                                       # below cols/128, above cols/128 + 15
        with pytest.raises(moe.MoeError):
            moe.fp8_quantize_pow2_rows(w, q, torch.empty(4, ld, dtype=torch.uint8, device=gpu))


def _down_case(cfg, gpu, dyn, seed):
    T, d, f, E, k, e0, NL = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local
    inp = synth.make_inputs(cfg, want=("w2",))
    idx = random_routing(np.random.default_rng(seed), T, E, k, skew=1.0)
    D = moe.make_desc(T, d, f, E, k, e0, NL, "bf16", 1, tile_counters=moe.new_tile_counters(gpu) if dyn else None)
    b = moe.Buffers(D, gather=True)
    moe.permute(D, to_dev(idx), None, b.counts, b.offsets, b.row_token, b.slot_row, None, b.ws_permute)
    _, off = oracle.count_tokens(idx, E, e0, NL)
    R = int(off[-1])
    # h: seeded bf16 rows, like the SwiGLU outputs in scale; rows past R stay
    # garbage and are left alone by the row quantiser
    h = synth.as_f32(synth.f32_to_bf16_bits(synth.normal_f32(seed, 7, (max(R, 1), f), 0.5)), "bf16")
    hd = torch.full((D.R_cap, f), float("nan"), dtype=torch.bfloat16, device=gpu)
    hd[:R] = to_dev(h[:R], "bf16")
    S8 = moe.fp8_scale_row_bytes(f)
    hq = torch.empty(D.R_cap, f, dtype=torch.uint8, device=gpu)
    hs = torch.empty(D.R_cap, S8, dtype=torch.uint8, device=gpu)
    moe.fp8_quantize_pow2_rows(hd, hq, hs, b.offsets[NL:])
    w2d = to_dev(inp["w2"])
    w2q = torch.empty(NL * d, f, dtype=torch.uint8, device=gpu)
    w2s = torch.empty(NL * d, S8, dtype=torch.uint8, device=gpu)
    moe.fp8_quantize_pow2_rows(w2d.view(NL * d, f), w2q, w2s)
    y = torch.empty(D.R_cap, d, dtype=torch.bfloat16, device=gpu)
    moe.expert_down_fp8mm(D, b.offsets, hq, hs, w2q, w2s, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(b.offsets), off)
    return inp, h[:R], off, R, (hq, hs, w2q, w2s), y


@pytest.mark.parametrize("dyn", [False, True])
@pytest.mark.parametrize("scale", [
    dict(T=512, d=256, f=128, E=32, num_local=8, expert_begin=8),
    dict(T=700, d=384, f=1792, E=16, num_local=16, expert_begin=0),      # 14 scale blocks per row: padded to 16
    dict(T=1500, d=320, f=640, E=64, num_local=24, expert_begin=40, k=6),  # ragged, empty experts
])
def test_fp8mm_down_matches_the_oracle(gpu, scale, dyn):
    # h and W2 quantised on the GPU (codes and scales checked bit-exact
    # against the oracle's), then y_perm against the oracle's down projection
    # on its own dequantised h and W2.
    cfg = synth.scaled(synth.CONFIGS["fwdbwd_1t"], **scale)
    print(f"[fp8mm down] {scale} dynamic={dyn}", flush=True)
    d, f, NL = cfg.d, cfg.f, cfg.num_local
    inp, h, off, R, (hq, hs, w2q, w2s), y = _down_case(cfg, gpu, dyn, cfg.T + f)
    cb = f // 128
    ch, eh = oracle.fp8_quantize_blocks_pow2(h)
    np.testing.assert_array_equal(hq[:R].cpu().numpy().reshape(-1), ch)
    np.testing.assert_array_equal(hs[:R, :cb].cpu().numpy().reshape(-1), eh)
    w2 = synth.as_f32(inp["w2"], "bf16")
    cw, ew = oracle.fp8_quantize_blocks_pow2(w2)
    np.testing.assert_array_equal(w2q.cpu().numpy().reshape(-1), cw)
    np.testing.assert_array_equal(w2s[:, :cb].cpu().numpy().reshape(-1), ew)
    hdq = oracle.fp8_dequantize_blocks_pow2(ch, eh).reshape(R, f)
    w2dq = oracle.fp8_dequantize_blocks_pow2(cw, ew).reshape(NL, d, f)
    want = oracle.expert_down(hdq, off, w2dq)
    assert max_row_rel_err(to_host(y)[:R], want) <= TOL["bf16"]


def test_fp8mm_down_rejects_unsupported_shapes(gpu):
    z = torch.zeros(1 << 16, dtype=torch.float32, device=gpu)
    D = _desc(64, 256, 192, 8, 2, 0, 8, "bf16")                 # f not a multiple of 128
    with pytest.raises(moe.MoeError):
        moe.expert_down_fp8mm(D, z, z, z, z, z, z)
    D = _desc(64, 256, 128, 8, 2, 0, 8, "f32")
    with pytest.raises(moe.MoeError):
        moe.expert_down_fp8mm(D, z, z, z, z, z, z)


def test_fp8mm_down_at_full_size_sampled(gpu):
    # The 1T share (T = 8192, d = 6144, 96 of 384 experts, f = 1792) in the
    # benchmark's launch configuration; the oracle quantises and multiplies
    # only what the sampled rows need (their h rows and their experts' W2).
    cfg = synth.CONFIGS["share_1t"]
    d, f, E, k, e0, NL = cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local
    print(f"[fp8mm down full size] T={cfg.T} d={d} f={f} E={E} NL={NL}", flush=True)
    inp, h, off, R, (hq, hs, w2q, w2s), y = _down_case(cfg, gpu, False, 3)
    rs = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(6).choice(R, 6, replace=False)]))
    seg = np.searchsorted(off, rs, side="right") - 1
    want = []
    for r, n in zip(rs, seg):
        hr = oracle.fp8_dequantize_blocks_pow2(*oracle.fp8_quantize_blocks_pow2(h[r]))
        w2n = synth.as_f32(inp["w2"][n], "bf16")
        wn = oracle.fp8_dequantize_blocks_pow2(*oracle.fp8_quantize_blocks_pow2(w2n)).reshape(d, f)
        want.append(oracle.expert_down(hr[None, :], np.array([0, 1]), wn[None])[0])
    got = to_host(y[torch.as_tensor(rs, device=y.device)])
    assert max_row_rel_err(got, np.array(want)) <= TOL["bf16"]


@pytest.mark.parametrize("scale", [
    dict(T=600, d=512, f=256, E=32, num_local=8, expert_begin=8),
    dict(T=700, d=512, f=1792, E=16, num_local=16, expert_begin=0),
])
def test_fp8mm_forward_layer_matches_the_oracle(gpu, scale):
    # The whole forward with both expert products on the FP8 matrix cores, as
    # the FP8 benchmark workload runs it: x, W1, W3, W2 and h quantised to
    # E4M3 with power-of-two block scales.  The oracle quantises at the same
    # points: x and the weights as given, and its own H after rounding it to
    # bf16.  The GPU's h is the bf16 rounding of its own G and U, an ulp away
    # from the oracle's here and there, and a value that sits near a code
    # boundary then takes the neighbouring code: a full code step where the
    # quantisation itself moves a value by at most half a step.  So y is held
    # to the bf16 bound plus twice the quantisation's own effect on y, q (the
    # oracle's y on quantised H against its y on the bf16 H); h itself, and
    # each product on identical codes (the tests above), meet the bf16 bound.
    cfg = synth.scaled(synth.CONFIGS["share_1t"], **scale)
    T, d, f, E, k, e0, NL = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.expert_begin, cfg.num_local
    print(f"[fp8mm layer] {scale}", flush=True)
    inp = synth.make_inputs(cfg, want=("x", "w1", "w3", "w2"))
    rng = np.random.default_rng(T + f)
    idx = random_routing(rng, T, E, k)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    D = _desc(T, d, f, E, k, e0, NL, "bf16")
    b = moe.Buffers(D, gather=True)
    moe.permute(D, to_dev(idx), None, b.counts, b.offsets, b.row_token, b.slot_row, None, b.ws_permute)
    xq, xs = _quant_pow2(to_dev(inp["x"]), gpu)
    wq = {n: _quant_pow2(to_dev(inp[n]), gpu) for n in ("w1", "w3")}
    moe.expert_gate_up_fp8mm(D, b.offsets, b.row_token, xq, xs, wq["w1"][0], wq["w1"][1], wq["w3"][0],
                             wq["w3"][1], None, b.h)
    S8 = moe.fp8_scale_row_bytes(f)
    hq = torch.empty(D.R_cap, f, dtype=torch.uint8, device=gpu)
    hs = torch.empty(D.R_cap, S8, dtype=torch.uint8, device=gpu)
    moe.fp8_quantize_pow2_rows(b.h, hq, hs, b.offsets[NL:])
    w2q = torch.empty(NL * d, f, dtype=torch.uint8, device=gpu)
    w2s = torch.empty(NL * d, S8, dtype=torch.uint8, device=gpu)
    moe.fp8_quantize_pow2_rows(to_dev(inp["w2"]).view(NL * d, f), w2q, w2s)
    moe.expert_down_fp8mm(D, b.offsets, hq, hs, w2q, w2s, b.y_perm)
    moe.combine(D, b.slot_row, to_dev(w), b.y_perm, b.y)
    torch.cuda.synchronize()
    deq = {}
    for n in ("x", "w1", "w3", "w2"):
        a = synth.as_f32(inp[n], "bf16")
        deq[n] = oracle.fp8_dequantize_blocks_pow2(*oracle.fp8_quantize_blocks_pow2(a)).reshape(a.shape)
    _, off = oracle.count_tokens(idx, E, e0, NL)
    rows, slot = oracle.generate_indices(idx, e0, NL, off)
    R = int(off[-1])
    _, _, H, _ = oracle.expert_ffn(oracle.permute(deq["x"], rows), off, deq["w1"], deq["w3"], np.zeros((NL, d, f)))
    assert max_row_rel_err(to_host(b.h)[:R], H) <= TOL["bf16"]
    Hb = oracle.bf16_round(H)
    Hq = oracle.fp8_dequantize_blocks_pow2(*oracle.fp8_quantize_blocks_pow2(Hb)).reshape(R, f)
    y = oracle.combine(oracle.expert_down(Hq, off, deq["w2"]), slot, w)
    q = max_row_rel_err(oracle.combine(oracle.expert_down(Hb, off, deq["w2"]), slot, w), y)
    err = max_row_rel_err(to_host(b.y), y)
    print(f"[fp8mm layer] y error {err:.4f}, quantisation effect q {q:.4f}", flush=True)
    assert err <= TOL["bf16"] + 2 * q
