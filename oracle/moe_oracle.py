"""Plain float64 CPU oracle of the MoE expert layer, forward and backward.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  It shares no code, header, table or helper with
the HIP library under mixture_experts_layer_02_amd/, and neither imports the
other.

Sources ("the pages"):
  [Aurora] "Scalable Pretraining of Large Mixture of Experts Language Models on
           Aurora Super Computer": section 3.1 (FastSparseMoE), its Algorithm 1
           (FastSparseMoEBlock with expert parallelism, stages 1-5) and Figure 5.
  [Domyn]  "Training a 1T-Params MoE on EU public infrastructure": the model
           table (hidden 6144, 384 routed experts, top-8, expert hidden 1792)
           and the sections on group-limited expert routing and on the FP8
           expert weight all-gather.

Arithmetic: every input is widened to float64 and every step runs in float64
with no intermediate rounding.  Matrix products use numpy's matmul as a
library step; everything else is written out as its definition.

Readings taken where the pages leave a step open (each is also listed in the
design notes):
  * Selection is made on the logits (softmax is strictly increasing, so the
    selected set equals the top-k of the probabilities), ties go to the lower
    expert index, +0.0 and -0.0 compare equal, and slot j holds the j-th
    selection in that order.
  * renormalize=1 (the default): the top-k probabilities are divided by their
    sum.  renormalize=0 keeps Algorithm 1's literal TopK(Softmax(logits)).
  * Local experts are the block [e0, e0 + NL).  Selections of other experts
    are counted but produce no row; their slots contribute nothing to y.
  * Rows of one expert's segment are in ascending token order (the order that
    Algorithm 1's blocked count/index kernels produce).
  * No capacity limit, no biases in the experts; the router may get an added
    per-expert logit bias (the Zipf-skewed workload).
  * The backward pass is not written out on the pages beyond stage 5; it is
    derived here by differentiating stages 1, 4 and 5.

Every function is pinned by a test in tests/test_oracle_*.py against brute
force, closed forms, invariants or finite differences; none is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "router_logits", "topk_route", "topk_route_grouped", "fp8_e4m3_decode", "fp8_e4m3_encode",
    "fp8_quantize_blocks", "fp8_dequantize_blocks", "fp8_quantize_blocks_pow2", "fp8_dequantize_blocks_pow2", "bf16_round", "count_tokens", "generate_indices", "permute",
    "silu", "silu_grad", "expert_ffn_rows", "expert_ffn", "expert_down", "combine",
    "combine_bwd", "expert_ffn_bwd_rows", "expert_ffn_bwd", "unpermute_bwd",
    "route_bwd", "router_bwd", "layer_forward", "layer_backward",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Stage 1 of Algorithm 1 [Aurora]: router, softmax, top-k.
# --------------------------------------------------------------------------

def router_logits(x, wr, bias=None):
    """logits[t][e] = sum_i x[t][i] * W_r[e][i]  (+ bias[e]).

    [Aurora] Algorithm 1, stage 1: the router is a linear layer mapping each of
    the tokens to one logit per expert.  W_r is stored out x in, i.e. [E][d].
    """
    L = _f64(x) @ _f64(wr).T
    if bias is not None:
        L = L + _f64(bias)[None, :]
    return L


def topk_route(logits, k, renormalize=1):
    """Per token: the k experts with the largest logits, and their weights.

    [Aurora] Algorithm 1, stage 1: probs = Softmax(logits); weights, indices =
    TopK(probs).  Returns idx [T][k] int32 (slot j = j-th largest, ties to the
    lower expert index) and w [T][k] float64: the softmax probabilities of the
    selected experts, divided by their sum when ``renormalize`` is 1.
    """
    L = _f64(logits)
    if not np.isfinite(L).all():
        raise ValueError("oracle: logits must be finite")
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("oracle: need 1 <= k <= E")
    # A stable sort of the negated logits keeps equal logits (including +0.0
    # against -0.0) in ascending expert order.
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    # Softmax over all experts, written out.
    z = np.exp(L - L.max(axis=1, keepdims=True))
    probs = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


def topk_route_grouped(logits, k, n_groups, renormalize=1):
    """Group-limited top-k: the same number of experts from every group.

    [Domyn] section "Group-limited expert routing": the E experts form
    n_groups groups of E/n_groups consecutive experts (one group per
    expert-parallel rank; 384 = 4 x 96 there), and the router takes k/n_groups
    experts from each group (2 per group at top-8), so that every group, and
    so every rank, receives exactly T*k/n_groups rows.  Within a group the
    experts taken are the group's best by the same order as topk_route (logit
    descending, lower index first on ties); the slots then hold all k taken
    experts in that order, and the weights are computed from the selection
    exactly as in topk_route (softmax probabilities of the selected experts,
    divided by their sum when ``renormalize`` is 1).
    """
    L = _f64(logits)
    if not np.isfinite(L).all():
        raise ValueError("oracle: logits must be finite")
    T, E = L.shape
    G = int(n_groups)
    if G < 1 or E % G or k % G or not 1 <= k <= E:
        raise ValueError("oracle: need n_groups dividing both E and k")
    Eg, kg = E // G, k // G
    chosen = []
    for g in range(G):
        block = L[:, g * Eg:(g + 1) * Eg]
        best = np.argsort(-block, axis=1, kind="stable")[:, :kg]
        chosen.append(best + g * Eg)
    sel = np.sort(np.concatenate(chosen, axis=1), axis=1)          # ascending expert index
    vals = np.take_along_axis(L, sel, axis=1)
    idx = np.take_along_axis(sel, np.argsort(-vals, axis=1, kind="stable"), axis=1).astype(np.int32)
    z = np.exp(L - L.max(axis=1, keepdims=True))
    probs = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


# --------------------------------------------------------------------------
# FP8 expert weights [Domyn] ("FP8 expert weight all-gather"): blocks of 128
# consecutive values, each scaled to the E4M3 range and cast, with one
# float32 scale per block; dequantised to bf16 before the expert GEMMs.
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def fp8_e4m3_decode(codes):
    """Value of every E4M3 code (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 is subnormal, m/8 * 2^-6; the code with
    all exponent and mantissa bits set is NaN; there is no infinity)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(x):
    """The E4M3 code nearest to each x (|x| <= 448), ties to an even mantissa.

    Positive codes are ordered like their values, and on each binade
    [2^e, 2^(e+1)) (e >= -6) the codes step by 2^(e-3); below 2^-6 they step by
    2^-9 (subnormals).  So the code is the binade's first code plus the
    rounded number of steps, and a carry into the next binade falls out of the
    contiguous numbering.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or not np.isfinite(x).all():
        raise ValueError("oracle: E4M3 input out of range")
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                                  # subnormals share the step of binade -6
    step = 2.0 ** (e - 3.0)
    steps = np.rint(a / step)                                # round half to even
    first = np.where(a < 2.0 ** -6, 0.0, (e + 7.0) * 8.0)    # code of 2^e (binade e >= -6)
    base = np.where(a < 2.0 ** -6, 0.0, 2.0 ** e)
    code = np.where(a < 2.0 ** -6, steps, first + (steps - base / step))
    code = code.astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)      # -0 and tiny negatives keep the sign


def fp8_quantize_blocks(w, block=128):
    """codes [n] uint8 and scales [n/block] float32 of w [n] (any shape, flattened).

    Per block: amax = max |w| (float32); scale = amax / 448 and inv = 448 / amax,
    both rounded to float32; each value is w * inv in float32, clamped to
    [-448, 448] (the product may exceed 448 by a rounding) and encoded to the
    nearest E4M3 code.  An all-zero block has scale 0 and all-zero codes.
    """
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    if w.size % block:
        raise ValueError("oracle: size must be a multiple of the block")
    wb = w.reshape(-1, block)
    amax = np.abs(wb).max(axis=1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    scale = np.where(nz, safe / np.float32(E4M3_MAX), np.float32(0)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    xs = (wb * inv[:, None]).astype(np.float32)
    xs = np.clip(xs, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = np.where(nz[:, None], fp8_e4m3_encode(xs), 0).astype(np.uint8)
    return codes.reshape(-1), scale


def bf16_round(v):
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32)


def fp8_dequantize_blocks(codes, scales, block=128):
    """bf16 weights (as float32 values) from codes and per-block scales:
    decode(code) * scale in float32, rounded to bf16."""
    dec = fp8_e4m3_decode(codes).astype(np.float32).reshape(-1, block)
    v = (dec * np.asarray(scales, np.float32)[:, None]).astype(np.float32)
    return bf16_round(v).reshape(-1)


def fp8_quantize_blocks_pow2(w, block=128):
    """codes [n] uint8 and power-of-two block scales [n/block] of w [n] (any
    shape, flattened), each scale given as its biased exponent e + 127 (the
    E8M0 byte: scale = 2^(byte - 127)).

    [Domyn] FP8 expert weights: blocks of 128 values scaled into the E4M3
    range and cast, one scale per block.  This form takes as the scale the
    smallest power of two 2^e with amax <= 448 * 2^e, so that the block
    maximum lands in (224, 448] and the scaling itself is exact; it is the
    scale a block-scaled FP8 matrix instruction applies (activations are
    quantised the same way, in blocks of 128 along a row).  Each value
    w * 2^-e is encoded to the nearest E4M3 code.  An all-zero block has
    e = 0 and zero codes (the sign of -0 is kept).
    """
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    if w.size % block:
        raise ValueError("oracle: size must be a multiple of the block")
    wb = w.reshape(-1, block).astype(np.float64)
    amax = np.abs(wb).max(axis=1)
    nz = amax > 0
    # amax = f 2^x with f in [0.5, 1), and 448 2^e = 0.875 2^(e+9): the least
    # e is x - 9 when f <= 0.875, else x - 8.
    f, x = np.frexp(np.where(nz, amax, 1.0))
    e = np.where(f <= 0.875, x - 9, x - 8)
    e = np.where(nz, e, 0).astype(np.int64)
    if np.any(e < -127) or np.any(e > 127):
        raise ValueError("oracle: block scale outside the E8M0 range")
    xs = wb * np.ldexp(1.0, -e)[:, None]                     # exact: a power of two
    codes = fp8_e4m3_encode(xs).astype(np.uint8)
    return codes.reshape(-1), (e + 127).astype(np.uint8)


def fp8_dequantize_blocks_pow2(codes, e8, block=128):
    """Values decode(code) * 2^(e8 - 127) of fp8_quantize_blocks_pow2's
    output, exactly (float64)."""
    dec = fp8_e4m3_decode(codes).reshape(-1, block)
    return (dec * np.ldexp(1.0, np.asarray(e8, np.int64) - 127)[:, None]).reshape(-1)


# --------------------------------------------------------------------------
# Stages 2 and 3 of Algorithm 1 [Aurora]: token counting, prefix sums and
# index generation, written as their plain definition (a stable counting sort
# of the local (token, slot) selections by expert).
# --------------------------------------------------------------------------

def _check_distinct(idx):
    """A token's k selections are k distinct experts (the top-k of stage 1
    never repeats one); a routing that repeats an expert is rejected."""
    for t, row in enumerate(np.asarray(idx).reshape(len(idx), -1)):
        if len(set(int(e) for e in row)) != len(row):
            raise ValueError(f"token {t} lists an expert more than once: {row.tolist()}")


def count_tokens(idx, E, e0, NL):
    """counts[e] for every expert e, and the local boundaries offsets[0..NL].

    [Aurora] Algorithm 1, stage 2: the per-expert token counts of the experts
    held locally, followed by a prefix sum that gives each expert's segment
    boundaries (cum_token_counts).  counts covers all E experts (selections
    of non-local experts are counted too); offsets[n] is the number of
    selections of local experts e0 .. e0+n-1, so offsets[NL] is the number of
    routed rows R.
    """
    idx = np.asarray(idx)
    _check_distinct(idx)
    counts = np.zeros(E, np.int64)
    for e in idx.reshape(-1):
        counts[int(e)] += 1
    offsets = np.zeros(NL + 1, np.int64)
    for n in range(NL):
        offsets[n + 1] = offsets[n] + counts[e0 + n]
    return counts, offsets


def generate_indices(idx, e0, NL, offsets):
    """row_token[R] and slot_row[T][k] of the permuted (expert-major) layout.

    [Aurora] Algorithm 1, stage 3: each selection of a local expert gets a row
    in that expert's segment; input_indices maps the row to its token and
    output_indices maps the token's local selection back to the row.
    Here slot_row[t][j] is the row of slot j of token t, or -1 when the slot's
    expert is not local; row_token[row] = t.  Tokens are visited in ascending
    order, so every segment lists its tokens in ascending order.
    """
    idx = np.asarray(idx)
    _check_distinct(idx)
    T, k = idx.shape
    R = int(offsets[NL])
    next_row = [int(offsets[n]) for n in range(NL)]
    row_token = np.full(R, -1, np.int64)
    slot_row = np.full((T, k), -1, np.int64)
    for t in range(T):
        for j in range(k):
            n = int(idx[t, j]) - e0
            if 0 <= n < NL:
                row = next_row[n]
                next_row[n] += 1
                row_token[row] = t
                slot_row[t, j] = row
    return row_token, slot_row


def permute(x, row_token):
    """mlp_in[row] = x[row_token[row]] ([Aurora] Algorithm 1, stage 4 gather)."""
    return np.asarray(x)[np.asarray(row_token, np.int64)]


# --------------------------------------------------------------------------
# Stage 4 of Algorithm 1 [Aurora]: the SwiGLU expert MLP on each segment.
# --------------------------------------------------------------------------

def silu(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    g = _f64(g)
    return g / (1.0 + np.exp(-g))


def silu_grad(g):
    """d silu / dg = s * (1 + g * (1 - s)) with s = sigmoid(g)."""
    g = _f64(g)
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def expert_ffn_rows(xr, w1e, w3e, w2e):
    """One expert's MLP on rows xr [m][d]: gate, up, silu(gate)*up, down.

    [Aurora] Algorithm 1, stage 4: gate_out = X W_gate, up_out = X W_up,
    mul_out = Silu(gate_out) * up_out, mlp_out = mul_out W_down, with the
    weights of a linear layer (out x in): w1e, w3e [f][d], w2e [d][f].
    """
    X = _f64(xr)
    G = X @ _f64(w1e).T
    U = X @ _f64(w3e).T
    H = silu(G) * U
    Y = H @ _f64(w2e).T
    return G, U, H, Y


def expert_ffn(x_perm, offsets, w1, w3, w2):
    """Stage 4 over all local experts: segment n is rows offsets[n]:offsets[n+1].

    [Aurora] Algorithm 1, stage 4 (Grouped_mm over the concatenated per-rank
    expert weights with the cum_token_counts boundaries).
    Returns G, U, H [R][f] and y_perm [R][d].
    """
    x_perm = _f64(x_perm)
    NL = len(offsets) - 1
    R = int(offsets[NL])
    f = np.asarray(w1).shape[1]
    d = np.asarray(w1).shape[2]
    G = np.zeros((R, f))
    U = np.zeros((R, f))
    H = np.zeros((R, f))
    Y = np.zeros((R, d))
    for n in range(NL):
        a, b = int(offsets[n]), int(offsets[n + 1])
        if b > a:
            G[a:b], U[a:b], H[a:b], Y[a:b] = expert_ffn_rows(x_perm[a:b], w1[n], w3[n], w2[n])
    return G, U, H, Y


def expert_down(h_perm, offsets, w2):
    """The down projection of stage 4 alone: y_perm[r] = h_perm[r] W_down^T
    with the weights of the expert whose segment holds row r.

    [Aurora] Algorithm 1, stage 4 (mlp_out = mul_out W_down, one Grouped_mm
    over the cum_token_counts segments); expert_ffn computes the same product
    after gate/up and SwiGLU.  h_perm [R][f], w2 [NL][d][f]; returns [R][d].
    """
    h_perm = _f64(h_perm)
    NL = len(offsets) - 1
    R = int(offsets[NL])
    d = np.asarray(w2).shape[1]
    Y = np.zeros((R, d))
    for n in range(NL):
        a, b = int(offsets[n]), int(offsets[n + 1])
        if b > a:
            Y[a:b] = h_perm[a:b] @ _f64(w2[n]).T
    return Y


# --------------------------------------------------------------------------
# Stage 5 of Algorithm 1 [Aurora]: weighted output reduction.
# --------------------------------------------------------------------------

def combine(y_perm, slot_row, w):
    """y[t] = sum over local slots j (ascending) of w[t][j] * y_perm[slot_row[t][j]].

    [Aurora] Algorithm 1, stage 5, ExpertOutputReductionForward: each output
    element accumulates the token's locally computed expert outputs scaled by
    their routing weights.  A token with no local slot gets y = 0.
    """
    y_perm = _f64(y_perm)
    w = _f64(w)
    slot_row = np.asarray(slot_row)
    T, k = slot_row.shape
    y = np.zeros((T, y_perm.shape[1]))
    for j in range(k):
        rows = slot_row[:, j]
        m = rows >= 0
        y[m] += w[m, j][:, None] * y_perm[rows[m]]
    return y


def combine_bwd(dy, y_perm, slot_row, w):
    """dy_perm[row] = w[t][j] dy[t];  dw[t][j] = <y_perm[row], dy[t]> (0 if non-local).

    [Aurora] Algorithm 1, stage 5, ExpertOutputReductionBackward (with the
    row/token indices read as the forward defines them).
    """
    dy = _f64(dy)
    y_perm = _f64(y_perm)
    w = _f64(w)
    slot_row = np.asarray(slot_row)
    T, k = slot_row.shape
    dy_perm = np.zeros_like(y_perm)
    dw = np.zeros((T, k))
    for j in range(k):
        rows = slot_row[:, j]
        m = rows >= 0
        t = np.nonzero(m)[0]
        dy_perm[rows[m]] = w[t, j][:, None] * dy[t]
        dw[t, j] = np.einsum("rd,rd->r", y_perm[rows[m]], dy[t])
    return dy_perm, dw


# --------------------------------------------------------------------------
# Backward of stage 4 (derived by differentiating the expert MLP).
# --------------------------------------------------------------------------

def expert_ffn_bwd_rows(xr, w1e, w3e, w2e, dyr):
    """Gradients of one expert's MLP for rows xr with upstream dyr [m][d].

    dH = dY W2, dU = dH * silu(G), dG = dH * U * silu'(G), dX = dG W1 + dU W3,
    dW1 = dG^T X, dW3 = dU^T X, dW2 = dY^T H (weights out x in).
    """
    X = _f64(xr)
    dY = _f64(dyr)
    G, U, H, _ = expert_ffn_rows(X, w1e, w3e, w2e)
    dH = dY @ _f64(w2e)
    dU = dH * silu(G)
    dG = dH * U * silu_grad(G)
    dX = dG @ _f64(w1e) + dU @ _f64(w3e)
    dW1 = dG.T @ X
    dW3 = dU.T @ X
    dW2 = dY.T @ H
    return dG, dU, dX, dW1, dW3, dW2


def expert_ffn_bwd(x_perm, offsets, w1, w3, w2, dy_perm):
    """Backward of stage 4 over all local experts.

    Returns dG, dU [R][f], dx_perm [R][d], dW1, dW3 [NL][f][d], dW2 [NL][d][f].
    An expert with no rows gets exactly zero weight gradients.
    """
    x_perm = _f64(x_perm)
    dy_perm = _f64(dy_perm)
    NL = len(offsets) - 1
    R = int(offsets[NL])
    NLw, f, d = np.asarray(w1).shape
    dG = np.zeros((R, f))
    dU = np.zeros((R, f))
    dX = np.zeros((R, d))
    dW1 = np.zeros((NLw, f, d))
    dW3 = np.zeros((NLw, f, d))
    dW2 = np.zeros((NLw, d, f))
    for n in range(NL):
        a, b = int(offsets[n]), int(offsets[n + 1])
        if b > a:
            dG[a:b], dU[a:b], dX[a:b], dW1[n], dW3[n], dW2[n] = expert_ffn_bwd_rows(
                x_perm[a:b], w1[n], w3[n], w2[n], dy_perm[a:b])
    return dG, dU, dX, dW1, dW3, dW2


def unpermute_bwd(dx_perm, slot_row):
    """dx[t] = sum over local slots j of dx_perm[slot_row[t][j]] (adjoint of the gather)."""
    dx_perm = _f64(dx_perm)
    slot_row = np.asarray(slot_row)
    T, k = slot_row.shape
    dx = np.zeros((T, dx_perm.shape[1]))
    for j in range(k):
        rows = slot_row[:, j]
        m = rows >= 0
        dx[m] += dx_perm[rows[m]]
    return dx


# --------------------------------------------------------------------------
# Backward of stage 1 (derived).
# --------------------------------------------------------------------------

def route_bwd(idx, w, dw, E, renormalize=1, logits=None):
    """dlogits [T][E] from the gradient dw [T][k] of the routing weights.

    renormalize=1: w_j = exp(L_j) / sum_{i in S} exp(L_i) over the selected set
    S, so dL_m = w_m (dw_m - <w, dw>) for m in S and 0 elsewhere (including
    selected experts that are not local: their dw is 0 but the normaliser
    still couples them).
    renormalize=0: w_j = p_{idx_j} with p the softmax over all E, so
    dL_e = p_e (g_e - <w, dw>) with g_e = dw_j where e = idx_j, else 0; this
    needs the logits.
    """
    idx = np.asarray(idx, np.int64)
    w = _f64(w)
    dw = _f64(dw)
    T, k = idx.shape
    s = (w * dw).sum(axis=1)
    dL = np.zeros((T, E))
    if renormalize:
        for j in range(k):
            dL[np.arange(T), idx[:, j]] = w[:, j] * (dw[:, j] - s)
    else:
        L = _f64(logits)
        z = np.exp(L - L.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        g = np.zeros((T, E))
        for j in range(k):
            g[np.arange(T), idx[:, j]] = dw[:, j]
        dL = p * (g - s[:, None])
    return dL


def router_bwd(x, wr, dlogits):
    """dx_router = dlogits W_r  [T][d];  dW_r = dlogits^T x  [E][d]."""
    dL = _f64(dlogits)
    return dL @ _f64(wr), dL.T @ _f64(x)


# --------------------------------------------------------------------------
# The whole layer.
# --------------------------------------------------------------------------

def layer_forward(x, wr, w1, w3, w2, k, e0, NL, renormalize=1, bias=None,
                  logits=None, routing=None, n_groups=1):
    """Stages 1-5 on one GPU's share.  Returns a dict of every intermediate.

    ``logits`` (optional) replaces stage 1's matmul, so that routing can be
    taken from a given logit tensor; ``routing=(idx, w)`` (optional) replaces
    stage 1 altogether (forced routing); ``n_groups`` > 1 selects with the
    group-limited rule (topk_route_grouped).
    """
    out = {}
    E = np.asarray(wr).shape[0]
    if routing is not None:
        idx, w = routing
        idx = np.asarray(idx, np.int32)
        w = _f64(w)
    else:
        L = router_logits(x, wr, bias) if logits is None else _f64(logits)
        out["logits"] = L
        if n_groups > 1:
            idx, w = topk_route_grouped(L, k, n_groups, renormalize)
        else:
            idx, w = topk_route(L, k, renormalize)
    out["idx"], out["w"] = idx, w
    counts, offsets = count_tokens(idx, E, e0, NL)
    row_token, slot_row = generate_indices(idx, e0, NL, offsets)
    out.update(counts=counts, offsets=offsets, row_token=row_token, slot_row=slot_row)
    x_perm = permute(_f64(x), row_token)
    G, U, H, Yp = expert_ffn(x_perm, offsets, w1, w3, w2)
    out.update(x_perm=x_perm, G=G, U=U, H=H, y_perm=Yp)
    out["y"] = combine(Yp, slot_row, w)
    return out


def layer_backward(fwd, x, wr, w1, w3, w2, dy, renormalize=1):
    """Gradients of <dy, y> with the routing (idx) held fixed.

    Returns dict with dy_perm, dw, dG, dU, dx_perm, dW1, dW3, dW2, dlogits,
    dx (expert path + router path) and dWr.
    """
    E = np.asarray(wr).shape[0]
    dy_perm, dw = combine_bwd(dy, fwd["y_perm"], fwd["slot_row"], fwd["w"])
    dG, dU, dXp, dW1, dW3, dW2 = expert_ffn_bwd(fwd["x_perm"], fwd["offsets"], w1, w3, w2, dy_perm)
    dx_moe = unpermute_bwd(dXp, fwd["slot_row"])
    dL = route_bwd(fwd["idx"], fwd["w"], dw, E, renormalize, fwd.get("logits"))
    dx_r, dWr = router_bwd(x, wr, dL)
    return dict(dy_perm=dy_perm, dw=dw, dG=dG, dU=dU, dx_perm=dXp, dW1=dW1, dW3=dW3,
                dW2=dW2, dlogits=dL, dx_router=dx_r, dx=dx_moe + dx_r, dWr=dWr)
