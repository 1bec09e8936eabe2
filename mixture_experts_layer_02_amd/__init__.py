"""Python binding of libmoe.so, the MI355X MoE expert-layer library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The
functions mirror the C ABI in include/moe.h one to one; ``Buffers``,
``forward`` and ``backward`` allocate the tensors of one layer pass and chain
the entry points in order.

There is no fallback: if libmoe.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported before libmoe.so so that the process holds one HIP runtime

__all__ = [
    "MoeError", "MoeDesc", "lib", "make_desc", "new_tile_counters", "SCHEDULE_STATIC", "SCHEDULE_DYNAMIC", "workspace_size", "router_logits", "route", "route_grouped", "hold_cus", "fp8_quantize", "fp8_dequantize", "permute", "permute_noalloc", "expert_gate_up_gather", "grouped_ffn_bwd_dw_gather", "expert_gate_up_fp8", "expert_down_fp8", "fp8_quantize_pow2", "expert_gate_up_fp8mm", "fp8_quantize_pow2_rows", "expert_down_fp8mm", "fp8_scale_row_bytes", "row_weights", "dtopk_w_from_parts", "dtopk_parts",
    "grouped_ffn", "expert_gate_up", "expert_down", "expert_bwd_dh", "expert_bwd_dx", "expert_bwd_dw_gate_up", "expert_bwd_dw_down", "combine_bwd_gather", "expert_bwd_dh_gather", "expert_bwd_dw_down_gather", "combine", "combine_bwd", "grouped_ffn_bwd_dx", "grouped_ffn_bwd_dw",
    "unpermute_bwd", "unpermute_router_bwd", "route_bwd", "router_bwd", "router_bwd_acc", "Buffers", "forward", "backward",
    "MOE_F32", "MOE_BF16",
]

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
OP_ROUTER_LOGITS, OP_PERMUTE, OP_GROUPED_FFN, OP_FFN_BWD_DX, OP_FFN_BWD_DW, OP_ROUTER_BWD = range(6)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

_vp = ctypes.c_void_p
SCHEDULE_STATIC, SCHEDULE_DYNAMIC = 0, 1
_sz = ctypes.c_size_t


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("T", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("f", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("expert_begin", ctypes.c_int32),
        ("num_local", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("tile_schedule", ctypes.c_int32),
        ("tile_counters", ctypes.c_void_p),
        ("wgrad_dtype", ctypes.c_int32),
    ]

    @property
    def R_cap(self) -> int:
        return self.T * min(self.k, self.num_local)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == MOE_BF16 else torch.float32


class MoeError(RuntimeError):
    def __init__(self, fn, rc):
        l = lib()
        msg = l.moe_status_str(rc).decode()
        if rc == MOE_ERR_HIP:
            msg += ": " + l.moe_last_error().decode()
        super().__init__(f"{fn} failed ({rc}): {msg}")
        self.rc = rc


# name -> argtypes (after the leading const moe_desc*)
_SIGS = {
    "moe_router_logits": [_vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_route": [_vp, _vp, _vp, _vp],
    "moe_route_grouped": [_vp, ctypes.c_int, _vp, _vp, _vp],
    "moe_permute": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_permute_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_grouped_ffn": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_expert_gate_up": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_gate_up_gather": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_gate_up_fp8": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_down_fp8": [_vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_gate_up_fp8mm": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_down_fp8mm": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_grouped_ffn_bwd_dw_gather": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_down": [_vp, _vp, _vp, _vp, _vp],
    "moe_expert_bwd_dh": [_vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_bwd_dx": [_vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_bwd_dw_gate_up": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_bwd_dw_down": [_vp, _vp, _vp, _vp, _vp],
    "moe_combine_bwd_gather": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_bwd_dh_gather": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_row_weights": [_vp, _vp, _vp, _vp],
    "moe_dtopk_w_from_parts": [_vp, _vp, _vp, _vp],
    "moe_expert_bwd_dw_down_gather": [_vp, _vp, _vp, _vp, _vp, _vp],
    "moe_combine": [_vp, _vp, _vp, _vp, _vp],
    "moe_combine_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_grouped_ffn_bwd_dx": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_grouped_ffn_bwd_dw": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_unpermute_bwd": [_vp, _vp, _vp, _vp, _vp],
    "moe_route_bwd": [_vp, _vp, _vp, _vp, _vp, _vp],
    "moe_router_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_router_bwd_acc": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_unpermute_router_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
}
EXPORTS = sorted(list(_SIGS) + ["moe_workspace_size", "moe_status_str", "moe_last_error", "moe_hold_cus",
                                 "moe_fp8_quantize", "moe_fp8_dequantize", "moe_fp8_quantize_pow2",
                                 "moe_fp8_quantize_pow2_rows"])

_lib = None


def lib():
    """Load libmoe.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = [ctypes.POINTER(MoeDesc)] + args
            fn.restype = ctypes.c_int
        l.moe_workspace_size.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        l.moe_workspace_size.restype = ctypes.c_int
        l.moe_status_str.argtypes = [ctypes.c_int]
        l.moe_status_str.restype = ctypes.c_char_p
        l.moe_fp8_quantize.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, _vp, _vp, _vp]
        l.moe_fp8_quantize.restype = ctypes.c_int
        l.moe_fp8_dequantize.argtypes = [_vp, _vp, ctypes.c_int64, _vp, _vp]
        l.moe_fp8_quantize_pow2.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, _vp, _vp, _vp]
        l.moe_fp8_quantize_pow2.restype = ctypes.c_int
        l.moe_fp8_quantize_pow2_rows.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp,
                                                 ctypes.c_int64, _vp]
        l.moe_fp8_quantize_pow2_rows.restype = ctypes.c_int
        l.moe_fp8_dequantize.restype = ctypes.c_int
        l.moe_hold_cus.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]
        l.moe_hold_cus.restype = ctypes.c_int
        l.moe_last_error.argtypes = []
        l.moe_last_error.restype = ctypes.c_char_p
        _lib = l
    return _lib


def make_desc(T, d, f, E, k, expert_begin=0, num_local=None, dtype=MOE_BF16, renormalize=1,
              tile_counters=None, wgrad_dtype=MOE_F32) -> MoeDesc:
    """The layer descriptor.  ``tile_counters`` (a zeroed int32 device tensor of
    16 elements, see new_tile_counters) selects the dynamic tile order of the
    grouped GEMMs; the descriptor keeps a reference to it.  ``wgrad_dtype``:
    the type of the expert weight gradients dW1, dW3, dW2 ("f32" or "bf16")."""
    if isinstance(dtype, str):
        dtype = MOE_BF16 if dtype == "bf16" else MOE_F32
    if isinstance(wgrad_dtype, str):
        wgrad_dtype = MOE_BF16 if wgrad_dtype == "bf16" else MOE_F32
    D = MoeDesc(ctypes.sizeof(MoeDesc), T, d, f, E, k, expert_begin, E if num_local is None else num_local,
                dtype, renormalize, SCHEDULE_STATIC, None, wgrad_dtype)
    if tile_counters is not None:
        if tile_counters.dtype != torch.int32 or tile_counters.numel() < 16 or not tile_counters.is_cuda:
            raise ValueError("tile_counters must be an int32 device tensor of 16 elements")
        D.tile_schedule = SCHEDULE_DYNAMIC
        D.tile_counters = tile_counters.data_ptr()
        D._tile_counters = tile_counters
    return D


def new_tile_counters(device="cuda"):
    """Zeroed counters for the dynamic tile order (every GEMM leaves them zero)."""
    return torch.zeros(16, dtype=torch.int32, device=device)


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("libmoe needs contiguous tensors")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _call(name, desc, *args):
    rc = getattr(lib(), name)(ctypes.byref(desc), *[_p(a) for a in args])
    if rc != MOE_OK:
        raise MoeError(name, rc)


def workspace_size(desc: MoeDesc, op: int) -> int:
    n = ctypes.c_size_t(0)
    rc = lib().moe_workspace_size(ctypes.byref(desc), op, ctypes.byref(n))
    if rc != MOE_OK:
        raise MoeError("moe_workspace_size", rc)
    return n.value


def _ws(ws):
    return (None, 0) if ws is None else (ws, ws.numel() * ws.element_size())


def router_logits(desc, x, wr, bias, logits, ws=None):
    if ws is None:  # a workspace of the queried size, when the shape needs one
        need = workspace_size(desc, OP_ROUTER_LOGITS)
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device) if need else None
    w, n = _ws(ws)
    _call("moe_router_logits", desc, x, wr, bias, logits, w, n, _stream())


def route(desc, logits, topk_idx, topk_w):
    _call("moe_route", desc, logits, topk_idx, topk_w, _stream())


def fp8_quantize(w, q, scales):
    """Blockwise-128 E4M3 codes q (uint8, w's size) and float32 scales (size/128) of w (bf16 or fp32)."""
    dt = MOE_BF16 if w.dtype == torch.bfloat16 else MOE_F32
    for t in (w, q, scales):
        if not t.is_contiguous():
            raise ValueError("libmoe needs contiguous tensors")
    rc = lib().moe_fp8_quantize(w.data_ptr(), dt, w.numel(), q.data_ptr(), scales.data_ptr(), _stream())
    if rc != MOE_OK:
        raise MoeError("moe_fp8_quantize", rc)


def fp8_quantize_pow2(w, q, e8):
    """E4M3 codes q (uint8, w's size) and power-of-two block scales e8 (uint8 E8M0 bytes, size/128) of w."""
    dt = MOE_BF16 if w.dtype == torch.bfloat16 else MOE_F32
    for t in (w, q, e8):
        if not t.is_contiguous():
            raise ValueError("libmoe needs contiguous tensors")
    rc = lib().moe_fp8_quantize_pow2(w.data_ptr(), dt, w.numel(), q.data_ptr(), e8.data_ptr(), _stream())
    if rc != MOE_OK:
        raise MoeError("moe_fp8_quantize_pow2", rc)


def fp8_scale_row_bytes(n):
    """Bytes per row of E8M0 block scales for rows of n codes, as the FP8 GEMMs read them."""
    return (n // 128 + 3) // 4 * 4


def fp8_quantize_pow2_rows(w, q, e8, nrows=None):
    """fp8_quantize_pow2 by rows of w [rows][cols]: codes q [rows][cols] and
    scales e8 [rows][e8_ld] (e8_ld = e8's row length, the bytes past cols/128
    zero); rows at or past the device int32 nrows (if given) are left alone."""
    dt = MOE_BF16 if w.dtype == torch.bfloat16 else MOE_F32
    for t in (w, q, e8):
        if not t.is_contiguous():
            raise ValueError("libmoe needs contiguous tensors")
    rows, cols = w.shape
    rc = lib().moe_fp8_quantize_pow2_rows(w.data_ptr(), dt, rows, cols, None if nrows is None else nrows.data_ptr(),
                                          q.data_ptr(), e8.data_ptr(), e8.shape[-1], _stream())
    if rc != MOE_OK:
        raise MoeError("moe_fp8_quantize_pow2_rows", rc)


def expert_down_fp8mm(desc, offsets, hq, hs, w2q, w2s, y_perm):
    """down on the FP8 matrix cores: h and W2 as codes with E8M0 block scales in rows of fp8_scale_row_bytes(f)."""
    _call("moe_expert_down_fp8mm", desc, offsets, hq, hs, w2q, w2s, y_perm, _stream())


def expert_gate_up_fp8mm(desc, offsets, row_token, xq, xs, w1q, w1s, w3q, w3s, gu, h):
    """gate/up + SwiGLU on the FP8 matrix cores: x and W1/W3 as codes with E8M0 block scales."""
    _call("moe_expert_gate_up_fp8mm", desc, offsets, row_token, xq, xs, w1q, w1s, w3q, w3s, gu, h, _stream())


def fp8_dequantize(q, scales, w):
    """bf16 weights w (q's size) = decode(q) * scale of each 128-value block."""
    for t in (w, q, scales):
        if not t.is_contiguous():
            raise ValueError("libmoe needs contiguous tensors")
    rc = lib().moe_fp8_dequantize(q.data_ptr(), scales.data_ptr(), q.numel(), w.data_ptr(), _stream())
    if rc != MOE_OK:
        raise MoeError("moe_fp8_dequantize", rc)


def hold_cus(workgroups, microseconds, lds_bytes=96 * 1024, stream=None):
    """Occupy `workgroups` compute units for `microseconds` (measurement aid:
    a stand-in for another kernel, such as a collective, holding part of the
    GPU while a grouped GEMM runs)."""
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = lib().moe_hold_cus(int(workgroups), int(lds_bytes), int(microseconds), s)
    if rc != MOE_OK:
        raise MoeError("moe_hold_cus", rc)


def route_grouped(desc, logits, n_groups, topk_idx, topk_w):
    _call("moe_route_grouped", desc, logits, int(n_groups), topk_idx, topk_w, _stream())


def permute(desc, topk_idx, x, counts, offsets, row_token, slot_row, x_perm, ws):
    w, n = _ws(ws)
    _call("moe_permute", desc, topk_idx, x, counts, offsets, row_token, slot_row, x_perm, w, n, _stream())


def permute_noalloc(desc, topk_idx, x, counts, offsets, row_token, slot_row, x_perm):
    """moe_permute with the library's fixed device scratch instead of a workspace."""
    _call("moe_permute_noalloc", desc, topk_idx, x, counts, offsets, row_token, slot_row, x_perm, _stream())


def grouped_ffn(desc, offsets, x_perm, w1, w3, w2, gu, h, y_perm, ws=None):
    w, n = _ws(ws)
    _call("moe_grouped_ffn", desc, offsets, x_perm, w1, w3, w2, gu, h, y_perm, w, n, _stream())


def expert_gate_up(desc, offsets, x_perm, w1, w3, gu, h):
    _call("moe_expert_gate_up", desc, offsets, x_perm, w1, w3, gu, h, _stream())


def expert_gate_up_gather(desc, offsets, row_token, x, w1, w3, gu, h):
    _call("moe_expert_gate_up_gather", desc, offsets, row_token, x, w1, w3, gu, h, _stream())


def grouped_ffn_bwd_dw_gather(desc, offsets, row_token, x, h, dgu, dy_perm, dw1, dw3, dw2):
    _call("moe_grouped_ffn_bwd_dw_gather", desc, offsets, row_token, x, h, dgu, dy_perm, dw1, dw3, dw2,
          _stream())


def expert_gate_up_fp8(desc, offsets, row_token, a, w1q, w1s, w3q, w3s, gu, h):
    """gate/up on FP8 weights (codes + block scales); row_token None: `a` is x_perm, else x."""
    _call("moe_expert_gate_up_fp8", desc, offsets, row_token, a, w1q, w1s, w3q, w3s, gu, h, _stream())


def expert_down_fp8(desc, offsets, h, w2q, w2s, y_perm):
    _call("moe_expert_down_fp8", desc, offsets, h, w2q, w2s, y_perm, _stream())


def expert_down(desc, offsets, h, w2, y_perm):
    _call("moe_expert_down", desc, offsets, h, w2, y_perm, _stream())


def expert_bwd_dh(desc, offsets, w2, gu, dy_perm, dgu):
    _call("moe_expert_bwd_dh", desc, offsets, w2, gu, dy_perm, dgu, _stream())


def expert_bwd_dx(desc, offsets, w1, w3, dgu, dx_perm):
    _call("moe_expert_bwd_dx", desc, offsets, w1, w3, dgu, dx_perm, _stream())


def expert_bwd_dw_gate_up(desc, offsets, row_token, a, dgu, dw1, dw3):
    """dW1 | dW3 alone; row_token None: `a` is x_perm, else x (read through row_token)."""
    _call("moe_expert_bwd_dw_gate_up", desc, offsets, row_token, a, dgu, dw1, dw3, _stream())


def expert_bwd_dw_down(desc, offsets, dy_perm, h, dw2):
    _call("moe_expert_bwd_dw_down", desc, offsets, dy_perm, h, dw2, _stream())


def combine_bwd_gather(desc, slot_row, topk_w, y_perm, dy, row_w, dtopk_w):
    """dtopk_w and the per-row routing weights row_w; no dy_perm."""
    _call("moe_combine_bwd_gather", desc, slot_row, topk_w, y_perm, dy, row_w, dtopk_w, _stream())


def expert_bwd_dh_gather(desc, offsets, row_token, row_w, dy, w2, gu, dgu, hw, dtopk_part=None):
    """dH from dy read through row_token, scaled by row_w, SwiGLU backward -> dgu; hw = row_w silu(G) U;
    dtopk_part: the rows' partial sums of (dy W2) silu(G) U (dtopk_parts(desc) per row)."""
    _call("moe_expert_bwd_dh_gather", desc, offsets, row_token, row_w, dy, w2, gu, dgu, hw, dtopk_part, _stream())


def dtopk_parts(desc):
    """Partial sums per row written by expert_bwd_dh_gather: two per 256-wide n-tile of f."""
    return 2 * ((desc.f + 255) // 256)


def row_weights(desc, slot_row, topk_w, row_w):
    """row_w[slot_row[t][j]] = topk_w[t][j] for every local slot."""
    _call("moe_row_weights", desc, slot_row, topk_w, row_w, _stream())


def dtopk_w_from_parts(desc, slot_row, dtopk_part, dtopk_w):
    """dtopk_w[t][j] = the sum of slot j's row's partial sums (0 for a non-local slot)."""
    _call("moe_dtopk_w_from_parts", desc, slot_row, dtopk_part, dtopk_w, _stream())


def expert_bwd_dw_down_gather(desc, offsets, row_token, dy, hw, dw2):
    """dW2 from dy read through row_token and hw."""
    _call("moe_expert_bwd_dw_down_gather", desc, offsets, row_token, dy, hw, dw2, _stream())


def combine(desc, slot_row, topk_w, y_perm, y):
    _call("moe_combine", desc, slot_row, topk_w, y_perm, y, _stream())


def combine_bwd(desc, slot_row, topk_w, y_perm, dy, dy_perm, dtopk_w):
    _call("moe_combine_bwd", desc, slot_row, topk_w, y_perm, dy, dy_perm, dtopk_w, _stream())


def grouped_ffn_bwd_dx(desc, offsets, w1, w3, w2, gu, dy_perm, dgu, dx_perm, ws=None):
    w, n = _ws(ws)
    _call("moe_grouped_ffn_bwd_dx", desc, offsets, w1, w3, w2, gu, dy_perm, dgu, dx_perm, w, n, _stream())


def grouped_ffn_bwd_dw(desc, offsets, x_perm, h, dgu, dy_perm, dw1, dw3, dw2, ws=None):
    w, n = _ws(ws)
    _call("moe_grouped_ffn_bwd_dw", desc, offsets, x_perm, h, dgu, dy_perm, dw1, dw3, dw2, w, n, _stream())


def unpermute_bwd(desc, slot_row, dx_perm, dx_add, dx):
    _call("moe_unpermute_bwd", desc, slot_row, dx_perm, dx_add, dx, _stream())


def unpermute_router_bwd(desc, slot_row, dx_perm, topk_idx, dlogits, wr, dx):
    _call("moe_unpermute_router_bwd", desc, slot_row, dx_perm, topk_idx, dlogits, wr, dx, _stream())


def route_bwd(desc, logits, topk_idx, topk_w, dtopk_w, dlogits):
    _call("moe_route_bwd", desc, logits, topk_idx, topk_w, dtopk_w, dlogits, _stream())


def router_bwd(desc, x, wr, dlogits, dx_router, dwr, ws):
    w, n = _ws(ws)
    _call("moe_router_bwd", desc, x, wr, dlogits, dx_router, dwr, w, n, _stream())


def router_bwd_acc(desc, x, wr, dlogits, dx, dwr, ws):
    w, n = _ws(ws)
    _call("moe_router_bwd_acc", desc, x, wr, dlogits, dx, dwr, w, n, _stream())


class Buffers:
    """Every device tensor of one forward (+ backward) pass of a layer, allocated once."""

    def __init__(self, desc: MoeDesc, device="cuda", backward=False, gather=False, gather_dy=None):
        """gather=True: the expert GEMMs read x through row_token (no x_perm).
        gather_dy (default: gather) = True: the backward reads dy through
        row_token (no dy_perm) and keeps the per-row routing weights row_w and
        hw = row_w silu(G) U instead."""
        dt = desc.torch_dtype
        T, d, f, E, k, NL, Rc = desc.T, desc.d, desc.f, desc.E, desc.k, desc.num_local, desc.R_cap
        z = dict(device=device)
        i32 = torch.int32
        self.desc = desc
        self.logits = torch.empty(T, E, dtype=torch.float32, **z)
        self.topk_idx = torch.empty(T, k, dtype=i32, **z)
        self.topk_w = torch.empty(T, k, dtype=torch.float32, **z)
        self.counts = torch.empty(E, dtype=i32, **z)
        self.offsets = torch.empty(NL + 1, dtype=i32, **z)
        self.row_token = torch.empty(Rc, dtype=i32, **z)
        self.slot_row = torch.empty(T, k, dtype=i32, **z)
        self.gather = gather
        self.gather_dy = gather if gather_dy is None else gather_dy
        gdy = self.gather_dy
        self.x_perm = None if gather else torch.empty(Rc, d, dtype=dt, **z)
        self.gu = torch.empty(Rc, 2 * f, dtype=dt, **z) if backward else None
        self.h = torch.empty(Rc, f, dtype=dt, **z)
        self.y_perm = torch.empty(Rc, d, dtype=dt, **z)
        self.y = torch.empty(T, d, dtype=dt, **z)
        self.ws_permute = torch.empty(max(16, workspace_size(desc, OP_PERMUTE)), dtype=torch.uint8, **z)
        self.ws_router = torch.empty(max(16, workspace_size(desc, OP_ROUTER_LOGITS)), dtype=torch.uint8, **z)
        if backward:
            self.dy_perm = None if gdy else torch.empty(Rc, d, dtype=dt, **z)
            self.row_w = torch.empty(Rc, dtype=torch.float32, **z) if gdy else None
            self.hw = torch.empty(Rc, f, dtype=dt, **z) if gdy else None
            self.dtopk_part = torch.empty(Rc, dtopk_parts(desc), dtype=torch.float32, **z) if gdy else None
            self.dtopk_w = torch.empty(T, k, dtype=torch.float32, **z)
            self.dgu = torch.empty(Rc, 2 * f, dtype=dt, **z)
            self.dx_perm = torch.empty(Rc, d, dtype=dt, **z)
            wdt = torch.bfloat16 if desc.wgrad_dtype == MOE_BF16 else torch.float32
            self.dW1 = torch.empty(NL, f, d, dtype=wdt, **z)
            self.dW3 = torch.empty(NL, f, d, dtype=wdt, **z)
            self.dW2 = torch.empty(NL, d, f, dtype=wdt, **z)
            self.dlogits = torch.empty(T, E, dtype=torch.float32, **z)
            self.dWr = torch.empty(E, d, dtype=torch.float32, **z)
            self.dx = torch.empty(T, d, dtype=dt, **z)
            self.ws_router_bwd = torch.empty(max(16, workspace_size(desc, OP_ROUTER_BWD)), dtype=torch.uint8, **z)


def forward(b: Buffers, x, wr, w1, w3, w2, bias=None, routing=None, n_groups=1):
    """Stages A1-A7.  ``routing=(topk_idx, topk_w)`` device tensors skip A1-A2;
    ``n_groups`` > 1 routes with the group-limited rule (route_grouped)."""
    D = b.desc
    if routing is None:
        router_logits(D, x, wr, bias, b.logits, b.ws_router)
        if n_groups > 1:
            route_grouped(D, b.logits, n_groups, b.topk_idx, b.topk_w)
        else:
            route(D, b.logits, b.topk_idx, b.topk_w)
        idx, w = b.topk_idx, b.topk_w
    else:
        idx, w = routing
    if b.gather:
        permute(D, idx, None, b.counts, b.offsets, b.row_token, b.slot_row, None, b.ws_permute)
        expert_gate_up_gather(D, b.offsets, b.row_token, x, w1, w3, b.gu, b.h)
        expert_down(D, b.offsets, b.h, w2, b.y_perm)
    else:
        permute(D, idx, x, b.counts, b.offsets, b.row_token, b.slot_row, b.x_perm, b.ws_permute)
        grouped_ffn(D, b.offsets, b.x_perm, w1, w3, w2, b.gu, b.h, b.y_perm)
    combine(D, b.slot_row, w, b.y_perm, b.y)
    return b.y


def backward(b: Buffers, x, wr, w1, w3, w2, dy, routing=None, fuse_router_dx=True):
    """Stages B1-B5 for upstream gradient dy (needs Buffers(backward=True)).
    fuse_router_dx: with renormalised weights, the router's share of dx is
    added in the unpermute pass (unpermute_router_bwd) instead of by the
    dx += dlogits Wr product."""
    D = b.desc
    idx, w = (b.topk_idx, b.topk_w) if routing is None else routing
    if b.gather_dy:
        # dtopk_w = <dy, y_perm> = <dy W2, h>: the row weights first, the dot
        # products as partial sums inside dH (y_perm is not read)
        row_weights(D, b.slot_row, w, b.row_w)
        expert_bwd_dh_gather(D, b.offsets, b.row_token, b.row_w, dy, w2, b.gu, b.dgu, b.hw, b.dtopk_part)
        dtopk_w_from_parts(D, b.slot_row, b.dtopk_part, b.dtopk_w)
        expert_bwd_dx(D, b.offsets, w1, w3, b.dgu, b.dx_perm)
        if b.gather:
            expert_bwd_dw_gate_up(D, b.offsets, b.row_token, x, b.dgu, b.dW1, b.dW3)
        else:
            expert_bwd_dw_gate_up(D, b.offsets, None, b.x_perm, b.dgu, b.dW1, b.dW3)
        expert_bwd_dw_down_gather(D, b.offsets, b.row_token, dy, b.hw, b.dW2)
    elif b.gather:
        combine_bwd(D, b.slot_row, w, b.y_perm, dy, b.dy_perm, b.dtopk_w)
        grouped_ffn_bwd_dx(D, b.offsets, w1, w3, w2, b.gu, b.dy_perm, b.dgu, b.dx_perm)
        grouped_ffn_bwd_dw_gather(D, b.offsets, b.row_token, x, b.h, b.dgu, b.dy_perm, b.dW1, b.dW3, b.dW2)
    else:
        combine_bwd(D, b.slot_row, w, b.y_perm, dy, b.dy_perm, b.dtopk_w)
        grouped_ffn_bwd_dx(D, b.offsets, w1, w3, w2, b.gu, b.dy_perm, b.dgu, b.dx_perm)
        grouped_ffn_bwd_dw(D, b.offsets, b.x_perm, b.h, b.dgu, b.dy_perm, b.dW1, b.dW3, b.dW2)
    if routing is None and fuse_router_dx and D.renormalize:
        route_bwd(D, b.logits, idx, w, b.dtopk_w, b.dlogits)
        unpermute_router_bwd(D, b.slot_row, b.dx_perm, idx, b.dlogits, wr, b.dx)
        router_bwd_acc(D, x, wr, b.dlogits, None, b.dWr, b.ws_router_bwd)
        return b.dx
    unpermute_bwd(D, b.slot_row, b.dx_perm, None, b.dx)
    if routing is None:
        route_bwd(D, b.logits, idx, w, b.dtopk_w, b.dlogits)
        router_bwd_acc(D, x, wr, b.dlogits, b.dx, b.dWr, b.ws_router_bwd)
    return b.dx
