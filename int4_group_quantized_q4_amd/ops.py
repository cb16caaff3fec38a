"""Python binding of libw4a16.so: same names and arguments as include/w4a16.h,
with torch device tensors in place of pointers.  Argument marshalling only --
every computation runs in the library's HIP kernels on the given stream
(default: torch's current stream).

A few allocating helpers (``repack``, ``dequant``, ``pack_codes``,
``linear``, ``moe_route``, ``moe_layer``) create the output tensors with
torch and then make the same calls.
"""

import contextlib
import ctypes

import torch

from . import _lib
from ._lib import (W4_EPI_NONE, W4_EPI_GEGLU_TANH, W4_EPI_SWIGLU, W4_OUT_BF16, W4_OUT_F32,
                   check, lib)

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t, name, dtypes=None, nullable=False):
    if t is None:
        if nullable:
            return None
        raise ValueError("%s must not be None" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ----------------------------------------------------------------- raw calls
def q4_group_repack(w, qweight, scales, group_status=None, counters=None, stream=None):
    rows, K = w.shape
    st = lib().q4_group_repack(
        _ptr(w, "w", _BF16_LIKE), rows, K, _ptr(qweight, "qweight", (torch.uint8,)),
        _ptr(scales, "scales", _BF16_LIKE), _ptr(group_status, "group_status", (torch.uint8,), True),
        _ptr(counters, "counters", (torch.int64,), True), _stream(stream))
    check(st, "q4_group_repack")


def q4_group_dequant_f32(qweight, scales, rows, K, out, stream=None):
    st = lib().q4_group_dequant_f32(
        _ptr(qweight, "qweight", (torch.uint8,)), _ptr(scales, "scales", _BF16_LIKE), rows, K,
        _ptr(out, "out", (torch.float32,)), _stream(stream))
    check(st, "q4_group_dequant_f32")


def q4_pack_codes(codes, qweight, stream=None):
    rows, K = codes.shape
    st = lib().q4_pack_codes(_ptr(codes, "codes", (torch.int8,)), rows, K,
                             _ptr(qweight, "qweight", (torch.uint8,)), _stream(stream))
    check(st, "q4_pack_codes")


def q4_pack_scales(scales, rows, K, scales_tiled, stream=None):
    st = lib().q4_pack_scales(_ptr(scales, "scales", _BF16_LIKE), rows, K,
                              _ptr(scales_tiled, "scales_tiled", _BF16_LIKE), _stream(stream))
    check(st, "q4_pack_scales")


def w4a16_set_gemm_kernel(kernel):
    """Process-wide GEMM kernel choice (W4_KERNEL_*); returns the previous one."""
    prev = lib().w4a16_set_gemm_kernel(int(kernel))
    if prev < 0:
        check(prev, "w4a16_set_gemm_kernel")
    return prev


@contextlib.contextmanager
def gemm_kernel(kernel):
    """Run the enclosed calls with the given W4_KERNEL_* choice, then restore."""
    prev = w4a16_set_gemm_kernel(kernel)
    try:
        yield
    finally:
        w4a16_set_gemm_kernel(prev)


def _ws(ws):
    return (_ptr(ws, "ws", None, True), 0 if ws is None else ws.numel() * ws.element_size())


def w4a16_linear_workspace(M, K, N):
    return int(lib().w4a16_linear_workspace(M, K, N))


def w4a16_linear(x, qweight, scales, N, y, ws=None, stream=None):
    M, K = x.shape
    wp, wn = _ws(ws)
    st = lib().w4a16_linear(_ptr(x, "x", _BF16_LIKE), M, K, _ptr(qweight, "qweight", (torch.uint8,)),
                            _ptr(scales, "scales", _BF16_LIKE), N, _ptr(y, "y", _BF16_LIKE), wp, wn, _stream(stream))
    check(st, "w4a16_linear")


def w4a16_moe_route_workspace(T, E, k):
    return int(lib().w4a16_moe_route_workspace(T, E, k))


def w4a16_moe_route(logits, k, topk_ids, topk_weights, expert_offsets, sorted_rows, sorted_tokens,
                    row_to_sorted, ws, stream=None):
    T, E = logits.shape
    i32 = (torch.int32,)
    st = lib().w4a16_moe_route(
        _ptr(logits, "logits", (torch.float32,)), T, E, k, _ptr(topk_ids, "topk_ids", i32),
        _ptr(topk_weights, "topk_weights", (torch.float32,)), _ptr(expert_offsets, "expert_offsets", i32),
        _ptr(sorted_rows, "sorted_rows", i32), _ptr(sorted_tokens, "sorted_tokens", i32),
        _ptr(row_to_sorted, "row_to_sorted", i32), _ptr(ws, "ws", None, True), ws.numel() * ws.element_size(),
        _stream(stream))
    check(st, "w4a16_moe_route")


def w4a16_moe_gmm_workspace(x_rows, R, E, K, N):
    return int(lib().w4a16_moe_gmm_workspace(x_rows, R, E, K, N))


def w4a16_moe_gmm(x, row_index, expert_offsets, E, R, K, N, qweight, scales, epilogue, out, out_dtype,
                  ws=None, stream=None):
    wp, wn = _ws(ws)
    st = lib().w4a16_moe_gmm(
        _ptr(x, "x", _BF16_LIKE), x.shape[0], _ptr(row_index, "row_index", (torch.int32,), True),
        _ptr(expert_offsets, "expert_offsets", (torch.int32,)), E, R, K, N,
        _ptr(qweight, "qweight", (torch.uint8,)), _ptr(scales, "scales", _BF16_LIKE), epilogue,
        _ptr(out, "out", (torch.float32,) + _BF16_LIKE), out_dtype, wp, wn, _stream(stream))
    check(st, "w4a16_moe_gmm")


def moe_gmm(x, row_index, expert_offsets, E, R, K, N, qweight, scales, epilogue, out, out_dtype, stream=None):
    """w4a16_moe_gmm with a freshly allocated workspace."""
    ws = torch.empty(max(16, w4a16_moe_gmm_workspace(x.shape[0], R, E, K, N)), dtype=torch.uint8, device=x.device)
    w4a16_moe_gmm(x, row_index, expert_offsets, E, R, K, N, qweight, scales, epilogue, out, out_dtype, ws, stream)


def w4a16_moe_combine(o, o_dtype, row_to_sorted, topk_weights, T, k, N, y, stream=None):
    st = lib().w4a16_moe_combine(
        _ptr(o, "o", (torch.float32,) + _BF16_LIKE), o_dtype, _ptr(row_to_sorted, "row_to_sorted", (torch.int32,)),
        _ptr(topk_weights, "topk_weights", (torch.float32,)), T, k, N, _ptr(y, "y", _BF16_LIKE), _stream(stream))
    check(st, "w4a16_moe_combine")


def w4a16_moe_layer_workspace(T, E, k, d, I):
    return int(lib().w4a16_moe_layer_workspace(T, E, k, d, I))


def w4a16_moe_layer_plan(T, E, k, d, I):
    arr = (ctypes.c_size_t * 9)()
    check(lib().w4a16_moe_layer_plan(T, E, k, d, I, arr), "w4a16_moe_layer_plan")
    return [int(v) for v in arr]


def w4a16_moe_layer(x, logits, k, I, w1_q, w1_s, w2_q, w2_s, activation, y, ws, stream=None):
    T, d = x.shape
    E = logits.shape[1]
    st = lib().w4a16_moe_layer(
        _ptr(x, "x", _BF16_LIKE), _ptr(logits, "logits", (torch.float32,)), T, E, k, d, I,
        _ptr(w1_q, "w1_q", (torch.uint8,)), _ptr(w1_s, "w1_s", _BF16_LIKE), _ptr(w2_q, "w2_q", (torch.uint8,)),
        _ptr(w2_s, "w2_s", _BF16_LIKE), activation, _ptr(y, "y", _BF16_LIKE), _ptr(ws, "ws", (torch.uint8,)),
        ws.numel(), _stream(stream))
    check(st, "w4a16_moe_layer")


# -------------------------------------------------------- allocating helpers
def repack(w, stream=None):
    """bf16 [rows, K] -> (qweight uint8 [rows*K/2], scales bf16 [rows*K/32]
    (tile16 scale layout), status uint8 [rows, K/32], counters int64 [2])."""
    rows, K = w.shape
    dev = w.device
    qweight = torch.empty(rows * K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(rows * K // 32, dtype=torch.bfloat16, device=dev)
    status = torch.empty(rows, K // 32, dtype=torch.uint8, device=dev)
    counters = torch.zeros(2, dtype=torch.int64, device=dev)
    q4_group_repack(w, qweight, scales, status, counters, stream)
    return qweight, scales, status, counters


def dequant(qweight, scales, rows, K, stream=None):
    out = torch.empty(rows, K, dtype=torch.float32, device=qweight.device)
    q4_group_dequant_f32(qweight, scales, rows, K, out, stream)
    return out


def pack_codes(codes, stream=None):
    rows, K = codes.shape
    qweight = torch.empty(rows * K // 2, dtype=torch.uint8, device=codes.device)
    q4_pack_codes(codes, qweight, stream)
    return qweight


def pack_scales(scales, stream=None):
    """plain bf16 [rows, K/32] -> tile16 scale layout (flat, rows*K/32)."""
    rows, G = scales.shape
    out = torch.empty(rows * G, dtype=scales.dtype, device=scales.device)
    q4_pack_scales(scales, rows, G * 32, out, stream)
    return out


def linear(x, qweight, scales, N, stream=None):
    M, K = x.shape
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    ws = torch.empty(max(16, w4a16_linear_workspace(M, K, N)), dtype=torch.uint8, device=x.device)
    w4a16_linear(x, qweight, scales, N, y, ws, stream)
    return y


def moe_route(logits, k, stream=None):
    T, E = logits.shape
    dev = logits.device
    R = T * k
    plan = {
        "topk_ids": torch.empty(T, k, dtype=torch.int32, device=dev),
        "topk_weights": torch.empty(T, k, dtype=torch.float32, device=dev),
        "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted_rows": torch.empty(R, dtype=torch.int32, device=dev),
        "sorted_tokens": torch.empty(R, dtype=torch.int32, device=dev),
        "row_to_sorted": torch.empty(R, dtype=torch.int32, device=dev),
    }
    ws = torch.empty(max(16, w4a16_moe_route_workspace(T, E, k)), dtype=torch.uint8, device=dev)
    w4a16_moe_route(logits, k, plan["topk_ids"], plan["topk_weights"], plan["expert_offsets"],
                    plan["sorted_rows"], plan["sorted_tokens"], plan["row_to_sorted"], ws, stream)
    return plan


def moe_layer(x, logits, k, I, w1_q, w1_s, w2_q, w2_s, activation=W4_EPI_GEGLU_TANH, ws=None, stream=None):
    """Whole MoE layer; returns (y, views) where views expose the routing plan
    and the intermediates left in the workspace."""
    T, d = x.shape
    E = logits.shape[1]
    need = w4a16_moe_layer_workspace(T, E, k, d, I)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    w4a16_moe_layer(x, logits, k, I, w1_q, w1_s, w2_q, w2_s, activation, y, ws, stream)
    p = w4a16_moe_layer_plan(T, E, k, d, I)
    R = T * k

    def view(i, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[p[i]:p[i] + nbytes].view(dt)

    views = {
        "topk_ids": view(0, R, torch.int32).view(T, k),
        "topk_weights": view(1, R, torch.float32).view(T, k),
        "expert_offsets": view(2, E + 1, torch.int32),
        "sorted_rows": view(3, R, torch.int32),
        "sorted_tokens": view(4, R, torch.int32),
        "row_to_sorted": view(5, R, torch.int32),
        "a": view(7, R * I, torch.bfloat16).view(R, I),
        "o": view(8, R * d, torch.float32).view(R, d),
    }
    return y, views
