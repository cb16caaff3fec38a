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


def _bytes(t):
    return t.numel() * t.element_size()


def _need(t, name, nbytes, device=None):
    """Raise ValueError unless tensor t (if given) holds at least nbytes and
    lives on `device`.  The library sees only pointers, so an undersized
    buffer would become an out-of-bounds device access: this check runs
    before any launch."""
    if t is None:
        return
    if _bytes(t) < nbytes:
        raise ValueError("%s holds %d bytes, the call needs %d" % (name, _bytes(t), nbytes))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _dims(*vals):
    for v in vals:
        if int(v) < 0:
            raise ValueError("sizes must be non-negative")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ----------------------------------------------------------------- raw calls
def q4_group_repack(w, qweight, scales, group_status=None, counters=None, stream=None):
    rows, K = w.shape
    d = w.device
    _need(qweight, "qweight", rows * K // 2, d)
    _need(scales, "scales", rows * K // 32 * 2, d)
    _need(group_status, "group_status", rows * K // 32, d)
    _need(counters, "counters", 16, d)
    st = lib().q4_group_repack(
        _ptr(w, "w", _BF16_LIKE), rows, K, _ptr(qweight, "qweight", (torch.uint8,)),
        _ptr(scales, "scales", _BF16_LIKE), _ptr(group_status, "group_status", (torch.uint8,), True),
        _ptr(counters, "counters", (torch.int64,), True), _stream(stream))
    check(st, "q4_group_repack")


def q4_group_dequant_f32(qweight, scales, rows, K, out, stream=None):
    _dims(rows, K)
    d = qweight.device
    _need(scales, "scales", rows * K // 32 * 2, d)
    _need(qweight, "qweight", rows * K // 2, d)
    _need(out, "out", rows * K * 4, d)
    st = lib().q4_group_dequant_f32(
        _ptr(qweight, "qweight", (torch.uint8,)), _ptr(scales, "scales", _BF16_LIKE), rows, K,
        _ptr(out, "out", (torch.float32,)), _stream(stream))
    check(st, "q4_group_dequant_f32")


def q4_pack_codes(codes, qweight, stream=None):
    rows, K = codes.shape
    _need(qweight, "qweight", rows * K // 2, codes.device)
    st = lib().q4_pack_codes(_ptr(codes, "codes", (torch.int8,)), rows, K,
                             _ptr(qweight, "qweight", (torch.uint8,)), _stream(stream))
    check(st, "q4_pack_codes")


def q4_pack_scales(scales, rows, K, scales_tiled, stream=None):
    _dims(rows, K)
    _need(scales, "scales", rows * K // 32 * 2)
    _need(scales_tiled, "scales_tiled", rows * K // 32 * 2, scales.device)
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
    _dims(N)
    d = x.device
    _need(qweight, "qweight", N * K // 2, d)
    _need(scales, "scales", N * K // 32 * 2, d)
    _need(y, "y", M * N * 2, d)
    _need(ws, "ws", 0, d)
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
    d = logits.device
    R = T * k
    for t, name in ((topk_ids, "topk_ids"), (topk_weights, "topk_weights"), (sorted_rows, "sorted_rows"),
                    (sorted_tokens, "sorted_tokens"), (row_to_sorted, "row_to_sorted")):
        _need(t, name, R * 4, d)
    _need(expert_offsets, "expert_offsets", (E + 1) * 4, d)
    _need(ws, "ws", 0, d)
    wp, wn = _ws(ws)
    st = lib().w4a16_moe_route(
        _ptr(logits, "logits", (torch.float32,)), T, E, k, _ptr(topk_ids, "topk_ids", i32),
        _ptr(topk_weights, "topk_weights", (torch.float32,)), _ptr(expert_offsets, "expert_offsets", i32),
        _ptr(sorted_rows, "sorted_rows", i32), _ptr(sorted_tokens, "sorted_tokens", i32),
        _ptr(row_to_sorted, "row_to_sorted", i32), wp, wn, _stream(stream))
    check(st, "w4a16_moe_route")


def w4a16_moe_topk(logits, k, topk_ids, topk_weights, stream=None):
    T, E = logits.shape
    d = logits.device
    _need(topk_ids, "topk_ids", T * k * 4, d)
    _need(topk_weights, "topk_weights", T * k * 4, d)
    st = lib().w4a16_moe_topk(_ptr(logits, "logits", (torch.float32,)), T, E, k,
                              _ptr(topk_ids, "topk_ids", (torch.int32,)),
                              _ptr(topk_weights, "topk_weights", (torch.float32,)), _stream(stream))
    check(st, "w4a16_moe_topk")


def w4a16_moe_gmm_ids(x, topk_ids, T, k, row_div, E, K, N, qweight, scales, epilogue, out, out_dtype, stream=None):
    _dims(T, k, E, K, N)
    if row_div not in (1, k):
        raise ValueError("row_div must be 1 or k")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [rows, K=%d], got %s" % (K, tuple(x.shape)))
    d = x.device
    _need(x, "x", (T * k // row_div) * K * 2, d)
    _need(topk_ids, "topk_ids", T * k * 4, d)
    _need(qweight, "qweight", E * N * K // 2, d)
    _need(scales, "scales", E * N * K // 32 * 2, d)
    ncol = N // 2 if epilogue in (W4_EPI_GEGLU_TANH, W4_EPI_SWIGLU) else N
    _need(out, "out", T * k * ncol * (4 if out_dtype == W4_OUT_F32 else 2), d)
    st = lib().w4a16_moe_gmm_ids(
        _ptr(x, "x", _BF16_LIKE), _ptr(topk_ids, "topk_ids", (torch.int32,)), T, k, row_div, E, K, N,
        _ptr(qweight, "qweight", (torch.uint8,)), _ptr(scales, "scales", _BF16_LIKE), epilogue,
        _ptr(out, "out", (torch.float32,) + _BF16_LIKE), out_dtype, _stream(stream))
    check(st, "w4a16_moe_gmm_ids")


def w4a16_moe_gmm_logits(x, logits, k, K, N, qweight, scales, epilogue, out, topk_ids, topk_weights, stream=None):
    """Gate/up matmul of a decode batch with its rows (and the top-k plan,
    written to topk_ids / topk_weights) from the router logits [T][E]."""
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    _dims(T, E, k, K, N)
    if x.dim() != 2 or x.shape[0] != T or x.shape[1] != K:
        raise ValueError("x must be [T=%d, K=%d], got %s" % (T, K, tuple(x.shape)))
    d = x.device
    _need(logits, "logits", T * E * 4, d)
    _need(qweight, "qweight", E * N * K // 2, d)
    _need(scales, "scales", E * N * K // 32 * 2, d)
    _need(out, "out", T * k * (N // 2) * 2, d)
    _need(topk_ids, "topk_ids", T * k * 4, d)
    _need(topk_weights, "topk_weights", T * k * 4, d)
    st = lib().w4a16_moe_gmm_logits(
        _ptr(x, "x", _BF16_LIKE), _ptr(logits, "logits", (torch.float32,)), T, E, k, K, N,
        _ptr(qweight, "qweight", (torch.uint8,)), _ptr(scales, "scales", _BF16_LIKE), epilogue,
        _ptr(out, "out", _BF16_LIKE), _ptr(topk_ids, "topk_ids", (torch.int32,)),
        _ptr(topk_weights, "topk_weights", (torch.float32,)), _stream(stream))
    check(st, "w4a16_moe_gmm_logits")


def w4a16_moe_gmm_workspace(x_rows, R, E, K, N):
    return int(lib().w4a16_moe_gmm_workspace(x_rows, R, E, K, N))


def w4a16_moe_gmm(x, row_index, expert_offsets, E, R, K, N, qweight, scales, epilogue, out, out_dtype,
                  ws=None, stream=None):
    _dims(E, R, K, N)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [x_rows, K=%d], got %s" % (K, tuple(x.shape)))
    d = x.device
    _need(row_index, "row_index", R * 4, d)
    _need(expert_offsets, "expert_offsets", (E + 1) * 4, d)
    _need(qweight, "qweight", E * N * K // 2, d)
    _need(scales, "scales", E * N * K // 32 * 2, d)
    ncol = N // 2 if epilogue in (W4_EPI_GEGLU_TANH, W4_EPI_SWIGLU) else N
    if out_dtype == W4_OUT_F32 and out.dtype != torch.float32:
        raise TypeError("out must be float32 for W4_OUT_F32")
    if out_dtype == W4_OUT_BF16 and out.dtype not in _BF16_LIKE:
        raise TypeError("out must be bf16 for W4_OUT_BF16")
    _need(out, "out", R * ncol * (4 if out_dtype == W4_OUT_F32 else 2), d)
    _need(ws, "ws", 0, d)
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
    _dims(T, k, N)
    d = o.device
    if o_dtype == W4_OUT_F32 and o.dtype != torch.float32:
        raise TypeError("o must be float32 for W4_OUT_F32")
    if o_dtype == W4_OUT_BF16 and o.dtype not in _BF16_LIKE:
        raise TypeError("o must be bf16 for W4_OUT_BF16")
    _need(o, "o", T * k * N * o.element_size(), d)
    _need(row_to_sorted, "row_to_sorted", T * k * 4, d)
    _need(topk_weights, "topk_weights", T * k * 4, d)
    _need(y, "y", T * N * 2, d)
    st = lib().w4a16_moe_combine(
        _ptr(o, "o", (torch.float32,) + _BF16_LIKE), o_dtype, _ptr(row_to_sorted, "row_to_sorted", (torch.int32,)),
        _ptr(topk_weights, "topk_weights", (torch.float32,)), T, k, N, _ptr(y, "y", _BF16_LIKE), _stream(stream))
    check(st, "w4a16_moe_combine")


def w4a16_moe_layer_workspace(T, E, k, d, I):
    return int(lib().w4a16_moe_layer_workspace(T, E, k, d, I))


def w4a16_moe_layer_sorted(T, E, k, d, I):
    """True when w4a16_moe_layer takes the sorted path for these sizes under
    the current kernel choice (it then writes the sort outputs of the plan)."""
    return bool(lib().w4a16_moe_layer_sorted(T, E, k, d, I))


def w4a16_moe_layer_plan(T, E, k, d, I):
    arr = (ctypes.c_size_t * 9)()
    check(lib().w4a16_moe_layer_plan(T, E, k, d, I, arr), "w4a16_moe_layer_plan")
    return [int(v) for v in arr]


def w4a16_moe_layer(x, logits, k, I, w1_q, w1_s, w2_q, w2_s, activation, y, ws, stream=None):
    T, d = x.shape
    E = logits.shape[1]
    _dims(k, I)
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError("logits must be [T=%d, E], got %s" % (T, tuple(logits.shape)))
    dv = x.device
    _need(logits, "logits", T * E * 4, dv)
    _need(w1_q, "w1_q", E * 2 * I * d // 2, dv)
    _need(w1_s, "w1_s", E * 2 * I * d // 32 * 2, dv)
    _need(w2_q, "w2_q", E * d * I // 2, dv)
    _need(w2_s, "w2_s", E * d * I // 32 * 2, dv)
    _need(y, "y", T * d * 2, dv)
    _need(ws, "ws", w4a16_moe_layer_workspace(T, E, k, d, I), dv)
    st = lib().w4a16_moe_layer(
        _ptr(x, "x", _BF16_LIKE), _ptr(logits, "logits", (torch.float32,)), T, E, k, d, I,
        _ptr(w1_q, "w1_q", (torch.uint8,)), _ptr(w1_s, "w1_s", _BF16_LIKE), _ptr(w2_q, "w2_q", (torch.uint8,)),
        _ptr(w2_s, "w2_s", _BF16_LIKE), activation, _ptr(y, "y", _BF16_LIKE), _ptr(ws, "ws", (torch.uint8,)),
        ws.numel(), _stream(stream))
    check(st, "w4a16_moe_layer")


def w4a16_moe_layer_noalloc(x, logits, k, I, w1_q, w1_s, w2_q, w2_s, activation, y, stream=None):
    """w4a16_moe_layer with the library's static device scratch in place of a
    workspace (no allocation in the call; calls on one GPU must not overlap)."""
    T, d = x.shape
    E = logits.shape[1]
    _dims(k, I)
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError("logits must be [T=%d, E], got %s" % (T, tuple(logits.shape)))
    dv = x.device
    _need(logits, "logits", T * E * 4, dv)
    _need(w1_q, "w1_q", E * 2 * I * d // 2, dv)
    _need(w1_s, "w1_s", E * 2 * I * d // 32 * 2, dv)
    _need(w2_q, "w2_q", E * d * I // 2, dv)
    _need(w2_s, "w2_s", E * d * I // 32 * 2, dv)
    _need(y, "y", T * d * 2, dv)
    st = lib().w4a16_moe_layer_noalloc(
        _ptr(x, "x", _BF16_LIKE), _ptr(logits, "logits", (torch.float32,)), T, E, k, d, I,
        _ptr(w1_q, "w1_q", (torch.uint8,)), _ptr(w1_s, "w1_s", _BF16_LIKE), _ptr(w2_q, "w2_q", (torch.uint8,)),
        _ptr(w2_s, "w2_s", _BF16_LIKE), activation, _ptr(y, "y", _BF16_LIKE), _stream(stream))
    check(st, "w4a16_moe_layer_noalloc")


# ------------------------------------------------------------- FP8 (W8A8)
def w8a8_quantize_rows(x, q, scale, stream=None):
    rows, K = x.shape
    d = x.device
    _need(q, "q", rows * K, d)
    _need(scale, "scale", rows * 4, d)
    st = lib().w8a8_quantize_rows(_ptr(x, "x", _BF16_LIKE), rows, K, _ptr(q, "q", (torch.uint8,)),
                                  _ptr(scale, "scale", (torch.float32,)), _stream(stream))
    check(st, "w8a8_quantize_rows")


def w8a8_moe_gmm(xq, x_scale, row_index, expert_offsets, E, R, K, N, wq, w_scale, epilogue, out, out_dtype,
                 stream=None):
    _dims(E, R, K, N)
    if xq.dim() != 2 or xq.shape[1] != K:
        raise ValueError("xq must be [x_rows, K=%d], got %s" % (K, tuple(xq.shape)))
    d = xq.device
    x_rows = xq.shape[0]
    _need(x_scale, "x_scale", x_rows * 4, d)
    _need(row_index, "row_index", R * 4, d)
    _need(expert_offsets, "expert_offsets", (E + 1) * 4, d)
    _need(wq, "wq", E * N * K, d)
    _need(w_scale, "w_scale", E * N * 4, d)
    ncol = N // 2 if epilogue in (W4_EPI_GEGLU_TANH, W4_EPI_SWIGLU) else N
    if out_dtype == W4_OUT_F32 and out.dtype != torch.float32:
        raise TypeError("out must be float32 for W4_OUT_F32")
    if out_dtype == W4_OUT_BF16 and out.dtype not in _BF16_LIKE:
        raise TypeError("out must be bf16 for W4_OUT_BF16")
    _need(out, "out", R * ncol * (4 if out_dtype == W4_OUT_F32 else 2), d)
    st = lib().w8a8_moe_gmm(
        _ptr(xq, "xq", (torch.uint8,)), _ptr(x_scale, "x_scale", (torch.float32,)), x_rows,
        _ptr(row_index, "row_index", (torch.int32,), True), _ptr(expert_offsets, "expert_offsets", (torch.int32,), True),
        E, R, K, N, _ptr(wq, "wq", (torch.uint8,)), _ptr(w_scale, "w_scale", (torch.float32,)), epilogue,
        _ptr(out, "out", (torch.float32,) + _BF16_LIKE), out_dtype, _stream(stream))
    check(st, "w8a8_moe_gmm")


def w8a8_moe_layer_plan(T, E, k, d, I):
    arr = (ctypes.c_size_t * 13)()
    check(lib().w8a8_moe_layer_plan(T, E, k, d, I, arr), "w8a8_moe_layer_plan")
    return [int(v) for v in arr]


def w8a8_moe_layer_workspace(T, E, k, d, I):
    return int(lib().w8a8_moe_layer_workspace(T, E, k, d, I))


def w8a8_moe_layer(x, logits, k, I, w1q, w1_scale, w2q, w2_scale, activation, y, ws, stream=None):
    T, d = x.shape
    E = logits.shape[1]
    _dims(k, I)
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError("logits must be [T=%d, E], got %s" % (T, tuple(logits.shape)))
    dv = x.device
    _need(logits, "logits", T * E * 4, dv)
    _need(w1q, "w1q", E * 2 * I * d, dv)
    _need(w1_scale, "w1_scale", E * 2 * I * 4, dv)
    _need(w2q, "w2q", E * d * I, dv)
    _need(w2_scale, "w2_scale", E * d * 4, dv)
    _need(y, "y", T * d * 2, dv)
    _need(ws, "ws", 0, dv)
    wp, wn = _ws(ws)
    st = lib().w8a8_moe_layer(
        _ptr(x, "x", _BF16_LIKE), _ptr(logits, "logits", (torch.float32,)), T, E, k, d, I,
        _ptr(w1q, "w1q", (torch.uint8,)), _ptr(w1_scale, "w1_scale", (torch.float32,)),
        _ptr(w2q, "w2q", (torch.uint8,)), _ptr(w2_scale, "w2_scale", (torch.float32,)), activation,
        _ptr(y, "y", _BF16_LIKE), wp, wn, _stream(stream))
    check(st, "w8a8_moe_layer")


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
    sorted_path = w4a16_moe_layer_sorted(T, E, k, d, I)

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
        "sorted": sorted_path,
    }
    return y, views


def fp8_moe_layer(x, logits, k, I, w1q, w1_scale, w2q, w2_scale, activation=W4_EPI_GEGLU_TANH, ws=None,
                  stream=None):
    """Whole FP8 MoE layer; returns (y, views) with the plan and intermediates."""
    T, d = x.shape
    E = logits.shape[1]
    need = w8a8_moe_layer_workspace(T, E, k, d, I)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    w8a8_moe_layer(x, logits, k, I, w1q, w1_scale, w2q, w2_scale, activation, y, ws, stream)
    p = w8a8_moe_layer_plan(T, E, k, d, I)
    R = T * k

    def view(i, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[p[i]:p[i] + nbytes].view(dt)

    views = {
        "topk_ids": view(0, R, torch.int32).view(T, k),
        "topk_weights": view(1, R, torch.float32).view(T, k),
        "expert_offsets": view(2, E + 1, torch.int32),
        "sorted_tokens": view(4, R, torch.int32),
        "row_to_sorted": view(5, R, torch.int32),
        "xq": view(7, T * d, torch.uint8).view(T, d),
        "x_scale": view(8, T, torch.float32),
        "a": view(9, R * I, torch.bfloat16).view(R, I),
        "aq": view(10, R * I, torch.uint8).view(R, I),
        "a_scale": view(11, R, torch.float32),
        "o": view(12, R * d, torch.float32).view(R, d),
    }
    return y, views
