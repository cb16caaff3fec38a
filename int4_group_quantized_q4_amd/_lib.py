"""ctypes loader of libw4a16.so (built in-tree by build.py).

The shared library is required: importing the package does not fail when it is
missing, but the first call of any entry point raises ``LibraryNotBuilt``.
There is no other implementation to fall back to.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

W4_OK = 0
W4_ERR_ARG = -1
W4_ERR_SHAPE = -2
W4_ERR_WORKSPACE = -3
W4_ERR_HIP = -4

W4_EPI_NONE = 0
W4_EPI_GEGLU_TANH = 1
W4_EPI_SWIGLU = 2

W4_OUT_BF16 = 0
W4_OUT_F32 = 1

W4_KERNEL_AUTO = 0
W4_KERNEL_STREAM = 1
W4_KERNEL_TILED = 2
W4_TILED_MIN_ROWS = 64

W4_NOALLOC_SCRATCH_BYTES = 32 << 20

W4_GROUP_OFF_GRID = 0
W4_GROUP_NONFINITE = 255

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/w4a16.h
SIGNATURES = {
    "w4a16_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a16_abi_version": (ctypes.c_int, []),
    "w4a16_set_gemm_kernel": (ctypes.c_int, [ctypes.c_int]),
    "q4_group_repack": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _p, _p]),
    "q4_group_dequant_f32": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p]),
    "q4_pack_codes": (ctypes.c_int, [_p, _i64, _i64, _p, _p]),
    "q4_pack_scales": (ctypes.c_int, [_p, _i64, _i64, _p, _p]),
    "w4a16_linear_workspace": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "w4a16_linear": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _i64, _p, _p, ctypes.c_size_t, _p]),
    "w4a16_moe_route_workspace": (_sz, [_i64, _i32, _i32]),
    "w4a16_moe_route": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "w4a16_moe_topk": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _p]),
    "w4a16_moe_gmm_ids": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _p, _p, _i32, _p, _i32, _p]),
    "w4a16_moe_gmm_logits": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _i64, _i64, _p, _p, _i32, _p, _p, _p, _p]),
    "w4a16_moe_gmm_workspace": (ctypes.c_size_t, [_i64, _i64, _i32, _i64, _i64]),
    "w4a16_moe_gmm": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _i64, _i64, _i64, _p, _p, _i32, _p, _i32, _p,
                                     ctypes.c_size_t, _p]),
    "w4a16_moe_combine": (ctypes.c_int, [_p, _i32, _p, _p, _i64, _i32, _i64, _p, _p]),
    "w4a16_moe_layer_workspace": (_sz, [_i64, _i32, _i32, _i64, _i64]),
    "w4a16_moe_layer_plan": (ctypes.c_int, [_i64, _i32, _i32, _i64, _i64, ctypes.POINTER(_sz)]),
    "w4a16_moe_layer_sorted": (ctypes.c_int, [_i64, _i32, _i32, _i64, _i64]),
    "w4a16_moe_layer": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p, _sz, _p]),
    "w4a16_moe_layer_noalloc": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p]),
    "w8a8_quantize_rows": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "w8a8_moe_gmm": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i32, _i64, _i64, _i64, _p, _p, _i32, _p, _i32, _p]),
    "w8a8_moe_layer_plan": (ctypes.c_int, [_i64, _i32, _i32, _i64, _i64, _p]),
    "w8a8_moe_layer_workspace": (ctypes.c_size_t, [_i64, _i32, _i32, _i64, _i64]),
    "w8a8_moe_layer": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _i64, _i64, _p, _p, _p, _p, _i32, _p, _p,
                                      ctypes.c_size_t, _p]),
}


class LibraryNotBuilt(RuntimeError):
    pass


class W4Error(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        super().__init__("%s failed: %s" % (name, status_string(status)))


_lib = None


def lib():
    """The loaded library (loads on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                "%s is missing: build it with `python -m int4_group_quantized_q4_amd.build` "
                "(or __graft_entry__.build())" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status):
    return lib().w4a16_status_string(int(status)).decode()


def check(status, name):
    if status != W4_OK:
        raise W4Error(status, name)
