"""C ABI contract checks that need no GPU: the library loads, exports every
function include/w4a16.h declares with a matching binding signature, and
rejects bad arguments on the host (those calls return before any HIP call)."""

import ctypes
import os
import re

import numpy as np
import pytest

import int4_group_quantized_q4_amd as w4
from int4_group_quantized_q4_amd import _lib
import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

FAKE = 0x10000  # a 16-byte aligned non-null address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for required in ("q4_group_repack", "w4a16_linear", "w4a16_moe_gmm", "w4a16_moe_route", "w4a16_moe_combine"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = _lib.lib()
    assert lib.w4a16_abi_version() == 2
    for st in (0, -1, -2, -3, -4):
        assert len(w4.status_string(st)) > 5
    assert "unknown" in w4.status_string(42)


def test_repack_argument_errors():
    lib = _lib.lib()
    f = lib.q4_group_repack
    assert f(FAKE, 16, 33, FAKE, FAKE, None, None, None) == w4.W4_ERR_SHAPE
    assert f(FAKE, 15, 32, FAKE, FAKE, None, None, None) == w4.W4_ERR_SHAPE
    assert f(FAKE, -16, 32, FAKE, FAKE, None, None, None) == w4.W4_ERR_ARG
    assert f(None, 16, 32, FAKE, FAKE, None, None, None) == w4.W4_ERR_ARG
    assert f(FAKE + 2, 16, 32, FAKE, FAKE, None, None, None) == w4.W4_ERR_ARG
    assert f(FAKE, 16, 32, FAKE, FAKE, None, FAKE + 4, None) == w4.W4_ERR_ARG
    assert f(FAKE, 1 << 30, 1 << 12, FAKE, FAKE, None, None, None) == w4.W4_ERR_SHAPE
    assert f(None, 0, 32, None, None, None, None, None) == w4.W4_OK      # empty: nothing enqueued


def test_linear_and_gmm_argument_errors():
    lib = _lib.lib()
    assert lib.w4a16_linear(FAKE, 4, 256, FAKE, FAKE, 500, FAKE, None, 0, None) == w4.W4_ERR_SHAPE
    assert lib.w4a16_linear(FAKE, 4, 250, FAKE, FAKE, 512, FAKE, None, 0, None) == w4.W4_ERR_SHAPE
    assert lib.w4a16_linear(FAKE, -1, 256, FAKE, FAKE, 512, FAKE, None, 0, None) == w4.W4_ERR_ARG
    assert lib.w4a16_linear(None, 4, 256, FAKE, FAKE, 512, FAKE, None, 0, None) == w4.W4_ERR_ARG
    assert lib.w4a16_linear(FAKE, 0, 256, None, None, 512, None, None, 0, None) == w4.W4_OK
    g = lib.w4a16_moe_gmm
    args = [FAKE, 64, FAKE, FAKE, 128, 512, 2816, 1408, FAKE, FAKE, w4.W4_EPI_GEGLU_TANH, FAKE, w4.W4_OUT_BF16, None, 0,
            None]
    bad = list(args); bad[10] = 7
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[12] = w4.W4_OUT_F32               # gated epilogue needs bf16 out
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[7] = 1424                          # N % 32 != 0 with a gated epilogue
    assert g(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[2] = None; bad[1] = 100            # no gather and too few x rows
    assert g(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[3] = None
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[4] = 0
    assert g(*bad) == w4.W4_ERR_ARG


def test_tiled_kernel_needs_workspace():
    """A prefill-shaped call (many rows per expert) selects the tiled kernel,
    whose fp16 activation rows live in the caller's workspace: without it the
    call fails on the host, before any launch."""
    lib = _lib.lib()
    need = lib.w4a16_moe_gmm_workspace(4096, 32768, 128, 2816, 1408)
    assert need >= 4096 * 2816 * 2 + 4096 * 4 and need % 256 == 0
    assert lib.w4a16_linear_workspace(300, 2816, 512) >= 300 * 2816 * 2
    args = [FAKE, 4096, FAKE, FAKE, 128, 32768, 2816, 1408, FAKE, FAKE, w4.W4_EPI_GEGLU_TANH, FAKE, w4.W4_OUT_BF16,
            None, 0, None]
    assert lib.w4a16_moe_gmm(*args) == w4.W4_ERR_WORKSPACE
    args[13], args[14] = FAKE, need - 1
    assert lib.w4a16_moe_gmm(*args) == w4.W4_ERR_WORKSPACE
    with w4.gemm_kernel(w4.W4_KERNEL_TILED):
        assert lib.w4a16_linear(FAKE, 300, 2816, FAKE, FAKE, 512, FAKE, None, 0, None) == w4.W4_ERR_WORKSPACE


def test_streaming_calls_argument_errors():
    lib = _lib.lib()
    assert lib.w4a16_moe_topk(FAKE, 64, 128, 17, FAKE, FAKE, None) == w4.W4_ERR_ARG
    assert lib.w4a16_moe_topk(None, 0, 128, 8, None, None, None) == w4.W4_OK
    g = lib.w4a16_moe_gmm_ids
    args = [FAKE, FAKE, 64, 8, 8, 128, 2816, 1408, FAKE, FAKE, w4.W4_EPI_GEGLU_TANH, FAKE, w4.W4_OUT_BF16, None]
    bad = list(args); bad[4] = 3                    # row_div must be 1 or k
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[2] = 257                  # more tokens than the ids scan holds
    assert g(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[12] = w4.W4_OUT_F32
    assert g(*bad) == w4.W4_ERR_ARG
    gl = lib.w4a16_moe_gmm_logits
    args = [FAKE, FAKE, 64, 128, 8, 2816, 1408, FAKE, FAKE, w4.W4_EPI_GEGLU_TANH, FAKE, FAKE, FAKE, None]
    bad = list(args); bad[9] = w4.W4_EPI_NONE       # gated epilogues only
    assert gl(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[2] = 257
    assert gl(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[1] = None
    assert gl(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[6] = 1400                 # N % 32
    assert gl(*bad) == w4.W4_ERR_SHAPE
    assert gl(None, None, 0, 128, 8, 2816, 1408, None, None, w4.W4_EPI_GEGLU_TANH, None, None, None, None) == w4.W4_OK


def test_route_combine_layer_argument_errors():
    lib = _lib.lib()
    assert lib.w4a16_moe_route_workspace(64, 128, 8) > 0
    assert lib.w4a16_moe_route_workspace(64, 4, 8) == 0
    r = lib.w4a16_moe_route
    assert r(FAKE, 64, 128, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == w4.W4_ERR_WORKSPACE
    assert r(FAKE, 64, 128, 17, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == w4.W4_ERR_ARG
    assert r(FAKE, 64, 300, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == w4.W4_ERR_ARG
    assert r(FAKE, 1 << 28, 128, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == w4.W4_ERR_SHAPE
    c = lib.w4a16_moe_combine
    assert c(FAKE, 1, FAKE, FAKE, 64, 8, 2812, FAKE, None) == w4.W4_ERR_SHAPE
    assert c(FAKE, 5, FAKE, FAKE, 64, 8, 2816, FAKE, None) == w4.W4_ERR_ARG
    ws = lib.w4a16_moe_layer_workspace(64, 128, 8, 2816, 704)
    R = 64 * 8
    assert ws >= R * 704 * 2 + R * 2816 * 4
    L = lib.w4a16_moe_layer
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 704, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, ws - 1, None) == w4.W4_ERR_WORKSPACE
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 704, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, ws, None) == w4.W4_ERR_ARG
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 700, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, ws, None) == w4.W4_ERR_SHAPE


def test_layer_plan_offsets():
    p = w4.w4a16_moe_layer_plan(64, 128, 8, 2816, 704)
    assert p[0] == 0 and all(b > a for a, b in zip(p, p[1:])) and all(v % 256 == 0 for v in p)


def test_layout_roundtrip_and_documented_offsets():
    rng = np.random.default_rng(0)
    for rows, K in [(16, 32), (32, 96), (48, 704), (16, 256), (32, 2816)]:
        c = rng.integers(-8, 8, (rows, K)).astype(np.int8)
        p = layout.encode(c)
        assert np.array_equal(layout.decode(p, rows, K), c)
    # the documented layout on one code: row 17 (tile 1, r 1), K = 256, column 37
    # (group 1 -> block 0, j 1; chunk 0; i 5) -> word at 8*256 + 4*4*(16*0 + 1) + 4*1,
    # bit 4*2 + 16 = 24 -> byte +3, low nibble; offset binary -3 + 8 = 5
    codes = np.full((32, 256), -8, dtype=np.int8)    # all-zero nibbles
    codes[17, 37] = -3
    p = layout.encode(codes)
    nz = np.nonzero(p)[0]
    assert list(nz) == [2048 + 16 + 4 + 3] and p[nz[0]] == 0x05
    # the documented scale position: row 17 (t 1, r 1), K = 704 (G = 22), group 21
    # (block 5, j 1, gb = 2) -> 1*16*22 + 64*5 + 1*2 + 1
    sc = np.zeros((32, 22), dtype=np.uint16)
    sc[17, 21] = 0x3F80
    ts = layout.encode_scales(sc)
    assert list(np.nonzero(ts)[0]) == [352 + 320 + 2 + 1]
    assert np.array_equal(layout.decode_scales(ts, 32, 704), sc)


def test_python_wrappers_reject_undersized_buffers():
    """The binding checks every buffer's size against the shapes it passes,
    before any launch: the library sees pointers only, so an undersized tensor
    would otherwise become an out-of-bounds device access.  (CPU tensors reach
    the size check first; a correctly sized CPU tensor would then be refused as
    not on the device.)"""
    import torch
    u8 = lambda n: torch.empty(n, dtype=torch.uint8)
    bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16)
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32)
    i32 = lambda n: torch.empty(n, dtype=torch.int32)
    size_err = pytest.raises(ValueError, match="holds .* bytes")
    with size_err:
        w4.q4_group_repack(bf(32, 64), u8(32 * 64 // 2 - 1), bf(64))
    with size_err:
        w4.q4_group_repack(bf(32, 64), u8(32 * 32), bf(63))
    with size_err:
        w4.q4_group_dequant_f32(u8(1024), bf(64), 32, 64, f32(32 * 64 - 1))
    with size_err:
        w4.w4a16_linear(bf(4, 256), u8(512 * 128), bf(512 * 8), 512, bf(4, 511))
    with size_err:
        w4.w4a16_linear(bf(4, 256), u8(512 * 128 - 16), bf(512 * 8), 512, bf(4, 512))
    with size_err:
        w4.w4a16_moe_route(f32(64, 128), 8, i32(512), f32(512), i32(128), i32(512), i32(512), i32(512), u8(1 << 16))
    E, R, K, N = 4, 40, 256, 128
    gmm = dict(x=bf(10, K), row_index=i32(R), expert_offsets=i32(E + 1), E=E, R=R, K=K, N=N,
               qweight=u8(E * N * K // 2), scales=bf(E * N * K // 32), epilogue=w4.W4_EPI_NONE,
               out=f32(R, N), out_dtype=w4.W4_OUT_F32)
    for key, bad in (("row_index", i32(R - 1)), ("expert_offsets", i32(E)), ("qweight", u8(E * N * K // 2 - 1)),
                     ("scales", bf(E * N * K // 32 - 1)), ("out", f32(R, N - 1))):
        with size_err:
            w4.w4a16_moe_gmm(**dict(gmm, **{key: bad}))
    with pytest.raises(ValueError, match="x must be"):
        w4.w4a16_moe_gmm(**dict(gmm, x=bf(10, K + 32)))
    with pytest.raises(TypeError):
        w4.w4a16_moe_gmm(**dict(gmm, out=bf(R, N)))
    with size_err:   # gated: out has N/2 columns
        w4.w4a16_moe_gmm(**dict(gmm, epilogue=w4.W4_EPI_GEGLU_TANH, out=bf(R, N // 2 - 1), out_dtype=w4.W4_OUT_BF16))
    with size_err:
        w4.w4a16_moe_combine(f32(8 * 2, 64), w4.W4_OUT_F32, i32(16), f32(16), 8, 2, 64, bf(8, 63))
    with size_err:
        w4.w4a16_moe_combine(f32(8 * 2 - 1, 64), w4.W4_OUT_F32, i32(16), f32(16), 8, 2, 64, bf(8, 64))
    T, E, k, d, I = 8, 16, 2, 64, 32
    need = w4.w4a16_moe_layer_workspace(T, E, k, d, I)
    layer = dict(x=bf(T, d), logits=f32(T, E), k=k, I=I, w1_q=u8(E * 2 * I * d // 2), w1_s=bf(E * 2 * I * d // 32),
                 w2_q=u8(E * d * I // 2), w2_s=bf(E * d * I // 32), activation=w4.W4_EPI_GEGLU_TANH, y=bf(T, d),
                 ws=u8(need))
    for key, bad in (("w1_q", u8(E * 2 * I * d // 2 - 1)), ("w2_s", bf(E * d * I // 32 - 1)), ("y", bf(T, d - 1)),
                     ("ws", u8(need - 1))):
        with size_err:
            w4.w4a16_moe_layer(**dict(layer, **{key: bad}))


def test_noalloc_layer_size_limit_on_host():
    """The no-allocation layer refuses, before touching any device, a layer
    whose workspace exceeds its static scratch; the limit is the header's."""
    lib = _lib.lib()
    assert w4.W4_NOALLOC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert "#define W4_NOALLOC_SCRATCH_BYTES (32u << 20)" in text
    assert lib.w4a16_moe_layer_workspace(290, 128, 8, 2816, 704) <= w4.W4_NOALLOC_SCRATCH_BYTES
    assert lib.w4a16_moe_layer_workspace(300, 128, 8, 2816, 704) > w4.W4_NOALLOC_SCRATCH_BYTES
    L = lib.w4a16_moe_layer_noalloc
    assert L(FAKE, FAKE, 300, 128, 8, 2816, 704, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None) == w4.W4_ERR_WORKSPACE
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 700, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None) == w4.W4_ERR_SHAPE
    assert L(FAKE, FAKE, 64, 128, 17, 2816, 704, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None) == w4.W4_ERR_ARG


def test_fp8_calls_argument_errors():
    """The FP8 comparison path's entry points reject bad shapes and pointers on
    the host, before any launch."""
    lib = _lib.lib()
    qr = lib.w8a8_quantize_rows
    assert qr(FAKE, 4, 48, FAKE, FAKE, None) == w4.W4_ERR_SHAPE       # K % 32
    assert qr(None, 4, 64, FAKE, FAKE, None) == w4.W4_ERR_ARG
    assert qr(None, 0, 64, None, None, None) == w4.W4_OK
    g = lib.w8a8_moe_gmm
    args = [FAKE, FAKE, 64, FAKE, FAKE, 128, 512, 2816, 1408, FAKE, FAKE, w4.W4_EPI_GEGLU_TANH, FAKE, w4.W4_OUT_BF16,
            None]
    bad = list(args); bad[7] = 2800                  # K % 32
    assert g(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[8] = 1400                  # N % 16
    assert g(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[13] = w4.W4_OUT_F32        # gated output is bf16
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[4] = None                  # E > 1 needs offsets
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[9] = None
    assert g(*bad) == w4.W4_ERR_ARG
    bad = list(args); bad[8] = 1392                  # 87 gate tiles... N/32 odd: gated pairs do not split
    assert g(*bad) == w4.W4_ERR_SHAPE
    bad = list(args); bad[6] = 0                     # R = 0: nothing to do
    assert g(*bad) == w4.W4_OK
    ws = lib.w8a8_moe_layer_workspace(64, 128, 8, 2816, 704)
    R = 64 * 8
    assert ws >= R * 704 * 3 + R * 2816 * 4 + 64 * 2816
    plan = (ctypes.c_size_t * 13)()
    assert lib.w8a8_moe_layer_plan(64, 128, 8, 2816, 704, plan) == w4.W4_OK
    assert list(plan) == sorted(plan) and all(v % 256 == 0 for v in plan)
    L = lib.w8a8_moe_layer
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 704, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, ws - 1, None) == w4.W4_ERR_WORKSPACE
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 704, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, ws, None) == w4.W4_ERR_ARG
    assert L(FAKE, FAKE, 64, 128, 8, 2816, 700, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, ws, None) == w4.W4_ERR_SHAPE
