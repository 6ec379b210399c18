"""The C-ABI library without a GPU: exported symbols, host-side validation, dispatch plan."""
import ctypes
import os
import re
import subprocess

import pytest

import weight_only_int4_w4a16_amd as w

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

OK, NULLP, SHAPE, GROUP, ALIGN, DEVICE, LAUNCH = range(7)
A = 0x10000          # a fake, 16-byte aligned address: validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:w4a16_status_t|const char \*|int32_t)\s*\*?\s*"
                                 r"(w4a16_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("w4a16_gemv", "w4a16_gemv_batched", "w4a16_moe_gemv", "w4a16_unpack_debug",
              "w4a16_describe_plan", "w4a16_status_string", "w4a16_abi_version",
              "w4a16_stream_read", "w4a16_moe_gemv_swiglu", "w4a16_moe_down_combine",
              "w4a16_describe_tail_plan", "w4a16_quantize_pack", "w4a16_moe_gemv_batched",
              "w4a16_describe_moe_batched_plan", "w4a16_moe_gemv3", "w4a16_unpack3_debug",
              "w4a16_describe_moe3_plan"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = w.library()
    out = subprocess.run(["nm", "-D", "--defined-only", w.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    for n in declared_functions():
        assert n in exported, n
        getattr(lib, n)
    assert lib.w4a16_abi_version() == 1


def test_library_has_no_oracle_dependency():
    out = subprocess.run(["nm", "-D", w.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    deps = subprocess.run(["ldd", w.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def test_status_strings():
    lib = w.library()
    for s in range(7):
        assert lib.w4a16_status_string(s)
    assert b"unknown" in lib.w4a16_status_string(99)


def gemv(qw=A, sc=A, x=A, y=A, N=64, K=256, G=128):
    return w.library().w4a16_gemv(qw, sc, x, y, N, K, G, None)


def batched(qw=A, sc=A, X=A, ldx=256, Y=A, ldy=64, M=4, N=64, K=256, G=128):
    return w.library().w4a16_gemv_batched(qw, sc, X, ldx, Y, ldy, M, N, K, G, None)


def moe(qw=A, sc=A, ids=A, topk=8, E=16, x=A, y=A, N=64, K=256, G=128):
    return w.library().w4a16_moe_gemv(qw, sc, ids, topk, E, x, y, N, K, G, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qw=None), NULLP), (dict(sc=None), NULLP), (dict(x=None), NULLP), (dict(y=None), NULLP),
    (dict(G=64), GROUP), (dict(G=0), GROUP),
    (dict(N=0), SHAPE), (dict(N=-5), SHAPE), (dict(N=1 << 31), SHAPE),
    (dict(K=0), SHAPE), (dict(K=64), SHAPE), (dict(K=200), SHAPE), (dict(K=65536 + 128), SHAPE),
    (dict(qw=A + 8), ALIGN), (dict(x=A + 4), ALIGN), (dict(sc=A + 1), ALIGN), (dict(y=A + 2), ALIGN),
])
def test_gemv_validation(kw, status):
    assert gemv(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), NULLP), (dict(M=0), SHAPE), (dict(M=17), SHAPE), (dict(ldx=255), SHAPE),
    (dict(ldy=63), SHAPE), (dict(ldx=260), ALIGN), (dict(X=A + 8), ALIGN), (dict(G=256), GROUP),
])
def test_batched_validation(kw, status):
    assert batched(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(ids=None), NULLP), (dict(topk=0), SHAPE), (dict(topk=1025), SHAPE), (dict(E=0), SHAPE),
    (dict(ids=A + 2), ALIGN), (dict(K=384 + 64), SHAPE), (dict(N=1 << 30, topk=4), SHAPE),
])
def test_moe_validation(kw, status):
    assert moe(**kw) == status


def swiglu(qw=A, sc=A, ids=A, topk=8, E=16, x=A, h=A, I=1024, K=2304, G=128):
    return w.library().w4a16_moe_gemv_swiglu(qw, sc, ids, topk, E, x, h, I, K, G, None)


def down(qw=A, sc=A, ids=A, rw=A, topk=8, E=16, h=A, out=A, H=2304, I=1024, G=128):
    return w.library().w4a16_moe_down_combine(qw, sc, ids, rw, topk, E, h, out, H, I, G, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qw=None), NULLP), (dict(sc=None), NULLP), (dict(ids=None), NULLP), (dict(x=None), NULLP),
    (dict(h=None), NULLP), (dict(G=64), GROUP), (dict(I=0), SHAPE), (dict(I=1 << 30), SHAPE),
    (dict(K=200), SHAPE), (dict(K=65536 + 128), SHAPE), (dict(topk=0), SHAPE),
    (dict(topk=1025), SHAPE), (dict(E=0), SHAPE), (dict(qw=A + 4), ALIGN), (dict(x=A + 2), ALIGN),
    (dict(h=A + 1), ALIGN), (dict(ids=A + 2), ALIGN),
])
def test_swiglu_validation(kw, status):
    assert swiglu(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(qw=None), NULLP), (dict(rw=None), NULLP), (dict(h=None), NULLP), (dict(out=None), NULLP),
    (dict(G=256), GROUP), (dict(H=0), SHAPE), (dict(I=64), SHAPE), (dict(I=1000), SHAPE),
    (dict(topk=0), SHAPE), (dict(topk=65, I=1024), SHAPE), (dict(E=0), SHAPE),
    (dict(h=A + 8), ALIGN), (dict(out=A + 2), ALIGN), (dict(rw=A + 1), ALIGN),
])
def test_down_combine_validation(kw, status):
    assert down(**kw) == status


@pytest.mark.parametrize("step,rows,K,I,topk,want", [
    (0, 0, 2304, 1024, 8, "valu_moe_swiglu tokens=1 lanes_per_row=8 chunks_per_item=3"),
    (0, 0, 2048, 1408, 8, "valu_moe_swiglu tokens=1 lanes_per_row=32 chunks_per_item=1"),
    (1, 2304, 0, 1024, 8, "splitk_moe_combine tokens=1 lanes_per_row=32 chunks_per_lane=1"),
    (1, 7168, 0, 1408, 8, "valu_moe_combine tokens=1 lanes_per_row=4 chunks_per_item=1"),
    (1, 5, 0, 128, 1, "valu_moe_combine tokens=1 lanes_per_row=4"),
])
def test_tail_dispatch(step, rows, K, I, topk, want):
    assert w.describe_tail_plan(step, rows, K, I, topk).startswith(want)


def quant(w_=A, ldw=256, qw=A, sc=A, N=64, K=256, G=128):
    return w.library().w4a16_quantize_pack(w_, ldw, qw, sc, N, K, G, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w_=None), NULLP), (dict(qw=None), NULLP), (dict(sc=None), NULLP), (dict(G=64), GROUP),
    (dict(N=0), SHAPE), (dict(K=200), SHAPE), (dict(K=0), SHAPE), (dict(ldw=128), SHAPE),
    (dict(K=(1 << 20) + 128, ldw=(1 << 20) + 128), SHAPE), (dict(w_=A + 8), ALIGN),
    (dict(ldw=260), ALIGN), (dict(qw=A + 2), ALIGN), (dict(sc=A + 1), ALIGN),
    (dict(N=1 << 24, K=1 << 20, ldw=1 << 20), SHAPE),
])
def test_quantize_validation(kw, status):
    assert quant(**kw) == status


def moeb(qw=A, sc=A, ids=A, M=4, topk=8, E=16, X=A, ldx=256, Y=A, N=64, K=256, G=128):
    return w.library().w4a16_moe_gemv_batched(qw, sc, ids, M, topk, E, X, ldx, Y, N, K, G, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qw=None), NULLP), (dict(ids=None), NULLP), (dict(X=None), NULLP), (dict(Y=None), NULLP),
    (dict(G=64), GROUP), (dict(M=0), SHAPE), (dict(M=17), SHAPE), (dict(topk=0), SHAPE),
    (dict(M=16, topk=17), SHAPE), (dict(E=0), SHAPE), (dict(ldx=128), SHAPE), (dict(K=200), SHAPE),
    (dict(ldx=260), ALIGN), (dict(ids=A + 2), ALIGN), (dict(X=A + 8), ALIGN),
])
def test_moe_batched_validation(kw, status):
    assert moeb(**kw) == status


def test_moe_batched_plans():
    # rows of 8k chunks take the 4x4x4-MFMA form (tokens of an expert share each decode) ...
    assert w.describe_moe_batched_plan(16, 2048, 2304, 8).startswith(
        "moe_batched_mfma4x4x4 slots=4 blocks_per_row=8 chunks_per_lane=3 threads=512")
    assert w.describe_moe_batched_plan(8, 300, 4096, 8).startswith(
        "moe_batched_mfma4x4x4 slots=4 blocks_per_row=16 chunks_per_lane=2")
    # ... the others the VALU form
    assert w.describe_moe_batched_plan(1, 5, 128, 256).startswith("moe_batched tokens_per_pass=1")
    assert w.describe_moe_batched_plan(3, 64, 384, 4).startswith("moe_batched tokens_per_pass=1")
    with pytest.raises(w.W4A16Error):
        w.describe_moe_batched_plan(16, 100, 8192, 8)    # activations do not fit in LDS


def moe3(qw=A, sc=A, ids=A, topk=8, E=16, x=A, y=A, N=64, K=256, G=128):
    return w.library().w4a16_moe_gemv3(qw, sc, ids, topk, E, x, y, N, K, G, None)


@pytest.mark.parametrize("kw,status", [
    (dict(qw=None), NULLP), (dict(sc=None), NULLP), (dict(ids=None), NULLP), (dict(x=None), NULLP),
    (dict(y=None), NULLP), (dict(G=64), GROUP), (dict(N=0), SHAPE), (dict(K=0), SHAPE),
    (dict(K=200), SHAPE), (dict(K=65536 + 128), SHAPE), (dict(topk=0), SHAPE),
    (dict(topk=1025), SHAPE), (dict(E=0), SHAPE), (dict(N=1 << 30, topk=4), SHAPE),
    (dict(qw=A + 2), ALIGN), (dict(x=A + 8), ALIGN), (dict(sc=A + 1), ALIGN),
    (dict(y=A + 2), ALIGN), (dict(ids=A + 2), ALIGN),
])
def test_moe3_validation(kw, status):
    assert moe3(**kw) == status


@pytest.mark.parametrize("N,K,topk,want", [
    (2048, 2304, 8, "moe3 lanes_per_row=8 blocks_per_item=3 threads=256 blocks=512 lds=4928"),
    (64, 384, 3, "moe3 lanes_per_row=4 blocks_per_item=3"),
    (100, 128, 5, "moe3 lanes_per_row=4 blocks_per_item=1"),
    (7, 65536, 1024, "moe3 lanes_per_row=8 blocks_per_item=1"),
])
def test_moe3_plans(N, K, topk, want):
    assert w.describe_moe3_plan(N, K, topk).startswith(want)


def test_every_valid_moe3_shape_has_a_plan():
    """Every K that is a multiple of 128 up to 65536 has an instantiated three-bit kernel."""
    for K in range(128, 65536 + 1, 128):
        assert w.describe_moe3_plan(33, K, 8).startswith("moe3 ")


def test_moe3_plan_rejects_bad_shapes():
    for args in ((0, 128, 1), (4, 100, 1), (4, 128, 0)):
        with pytest.raises(w.W4A16Error):
            w.describe_moe3_plan(*args)


def test_unpack3_validation():
    lib = w.library()
    assert lib.w4a16_unpack3_debug(None, A, 4, 64, None) == NULLP
    assert lib.w4a16_unpack3_debug(A, None, 4, 64, None) == NULLP
    assert lib.w4a16_unpack3_debug(A, A, 4, 48, None) == SHAPE
    assert lib.w4a16_unpack3_debug(A, A, 0, 64, None) == SHAPE
    assert lib.w4a16_unpack3_debug(A + 2, A, 4, 64, None) == ALIGN


def test_unpack_validation():
    lib = w.library()
    assert lib.w4a16_unpack_debug(None, A, 4, 64, None) == NULLP
    assert lib.w4a16_unpack_debug(A, A, 4, 12, None) == SHAPE
    assert lib.w4a16_unpack_debug(A, A, 0, 64, None) == SHAPE
    assert lib.w4a16_unpack_debug(A + 2, A, 4, 64, None) == ALIGN


def test_stream_read_validation():
    lib = w.library()
    assert lib.w4a16_stream_read(None, 64, A, 1, 4, None) == NULLP
    assert lib.w4a16_stream_read(A, 64, None, 1, 4, None) == NULLP
    assert lib.w4a16_stream_read(A, 8, A, 1, 4, None) == SHAPE
    assert lib.w4a16_stream_read(A, 72, A, 1, 4, None) == SHAPE
    assert lib.w4a16_stream_read(A, 64, A, 0, 4, None) == SHAPE
    assert lib.w4a16_stream_read(A, 64, A, 1, 3, None) == SHAPE
    assert lib.w4a16_stream_read(A + 4, 64, A, 1, 4, None) == ALIGN
    assert lib.w4a16_stream_read(A, 64, A + 2, 1, 4, None) == ALIGN


def test_valid_arguments_reach_the_device_check_only():
    # With well-formed arguments the call gets past validation; on a host without a gfx950 GPU
    # it must stop at the device check and enqueue nothing.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert gemv() == DEVICE
    assert batched() == DEVICE
    assert moe() == DEVICE
    assert w.library().w4a16_stream_read(A, 64, A, 1, 4, None) == DEVICE
    assert swiglu() == DEVICE
    assert down() == DEVICE
    assert quant() == DEVICE
    assert moeb() == DEVICE
    assert moe3() == DEVICE
    assert w.library().w4a16_unpack3_debug(A, A, 4, 64, None) == DEVICE


@pytest.mark.parametrize("M,N,K,topk,kind", [
    (1, 1024, 2048, 0, "splitk "), (1, 4096, 7168, 0, "splitk "), (1, 16384, 3072, 0, "splitk "),
    (1, 16384, 1536, 0, "valu tokens=1 lanes_per_row=8 chunks_per_item=3"),
    (1, 8192, 1024, 0, "valu "), (1, 4096, 4096, 0, "splitk "),
    (1, 28672, 4096, 0, "splitk tokens=1 lanes_per_row=32 chunks_per_lane=1 row_steps=4"),
    (1, 14336, 2048, 0, "valu tokens=1 lanes_per_row=32 chunks_per_item=2"),
    (1, 4096, 14336, 0, "splitk "), (1, 8192, 8192, 0, "splitk "), (1, 163840, 2304, 0, "valu "),
    (1, 2048, 2304, 8, "valu_moe"), (1, 5, 128, 0, "valu "), (1, 64, 65536, 0, "splitk "),
    (2, 8192, 8192, 0, "splitk "),
    (4, 163840, 2304, 0, "mfma4x4x4_splitk token_groups=1 chunks_per_lane=3 row_steps=1 "
                         "blocks_per_row=8 threads=192 blocks=1024"),
    (5, 163840, 2304, 0, "mfma16x16x32_lds8_lines tiles_per_wave=1 k_split=1 groups_per_item=2 "
                         "threads=512 blocks=512"),
    (1, 163840, 2304, 0, "valu tokens=1 lanes_per_row=8 chunks_per_item=1 row_steps=2"),
    (6, 163840, 2304, 0, "mfma16x16x32_lds8_lines"),
    (2, 163840, 2304, 0, "mfma4x4x4_splitk"), (4, 32768, 2048, 0, "mfma4x4x4_splitk"),
    (8, 163840, 2304, 0, "mfma16x16x32_lds8_lines"), (3, 100, 384, 0, "valu "),
    (4, 28672, 4096, 0, "mfma4x4x4_splitk token_groups=1 chunks_per_lane=2 row_steps=2 "
                        "blocks_per_row=16"),
    (3, 8192, 8192, 0, "mfma4x4x4_splitk token_groups=1 chunks_per_lane=2"),
    (8, 4096, 14336, 0, "mfma4x4x4_splitk token_groups=2 chunks_per_lane=4"),
    (5, 7, 256, 0, "mfma4x4x4_splitk token_groups=2 chunks_per_lane=1 row_steps=1 blocks_per_row=8"),
    (8, 14336, 2048, 0, "mfma4x4x4_splitk token_groups=2 chunks_per_lane=1 row_steps=1"),
    (8, 28672, 4096, 0, "mfma16x16x32_lds_lines"), (2, 28672, 4096, 0, "splitk "),
    (2, 14336, 2048, 0, "splitk tokens=2"), (4, 14336, 2048, 0, "mfma4x4x4_splitk token_groups=1 "
                                                              "chunks_per_lane=1 row_steps=2"),
    (16, 8192, 8192, 0, "mfma16x16x32_rows tiles_per_wave=2 k_split=4 groups_per_item=2 threads=256"),
    (12, 8192, 8192, 0, "mfma16x16x32_rows tiles_per_wave=2 k_split=4"),
    (8, 8192, 8192, 0, "mfma16x16x32_rows8 tiles_per_wave=2 k_split=4 groups_per_item=2 threads=256"),
    (5, 8192, 8192, 0, "mfma16x16x32_rows8 tiles_per_wave=2 k_split=4"),
    (8, 16384, 4096, 0, "mfma16x16x32_rows8 tiles_per_wave=2 k_split=4"),
    (8, 12288, 8192, 0, "mfma4x4x4_splitk token_groups=2"),
    (16, 4096, 14336, 0, "mfma16x16x32_rows tiles_per_wave=1 k_split=8 groups_per_item=2 threads=512"),
    (16, 14336, 2048, 0, "mfma16x16x32_lines tiles_per_wave=4 k_split=4"),
    (16, 300, 2688, 0, "mfma16x16x32 tiles_per_wave=1 k_split=1 groups_per_item=1"),
    (16, 163840, 2304, 0, "mfma16x16x32_lds_lines tiles_per_wave=1 k_split=1 groups_per_item=2"),
    (16, 2048, 4096, 0, "mfma16x16x32_rows tiles_per_wave=1 k_split=8"),
    (16, 4096, 2304, 0, "mfma16x16x32_lds_lines tiles_per_wave=1 k_split=1 groups_per_item=6 threads=256"),
])
def test_default_dispatch(M, N, K, topk, kind):
    """The shipped entry points pick the tuned kernels with no configuration (no env switch)."""
    plan = w.describe_plan(M, N, K, topk, cus=256)
    assert plan.startswith(kind), plan
    if not kind.startswith("mfma"):
        assert f"tokens={M}" in plan


def test_every_valid_shape_has_a_plan():
    for M in range(1, 17):
        for K in (128, 256, 384, 1152, 2304, 4096, 14336, 65536 if M == 1 else 131072):
            assert w.describe_plan(M, 777, K, 0, 256)
    for K in (128, 2304, 65536):
        assert "_moe " in w.describe_plan(1, 33, K, 8, 256)


def test_describe_rejects_bad_shapes():
    for args in ((0, 10, 128), (17, 10, 128), (1, 0, 128), (1, 10, 100), (2, 10, 128, 4)):
        with pytest.raises(w.W4A16Error):
            w.describe_plan(*args)


def test_binding_refuses_host_tensors_and_wrong_dtypes():
    """The Python layer checks dtypes, devices and ranks before calling the library."""
    import torch
    q = torch.zeros((4, 16), dtype=torch.int32)
    s = torch.zeros((4, 1), dtype=torch.float16)
    x = torch.zeros(128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        w.gemv(q, s, x)                       # host tensors
    with pytest.raises(TypeError, match="qweight"):
        w.gemv(q.float(), s, x)
    for args in ((q, s.float(), x), (q, s, x.half()), (q.reshape(-1), s, x)):
        with pytest.raises((TypeError, ValueError)):
            w.gemv(*args)
    with pytest.raises(TypeError, match="qweight"):
        w.moe_gemv(q.reshape(1, 4, 16).float(), s.reshape(1, 4, 1), torch.zeros(2), x)
