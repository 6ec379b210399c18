"""MI355X (gfx950) W4A16 decode GEMV.

Thin ctypes binding over libw4a16.so (C ABI in include/w4a16.h). This module only checks and
marshals arguments; every step of the computation runs in the HIP kernels of the library.
PyTorch supplies device memory and the current stream.

Tensor conventions:
  qweight  torch.int32  [N, K/8]       packed signed 4-bit values (uint32 bit patterns)
  scales   torch.float16 [N, K/128]    one scale per 128-wide K group
  x        torch.bfloat16 [K]          activations (batched: [M, ldx], unit stride along K)
  out      torch.float32 [N]           (batched: [M, N] with any row stride >= N)
  MoE      qweight [E, N, K/8], scales [E, N, K/128], expert_ids torch.int32 [topk] on the GPU,
           out [topk, N]

If libw4a16.so has not been built, every call raises ImportError; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["gemv", "gemv_batched", "moe_gemv", "moe_gemv_batched", "moe_gemv_swiglu",
           "moe_down_combine", "describe_moe_batched_plan",
           "quantize_pack", "unpack_debug", "describe_plan", "describe_tail_plan", "stream_read",
           "W4A16Error",
           "library", "LIB_PATH", "GROUP_SIZE", "MAX_BATCH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")
GROUP_SIZE = 128
MAX_BATCH = 16

_lib: Optional[ctypes.CDLL] = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library() -> ctypes.CDLL:
    """The loaded libw4a16.so; raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m weight_only_int4_w4a16_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.w4a16_gemv.argtypes = [P, P, P, P, i64, i64, i32, P]
    lib.w4a16_gemv_batched.argtypes = [P, P, P, i64, P, i64, i32, i64, i64, i32, P]
    lib.w4a16_moe_gemv.argtypes = [P, P, P, i32, i32, P, P, i64, i64, i32, P]
    lib.w4a16_unpack_debug.argtypes = [P, P, i64, i64, P]
    lib.w4a16_describe_plan.argtypes = [i32, i64, i64, i32, i32, ctypes.c_char_p, i64]
    lib.w4a16_stream_read.argtypes = [P, i64, P, i32, i32, P]
    lib.w4a16_moe_gemv_swiglu.argtypes = [P, P, P, i32, i32, P, P, i64, i64, i32, P]
    lib.w4a16_moe_down_combine.argtypes = [P, P, P, P, i32, i32, P, P, i64, i64, i32, P]
    lib.w4a16_describe_tail_plan.argtypes = [i32, i64, i64, i64, i32, i32, ctypes.c_char_p, i64]
    lib.w4a16_quantize_pack.argtypes = [P, i64, P, P, i64, i64, i32, P]
    lib.w4a16_moe_gemv_batched.argtypes = [P, P, P, i32, i32, i32, P, i64, P, i64, i64, i32, P]
    lib.w4a16_describe_moe_batched_plan.argtypes = [i32, i64, i64, i32, i32, ctypes.c_char_p,
                                                    i64]
    lib.w4a16_moe_gemv3.argtypes = [P, P, P, i32, i32, P, P, i64, i64, i32, P]
    lib.w4a16_unpack3_debug.argtypes = [P, P, i64, i64, P]
    lib.w4a16_describe_moe3_plan.argtypes = [i64, i64, i32, i32, ctypes.c_char_p, i64]
    lib.w4a16_status_string.argtypes = [ctypes.c_int]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    lib.w4a16_abi_version.argtypes = []
    for f in (lib.w4a16_gemv, lib.w4a16_gemv_batched, lib.w4a16_moe_gemv,
              lib.w4a16_unpack_debug, lib.w4a16_describe_plan, lib.w4a16_stream_read,
              lib.w4a16_moe_gemv_swiglu, lib.w4a16_moe_down_combine,
              lib.w4a16_describe_tail_plan, lib.w4a16_quantize_pack, lib.w4a16_moe_gemv_batched,
              lib.w4a16_describe_moe_batched_plan, lib.w4a16_abi_version):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().w4a16_status_string(int(status)).decode()


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")


def _ok(status: int, where: str):
    if status != 0:
        raise W4A16Error(status, where)


def gemv(qweight: torch.Tensor, scales: torch.Tensor, x: torch.Tensor,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = W x for one token. Returns out (allocated as float32 [N] when not given)."""
    _need(qweight, torch.int32, "qweight", 2)
    _need(scales, torch.float16, "scales", 2)
    _need(x, torch.bfloat16, "x", 1)
    N, K = qweight.shape[0], qweight.shape[1] * 8
    if not (qweight.is_contiguous() and scales.is_contiguous() and x.is_contiguous()):
        raise ValueError("qweight, scales and x must be contiguous")
    if tuple(scales.shape) != (N, K // GROUP_SIZE) or x.numel() != K:
        raise ValueError(f"shape mismatch: qweight {tuple(qweight.shape)}, scales "
                         f"{tuple(scales.shape)}, x {tuple(x.shape)}")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=qweight.device)
    _need(out, torch.float32, "out", 1)
    if out.numel() != N or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of N elements")
    _ok(library().w4a16_gemv(qweight.data_ptr(), scales.data_ptr(), x.data_ptr(),
                             out.data_ptr(), N, K, GROUP_SIZE, _stream(stream)), "w4a16_gemv")
    return out


def gemv_batched(qweight: torch.Tensor, scales: torch.Tensor, X: torch.Tensor,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = X W^T for M <= 16 tokens. X [M, >=K] bf16 with unit stride along K."""
    _need(qweight, torch.int32, "qweight", 2)
    _need(scales, torch.float16, "scales", 2)
    _need(X, torch.bfloat16, "X", 2)
    N, K = qweight.shape[0], qweight.shape[1] * 8
    M = X.shape[0]
    if not (qweight.is_contiguous() and scales.is_contiguous()):
        raise ValueError("qweight and scales must be contiguous")
    if tuple(scales.shape) != (N, K // GROUP_SIZE) or X.shape[1] < K or X.stride(1) != 1:
        raise ValueError("shape mismatch between qweight, scales and X")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=qweight.device)
    _need(out, torch.float32, "out", 2)
    if out.shape[0] != M or out.shape[1] != N or out.stride(1) != 1:
        raise ValueError("out must be float32 [M, N] with unit stride along N")
    ldx = X.stride(0) if M > 1 else max(X.stride(0), K)
    ldy = out.stride(0) if M > 1 else max(out.stride(0), N)
    _ok(library().w4a16_gemv_batched(qweight.data_ptr(), scales.data_ptr(), X.data_ptr(), ldx,
                                     out.data_ptr(), ldy, M, N, K, GROUP_SIZE, _stream(stream)),
        "w4a16_gemv_batched")
    return out


def moe_gemv(qweight: torch.Tensor, scales: torch.Tensor, expert_ids: torch.Tensor,
             x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[t] = W_{expert_ids[t]} x for every selected expert; reads only those experts."""
    _need(qweight, torch.int32, "qweight", 3)
    _need(scales, torch.float16, "scales", 3)
    _need(expert_ids, torch.int32, "expert_ids", 1)
    _need(x, torch.bfloat16, "x", 1)
    E, N, K = qweight.shape[0], qweight.shape[1], qweight.shape[2] * 8
    topk = expert_ids.numel()
    if not all(t.is_contiguous() for t in (qweight, scales, expert_ids, x)):
        raise ValueError("qweight, scales, expert_ids and x must be contiguous")
    if tuple(scales.shape) != (E, N, K // GROUP_SIZE) or x.numel() != K:
        raise ValueError("shape mismatch between qweight, scales and x")
    if out is None:
        out = torch.empty((topk, N), dtype=torch.float32, device=qweight.device)
    _need(out, torch.float32, "out", 2)
    if tuple(out.shape) != (topk, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [topk, N] tensor")
    _ok(library().w4a16_moe_gemv(qweight.data_ptr(), scales.data_ptr(), expert_ids.data_ptr(),
                                 topk, E, x.data_ptr(), out.data_ptr(), N, K, GROUP_SIZE,
                                 _stream(stream)), "w4a16_moe_gemv")
    return out


def moe_gemv3(qweight3: torch.Tensor, scales: torch.Tensor, expert_ids: torch.Tensor,
              x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[t] = W3_{expert_ids[t]} x over three-bit experts qweight3 int32 [E, N, 3K/32] (32 codes
    per three words); reads only the selected experts. Returns float32 [topk, N]."""
    _need(qweight3, torch.int32, "qweight3", 3)
    _need(scales, torch.float16, "scales", 3)
    _need(expert_ids, torch.int32, "expert_ids", 1)
    _need(x, torch.bfloat16, "x", 1)
    E, N = qweight3.shape[0], qweight3.shape[1]
    if qweight3.shape[2] % 3:
        raise ValueError("qweight3 rows must hold whole 3-word blocks")
    K = qweight3.shape[2] // 3 * 32
    topk = expert_ids.numel()
    if not all(t.is_contiguous() for t in (qweight3, scales, expert_ids, x)):
        raise ValueError("qweight3, scales, expert_ids and x must be contiguous")
    if tuple(scales.shape) != (E, N, K // GROUP_SIZE) or x.numel() != K:
        raise ValueError("shape mismatch between qweight3, scales and x")
    if out is None:
        out = torch.empty((topk, N), dtype=torch.float32, device=qweight3.device)
    _need(out, torch.float32, "out", 2)
    if tuple(out.shape) != (topk, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [topk, N] tensor")
    _ok(library().w4a16_moe_gemv3(qweight3.data_ptr(), scales.data_ptr(), expert_ids.data_ptr(),
                                  topk, E, x.data_ptr(), out.data_ptr(), N, K, GROUP_SIZE,
                                  _stream(stream)), "w4a16_moe_gemv3")
    return out


def unpack3_debug(qweight3: torch.Tensor, stream=None) -> torch.Tensor:
    """int8 [N, K]: every three-bit code of qweight3 int32 [N, 3K/32], decoded by the GEMV's
    decode steps."""
    _need(qweight3, torch.int32, "qweight3", 2)
    if not qweight3.is_contiguous() or qweight3.shape[1] % 3:
        raise ValueError("qweight3 must be contiguous with whole 3-word blocks per row")
    N, K = qweight3.shape[0], qweight3.shape[1] // 3 * 32
    out = torch.empty((N, K), dtype=torch.int8, device=qweight3.device)
    _ok(library().w4a16_unpack3_debug(qweight3.data_ptr(), out.data_ptr(), N, K,
                                      _stream(stream)), "w4a16_unpack3_debug")
    return out


def describe_moe3_plan(N: int, K: int, topk: int, cus: int = 256) -> str:
    """Launch shape of w4a16_moe_gemv3 (host-only)."""
    buf = ctypes.create_string_buffer(256)
    _ok(library().w4a16_describe_moe3_plan(N, K, topk, cus, buf, len(buf)),
        "w4a16_describe_moe3_plan")
    return buf.value.decode()


def moe_gemv_batched(qweight: torch.Tensor, scales: torch.Tensor, expert_ids: torch.Tensor,
                     X: torch.Tensor, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Y[m, t] = W_{expert_ids[m, t]} X[m] for M <= 16 tokens with their own experts; every
    selected expert is read once. expert_ids int32 [M, topk]; returns float32 [M, topk, N]."""
    _need(qweight, torch.int32, "qweight", 3)
    _need(scales, torch.float16, "scales", 3)
    _need(expert_ids, torch.int32, "expert_ids", 2)
    _need(X, torch.bfloat16, "X", 2)
    E, N, K = qweight.shape[0], qweight.shape[1], qweight.shape[2] * 8
    M, topk = expert_ids.shape
    if not all(t.is_contiguous() for t in (qweight, scales, expert_ids)):
        raise ValueError("qweight, scales and expert_ids must be contiguous")
    if (tuple(scales.shape) != (E, N, K // GROUP_SIZE) or X.shape[0] != M or X.shape[1] < K
            or X.stride(1) != 1):
        raise ValueError("shape mismatch between qweight, scales, expert_ids and X")
    if out is None:
        out = torch.empty((M, topk, N), dtype=torch.float32, device=qweight.device)
    _need(out, torch.float32, "out", 3)
    if tuple(out.shape) != (M, topk, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [M, topk, N] tensor")
    ldx = X.stride(0) if M > 1 else max(X.stride(0), K)
    _ok(library().w4a16_moe_gemv_batched(qweight.data_ptr(), scales.data_ptr(),
                                         expert_ids.data_ptr(), M, topk, E, X.data_ptr(), ldx,
                                         out.data_ptr(), N, K, GROUP_SIZE, _stream(stream)),
        "w4a16_moe_gemv_batched")
    return out


def moe_gemv_swiglu(qweight: torch.Tensor, scales: torch.Tensor, expert_ids: torch.Tensor,
                    x: torch.Tensor, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """h[t] = bf16(silu(W_e[:I] x) * (W_e[I:] x)), e = expert_ids[t], for gate+up experts
    qweight [E, 2I, K/8]. Returns h as torch.bfloat16 [topk, I]."""
    _need(qweight, torch.int32, "qweight", 3)
    _need(scales, torch.float16, "scales", 3)
    _need(expert_ids, torch.int32, "expert_ids", 1)
    _need(x, torch.bfloat16, "x", 1)
    E, N2, K = qweight.shape[0], qweight.shape[1], qweight.shape[2] * 8
    if N2 % 2:
        raise ValueError("gate+up experts need an even number of rows")
    I, topk = N2 // 2, expert_ids.numel()
    if not all(t.is_contiguous() for t in (qweight, scales, expert_ids, x)):
        raise ValueError("qweight, scales, expert_ids and x must be contiguous")
    if tuple(scales.shape) != (E, N2, K // GROUP_SIZE) or x.numel() != K:
        raise ValueError("shape mismatch between qweight, scales and x")
    if out is None:
        out = torch.empty((topk, I), dtype=torch.bfloat16, device=qweight.device)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (topk, I) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [topk, I] tensor")
    _ok(library().w4a16_moe_gemv_swiglu(qweight.data_ptr(), scales.data_ptr(),
                                        expert_ids.data_ptr(), topk, E, x.data_ptr(),
                                        out.data_ptr(), I, K, GROUP_SIZE, _stream(stream)),
        "w4a16_moe_gemv_swiglu")
    return out


def moe_down_combine(qweight: torch.Tensor, scales: torch.Tensor, expert_ids: torch.Tensor,
                     route_weights: torch.Tensor, h: torch.Tensor,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out = sum_t route_weights[t] * W_{expert_ids[t]} h[t] for down experts qweight [E, H, I/8]
    and h bfloat16 [topk, I]. Returns float32 [H]."""
    _need(qweight, torch.int32, "qweight", 3)
    _need(scales, torch.float16, "scales", 3)
    _need(expert_ids, torch.int32, "expert_ids", 1)
    _need(route_weights, torch.float32, "route_weights", 1)
    _need(h, torch.bfloat16, "h", 2)
    E, H, I = qweight.shape[0], qweight.shape[1], qweight.shape[2] * 8
    topk = expert_ids.numel()
    if not all(t.is_contiguous() for t in (qweight, scales, expert_ids, route_weights, h)):
        raise ValueError("all operands must be contiguous")
    if (tuple(scales.shape) != (E, H, I // GROUP_SIZE) or tuple(h.shape) != (topk, I)
            or route_weights.numel() != topk):
        raise ValueError("shape mismatch between qweight, scales, h, ids and weights")
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=qweight.device)
    _need(out, torch.float32, "out", 1)
    if out.numel() != H or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [H] tensor")
    _ok(library().w4a16_moe_down_combine(qweight.data_ptr(), scales.data_ptr(),
                                         expert_ids.data_ptr(), route_weights.data_ptr(), topk,
                                         E, h.data_ptr(), out.data_ptr(), H, I, GROUP_SIZE,
                                         _stream(stream)), "w4a16_moe_down_combine")
    return out


def quantize_pack(w_bf16: torch.Tensor, out=None, stream=None):
    """Quantise bf16 weights [N, >=K] (unit stride along K; K = w.shape[1] unless out says
    otherwise) into (qweight int32 [N, K/8], scales float16 [N, K/128])."""
    _need(w_bf16, torch.bfloat16, "w", 2)
    N = w_bf16.shape[0]
    if w_bf16.stride(1) != 1:
        raise ValueError("w must have unit stride along K")
    if out is None:
        K = w_bf16.shape[1]
        qweight = torch.empty((N, K // 8), dtype=torch.int32, device=w_bf16.device)
        scales = torch.empty((N, K // GROUP_SIZE), dtype=torch.float16, device=w_bf16.device)
    else:
        qweight, scales = out
        K = qweight.shape[1] * 8
    _need(qweight, torch.int32, "qweight", 2)
    _need(scales, torch.float16, "scales", 2)
    if (tuple(qweight.shape) != (N, K // 8) or tuple(scales.shape) != (N, K // GROUP_SIZE)
            or not qweight.is_contiguous() or not scales.is_contiguous()
            or K > w_bf16.shape[1]):
        raise ValueError("qweight [N, K/8] and scales [N, K/128] must be contiguous")
    ldw = w_bf16.stride(0) if N > 1 else max(w_bf16.stride(0), K)
    _ok(library().w4a16_quantize_pack(w_bf16.data_ptr(), ldw, qweight.data_ptr(),
                                      scales.data_ptr(), N, K, GROUP_SIZE, _stream(stream)),
        "w4a16_quantize_pack")
    return qweight, scales


def unpack_debug(qweight: torch.Tensor, stream=None) -> torch.Tensor:
    """int8 [N, K]: the signed value of every packed nibble, decoded by the GEMV unpack."""
    _need(qweight, torch.int32, "qweight", 2)
    if not qweight.is_contiguous():
        raise ValueError("qweight must be contiguous")
    N, K = qweight.shape[0], qweight.shape[1] * 8
    out = torch.empty((N, K), dtype=torch.int8, device=qweight.device)
    _ok(library().w4a16_unpack_debug(qweight.data_ptr(), out.data_ptr(), N, K, _stream(stream)),
        "w4a16_unpack_debug")
    return out


def describe_moe_batched_plan(M: int, N: int, K: int, topk: int, cus: int = 256) -> str:
    """Launch shape of w4a16_moe_gemv_batched (host-only)."""
    buf = ctypes.create_string_buffer(256)
    _ok(library().w4a16_describe_moe_batched_plan(M, N, K, topk, cus, buf, len(buf)),
        "w4a16_describe_moe_batched_plan")
    return buf.value.decode()


def describe_tail_plan(step: int, rows: int, K: int, I: int, topk: int, cus: int = 256) -> str:
    """Launch shape of the expert-tail steps: 0 = SwiGLU gate+up (I, K), 1 = down + combine
    (rows = H, I). Host-only."""
    buf = ctypes.create_string_buffer(256)
    _ok(library().w4a16_describe_tail_plan(step, rows, K, I, topk, cus, buf, len(buf)),
        "w4a16_describe_tail_plan")
    return buf.value.decode()


def describe_plan(M: int, N: int, K: int, topk: int = 0, cus: int = 256) -> str:
    """The kernel and launch shape the library picks for a call (host-only, no device)."""
    buf = ctypes.create_string_buffer(256)
    _ok(library().w4a16_describe_plan(M, N, K, topk, cus, buf, len(buf)), "w4a16_describe_plan")
    return buf.value.decode()


def stream_read(buf: torch.Tensor, nbytes: int, out: torch.Tensor, blocks: int, unroll: int,
                stream=None) -> None:
    """Measurement support: stream `nbytes` bytes of `buf` once (the plain read ceiling).
    out is a uint32-sized tensor (torch.int32) of at least blocks * 4 elements."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous GPU tensor")
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    _need(out, torch.int32, "out", 1)
    if out.numel() < blocks * 4:
        raise ValueError("out needs blocks * 4 elements")
    _ok(library().w4a16_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, unroll,
                                    _stream(stream)), "w4a16_stream_read")
