"""Seeded synthetic inputs for the W4A16 decode GEMV (test and bench infrastructure).

This module only draws random bits. It holds none of the product's arithmetic: no
nibble decoding, no scale application, no dot product. Both the CPU oracle and the
HIP path are fed from it, and nothing else is shared between them.

Storage format (the local-kimi README, technical-detail section, says only that the
fast W4A16 GEMV keeps the reduction axis contiguous and reads packed INT4 weights;
the concrete layout below is the plainest reading of that plus the workload sizes):

  qweight  uint32[N][K/8]      8 signed 4-bit values per word along K, value k=8w+i
                               in bits [4i, 4i+3] of word w (low nibble first),
                               two's complement, no zero point
  scales   fp16 bits [N][K/128] one scale per 128-wide K group, row-major
  x        bf16 bits [K]        (batched: X bf16 bits [M][K])
  MoE      qweight uint32[E][N][K/8], scales fp16 bits [E][N][K/128], ids int32[topk]
  3-bit    qweight3 uint32[E][N][3K/32]: 32 three-bit codes per three words; any bits are
           valid codes, so uniform words give codes uniform over [-4, 3]

Draw recipe, per (config id, seed): numpy PCG64 seeded with [config_id, seed];
draw order words, then scales, then activations, then expert ids.
  * words: uniform uint32, so each nibble is uniform over the 16 codes, i.e. the
    signed value is uniform over [-8, 7];
  * scales: float64 uniform in [0.001, 0.01], rounded to fp16 (round-to-nearest-even);
  * activations: float32 standard normal, rounded to bf16 (round-to-nearest-even);
  * expert ids: uniform without replacement from [0, E).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

GROUP = 128

# Workload shapes: name -> (config id, N, K). The MoE entry is per expert.
SHAPES: Dict[str, Tuple[int, int, int]] = {
    "c1": (1, 1024, 2048),      # single GEMV
    "c2": (2, 4096, 4096),      # dense projection
    "c3a": (31, 28672, 4096),   # fused gate+up projection
    "c3b": (32, 4096, 14336),   # down projection
    "c4": (4, 2048, 2304),      # one MoE expert (fused gate+up); 256 experts, top-8
    "c5a": (51, 8192, 8192),    # square projection, M in {1,2,4,8,16}
    "c5b": (52, 163840, 2304),  # wide output head, M in {1,2,4,8,16}
}
MOE_EXPERTS = 256
MOE_TOPK = 8
# Expert tail after the grouped gate+up product: the c4 experts (2I = 2048 gate+up rows over
# K = 2304) followed by down experts of H = 2304 rows over I = 1024.
TAIL = {"config_id": 41, "E": MOE_EXPERTS, "I": 1024, "H": 2304, "K": 2304, "topk": MOE_TOPK}
BATCH_SIZES = (1, 2, 4, 8, 16)


def rng_for(config_id: int, seed: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(seed)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the 16-bit patterns.

    Only used to turn random normal draws into stored activations; NaN is not
    produced by the draws. The stored bits are the ground truth for both sides.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def draw_words(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)


def draw_scales(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.uniform(0.001, 0.01, size=shape).astype(np.float16).view(np.uint16)


def draw_acts(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclasses.dataclass
class Dense:
    qweight: np.ndarray   # uint32 [N][K/8]
    scales: np.ndarray    # uint16 (fp16 bits) [N][K/128]
    x: np.ndarray         # uint16 (bf16 bits) [M][K] (M=1 for single-token)
    N: int
    K: int
    M: int


@dataclasses.dataclass
class Moe:
    qweight: np.ndarray   # uint32 [E][N][K/8]
    scales: np.ndarray    # uint16 [E][N][K/128]
    x: np.ndarray         # uint16 [K]
    ids: np.ndarray       # int32 [topk]
    E: int
    N: int
    K: int
    topk: int


def dense(N: int, K: int, seed: int, M: int = 1, config_id: int = 0) -> Dense:
    """Dense W4A16 operands of shape N x K with M activation rows."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    rng = rng_for(config_id, seed)
    qw = draw_words(rng, (N, K // 8))
    sc = draw_scales(rng, (N, K // GROUP))
    x = draw_acts(rng, (M, K))
    return Dense(qw, sc, x, N, K, M)


def moe(E: int, N: int, K: int, topk: int, seed: int, config_id: int = 0) -> Moe:
    rng = rng_for(config_id, seed)
    qw = draw_words(rng, (E, N, K // 8))
    sc = draw_scales(rng, (E, N, K // GROUP))
    x = draw_acts(rng, (K,))
    ids = rng.choice(E, size=topk, replace=False).astype(np.int32)
    return Moe(qw, sc, x, ids, E, N, K, topk)


def moe3(E: int, N: int, K: int, topk: int, seed: int, config_id: int = 0) -> Moe:
    """Three-bit grouped-expert operands: Moe with qweight uint32 [E][N][3K/32] (same draw
    order as moe)."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    rng = rng_for(config_id, seed)
    qw = draw_words(rng, (E, N, 3 * K // 32))
    sc = draw_scales(rng, (E, N, K // GROUP))
    x = draw_acts(rng, (K,))
    ids = rng.choice(E, size=topk, replace=False).astype(np.int32)
    return Moe(qw, sc, x, ids, E, N, K, topk)


@dataclasses.dataclass
class MoeTail:
    gu_qweight: np.ndarray    # uint32 [E][2I][K/8], rows [0, I) gate, [I, 2I) up
    gu_scales: np.ndarray     # uint16 [E][2I][K/128]
    x: np.ndarray             # uint16 (bf16) [K]
    ids: np.ndarray           # int32 [topk]
    route_w: np.ndarray       # float32 [topk], positive, summing to about 1
    down_qweight: np.ndarray  # uint32 [E][H][I/8]
    down_scales: np.ndarray   # uint16 [E][H][I/128]
    h: np.ndarray             # uint16 (bf16) [topk][I], an activation draw for the down step alone
    E: int
    I: int
    H: int
    K: int
    topk: int


def moe_tail(E: int, I: int, H: int, K: int, topk: int, seed: int,
             config_id: int = 0) -> MoeTail:
    """Operands of the expert tail. Draw order: gate+up words, gate+up scales, x, ids, router
    weights (uniform in [0.05, 1), then divided by their sum in float64 and stored as float32),
    down words, down scales, h (standard normal rounded to bf16)."""
    if K % GROUP or I % GROUP:
        raise ValueError("K and I must be multiples of 128")
    rng = rng_for(config_id, seed)
    gq = draw_words(rng, (E, 2 * I, K // 8))
    gs = draw_scales(rng, (E, 2 * I, K // GROUP))
    x = draw_acts(rng, (K,))
    ids = rng.choice(E, size=topk, replace=False).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=topk)
    w = (w / w.sum()).astype(np.float32)
    dq = draw_words(rng, (E, H, I // 8))
    ds = draw_scales(rng, (E, H, I // GROUP))
    h = draw_acts(rng, (topk, I))
    return MoeTail(gq, gs, x, ids, w, dq, ds, h, E, I, H, K, topk)


def tail_config(seed: int, experts: Optional[int] = None) -> MoeTail:
    t = TAIL
    return moe_tail(experts or t["E"], t["I"], t["H"], t["K"], t["topk"], seed,
                    config_id=t["config_id"])


def config(name: str, seed: int, M: int = 1, experts: Optional[int] = None):
    """Operands of a named workload (see SHAPES) for a given seed."""
    cid, N, K = SHAPES[name]
    if name == "c4":
        return moe(experts or MOE_EXPERTS, N, K, MOE_TOPK, seed, config_id=cid)
    return dense(N, K, seed, M=M, config_id=cid * 100 + M)


def algorithmic_bytes(N: int, K: int, M: int = 1) -> int:
    """Bytes a W4A16 GEMV must move: packed weights + fp16 scales + bf16 activations."""
    return N * K // 2 + N * (K // GROUP) * 2 + M * K * 2


def algorithmic_bytes3(N: int, K: int, topk: int) -> int:
    """Bytes a one-token three-bit grouped-expert GEMV must move: topk experts' packed codes and
    fp16 scales, the bf16 activation, and the topk ids."""
    return topk * (N * 3 * K // 8 + N * (K // GROUP) * 2) + K * 2 + 4 * topk
