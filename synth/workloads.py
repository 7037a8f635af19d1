"""The five synthetic 27B-class workloads of the quantized weight sweep.

Shapes follow the 27B hybrid model described on the Qwen3.8 model pages
(hidden size 5120, MLP width 17408, 64 decoder layers): per layer a fused
q/k/v-style projection 5120 -> 7168, an output projection 5120 -> 5120, a fused
gate+up projection 5120 -> 34816 and a down projection 17408 -> 5120.  Weights
are N(0, 0.02)-distributed fp32 (Irwin-Hall-12 variates, see ``synth.py``),
activations are N(0, 1) rounded to fp16.

Seeds: workload 1 uses seed 0.  Otherwise a matrix of layer L, projection P
in workload C has seed 1_000_000*C + 1_000*L + 10*P, and the activation panel
for inner size K has seed 1_000_000*C + 900_000 + K.  Streams inside a seed
separate weights, outlier mask and activations.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SIGMA = 0.02
# Bernoulli(0.001) outlier mask: threshold floor(0.001 * 2**32) on a 32-bit word.
OUTLIER_THRESH = 4294967
OUTLIER_MULT = 20.0

HIDDEN = 5120
LAYERS = 64
# (name, N = output features, K = input features)
LAYER_PROJS = (
    ("qkv", 7168, 5120),
    ("o", 5120, 5120),
    ("gate_up", 34816, 5120),
    ("down", 5120, 17408),
)


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    N: int
    K: int
    bits: int
    seed: int
    outliers: bool = False

    @property
    def thresh(self) -> int:
        return OUTLIER_THRESH if self.outliers else 0


@dataclass
class Workload:
    cfg: int
    name: str
    matrices: list
    Ms: list
    x_seeds: dict = field(default_factory=dict)

    def x_seed(self, K: int) -> int:
        return self.x_seeds[K]

    @property
    def distinct_K(self):
        return sorted({m.K for m in self.matrices})


def _xseeds(cfg: int, Ks) -> dict:
    if cfg == 1:
        return {k: 0 for k in Ks}
    return {k: 1_000_000 * cfg + 900_000 + k for k in Ks}


def _stack(cfg: int, bits: int, outliers: bool, layers: int = LAYERS) -> list:
    mats = []
    for L in range(layers):
        for P, (name, N, K) in enumerate(LAYER_PROJS):
            mats.append(MatrixSpec(f"L{L}.{name}", N, K, bits,
                                   1_000_000 * cfg + 1_000 * L + 10 * P, outliers))
    return mats


VOCAB = 248320  # output rows of the lm_head-class verify head


FMT_G64 = 0x104   # 4-bit symmetric, one scale per 64 weights
FMT_ZP = 0x204    # 4-bit group-32 asymmetric with 4-bit zero points


def workload(cfg: int, layers: int = LAYERS) -> Workload:
    """Workload ``cfg`` (1..8).  ``layers`` shrinks workloads 4/5/7/8 for tests.
    Workload 6 is the verify head: the lm_head-class matrix 5120 -> 248320,
    4-bit, at M = 6 (one slot, five drafts) and M = 48 (eight such slots).
    Workloads 7 and 8 are the 64-layer stack in the group-64 and the
    zero-point 4-bit formats, swept at M = 1, 8 and 48."""
    if cfg == 1:
        mats = [MatrixSpec("linear", 1024, 1024, 4, 0)]
        return Workload(1, "linear 1024x1024 4-bit M=1", mats, [1], _xseeds(1, [1024]))
    if cfg == 2:
        mats = [MatrixSpec("gate_up", 34816, HIDDEN, 4, 2_000_000)]
        return Workload(2, "gate+up 5120->34816 4-bit M=1", mats, [1], _xseeds(2, [HIDDEN]))
    if cfg == 3:
        mats = [MatrixSpec("gate_up", 34816, HIDDEN, 4, 3_000_000),
                MatrixSpec("down", HIDDEN, 17408, 5, 3_000_010)]
        return Workload(3, "gate+up 4-bit + down 5-bit M=6", mats, [6],
                        _xseeds(3, [HIDDEN, 17408]))
    if cfg == 4:
        mats = _stack(4, 4, True, layers)
        return Workload(4, f"{layers}-layer stack 4-bit M=48", mats, [48],
                        _xseeds(4, [HIDDEN, 17408]))
    if cfg == 5:
        mats = _stack(5, 5, True, layers)
        return Workload(5, f"{layers}-layer stack 5-bit M sweep", mats,
                        [1, 2, 4, 8, 16, 32, 48, 64], _xseeds(5, [HIDDEN, 17408]))
    if cfg == 6:
        mats = [MatrixSpec("lm_head", VOCAB, HIDDEN, 4, 6_000_000)]
        return Workload(6, "verify head 5120->248320 4-bit", mats, [6, 48], _xseeds(6, [HIDDEN]))
    if cfg == 7:
        mats = _stack(7, FMT_G64, True, layers)
        return Workload(7, f"{layers}-layer stack 4-bit group-64 M sweep", mats, [1, 8, 48],
                        _xseeds(7, [HIDDEN, 17408]))
    if cfg == 8:
        mats = _stack(8, FMT_ZP, True, layers)
        return Workload(8, f"{layers}-layer stack 4-bit zero-point M sweep", mats, [1, 8, 48],
                        _xseeds(8, [HIDDEN, 17408]))
    raise ValueError(f"unknown workload {cfg}")


def ragged_slots(M: int, seed: int = 5_000_777) -> list:
    """Slot table for an M-row verify panel: slots with d ~ U{1..6} drafts each
    (1 + d rows), drawn until M rows are covered; the last slot is truncated.
    Rows are independent in the sweep, so this is bookkeeping only."""
    rng = np.random.Generator(np.random.PCG64(seed + M))
    slots, rows = [], 0
    while rows < M:
        d = int(rng.integers(1, 7))
        take = min(1 + d, M - rows)
        slots.append(take)
        rows += take
    return slots


def weight_bytes(bits: int, N: int, K: int) -> int:
    """Algorithmic code + scale bytes of a format (4, 5 or a variant code):
    bits/8 per weight plus one fp16 per group (32, or 64 for the group-64
    format), plus half a byte per group of zero points in the zero-point one."""
    if bits == FMT_G64:
        return N * K // 2 + N * (K // 64) * 2
    if bits == FMT_ZP:
        return N * K // 2 + N * (K // 32) * 2 + N * (K // 32) // 2
    return N * K * bits // 8 + N * (K // 32) * 2
