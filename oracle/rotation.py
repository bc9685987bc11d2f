"""Randomised Walsh-Hadamard rotation and the seeded state generator (oracle).

Rotation (TurboQuant-MLX page, core technique item 1; vllm-metal TurboQuant guide,
quantisation principle section; TurboQuant vLLM guide section 2 step 1): a vector
is multiplied by a random orthogonal matrix built from the Walsh-Hadamard
transform and a random sign flip,
    Pi = H_d diag(s) / sqrt(d),   s in {+1,-1}^d,
with H_d the Sylvester Hadamard matrix (H_1 = [1], H_2m = [[H, H], [H, -H]]).
The head dimension must be a power of two (64/128/256/512 per the vllm-metal
guide's support-limits section).  H_d is symmetric, so Pi^T = diag(s) H_d / sqrt(d).

The oracle applies Pi as a dense matrix: no fast transform, no fusion.

``reference_rotation_state`` restates the library's documented seeded generator
(SplitMix64 followed by Box-Muller) from the published definitions of those two
algorithms, so the library's ``tq_make_rotation`` can be pinned bit for bit.
"""
from __future__ import annotations

import math

import numpy as np


def sylvester_hadamard(d: int) -> np.ndarray:
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(signs: np.ndarray) -> np.ndarray:
    """Pi = H diag(s) / sqrt(d) as a dense float64 matrix."""
    s = np.asarray(signs, dtype=np.float64)
    d = len(s)
    return sylvester_hadamard(d) * s[None, :] / math.sqrt(d)


# ---------------------------------------------------------------------------
# Seeded state generator (restated from the algorithms' published definitions)
# ---------------------------------------------------------------------------
_M64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64 (Steele, Lea and Flood, 2014): Weyl step, then a 64-bit finaliser."""

    def __init__(self, seed: int):
        self.state = seed & _M64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & _M64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        return z ^ (z >> 31)


def reference_rotation_state(d: int, seed: int):
    """(sign mask words, QJL matrix) as the library documents them.

    * sign words: word w = low 32 bits of the w-th SplitMix64 output
      (bit j%32 of word j/32 set <=> s_j = -1);
    * QJL matrix (row-major, d*d fp16): entries filled in pairs by Box-Muller
      (Box and Muller, 1958) from the next two outputs x1, x2:
      u1 = ((x1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (x2 >> 11) * 2^-53 in [0, 1),
      rho = sqrt(-2 ln u1), pair = (rho cos(2 pi u2), rho sin(2 pi u2)),
      each rounded from float64 to fp16 (nearest even).
    """
    g = SplitMix64(seed)
    words = np.array([g.next() & 0xFFFFFFFF for _ in range(d // 32)], dtype=np.uint32)
    out = np.empty(d * d, dtype=np.float64)
    for i in range(0, d * d, 2):
        x1, x2 = g.next(), g.next()
        u1 = ((x1 >> 11) + 1) * 2.0 ** -53
        u2 = (x2 >> 11) * 2.0 ** -53
        rho = math.sqrt(-2.0 * math.log(u1))
        out[i] = rho * math.cos(2.0 * math.pi * u2)
        out[i + 1] = rho * math.sin(2.0 * math.pi * u2)
    return words, out.astype(np.float16).reshape(d, d)


def mask_to_signs(words: np.ndarray, d: int) -> np.ndarray:
    s = np.ones(d, dtype=np.int8)
    for j in range(d):
        if (int(words[j // 32]) >> (j % 32)) & 1:
            s[j] = -1
    return s
