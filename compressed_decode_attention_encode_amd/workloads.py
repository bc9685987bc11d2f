"""Seeded synthetic workloads for the TurboQuant KV encode / decode path.

This module only draws random numbers and fixes shapes. It holds none of the
method's arithmetic (no rotation, quantisation, packing or attention), so both
the HIP path and the CPU oracle can take their inputs from it without sharing
any of the computation under test.

Every tensor is generated per (batch, kv-head) slice from its own seed, so a
single slice of a large workload can be regenerated exactly without producing
the rest. The random numbers the method itself draws (the rotation sign
vectors and the Gaussian QJL projection) are produced here too and handed to
both sides as inputs.

Workloads stand in for the model geometries the pages quote (Llama-3.2-1B,
Qwen3-0.6B, Qwen2.5-7B and Qwen2.5-32B attention layers); values are synthetic
N(0,1) with the outlier structure described per workload.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Seed roles.  A tensor's seed is (workload seed, role, b, g).
ROLE_K, ROLE_V, ROLE_Q = 0, 1, 2
ROLE_OUTLIER_CH = 5
ROLE_SIGNS_K, ROLE_SIGNS_V, ROLE_QJL = 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_ctx: int            # total cached tokens (compressed + recent buffer)
    n_recent: int         # last n_recent tokens stay exact in the recent buffer
    k_kind: str           # "lm_qjl" | "affine8" | "lm_mse" | "f16" (keys kept 16-bit, k_bits 16)
    k_bits: int
    v_kind: str           # "group_sym" | "lm_rot" | "group_asym" (group-32 min/max)
    v_bits: int
    in_dtype: str         # "f16" | "bf16"   (K/V/Q as produced by the model)
    recent_dtype: str     # "f16"
    outliers: str = "none"   # "none" | "const10" | "studentt3x10"
    n_outlier_ch: int = 0
    flush_tokens: int = 0    # >0: encode in flushes of this many tokens

    @property
    def n_rep(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_compressed(self) -> int:
        return self.n_ctx - self.n_recent

    def scaled(self, n_ctx: int, batch: int | None = None, name: str | None = None) -> "Workload":
        """Same geometry and encoding at a different context length (parity sizes)."""
        n_recent = min(self.n_recent, n_ctx)
        return dataclasses.replace(self, n_ctx=n_ctx, n_recent=n_recent,
                                   batch=self.batch if batch is None else batch,
                                   name=name or f"{self.name}@{n_ctx}")


# The five synthetic workloads.  Names state what they are.
WORKLOADS = {
    "tiny_h1_d128_t512": Workload(
        "tiny_h1_d128_t512", 101, 1, 1, 1, 128, 512, 0,
        "lm_qjl", 3, "group_sym", 2, "f16", "f16"),
    "llama1b_h32x8_d64_t32k": Workload(
        "llama1b_h32x8_d64_t32k", 102, 1, 32, 8, 64, 32768, 128,
        "lm_qjl", 3, "group_sym", 2, "f16", "f16", "const10", 4),
    "qwen0p6b_h16x4_d128_b8_t64k": Workload(
        "qwen0p6b_h16x4_d128_b8_t64k", 103, 8, 16, 4, 128, 65536, 0,
        "affine8", 8, "lm_rot", 3, "f16", "f16"),
    "qwen7b_h28x4_d128_b16_t32k": Workload(
        "qwen7b_h28x4_d128_b16_t32k", 104, 16, 28, 4, 128, 32768, 128,
        "lm_qjl", 3, "group_sym", 2, "bf16", "f16", "studentt3x10", 4, flush_tokens=128),
    "qwen32b_h40x8_d128_b4_t128k": Workload(
        "qwen32b_h40x8_d128_b4_t128k", 105, 4, 40, 8, 128, 131072, 0,
        "lm_qjl", 4, "group_sym", 4, "bf16", "f16"),
    "qwen32b_h40x8_d256_b4_t128k": Workload(
        "qwen32b_h40x8_d256_b4_t128k", 106, 4, 40, 8, 256, 131072, 0,
        "lm_qjl", 4, "group_sym", 4, "bf16", "f16"),
    # the pages' other modes on the same geometries: MSE-only 3-bit keys (no QJL sketch) on
    # the Llama-like layer, and K8+V4 (per-block affine 8-bit keys, rotated 4-bit Lloyd-Max
    # values; the MLX page's mixed mode, quoted on a Qwen2.5-7B at 32K)
    "llama1b_mse3_h32x8_d64_t32k": Workload(
        "llama1b_mse3_h32x8_d64_t32k", 107, 1, 32, 8, 64, 32768, 128,
        "lm_mse", 3, "group_sym", 2, "f16", "f16", "const10", 4),
    # V-only mode (MLX page): keys kept 16-bit, values rotated 3-bit Lloyd-Max
    "llama1b_vonly_h32x8_d64_t32k": Workload(
        "llama1b_vonly_h32x8_d64_t32k", 109, 1, 32, 8, 64, 32768, 128,
        "f16", 16, "lm_rot", 3, "f16", "f16", "const10", 4),
    # the benchmark page's layout under the 2 + 1 bit reading of "3-bit keys" (2 Lloyd-Max
    # bits + the QJL sign) with group-32 min/max 2-bit values, on the Qwen2.5-32B-like geometry
    # (its memory table comes out of this layout: 100 bytes per token and kv-head)
    "qwen32b_r1_h40x8_d128_b4_t32k": Workload(
        "qwen32b_r1_h40x8_d128_b4_t32k", 110, 4, 40, 8, 128, 32768, 128,
        "lm_qjl", 2, "group_asym", 2, "bf16", "f16"),
    # the vllm-metal guide's low-memory row (q4_0 keys, q3_0 values) on the Qwen3-0.6B-like geometry
    "qwen0p6b_q4k_h16x4_d128_b8_t64k": Workload(
        "qwen0p6b_q4k_h16x4_d128_b8_t64k", 111, 8, 16, 4, 128, 65536, 0,
        "affine8", 4, "lm_rot", 3, "f16", "f16"),
    "qwen7b_k8v4_h28x4_d128_b16_t32k": Workload(
        "qwen7b_k8v4_h28x4_d128_b16_t32k", 108, 16, 28, 4, 128, 32768, 128,
        "affine8", 8, "lm_rot", 4, "bf16", "f16", "studentt3x10", 4, flush_tokens=128),
}

# The workload the benchmark line is quoted on (Llama-3.2-1B-like layer, 32K context).
BENCH_WORKLOAD = "llama1b_h32x8_d64_t32k"


# ----------------------------------------------------------------------------------
# dtype helpers (value rounding of the synthetic inputs; no method arithmetic)
# ----------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> uint16 storage bits of fp16 or bf16 (nearest-even)."""
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 storage bits -> exact float64 values."""
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------------

def _rng(wl: Workload, role: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, role, *idx])))


def outlier_channels(wl: Workload, g: int) -> np.ndarray:
    """Channels of kv-head g that carry outliers (distinct, fixed over tokens and batch)."""
    if wl.n_outlier_ch == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(wl, ROLE_OUTLIER_CH, g).choice(wl.head_dim, wl.n_outlier_ch, replace=False))


def kv_slice_f32(wl: Workload, role: int, b: int, g: int, n_tokens: int | None = None) -> np.ndarray:
    """Float32 values of K (role 0) or V (role 1) for slice (b, g): [n_ctx, d] before rounding."""
    T = wl.n_ctx if n_tokens is None else n_tokens
    rng = _rng(wl, role, b, g)
    x = rng.standard_normal((T, wl.head_dim), dtype=np.float32)
    ch = outlier_channels(wl, g)
    if len(ch):
        if wl.outliers == "const10":
            x[:, ch] *= np.float32(10.0)
        elif wl.outliers == "studentt3x10":
            x[:, ch] = (rng.standard_t(3.0, size=(T, len(ch))) * 10.0).astype(np.float32)
        else:
            raise ValueError(wl.outliers)
    # keep every value inside fp16 range so fp16 norms and scales stay finite
    np.clip(x, -6.0e4, 6.0e4, out=x)
    return x


def kv_slice_bits(wl: Workload, role: int, b: int, g: int, n_tokens: int | None = None) -> np.ndarray:
    """Storage bits (uint16, wl.in_dtype) of K or V for slice (b, g): [n_ctx, d]."""
    return to_storage(kv_slice_f32(wl, role, b, g, n_tokens), wl.in_dtype)


def kv_bits(wl: Workload, role: int, threads: int = 8) -> np.ndarray:
    """Full K or V as storage bits [B, Hkv, n_ctx, d] (uint16)."""
    out = np.empty((wl.batch, wl.n_kv_heads, wl.n_ctx, wl.head_dim), dtype=np.uint16)

    def one(bg):
        b, g = bg
        out[b, g] = kv_slice_bits(wl, role, b, g)

    jobs = [(b, g) for b in range(wl.batch) for g in range(wl.n_kv_heads)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, jobs))
    return out


def q_bits(wl: Workload, variant: str = "normal") -> np.ndarray:
    """Decode queries [B, Hq, d] as storage bits.

    variant "normal": N(0,1).  variant "needle": each head's query is a scaled copy
    of one cached key of its kv-head, so one score dominates the softmax (peaked case).
    """
    rng = _rng(wl, ROLE_Q, 0)
    q = rng.standard_normal((wl.batch, wl.n_q_heads, wl.head_dim), dtype=np.float32)
    if variant == "needle":
        pick = rng.integers(0, max(wl.n_compressed, 1), size=(wl.batch, wl.n_q_heads))
        for b in range(wl.batch):
            for g in range(wl.n_kv_heads):
                keys = kv_slice_f32(wl, ROLE_K, b, g)
                for h in range(g * wl.n_rep, (g + 1) * wl.n_rep):
                    k = keys[int(pick[b, h])].astype(np.float64)
                    # q.k/sqrt(d) of the picked key is 12; the other scores stay O(1)
                    alpha = 12.0 * np.sqrt(wl.head_dim) / max(float(np.dot(k, k)), 1e-6)
                    q[b, h] = (alpha * k).astype(np.float32)
    elif variant != "normal":
        raise ValueError(variant)
    return to_storage(q, wl.in_dtype)


def q_bits_multi(wl: Workload, n_query: int) -> np.ndarray:
    """Queries of a multi-query decode step [B, n_query, Hq, d] as storage bits, N(0,1)."""
    rng = _rng(wl, ROLE_Q, 1 + n_query)
    q = rng.standard_normal((wl.batch, n_query, wl.n_q_heads, wl.head_dim), dtype=np.float32)
    return to_storage(q, wl.in_dtype)


def rotation_signs(wl: Workload, which: str) -> np.ndarray:
    """Random sign vector s in {+1,-1}^d of one rotation (shared by all heads and tokens).

    Returned as int8 +1/-1; the C-ABI takes it as a bitmask (bit j set <=> s_j = -1).
    """
    role = ROLE_SIGNS_K if which == "k" else ROLE_SIGNS_V
    bits = _rng(wl, role, 0).integers(0, 2, size=wl.head_dim)
    return np.where(bits == 1, -1, 1).astype(np.int8)


def signs_to_mask(s: np.ndarray) -> np.ndarray:
    """int8 +1/-1 vector -> uint32 words, bit (j mod 32) of word j/32 set where s_j = -1."""
    d = len(s)
    words = np.zeros(d // 32, dtype=np.uint32)
    for j in range(d):
        if s[j] < 0:
            words[j // 32] |= np.uint32(1 << (j % 32))
    return words


def qjl_matrix(wl: Workload) -> np.ndarray:
    """QJL projection S in R^{d x d}, i.i.d. N(0,1) drawn in float64 and stored as fp16
    (rounded to nearest even), row-major."""
    return _rng(wl, ROLE_QJL, 0).standard_normal((wl.head_dim, wl.head_dim)).astype(np.float16)
