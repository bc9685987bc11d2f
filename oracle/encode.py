"""TurboQuant encode (oracle): per-vector quantisers, in the pages' order.

Inputs are the exact float64 values of the fp16/bf16 K/V vectors, shape (..., d).
Every function also returns which decisions sit within ``BAND`` (1e-6) of a
decision threshold, measured in that quantiser's normalised input; the GPU
comparison excludes exactly those and reports how many there were.

Keys, LM + QJL (TurboQuant vLLM guide, section 2 steps 1-3; TurboQuant benchmark
page, compression algorithm details): rotate, quantise every coordinate with the
Lloyd-Max codebook, then keep one sign bit per dimension of a Gaussian projection
of the quantisation residual so that the inner-product estimate is unbiased.

Values, group-32 symmetric (TurboQuant vLLM guide, section 2 step 4): each group
of 32 consecutive channels gets one scale and symmetric 2- or 4-bit levels.

Values, group-32 min/max (TurboQuant benchmark page, compression algorithm details:
values keep a per-group minimum and maximum): each group of 32 channels gets an
fp16 step a = (max - min)/(L-1) and offset m = min, and codes 0 .. L-1 -- the same
quantiser as the per-block affine keys below, at 2 or 4 bits.

Keys, per-block affine 8-bit (and 5/4/2-bit, the guide's compression-ratio table) and
values, rotated Lloyd-Max 3-bit (vllm-metal TurboQuant guide, quantisation principle
table): keys keep their own scale and offset per block with no rotation; values are
rotated, then mapped to the 8-centroid codebook.

Readings where the pages are silent (each also listed in the design notes):
  * the vector is normalised before rotation; its norm n (and the residual norm
    gamma) are kept as fp16, rounded to nearest-even; the rotated-LM value norm is fp32;
  * LM decision: idx_j = #{i : t_i < y_j} with float32 thresholds t_i (ties go low);
  * the QJL projection acts on the rotated-domain residual r = y - c[idx];
    S is d x d i.i.d. N(0,1) (any S passed in is used exactly as given); stored
    bit = (z_j >= 0), z = S r, with z evaluated in float64 on the float64 residual;
  * group scale Delta = fp16(2 amax / (L-1)), idx = clamp(rne(v/Delta + (L-1)/2), 0, L-1)
    with the stored Delta; Delta = 0 gives idx = L-1, 0, L/2 for v > 0, v < 0, v = 0;
  * affine scale a = fp16((max-min)/(2^b-1)), offset m = fp16(min), q = clamp(rne((k-m)/a), 0, 2^b-1)
    for keys of b = 8, 5, 4, 2 bits; a = 0 gives q = 0; min/max values alike with L - 1 = 3 or 15;
  * a quotient lying exactly on a half-integer is an exact tie, decided by round-half-
    to-even and compared like any other element; only inexact values within BAND of a
    boundary are marked near.  Exact ties are common with fp16 inputs (a value that is
    an exact multiple of the stored scale), and they are detected in exact arithmetic:
    the doubled quotient is an integer r with r * scale reproducing the doubled numerator.
"""
from __future__ import annotations

import numpy as np

from .rotation import rotation_matrix

BAND = 1e-6


def _exact_half(num: np.ndarray, den: np.ndarray, off: float) -> np.ndarray:
    """num/den + off lies exactly on a half-integer (num, den dyadic; num exact in float64).

    2 num/den + 2 off must be an odd integer r' ; with r = 2 num/den rounded to an integer,
    r * den == 2 num is an exact float64 identity for the small integers involved.
    """
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(2.0 * num / den)
        exact = (den != 0) & (r * den == 2.0 * num)
    odd = np.mod(r + 2.0 * off, 2.0) == 1.0
    return exact & odd


def _lm_decide(y: np.ndarray, thresholds32: np.ndarray):
    t = thresholds32.astype(np.float64)
    idx = np.zeros(y.shape, dtype=np.int64)
    near = np.zeros(y.shape, dtype=bool)
    for ti in t:
        idx += (y > ti)
        near |= np.abs(y - ti) < BAND
    return idx, near


def encode_k_lm_qjl(k: np.ndarray, signs: np.ndarray, S: np.ndarray,
                    centroids32: np.ndarray, thresholds32: np.ndarray) -> dict:
    d = k.shape[-1]
    # norm and unit vector
    n = np.sqrt(np.sum(k * k, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[..., None] > 0, k / safe[..., None], 0.0)
    # step 1: random rotation
    y = u @ rotation_matrix(signs).T
    # step 2: Lloyd-Max indices
    idx, near_lm = _lm_decide(y, thresholds32)
    # step 3: residual and its sign sketch
    r = y - centroids32.astype(np.float64)[idx]
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    z = r @ np.asarray(S, dtype=np.float64).T
    bits = z >= 0
    near_qjl = np.abs(z) < BAND
    # a vector with a near-threshold LM index may legitimately differ in its residual,
    # so all of its sign bits are excluded too
    near_qjl |= np.any(near_lm, axis=-1, keepdims=True)
    return {
        "idx": idx, "qjl": bits,
        "n16": n.astype(np.float16), "g16": gamma.astype(np.float16),
        "near_idx": near_lm, "near_qjl": near_qjl,
        "y": y, "z": z,
    }


def encode_v_group_sym(v: np.ndarray, bits: int) -> dict:
    d = v.shape[-1]
    L = 1 << bits
    vg = v.reshape(v.shape[:-1] + (d // 32, 32))
    amax = np.max(np.abs(vg), axis=-1)
    scale16 = (2.0 * amax / (L - 1)).astype(np.float16)
    delta = scale16.astype(np.float64)[..., None]
    off = (L - 1) / 2.0
    with np.errstate(divide="ignore", invalid="ignore"):
        x = vg / delta + off
    idx = np.clip(np.rint(x), 0, L - 1)
    zero = np.broadcast_to(delta == 0, vg.shape)
    idx = np.where(zero, np.where(vg > 0, L - 1, np.where(vg < 0, 0, L // 2)), idx).astype(np.int64)
    frac = x - np.floor(x)
    near = (~zero) & (np.abs(frac - 0.5) < BAND) & ~_exact_half(vg, delta, (L - 1) / 2.0)
    return {"idx": idx.reshape(v.shape), "scale16": scale16,
            "near_idx": near.reshape(v.shape)}


def _group_minmax(x: np.ndarray, top: int):
    """Per group of 32: a = fp16((max-min)/top), m = fp16(min), q = clamp(rne((x-m)/a), 0, top)
    with the stored a and m (a = 0: q = 0)."""
    d = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (d // 32, 32))
    lo = np.min(xg, axis=-1)
    hi = np.max(xg, axis=-1)
    a16 = ((hi - lo) / float(top)).astype(np.float16)
    m16 = lo.astype(np.float16)
    a = a16.astype(np.float64)[..., None]
    m = m16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        xq = (xg - m) / a
    q = np.where(a == 0, 0, np.clip(np.rint(xq), 0, top)).astype(np.int64)
    frac = xq - np.floor(xq)
    near = (a != 0) & (np.abs(frac - 0.5) < BAND) & ~_exact_half(xg - m, a, 0.0)
    return q.reshape(x.shape), a16, m16, near.reshape(x.shape)


def encode_k_affine(k: np.ndarray, bits: int = 8) -> dict:
    """Per-block affine keys (vllm-metal guide, quantisation principle and compression-ratio
    table: q8_0, q5_0, q4_0 and the 2-bit uint2/int2 keys): per block of 32, a = fp16((max -
    min)/(2^bits - 1)), m = fp16(min), q = clamp(rne((k - m)/a), 0, 2^bits - 1)."""
    q, a16, m16, near = _group_minmax(k, (1 << bits) - 1)
    return {"q": q, "a16": a16, "m16": m16, "near_idx": near}


def encode_v_group_asym(v: np.ndarray, bits: int) -> dict:
    """Group-32 min/max values (benchmark page): v_hat = m + a idx."""
    idx, a16, m16, near = _group_minmax(v, (1 << bits) - 1)
    return {"idx": idx, "a16": a16, "m16": m16, "near_idx": near}


def encode_k_lm_mse(k: np.ndarray, signs: np.ndarray,
                    centroids32: np.ndarray, thresholds32: np.ndarray) -> dict:
    """MSE-only keys (vLLM guide section 2, steps 1-2 without the QJL residual step): the
    norm, the rotation and the Lloyd-Max decision, exactly the steps of the rotated values
    below, with the key rotation and codebook."""
    return encode_v_lm_rot(k, signs, centroids32, thresholds32)


def encode_v_lm_rot(v: np.ndarray, signs: np.ndarray,
                    centroids32: np.ndarray, thresholds32: np.ndarray) -> dict:
    n = np.sqrt(np.sum(v * v, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[..., None] > 0, v / safe[..., None], 0.0)
    y = u @ rotation_matrix(signs).T
    idx, near = _lm_decide(y, thresholds32)
    return {"idx": idx, "n32": n.astype(np.float32), "near_idx": near, "y": y}
