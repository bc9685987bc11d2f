"""Bit packing and plane sizes of the packed cache (oracle's own packer/unpacker).

Packing (TurboQuant vLLM guide, section 2 step 5: 2-bit codes four to a byte;
TurboQuant-MLX page, core technique item 3: ten 3-bit indices per uint32):

* codes of b bits are packed little-endian into uint32 words, code j in bits
  [b*(j mod P), b*(j mod P) + b) of word floor(j / P), with P = 16, 10, 8 codes
  per word for b = 2, 3, 4 (for b = 3 bits 30..31 of each word stay zero);
* affine 8-bit codes: one byte per code, byte j of the row (4 per word, LSB first);
* affine 5-bit codes: two planes in the row -- d/8 words of low nibbles (code j's low 4 bits
  at bits 4 (j mod 8) of word floor(j / 8)), then d/32 words of fifth bits (code j's bit 4
  at bit j mod 32 of word d/8 + floor(j / 32)); 5 bits per code, no padding;
* affine 4- and 2-bit codes pack like the other 4- and 2-bit codes;
* QJL signs: bit (j mod 32) of word floor(j / 32) is 1 iff the projection is >= 0.

Planes (all token-major, [B][Hkv][capacity][...]):
  k_codes u32[W_k]; k_signs u32[d/32] (LM+QJL keys only);
  k_aux   fp16 (n, gamma) for LM+QJL keys, fp16 (scale, min) per 32-block for affine keys;
  v_codes u32[W_v];
  v_aux   fp16 scale per 32-group for group values, fp32 norm for rotated-LM values.
"""
from __future__ import annotations

import numpy as np

CODES_PER_WORD = {2: 16, 3: 10, 4: 8}


def words_for(d: int, bits: int) -> int:
    if bits == 8:
        return d // 4
    if bits == 5:
        return d // 8 + d // 32
    p = CODES_PER_WORD[bits]
    return -(-d // p)


def _pack5(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint64)
    d = codes.shape[-1]
    assert d % 32 == 0 and codes.max(initial=0) < 32
    out = np.zeros(codes.shape[:-1] + (d // 8 + d // 32,), dtype=np.uint64)
    for j in range(d):
        out[..., j // 8] |= (codes[..., j] & np.uint64(15)) << np.uint64(4 * (j % 8))
        out[..., d // 8 + j // 32] |= (codes[..., j] >> np.uint64(4)) << np.uint64(j % 32)
    return out.astype(np.uint32)


def _unpack5(words: np.ndarray, d: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    out = np.empty(w.shape[:-1] + (d,), dtype=np.int64)
    for j in range(d):
        lo = (w[..., j // 8] >> np.uint64(4 * (j % 8))) & np.uint64(15)
        hi = (w[..., d // 8 + j // 32] >> np.uint64(j % 32)) & np.uint64(1)
        out[..., j] = lo | (hi << np.uint64(4))
    return out


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """(..., d) integer codes -> (..., W) uint32 words."""
    if bits == 5:
        return _pack5(codes)
    codes = np.asarray(codes, dtype=np.uint64)
    d = codes.shape[-1]
    if bits == 8:
        per, width = 4, 8
    else:
        per, width = CODES_PER_WORD[bits], bits
    assert codes.max(initial=0) < (1 << width)
    nw = -(-d // per)
    out = np.zeros(codes.shape[:-1] + (nw,), dtype=np.uint64)
    for j in range(d):
        out[..., j // per] |= codes[..., j] << np.uint64(width * (j % per))
    return out.astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    if bits == 5:
        return _unpack5(words, d)
    words = np.asarray(words, dtype=np.uint64)
    if bits == 8:
        per, width = 4, 8
    else:
        per, width = CODES_PER_WORD[bits], bits
    mask = np.uint64((1 << width) - 1)
    out = np.empty(words.shape[:-1] + (d,), dtype=np.int64)
    for j in range(d):
        out[..., j] = (words[..., j // per] >> np.uint64(width * (j % per))) & mask
    return out


def pack_signs(bits_set: np.ndarray) -> np.ndarray:
    """(..., d) bool -> (..., d/32) uint32."""
    b = np.asarray(bits_set, dtype=np.uint64)
    d = b.shape[-1]
    out = np.zeros(b.shape[:-1] + (d // 32,), dtype=np.uint64)
    for j in range(d):
        out[..., j // 32] |= b[..., j] << np.uint64(j % 32)
    return out.astype(np.uint32)


def unpack_signs(words: np.ndarray, d: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    out = np.empty(w.shape[:-1] + (d,), dtype=bool)
    for j in range(d):
        out[..., j] = ((w[..., j // 32] >> np.uint64(j % 32)) & np.uint64(1)) == 1
    return out


def bytes_per_token_head(d: int, k_kind: str, k_bits: int, v_kind: str, v_bits: int) -> dict:
    """Bytes of each plane for one token of one kv-head."""
    if k_kind == "lm_qjl":
        k = {"k_codes": 4 * words_for(d, k_bits), "k_signs": d // 8, "k_aux": 4}
    elif k_kind == "f16":
        k = {"k_codes": 2 * d, "k_signs": 0, "k_aux": 0}
    elif k_kind == "lm_mse":
        k = {"k_codes": 4 * words_for(d, k_bits), "k_signs": 0, "k_aux": 4}
    elif k_kind == "affine8":
        # per-block affine keys at k_bits 8 / 5 / 4 / 2, one (scale, min) fp16 pair per 32
        k = {"k_codes": 4 * words_for(d, k_bits), "k_signs": 0, "k_aux": (d // 32) * 4}
    else:
        raise ValueError(k_kind)
    if v_kind == "group_sym":
        v = {"v_codes": 4 * words_for(d, v_bits), "v_aux": (d // 32) * 2}
    elif v_kind == "group_asym":
        v = {"v_codes": 4 * words_for(d, v_bits), "v_aux": (d // 32) * 4}
    elif v_kind == "lm_rot":
        v = {"v_codes": 4 * words_for(d, v_bits), "v_aux": 4}
    else:
        raise ValueError(v_kind)
    return {**k, **v}


def compression_ratio(d: int, k_kind: str, k_bits: int, v_kind: str, v_bits: int) -> float:
    """fp16 K+V bytes (4d) over packed bytes, per token and kv-head."""
    return 4.0 * d / sum(bytes_per_token_head(d, k_kind, k_bits, v_kind, v_bits).values())
