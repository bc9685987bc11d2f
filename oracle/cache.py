"""Assemble / read the packed cache planes (oracle).

``encode_planes`` runs the oracle encoders over a [B, Hkv, T, d] tensor and writes
the planes in the documented layout (see ``oracle.layout``); ``read_planes``
unpacks one (b, kv-head) slice back to codes and side values.  ``lay`` is any
object with attributes head_dim, k_kind, k_bits, v_kind, v_bits.
"""
from __future__ import annotations

import numpy as np

from . import encode as enc
from . import layout as L


def encode_k(lay, k: np.ndarray, state: dict) -> dict:
    """k: float64 [..., d] -> dict of K planes [..., ...] and band masks."""
    if lay.k_kind == "lm_qjl":
        c, t = state["cb_k"]
        e = enc.encode_k_lm_qjl(k, state["signs_k"], state["S"], c, t)
        aux = np.stack([e["n16"].view(np.uint16), e["g16"].view(np.uint16)], axis=-1)
        return {"k_codes": L.pack_codes(e["idx"], lay.k_bits), "k_signs": L.pack_signs(e["qjl"]),
                "k_aux": aux, "near_idx": e["near_idx"], "near_qjl": e["near_qjl"], "enc": e}
    if lay.k_kind == "f16":
        # V-only mode (MLX page): the key row kept as its 16-bit storage value; k holds
        # values of that type exactly, so the conversion back to bits is exact
        dt = getattr(lay, "in_dtype", "f16")
        if dt == "f16":
            bits = np.asarray(k).astype(np.float16).view(np.uint16)
        else:
            bits = (np.asarray(k).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(_bits_to_f64(bits, dt), np.asarray(k)), "keys not representable in the storage type"
        return {"k_codes": np.ascontiguousarray(bits).view(np.uint32), "near_idx": np.zeros(np.shape(k), bool),
                "enc": {"bits": bits}}
    if lay.k_kind == "lm_mse":
        c, t = state["cb_k"]
        e = enc.encode_k_lm_mse(k, state["signs_k"], c, t)
        return {"k_codes": L.pack_codes(e["idx"], lay.k_bits), "k_aux": e["n32"],
                "near_idx": e["near_idx"], "enc": e}
    if lay.k_kind == "affine8":
        e = enc.encode_k_affine(k, lay.k_bits)
        aux = np.stack([e["a16"].view(np.uint16), e["m16"].view(np.uint16)], axis=-1)
        return {"k_codes": L.pack_codes(e["q"], lay.k_bits), "k_aux": aux,
                "near_idx": e["near_idx"], "enc": e}
    raise ValueError(lay.k_kind)


def encode_v(lay, v: np.ndarray, state: dict) -> dict:
    if lay.v_kind == "group_sym":
        e = enc.encode_v_group_sym(v, lay.v_bits)
        return {"v_codes": L.pack_codes(e["idx"], lay.v_bits), "v_aux": e["scale16"].view(np.uint16),
                "near_idx": e["near_idx"], "enc": e}
    if lay.v_kind == "group_asym":
        e = enc.encode_v_group_asym(v, lay.v_bits)
        aux = np.stack([e["a16"].view(np.uint16), e["m16"].view(np.uint16)], axis=-1)
        return {"v_codes": L.pack_codes(e["idx"], lay.v_bits), "v_aux": aux,
                "near_idx": e["near_idx"], "enc": e}
    if lay.v_kind == "lm_rot":
        c, t = state["cb_v"]
        e = enc.encode_v_lm_rot(v, state["signs_v"], c, t)
        return {"v_codes": L.pack_codes(e["idx"], lay.v_bits), "v_aux": e["n32"],
                "near_idx": e["near_idx"], "enc": e}
    raise ValueError(lay.v_kind)


def _bits_to_f64(bits: np.ndarray, dt: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def read_k(lay, planes: dict, state: dict) -> dict:
    """Unpack K planes of shape [..., W] to codes and float64 side values."""
    d = lay.head_dim
    if lay.k_kind == "f16":
        bits = np.ascontiguousarray(planes["k_codes"], dtype=np.uint32).view(np.uint16)
        return {"k": _bits_to_f64(bits, getattr(lay, "in_dtype", "f16"))}
    if lay.k_kind == "lm_qjl":
        aux = np.asarray(planes["k_aux"], dtype=np.uint16)
        return {"idx": L.unpack_codes(planes["k_codes"], lay.k_bits, d),
                "sigma": np.where(L.unpack_signs(planes["k_signs"], d), 1.0, -1.0),
                "n": aux[..., 0].view(np.float16).astype(np.float64),
                "gamma": aux[..., 1].view(np.float16).astype(np.float64)}
    if lay.k_kind == "lm_mse":
        return {"idx": L.unpack_codes(planes["k_codes"], lay.k_bits, d),
                "n": np.asarray(planes["k_aux"], dtype=np.float32).astype(np.float64)}
    aux = np.asarray(planes["k_aux"], dtype=np.uint16)
    return {"q": L.unpack_codes(planes["k_codes"], lay.k_bits, d),
            "a": aux[..., 0].view(np.float16).astype(np.float64),
            "m": aux[..., 1].view(np.float16).astype(np.float64)}


def read_v(lay, planes: dict, state: dict) -> dict:
    d = lay.head_dim
    idx = L.unpack_codes(planes["v_codes"], lay.v_bits, d)
    if lay.v_kind == "group_sym":
        return {"idx": idx, "scale": np.asarray(planes["v_aux"], dtype=np.uint16).view(np.float16).astype(np.float64)}
    if lay.v_kind == "group_asym":
        aux = np.asarray(planes["v_aux"], dtype=np.uint16)
        return {"idx": idx, "a": aux[..., 0].view(np.float16).astype(np.float64),
                "m": aux[..., 1].view(np.float16).astype(np.float64)}
    return {"idx": idx, "n": np.asarray(planes["v_aux"], dtype=np.float32).astype(np.float64)}


def make_state(lay, signs_k, signs_v, S) -> dict:
    """Oracle state: its own codebooks plus the drawn random numbers (signs, QJL matrix)."""
    from .codebook import codebook_f32
    st = {"signs_k": np.asarray(signs_k), "signs_v": np.asarray(signs_v), "S": np.asarray(S)}
    if lay.k_kind in ("lm_qjl", "lm_mse"):
        st["cb_k"] = codebook_f32(lay.head_dim, lay.k_bits)
    if lay.v_kind == "lm_rot":
        st["cb_v"] = codebook_f32(lay.head_dim, lay.v_bits)
    return st
