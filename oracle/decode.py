"""Single-query decode attention on the packed cache (oracle, float64).

For query head h of batch b, with kv-head g = floor(h / n_rep) (GQA: the n_rep
query heads of a group read the same cached keys and values; TurboQuant-MLX
page, GPU kernel optimisation section, n_rep item):

  compressed tokens t < N_c, LM+QJL keys (TurboQuant vLLM guide, section 2: the
  unbiased inner-product estimate; TurboQuant-MLX page: the query is rotated once
  and scored against the rotated codes):
      q_r = Pi q,  q_s = S q_r,
      s_t = n_t / sqrt(d) * ( <q_r, c[idx_t]> + gamma_t sqrt(pi/2)/d <q_s, sigma_t> )
  compressed tokens, affine keys:   s_t = <q, m + a * q_t> / sqrt(d)
  recent-buffer tokens (exact fp16; TurboQuant vLLM guide section 5, benchmark page
  buffering strategy):             s_r = <q, k_r> / sqrt(d)
  p = softmax over all N_c + R scores;
  group values:        out = sum_t p_t Delta_t (idx_t - (L-1)/2) + sum_r p_r v_r
  min/max values:      out = sum_t p_t (m_t + a_t idx_t) + sum_r p_r v_r  (per 32-group a, m)
  rotated-LM values:   out = Pi_v^T ( sum_t p_t n_t c[idx_t] ) + sum_r p_r v_r
  (the weighted sum is formed in the rotated domain and rotated back once:
  TurboQuant-MLX page, GPU kernel optimisation section, butterfly item).

``decode_attention_bruteforce`` instead reconstructs every key and value vector
explicitly in the natural domain and runs plain softmax attention; the two must
agree to rounding.  ``exact_attention`` is plain attention on the original values.
"""
from __future__ import annotations

import math

import numpy as np

from . import cache as C
from .rotation import rotation_matrix


def _slice(planes: dict, b: int, g: int, n: int) -> dict:
    return {k: np.asarray(v)[b, g, :n] for k, v in planes.items()
            if k in ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")}


def _scores_compressed(lay, q: np.ndarray, kd: dict, state: dict) -> np.ndarray:
    d = lay.head_dim
    if lay.k_kind == "lm_qjl":
        c = state["cb_k"][0].astype(np.float64)
        q_r = rotation_matrix(state["signs_k"]) @ q
        q_s = state["S"].astype(np.float64) @ q_r
        lm = c[kd["idx"]] @ q_r
        qjl = kd["sigma"] @ q_s
        return kd["n"] / math.sqrt(d) * (lm + kd["gamma"] * math.sqrt(math.pi / 2.0) / d * qjl)
    if lay.k_kind == "f16":
        # 16-bit keys (V-only mode): the plain scaled dot product
        return kd["k"] @ q / math.sqrt(d)
    if lay.k_kind == "lm_mse":
        # MSE-only keys: the codebook term alone, n / sqrt(d) <Pi q, c[idx]>
        c = state["cb_k"][0].astype(np.float64)
        q_r = rotation_matrix(state["signs_k"]) @ q
        return kd["n"] / math.sqrt(d) * (c[kd["idx"]] @ q_r)
    # per-block affine keys: k_hat = m + a * q per 32-block
    k_hat = _affine_k_hat(kd, d)
    return k_hat @ q / math.sqrt(d)


def _affine_k_hat(kd: dict, d: int) -> np.ndarray:
    a = np.repeat(kd["a"], 32, axis=-1)
    m = np.repeat(kd["m"], 32, axis=-1)
    return m + a * kd["q"]


def _v_hat_group(lay, vd: dict) -> np.ndarray:
    if lay.v_kind == "group_asym":
        return np.repeat(vd["m"], 32, axis=-1) + np.repeat(vd["a"], 32, axis=-1) * vd["idx"]
    Lv = 1 << lay.v_bits
    scale = np.repeat(vd["scale"], 32, axis=-1)
    return scale * (vd["idx"] - (Lv - 1) / 2.0)


def decode_attention(lay, q: np.ndarray, planes: dict, n_compressed: int, state: dict,
                     recent_k: np.ndarray | None = None, recent_v: np.ndarray | None = None,
                     heads: list | None = None) -> np.ndarray:
    """q: float64 [B, Hq, d]; planes: packed [B, Hkv, cap, ...]; recent_*: float64 [B, Hkv, R, d].

    Returns float64 [B, Hq, d] (rows not listed in ``heads`` -- (b, h) pairs -- are NaN).
    """
    B, Hq, d = q.shape
    n_rep = lay.n_q_heads // lay.n_kv_heads
    R = 0 if recent_k is None else recent_k.shape[2]
    out = np.full((B, Hq, d), np.nan)
    want = None if heads is None else set(map(tuple, heads))
    for b in range(B):
        for g in range(lay.n_kv_heads):
            hs = [h for h in range(g * n_rep, (g + 1) * n_rep) if want is None or (b, h) in want]
            if not hs:
                continue
            sl = _slice(planes, b, g, n_compressed)
            kd = C.read_k(lay, sl, state) if n_compressed else None
            vd = C.read_v(lay, sl, state) if n_compressed else None
            for h in hs:
                parts = []
                if n_compressed:
                    parts.append(_scores_compressed(lay, q[b, h], kd, state))
                if R:
                    parts.append(recent_k[b, g] @ q[b, h] / math.sqrt(d))
                s = np.concatenate(parts)
                p = np.exp(s - np.max(s))
                p /= np.sum(p)
                pc, pr = p[:n_compressed], p[n_compressed:]
                o = np.zeros(d)
                if n_compressed:
                    if lay.v_kind in ("group_sym", "group_asym"):
                        o += pc @ _v_hat_group(lay, vd)
                    else:
                        c = state["cb_v"][0].astype(np.float64)
                        acc_rot = (pc * vd["n"]) @ c[vd["idx"]]
                        o += rotation_matrix(state["signs_v"]).T @ acc_rot
                if R:
                    o += pr @ recent_v[b, g]
                out[b, h] = o
    return out


def decode_attention_multi(lay, q: np.ndarray, planes: dict, n_compressed: int, state: dict,
                           recent_k: np.ndarray, recent_v: np.ndarray) -> np.ndarray:
    """Several consecutive queries per step (vllm-metal guide, prefill section: a short suffix
    or the draft tokens of speculative verification read the compressed cache directly).

    q: float64 [B, NQ, Hq, d]; recent_*: float64 [B, Hkv, R, d] whose last NQ tokens are the
    queries' own keys/values, in order.  Query j attends to every compressed token and to
    recent tokens 0 .. R - NQ + j (causal inside the suffix): it is the single-query decode
    with the recent buffer cut after its own token.  Returns float64 [B, NQ, Hq, d].
    """
    B, NQ, Hq, d = q.shape
    R = recent_k.shape[2]
    assert R >= NQ, "the queries' own tokens are the last NQ recent tokens"
    out = np.empty((B, NQ, Hq, d))
    for j in range(NQ):
        lim = R - NQ + j + 1
        out[:, j] = decode_attention(lay, q[:, j], planes, n_compressed, state, recent_k[:, :, :lim], recent_v[:, :, :lim])
    return out


def reconstruct_k(lay, kd: dict, state: dict) -> np.ndarray:
    """Explicit natural-domain key estimate n Pi^T (c[idx] + gamma sqrt(pi/2)/d S^T sigma)."""
    d = lay.head_dim
    if lay.k_kind == "affine8":
        return _affine_k_hat(kd, d)
    if lay.k_kind == "f16":
        return kd["k"]
    c = state["cb_k"][0].astype(np.float64)
    if lay.k_kind == "lm_mse":
        return kd["n"][:, None] * (c[kd["idx"]] @ rotation_matrix(state["signs_k"]))
    S = state["S"].astype(np.float64)
    rot = c[kd["idx"]] + kd["gamma"][:, None] * math.sqrt(math.pi / 2.0) / d * (kd["sigma"] @ S)
    return kd["n"][:, None] * (rot @ rotation_matrix(state["signs_k"]))


def reconstruct_v(lay, vd: dict, state: dict) -> np.ndarray:
    if lay.v_kind in ("group_sym", "group_asym"):
        return _v_hat_group(lay, vd)
    c = state["cb_v"][0].astype(np.float64)
    return vd["n"][:, None] * (c[vd["idx"]] @ rotation_matrix(state["signs_v"]))


def decode_attention_bruteforce(lay, q, planes, n_compressed, state, recent_k=None, recent_v=None):
    B, Hq, d = q.shape
    n_rep = lay.n_q_heads // lay.n_kv_heads
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for g in range(lay.n_kv_heads):
            sl = _slice(planes, b, g, n_compressed)
            K = [reconstruct_k(lay, C.read_k(lay, sl, state), state)] if n_compressed else []
            V = [reconstruct_v(lay, C.read_v(lay, sl, state), state)] if n_compressed else []
            if recent_k is not None and recent_k.shape[2]:
                K.append(recent_k[b, g])
                V.append(recent_v[b, g])
            K, V = np.concatenate(K), np.concatenate(V)
            for h in range(g * n_rep, (g + 1) * n_rep):
                out[b, h] = exact_attention_1(q[b, h], K, V)
    return out


def exact_attention_1(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    s = K @ q / math.sqrt(q.shape[-1])
    p = np.exp(s - np.max(s))
    return (p / np.sum(p)) @ V


def exact_attention(lay, q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Plain softmax attention of q [B,Hq,d] over the original k, v [B,Hkv,T,d] (float64)."""
    B, Hq, d = q.shape
    n_rep = lay.n_q_heads // lay.n_kv_heads
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            out[b, h] = exact_attention_1(q[b, h], k[b, g], v[b, g])
    return out
