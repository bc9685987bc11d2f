"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the CPU
oracle on the same seeded inputs, and compare them element by element.

Encode: packed indices and QJL sign bits must match bit for bit except elements the
oracle marks as within 1e-6 of a decision threshold (counted and returned); the fp16 n and
gamma of LM+QJL keys within one ulp (counted), every other side value exactly.  Decode: max over (b, h) of max_j |o_gpu - o_ref| /
max_j |o_ref| <= 2e-3, with the GPU decoding the oracle's own packed planes (identical
codes), plus an end-to-end run where each side encodes for itself.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np

from compressed_decode_attention_encode_amd import workloads as W
from oracle import cache as OC
from oracle import decode as OD
from oracle import layout as OL

ATTN_TOL = 2e-3
FILL = 0xAB


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def torch_mod():
    import torch
    return torch


def dev_u16(bits: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def plane_shapes(wl, batch, cap):
    d = wl.head_dim
    wk = d // 2 if wl.k_kind == "f16" else OL.words_for(d, wl.k_bits)   # 16-bit keys: the row itself
    wv = OL.words_for(d, wl.v_bits)
    s = {"k_codes": (np.uint32, (batch, wl.n_kv_heads, cap, wk)),
         "v_codes": (np.uint32, (batch, wl.n_kv_heads, cap, wv))}
    if wl.k_kind == "lm_qjl":
        s["k_signs"] = (np.uint32, (batch, wl.n_kv_heads, cap, d // 32))
        s["k_aux"] = (np.uint16, (batch, wl.n_kv_heads, cap, 2))
    elif wl.k_kind == "lm_mse":
        s["k_aux"] = (np.float32, (batch, wl.n_kv_heads, cap))
    elif wl.k_kind == "f16":
        pass
    else:
        s["k_aux"] = (np.uint16, (batch, wl.n_kv_heads, cap, d // 32, 2))
    if wl.v_kind == "group_sym":
        s["v_aux"] = (np.uint16, (batch, wl.n_kv_heads, cap, d // 32))
    elif wl.v_kind == "group_asym":
        s["v_aux"] = (np.uint16, (batch, wl.n_kv_heads, cap, d // 32, 2))
    else:
        s["v_aux"] = (np.float32, (batch, wl.n_kv_heads, cap))
    return s


def download(cache, wl, batch, cap) -> dict:
    torch_mod().cuda.synchronize()
    out = {}
    for name, (dt, shape) in plane_shapes(wl, batch, cap).items():
        out[name] = cache.planes[name].cpu().numpy().view(dt).reshape(shape)
    return out


def upload_planes(cache, planes: dict):
    torch = torch_mod()
    for name, arr in planes.items():
        if name in cache.planes:
            src = torch.from_numpy(np.ascontiguousarray(arr).view(np.uint8).reshape(-1))
            assert src.numel() == cache.planes[name].numel(), name
            cache.planes[name].copy_(src.cuda())


def upload_slice(cache, wl, planes: dict, b: int, g: int, cap: int):
    """Overwrite slice (b, g) of every plane of a device cache [B][Hkv][cap][row] with the
    given planes of shape [1, 1, cap, ...] (the oracle's encoding of that slice)."""
    torch = torch_mod()
    for name, (dt, shape) in plane_shapes(wl, cache.struct.batch, cap).items():
        if name not in planes or name not in cache.planes:
            continue
        row = int(np.prod(shape[3:], dtype=np.int64)) * np.dtype(dt).itemsize
        src = np.ascontiguousarray(planes[name]).view(np.uint8).reshape(-1)
        assert src.size == cap * row, (name, src.size, cap * row)
        off = ((b * wl.n_kv_heads + g) * cap) * row
        cache.planes[name][off:off + cap * row].copy_(torch.from_numpy(src).cuda())


class Setup:
    """Seeded inputs, GPU state and oracle state of one workload."""

    def __init__(self, wl: W.Workload, signs_from_library: bool = False):
        from compressed_decode_attention_encode_amd import tq
        self.wl = wl
        self.tq = tq
        self.layout = tq.layout_of(wl)
        self.sk = W.rotation_signs(wl, "k")
        self.sv = W.rotation_signs(wl, "v")
        self.S = W.qjl_matrix(wl)
        self.dstate = tq.upload_state(self.layout, W.signs_to_mask(self.sk), W.signs_to_mask(self.sv), self.S)
        self.ostate = OC.make_state(wl, self.sk, self.sv, self.S)

    # --- inputs -------------------------------------------------------------------------
    def kv(self):
        t = time.time()
        K = W.kv_bits(self.wl, W.ROLE_K)
        V = W.kv_bits(self.wl, W.ROLE_V)
        log(f"  inputs {self.wl.name}: {K.shape} in {time.time() - t:.1f}s")
        return K, V

    def recent(self, K, V):
        """Recent buffer (the last n_recent tokens) as recent_dtype bits, [B, Hkv, 128, d] ring slots."""
        wl = self.wl
        R = wl.n_recent
        if R == 0:
            return None, None, 0
        ring = max(R, 1)
        out = []
        for X in (K, V):
            vals = W.storage_to_f64(X[:, :, wl.n_compressed:wl.n_ctx], wl.in_dtype).astype(np.float32)
            assert np.all(np.abs(vals) < 65504.0)
            buf = np.zeros(X.shape[:2] + (ring, wl.head_dim), dtype=np.uint16)
            buf[:, :, :R] = W.to_storage(vals, wl.recent_dtype)
            out.append(buf)
        return out[0], out[1], R

    # --- GPU ---------------------------------------------------------------------------
    def gpu_encode(self, K, V, n_tokens, cap, dst_offset=0, fill=FILL):
        tq = self.tq
        wl = self.wl
        B = K.shape[0]
        cache = tq.alloc_cache(self.layout, B, cap, fill=fill)
        step = wl.flush_tokens or n_tokens
        for off in range(0, n_tokens, step):
            n = min(step, n_tokens - off)
            kd = dev_u16(K[:, :, off:off + n])
            vd = dev_u16(V[:, :, off:off + n])
            tq.tq_encode(self.layout, self.dstate.struct, kd, vd, B, n, dst_offset + off, cache.struct)
        torch_mod().cuda.synchronize()
        return cache

    def gpu_decode(self, cache, Q, n_c, rk=None, rv=None, n_recent=0):
        tq = self.tq
        torch = torch_mod()
        B = Q.shape[0]
        ws_bytes = tq.tq_decode_workspace_bytes(self.layout, B, n_c)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        out = torch.full((B, self.wl.n_q_heads, self.wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        qd = dev_u16(Q)
        rkd = dev_u16(rk) if rk is not None else None
        rvd = dev_u16(rv) if rv is not None else None
        rcap = rk.shape[2] if rk is not None else 0
        tq.tq_decode_attn(self.layout, self.dstate.struct, qd, cache.struct, n_c, rkd, rvd, n_recent, rcap, out, ws,
                          ws_bytes)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    # --- oracle ------------------------------------------------------------------------
    def oracle_encode(self, K, V):
        """K, V storage bits [..., T, d] -> (planes dict, K encoding, V encoding)."""
        wl = self.wl
        ek = OC.encode_k(wl, W.storage_to_f64(K, wl.in_dtype), self.ostate)
        ev = OC.encode_v(wl, W.storage_to_f64(V, wl.in_dtype), self.ostate)
        planes = {n: a for n, a in {**ek, **ev}.items() if n in OL_PLANES}
        return planes, ek, ev

    def oracle_decode(self, planes, Q, n_c, rk=None, rv=None, n_recent=0, heads=None):
        wl = self.wl
        q = W.storage_to_f64(Q, wl.in_dtype)
        rkf = W.storage_to_f64(rk[:, :, :n_recent], wl.recent_dtype) if n_recent else None
        rvf = W.storage_to_f64(rv[:, :, :n_recent], wl.recent_dtype) if n_recent else None
        return OD.decode_attention(wl, q, planes, n_c, self.ostate, rkf, rvf, heads=heads)


OL_PLANES = ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")


def compare_encode(wl, gpu: dict, ek: dict, ev: dict, rows=slice(None)) -> dict:
    """Compare GPU planes (restricted to `rows` of the token axis) with the oracle encoding.

    Returns counts; raises AssertionError on any mismatch outside the exclusion band."""
    d = wl.head_dim
    st = {}
    g = {n: a[:, :, rows] for n, a in gpu.items()}
    if wl.k_kind == "lm_qjl":
        idx = OL.unpack_codes(g["k_codes"], wl.k_bits, d)
        near = ek["near_idx"]
        diff = idx != ek["enc"]["idx"]
        st["k_idx_mismatch"] = int((diff & ~near).sum())
        st["k_idx_excluded"] = int(near.sum())
        st["k_idx_excluded_differ"] = int((diff & near).sum())
        # sign bits: excluded where |z| < band, and for a vector whose LM codes differ
        # (a different index means a different residual)
        sg = OL.unpack_signs(g["k_signs"], d)
        nq = (np.abs(ek["enc"]["z"]) < 1e-6) | np.any(diff, axis=-1, keepdims=True)
        sdiff = sg != ek["enc"]["qjl"]
        st["k_sign_mismatch"] = int((sdiff & ~nq).sum())
        st["k_sign_excluded"] = int(nq.sum())
        st["k_sign_excluded_differ"] = int((sdiff & nq).sum())
        row_ok = ~np.any(diff, axis=-1)
        # fp16 n and gamma within one ulp of the float64 values rounded to fp16 (both are
        # non-negative, so one ulp is a bit-pattern difference of 1); rows whose codes differ
        # have a different residual and are left out
        ulps = np.abs(g["k_aux"].astype(np.int32) - ek["k_aux"].astype(np.int32))
        st["k_aux_mismatch"] = int(((ulps > 1).any(axis=-1) & row_ok).sum())
        st["k_aux_one_ulp"] = int(((ulps == 1).any(axis=-1) & row_ok).sum())
        # whole rows with no excluded element must be identical words (padding bits included)
        st["k_word_mismatch"] = int(((g["k_codes"] != ek["k_codes"]).any(axis=-1) & row_ok).sum())
    elif wl.k_kind == "f16":
        st["k_word_mismatch"] = int((g["k_codes"] != ek["k_codes"]).sum())
    elif wl.k_kind == "lm_mse":
        idx = OL.unpack_codes(g["k_codes"], wl.k_bits, d)
        near = ek["near_idx"]
        diff = idx != ek["enc"]["idx"]
        st["k_idx_mismatch"] = int((diff & ~near).sum())
        st["k_idx_excluded"] = int(near.sum())
        st["k_idx_excluded_differ"] = int((diff & near).sum())
        st["k_aux_mismatch"] = int((g["k_aux"].view(np.uint32) != ek["k_aux"].view(np.uint32)).sum())
    else:
        qa = OL.unpack_codes(g["k_codes"], wl.k_bits, d)
        near = ek["near_idx"]
        diff = qa != ek["enc"]["q"]
        st["k_idx_mismatch"] = int((diff & ~near).sum())
        st["k_idx_excluded"] = int(near.sum())
        st["k_idx_excluded_differ"] = int((diff & near).sum())
        st["k_aux_mismatch"] = int((g["k_aux"] != ek["k_aux"]).sum())
    if wl.v_kind in ("group_sym", "group_asym"):
        vi = OL.unpack_codes(g["v_codes"], wl.v_bits, d)
        near = ev["near_idx"]
        diff = vi != ev["enc"]["idx"]
        st["v_idx_mismatch"] = int((diff & ~near).sum())
        st["v_idx_excluded"] = int(near.sum())
        st["v_idx_excluded_differ"] = int((diff & near).sum())
        st["v_aux_mismatch"] = int((g["v_aux"] != ev["v_aux"]).sum())
    else:
        vi = OL.unpack_codes(g["v_codes"], wl.v_bits, d)
        near = ev["near_idx"]
        diff = vi != ev["enc"]["idx"]
        st["v_idx_mismatch"] = int((diff & ~near).sum())
        st["v_idx_excluded"] = int(near.sum())
        st["v_idx_excluded_differ"] = int((diff & near).sum())
        st["v_aux_mismatch"] = int((g["v_aux"].view(np.uint32) != ev["v_aux"].view(np.uint32)).sum())
    for k, v in st.items():
        if k.endswith("mismatch"):
            assert v == 0, (wl.name, st)
    return st


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over (b, h) of max_j |out - ref| / max_j |ref| (rows of ref that are NaN are skipped)."""
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            r = ref[b, h]
            if np.isnan(r).any():
                continue
            assert np.all(np.isfinite(out[b, h])), (b, h)
            worst = max(worst, float(np.max(np.abs(out[b, h] - r)) / max(np.max(np.abs(r)), 1e-300)))
    return worst


def untouched(gpu: dict, rows_written: slice, cap: int) -> bool:
    """Slots outside the written token range still hold the fill byte."""
    ok = True
    for n, a in gpu.items():
        raw = a.view(np.uint8).reshape(a.shape[0], a.shape[1], cap, -1)
        mask = np.ones(cap, dtype=bool)
        mask[rows_written] = False
        ok &= bool(np.all(raw[:, :, mask] == FILL))
    return ok
