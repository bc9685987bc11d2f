"""ctypes binding of libtq.so (include/tq.h) -- argument marshalling only.

Every step of encode and decode runs in the library's HIP kernels.  PyTorch is used
only to own device memory and to name the HIP stream.  If libtq.so has not been
built, importing this module raises immediately: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m compressed_decode_attention_encode_amd.build`")

# Device memory and streams come from torch, so libtq must run on torch's HIP runtime.
# torch ships its own libamdhip64 whose soname matches the one libtq links; importing
# torch first makes the loader bind libtq to that copy instead of loading a second one.
try:
    import torch  # noqa: F401
except ImportError:   # plain C-ABI use without torch: libtq loads the system runtime
    torch = None
_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_loaded():
    try:
        with open(f"/proc/{os.getpid()}/maps") as fh:
            return sorted({ln.split()[-1] for ln in fh if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes_loaded()) > 1:
    raise ImportError(f"two HIP runtimes are loaded in this process: {_hip_runtimes_loaded()}; "
                      "import torch before anything that loads another libamdhip64")

TQ_OK, TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP = 0, -1, -2, -3, -4
TQ_F16, TQ_BF16 = 0, 1
TQ_K_LM_QJL, TQ_K_AFFINE8, TQ_K_LM_MSE, TQ_K_F16 = 0, 1, 2, 3
TQ_V_GROUP_SYM, TQ_V_LM_ROT, TQ_V_GROUP_ASYM = 0, 1, 2

EXPORTED = ("tq_make_codebook", "tq_make_rotation", "tq_cache_plane_bytes", "tq_encode",
            "tq_decode_workspace_bytes", "tq_decode_attn", "tq_decode_multi_workspace_bytes", "tq_decode_attn_multi",
            "tq_materialize", "tq_strerror", "tq_last_error", "tq_probe_stream_read", "tq_decode_attn_noalloc",
            "tq_decode_noalloc_max_scratch_bytes")


class tq_layout(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("k_kind", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_kind", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("recent_dtype", ctypes.c_int32)]


class tq_state(ctypes.Structure):
    _fields_ = [("k_centroids", ctypes.c_void_p), ("k_thresholds", ctypes.c_void_p),
                ("v_centroids", ctypes.c_void_p), ("v_thresholds", ctypes.c_void_p),
                ("k_signs", ctypes.c_void_p), ("v_signs", ctypes.c_void_p), ("qjl", ctypes.c_void_p)]


class tq_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_signs", ctypes.c_void_p), ("k_aux", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_aux", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("capacity", ctypes.c_int32)]


_P = ctypes.c_void_p
_lib.tq_make_codebook.argtypes = [ctypes.c_int, ctypes.c_int, _P, _P, _P]
_lib.tq_make_rotation.argtypes = [ctypes.c_int, ctypes.c_uint64, _P, _P]
_lib.tq_cache_plane_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.c_int, ctypes.c_int, _P]
_lib.tq_encode.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_state), _P, _P, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int, ctypes.POINTER(tq_cache), _P]
_lib.tq_decode_workspace_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.c_int, ctypes.c_int]
_lib.tq_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.tq_decode_attn.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_state), _P, ctypes.POINTER(tq_cache),
                                ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_size_t, _P]
_lib.tq_decode_multi_workspace_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.tq_decode_multi_workspace_bytes.restype = ctypes.c_size_t
_lib.tq_decode_attn_multi.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_state), _P, ctypes.c_int,
                                      ctypes.POINTER(tq_cache), ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int, _P, _P,
                                      ctypes.c_size_t, _P]
_lib.tq_materialize.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_state), ctypes.POINTER(tq_cache),
                                ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_int, _P]
_lib.tq_probe_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.tq_decode_attn_noalloc.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_state), _P,
                                        ctypes.POINTER(tq_cache), ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int, _P,
                                        _P]
_lib.tq_decode_noalloc_max_scratch_bytes.argtypes = []
_lib.tq_decode_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
_lib.tq_strerror.argtypes = [ctypes.c_int]
_lib.tq_strerror.restype = ctypes.c_char_p
_lib.tq_last_error.argtypes = []
_lib.tq_last_error.restype = ctypes.c_char_p


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def _check(rc: int) -> None:
    if rc != TQ_OK:
        raise TQError(rc, tq_last_error())


def _ptr(x) -> int | None:
    """Device/host address of a tensor/array, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(type(x))


def _stream(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream   # torch.cuda.Stream on ROCm: the hipStream_t


# ---------------------------------------------------------------------------- entry points
def tq_strerror(status: int) -> str:
    return _lib.tq_strerror(status).decode()


def tq_last_error() -> str:
    return _lib.tq_last_error().decode()


def tq_make_codebook(head_dim: int, bits: int):
    """-> (centroids float32[2^bits], thresholds float32[2^bits-1], distortion)."""
    L = 1 << bits if 1 <= bits <= 4 else 2
    c = np.zeros(L, dtype=np.float32)
    t = np.zeros(max(L - 1, 1), dtype=np.float32)
    dist = ctypes.c_double(0.0)
    _check(_lib.tq_make_codebook(head_dim, bits, c.ctypes.data, t.ctypes.data, ctypes.addressof(dist)))
    return c, t[:L - 1], dist.value


def tq_make_rotation(head_dim: int, seed: int, with_qjl: bool = True):
    """-> (sign mask uint32[d/32], QJL matrix float16[d, d] or None)."""
    s = np.zeros(max(head_dim // 32, 1), dtype=np.uint32)
    q = np.zeros((head_dim, head_dim), dtype=np.uint16) if with_qjl and head_dim > 0 else None
    _check(_lib.tq_make_rotation(head_dim, seed, s.ctypes.data, None if q is None else q.ctypes.data))
    return s, (None if q is None else q.view(np.float16))


def tq_cache_plane_bytes(layout: tq_layout, batch: int, capacity: int):
    out = (ctypes.c_size_t * 5)()
    _check(_lib.tq_cache_plane_bytes(ctypes.byref(layout), batch, capacity, ctypes.addressof(out)))
    return list(out)


def tq_encode(layout: tq_layout, state: tq_state, k, v, batch: int, n_tokens: int, dst_offset: int,
              cache: tq_cache, stream=None) -> None:
    _check(_lib.tq_encode(ctypes.byref(layout), ctypes.byref(state), _ptr(k), _ptr(v), batch, n_tokens, dst_offset,
                          ctypes.byref(cache), _stream(stream)))


def tq_decode_workspace_bytes(layout: tq_layout, batch: int, max_compressed: int) -> int:
    return int(_lib.tq_decode_workspace_bytes(ctypes.byref(layout), batch, max_compressed))


def tq_decode_attn(layout: tq_layout, state: tq_state, q, cache: tq_cache, n_compressed: int, recent_k, recent_v,
                   n_recent: int, recent_capacity: int, out, workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.tq_decode_attn(ctypes.byref(layout), ctypes.byref(state), _ptr(q), ctypes.byref(cache), n_compressed,
                               _ptr(recent_k), _ptr(recent_v), n_recent, recent_capacity, _ptr(out), _ptr(workspace),
                               workspace_bytes, _stream(stream)))


def tq_decode_attn_noalloc(layout: tq_layout, state: tq_state, q, cache: tq_cache, n_compressed: int, recent_k,
                           recent_v, n_recent: int, recent_capacity: int, out, stream=None) -> None:
    _check(_lib.tq_decode_attn_noalloc(ctypes.byref(layout), ctypes.byref(state), _ptr(q), ctypes.byref(cache),
                                       n_compressed, _ptr(recent_k), _ptr(recent_v), n_recent, recent_capacity,
                                       _ptr(out), _stream(stream)))


def tq_decode_noalloc_max_scratch_bytes() -> int:
    return int(_lib.tq_decode_noalloc_max_scratch_bytes())


def tq_decode_multi_workspace_bytes(layout: tq_layout, batch: int, n_query: int, max_compressed: int) -> int:
    return int(_lib.tq_decode_multi_workspace_bytes(ctypes.byref(layout), batch, n_query, max_compressed))


def tq_decode_attn_multi(layout: tq_layout, state: tq_state, q, n_query: int, cache: tq_cache, n_compressed: int,
                         recent_k, recent_v, n_recent: int, recent_capacity: int, out, workspace, workspace_bytes: int,
                         stream=None) -> None:
    _check(_lib.tq_decode_attn_multi(ctypes.byref(layout), ctypes.byref(state), _ptr(q), n_query, ctypes.byref(cache),
                                     n_compressed, _ptr(recent_k), _ptr(recent_v), n_recent, recent_capacity, _ptr(out),
                                     _ptr(workspace), workspace_bytes, _stream(stream)))


def tq_materialize(layout: tq_layout, state: tq_state, cache: tq_cache, t0: int, n_tokens: int, out_k, out_v,
                   out_dtype: int = TQ_F16, stream=None) -> None:
    _check(_lib.tq_materialize(ctypes.byref(layout), ctypes.byref(state), ctypes.byref(cache), t0, n_tokens,
                               _ptr(out_k), _ptr(out_v), out_dtype, _stream(stream)))


def tq_probe_stream_read(src, nbytes: int, sink, stream=None) -> None:
    """Measurement helper (include/tq_probe.h): one streaming read of `nbytes` device bytes."""
    rc = _lib.tq_probe_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream))
    if rc != TQ_OK:
        raise TQError(rc, "tq_probe_stream_read failed")


# ---------------------------------------------------------------------------- marshalling helpers
_KIND_K = {"lm_qjl": TQ_K_LM_QJL, "affine8": TQ_K_AFFINE8, "lm_mse": TQ_K_LM_MSE, "f16": TQ_K_F16}
_KIND_V = {"group_sym": TQ_V_GROUP_SYM, "lm_rot": TQ_V_LM_ROT, "group_asym": TQ_V_GROUP_ASYM}
_DT = {"f16": TQ_F16, "bf16": TQ_BF16}


def make_layout(head_dim, n_q_heads, n_kv_heads, k_kind, k_bits, v_kind, v_bits, in_dtype="f16",
                recent_dtype="f16") -> tq_layout:
    return tq_layout(head_dim, n_q_heads, n_kv_heads, _KIND_K.get(k_kind, k_kind), k_bits, _KIND_V.get(v_kind, v_kind),
                     v_bits, _DT.get(in_dtype, in_dtype), _DT.get(recent_dtype, recent_dtype))


def layout_of(wl) -> tq_layout:
    """Layout of a workload-like object (attributes as in workloads.Workload)."""
    return make_layout(wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.k_kind, wl.k_bits, wl.v_kind, wl.v_bits,
                       wl.in_dtype, wl.recent_dtype)


@dataclass
class DeviceState:
    """Method state uploaded to the device (torch tensors keep the memory alive)."""
    tensors: dict
    struct: tq_state


def upload_state(layout: tq_layout, signs_k, signs_v, qjl, device="cuda") -> DeviceState:
    """Codebooks from tq_make_codebook plus the given sign masks / QJL matrix, on `device`."""
    import torch
    t = {}
    d = layout.head_dim
    if layout.k_kind in (TQ_K_LM_QJL, TQ_K_LM_MSE):
        c, th, _ = tq_make_codebook(d, layout.k_bits)
        t["k_centroids"] = torch.from_numpy(c).to(device)
        t["k_thresholds"] = torch.from_numpy(th.copy()).to(device)
        t["k_signs"] = torch.from_numpy(np.asarray(signs_k, dtype=np.uint32).view(np.int32).copy()).to(device)
    if layout.k_kind == TQ_K_LM_QJL:
        # fp16 S (a float16 array is passed through; other dtypes are rounded to nearest even)
        t["qjl"] = torch.from_numpy(np.ascontiguousarray(qjl, dtype=np.float16).view(np.int16).copy()).to(device)
    if layout.v_kind == TQ_V_LM_ROT:
        c, th, _ = tq_make_codebook(d, layout.v_bits)
        t["v_centroids"] = torch.from_numpy(c).to(device)
        t["v_thresholds"] = torch.from_numpy(th.copy()).to(device)
        t["v_signs"] = torch.from_numpy(np.asarray(signs_v, dtype=np.uint32).view(np.int32).copy()).to(device)
    st = tq_state(*[(t[n].data_ptr() if n in t else None) for n, _ in tq_state._fields_])
    return DeviceState(t, st)


@dataclass
class DeviceCache:
    planes: dict       # name -> torch.uint8 tensor (flat bytes)
    struct: tq_cache


PLANES = ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")


def alloc_cache(layout: tq_layout, batch: int, capacity: int, device="cuda", fill: int | None = None) -> DeviceCache:
    import torch
    sizes = tq_cache_plane_bytes(layout, batch, capacity)
    planes = {}
    for name, nb in zip(PLANES, sizes):
        if nb == 0:
            continue
        planes[name] = (torch.empty(nb, dtype=torch.uint8, device=device) if fill is None
                        else torch.full((nb,), fill, dtype=torch.uint8, device=device))
    st = tq_cache(*[(planes[n].data_ptr() if n in planes else None) for n in PLANES], batch, capacity)
    return DeviceCache(planes, st)
