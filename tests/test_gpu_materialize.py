"""GPU parity of tq_materialize against the oracle's explicit reconstruction.

The GPU dequantises the oracle's packed planes (identical codes) and its fp16 / bf16 rows
are compared with the oracle's float64 reconstruction:

  * group-scaled values are exact in float32 (a fp16 scale times a half-integer), so
    the GPU's rounded row must equal the reference rounded to the output type, bit for
    bit;
  * the other kinds go through float32 arithmetic (butterflies, the S^T sigma sums,
    m + a q).  Its error is relative to the row's scale, not to each element: a float32
    emulation of the kernel's steps on the tiny workload lands within 1.1e-7 x max|row|
    of the float64 reference.  A GPU element may therefore differ from the rounded
    reference by one output ulp where the reference lies near a rounding boundary, and
    small elements (far below the row's largest) by that absolute float32 error.  The
    bound asserted is |gpu - ref| <= ulp(ref) + 2^-20 max|ref row| (8x the emulated
    error), and the count of elements that are not the nearest value is logged.
"""
import dataclasses

import numpy as np
import pytest

from compressed_decode_attention_encode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _gpu_ok():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


if not _gpu_ok():
    pytest.skip("no GPU", allow_module_level=True)

import gpu_harness as H  # noqa: E402
from oracle import cache as OC  # noqa: E402
from oracle import decode as OD  # noqa: E402

FMT = {"f16": 0, "bf16": 1}


def ref_rows(s, planes, b, g, t0, n, half):
    """Oracle float64 reconstruction of rows [t0, t0 + n) of slice (b, g)."""
    sl = {k: np.asarray(v)[b, g, t0:t0 + n] for k, v in planes.items() if k in H.OL_PLANES}
    if half == "k":
        return OD.reconstruct_k(s.wl, OC.read_k(s.wl, sl, s.ostate), s.ostate)
    return OD.reconstruct_v(s.wl, OC.read_v(s.wl, sl, s.ostate), s.ostate)


def bits_to_f64(bits, fmt):
    bits = np.asarray(bits).astype(np.uint16)
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nearest_bits(ref, fmt):
    """ref (float64) rounded to the output type, nearest-even."""
    if fmt == "f16":
        return ref.astype(np.float16).view(np.uint16)
    # float64 -> bf16 directly: round the float64 significand to 8 bits
    m, e = np.frexp(ref)                                   # ref = m 2^e, |m| in [0.5, 1)
    e = np.maximum(e, -125)                                 # bf16 subnormals: fixed quantum 2^-133
    q = np.ldexp(1.0, e - 8)
    r = np.round(ref / q) * q                               # numpy rounds half to even
    return W.f32_to_bf16_bits(r.astype(np.float32))


def ulp_at(ref, fmt):
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    if fmt == "f16":
        return 2.0 ** np.maximum(e - 10, -24)
    return 2.0 ** np.maximum(e - 7, -133)


def compare(got_bits, ref, fmt, exact):
    """Assert the bound; return (elements, not-nearest count)."""
    got = bits_to_f64(got_bits, fmt)
    assert np.all(np.isfinite(got)), "non-finite output"
    near = nearest_bits(ref, fmt)
    not_nearest = int(np.count_nonzero(np.asarray(got_bits).astype(np.uint16) != near))
    if exact:
        assert not_nearest == 0, f"{not_nearest} elements differ from the exactly rounded reference"
    else:
        err = np.abs(got - ref)
        row_scale = np.max(np.abs(ref), axis=-1, keepdims=True)
        bad = err > ulp_at(ref, fmt) + 2.0 ** -20 * row_scale
        assert not bad.any(), (f"{int(bad.sum())} elements beyond one ulp; worst {float(err.max()):.3e} at "
                               f"{np.unravel_index(int(np.argmax(err)), err.shape)}")
    return got.size, not_nearest


def run_case(wl, fmt="f16", t0=3, trim=7):
    import torch
    s = H.Setup(wl)
    K, V = s.kv()
    n_c = wl.n_compressed
    planes, _, _ = s.oracle_encode(K[:, :, :n_c], V[:, :, :n_c])
    B, Hkv, d = K.shape[0], wl.n_kv_heads, wl.head_dim
    cache = s.tq.alloc_cache(s.layout, B, n_c)
    H.upload_planes(cache, planes)
    n = n_c - t0 - trim
    ok = torch.empty((B, Hkv, n, d), dtype=torch.int16, device="cuda")
    ov = torch.empty((B, Hkv, n, d), dtype=torch.int16, device="cuda")
    s.tq.tq_materialize(s.layout, s.dstate.struct, cache.struct, t0, n, ok, ov, FMT[fmt])
    torch.cuda.synchronize()
    gk = ok.cpu().numpy().view(np.uint16)
    gv = ov.cpu().numpy().view(np.uint16)
    tot = {"k": [0, 0], "v": [0, 0]}
    for b in range(B):
        for g in range(Hkv):
            for half, got in (("k", gk), ("v", gv)):
                ref = ref_rows(s, planes, b, g, t0, n, half)
                exact = half == "v" and wl.v_kind == "group_sym"
                c, nn = compare(got[b, g], ref, fmt, exact)
                tot[half][0] += c
                tot[half][1] += nn
    H.log(f"[materialize] {wl.name} {fmt} t0={t0} n={n}: keys {tot['k'][1]}/{tot['k'][0]} not nearest, "
          f"values {tot['v'][1]}/{tot['v'][0]}")
    return s, cache


def small(name):
    wl = W.WORKLOADS[name]
    return wl.scaled(357 + wl.n_recent, batch=min(wl.batch, 2))


NAMES = list(W.WORKLOADS)


@pytest.mark.parametrize("name", NAMES)
def test_materialize_workloads_f16(name):
    run_case(small(name), "f16")


@pytest.mark.parametrize("name", ["llama1b_h32x8_d64_t32k", "qwen0p6b_h16x4_d128_b8_t64k",
                                  "qwen32b_h40x8_d256_b4_t128k"])
def test_materialize_workloads_bf16(name):
    run_case(small(name), "bf16", t0=0, trim=1)


VARIANTS = [
    (64, "lm_qjl", 2, "group_sym", 4, 4, 2, "f16"),
    (64, "lm_qjl", 4, "group_sym", 2, 8, 2, "bf16"),
    (128, "lm_qjl", 2, "group_sym", 2, 4, 2, "f16"),
    (256, "lm_qjl", 3, "group_sym", 2, 2, 2, "f16"),
    (256, "lm_qjl", 2, "group_sym", 4, 4, 1, "f16"),
    (64, "affine8", 8, "lm_rot", 2, 4, 2, "f16"),
    (64, "affine8", 8, "lm_rot", 4, 2, 2, "bf16"),
    (256, "affine8", 8, "lm_rot", 4, 4, 2, "f16"),
    (256, "affine8", 8, "lm_rot", 2, 2, 1, "f16"),
    (64, "lm_mse", 3, "lm_rot", 3, 4, 2, "f16"),
    (128, "lm_mse", 4, "group_sym", 4, 4, 2, "bf16"),
    (256, "lm_mse", 2, "lm_rot", 4, 2, 1, "f16"),
    (128, "f16", 16, "lm_rot", 3, 4, 2, "bf16"),
    (256, "f16", 16, "group_sym", 2, 2, 2, "f16"),
    (256, "f16", 16, "lm_rot", 4, 2, 2, "bf16"),
    (128, "lm_qjl", 2, "group_asym", 2, 4, 2, "f16"),
    (64, "lm_qjl", 3, "group_asym", 4, 4, 2, "bf16"),
    # 5/4/2-bit affine keys (the vllm-metal compression-ratio table's q5_0, q4_0, uint2/int2)
    (128, "affine8", 5, "lm_rot", 3, 4, 2, "f16"),
    (64, "affine8", 5, "lm_rot", 4, 8, 2, "bf16"),
    (64, "affine8", 4, "lm_rot", 2, 4, 2, "bf16"),
    (128, "affine8", 2, "lm_rot", 2, 2, 2, "f16"),
    # head_dim 512
    (512, "lm_qjl", 3, "group_sym", 2, 4, 2, "f16"),
    (512, "lm_qjl", 2, "lm_rot", 4, 2, 1, "bf16"),
    (512, "lm_mse", 4, "lm_rot", 3, 2, 2, "f16"),
    (512, "affine8", 5, "group_asym", 4, 4, 2, "bf16"),
    (512, "affine8", 8, "group_sym", 4, 2, 1, "f16"),
    (512, "f16", 16, "lm_rot", 2, 2, 2, "bf16"),
]


def make_variant(v):
    d, kk, kb, vk, vb, hq, hkv, dt = v
    return W.Workload(name=f"mat_d{d}_{kk}{kb}_{vk}{vb}_{dt}", seed=777, batch=2, n_q_heads=hq, n_kv_heads=hkv,
                      head_dim=d, n_ctx=290, n_recent=0, k_kind=kk, k_bits=kb, v_kind=vk, v_bits=vb, in_dtype=dt,
                      recent_dtype="f16")


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: make_variant(v).name)
def test_materialize_variants(v):
    run_case(make_variant(v), "f16", t0=11, trim=0)


@pytest.mark.parametrize("t0,n", [(0, 1), (200, 57), (256, 1)])
def test_materialize_edge_lengths(t0, n):
    """Single rows, a ragged last tile, the last slot; n = 0 writes nothing."""
    import torch
    wl = dataclasses.replace(W.WORKLOADS["qwen32b_h40x8_d128_b4_t128k"].scaled(257, batch=1), n_recent=0)
    s = H.Setup(wl)
    K, V = s.kv()
    planes, _, _ = s.oracle_encode(K, V)
    cache = s.tq.alloc_cache(s.layout, 1, 257)
    H.upload_planes(cache, planes)
    ok = torch.empty((1, wl.n_kv_heads, n, wl.head_dim), dtype=torch.int16, device="cuda")
    ov = torch.empty_like(ok)
    s.tq.tq_materialize(s.layout, s.dstate.struct, cache.struct, t0, n, ok, ov, 0)
    torch.cuda.synchronize()
    for g in range(wl.n_kv_heads):
        compare(ok.cpu().numpy().view(np.uint16)[0, g], ref_rows(s, planes, 0, g, t0, n, "k"), "f16", False)
        compare(ov.cpu().numpy().view(np.uint16)[0, g], ref_rows(s, planes, 0, g, t0, n, "v"), "f16", True)
    sentinel = torch.full((1, wl.n_kv_heads, 4, wl.head_dim), 0x1234, dtype=torch.int16, device="cuda")
    s.tq.tq_materialize(s.layout, s.dstate.struct, cache.struct, 5, 0, sentinel, sentinel, 0)
    torch.cuda.synchronize()
    assert bool((sentinel == 0x1234).all())


def _put_slice(cache, planes, wl, b, g, cap):
    """Overwrite slice (b, g) of a full-size GPU cache with the oracle's planes of it."""
    import torch
    for name, arr in planes.items():
        if name not in cache.planes:
            continue
        row = np.ascontiguousarray(arr[0, 0]).view(np.uint8).reshape(-1)
        rb = row.size // arr.shape[2]               # bytes per token row of this plane
        off = ((b * wl.n_kv_heads + g) * cap) * rb
        cache.planes[name][off:off + row.size].copy_(torch.from_numpy(row).cuda())


FULL = [("llama1b_h32x8_d64_t32k", (0, 5)),
        ("qwen0p6b_h16x4_d128_b8_t64k", (6, 2)),
        ("qwen32b_h40x8_d256_b4_t128k", (2, 7))]


@pytest.mark.parametrize("name,sl", FULL)
def test_materialize_full_size_sampled(name, sl):
    """Whole cache materialised in the launch configuration of the full workload; one slice
    carries the oracle's planes (identical codes) and is checked against the oracle."""
    import torch
    wl = W.WORKLOADS[name]
    s = H.Setup(wl)
    n = wl.n_compressed
    B = wl.batch
    b, g = sl
    K, V = s.kv()
    cache = s.gpu_encode(K[:, :, :n], V[:, :, :n], n, n)
    planes, _, _ = s.oracle_encode(K[b:b + 1, g:g + 1, :n], V[b:b + 1, g:g + 1, :n])
    _put_slice(cache, planes, wl, b, g, n)
    del K, V
    ok = torch.empty((B, wl.n_kv_heads, n, wl.head_dim), dtype=torch.int16, device="cuda")
    ov = torch.empty_like(ok)
    s.tq.tq_materialize(s.layout, s.dstate.struct, cache.struct, 0, n, ok, ov, 0)
    torch.cuda.synchronize()
    sub = dataclasses.replace(wl, batch=1, n_kv_heads=1, n_q_heads=wl.n_rep)
    s_sub = H.Setup.__new__(H.Setup)
    s_sub.wl, s_sub.ostate = sub, s.ostate
    ck, nk = compare(ok[b, g].cpu().numpy().view(np.uint16), ref_rows(s_sub, planes, 0, 0, 0, n, "k"), "f16", False)
    cv, nv = compare(ov[b, g].cpu().numpy().view(np.uint16), ref_rows(s_sub, planes, 0, 0, 0, n, "v"), "f16",
                     wl.v_kind == "group_sym")
    H.log(f"[materialize full] {name} slice {sl}: keys {nk}/{ck} not nearest, values {nv}/{cv}")
    del cache, ok, ov
    torch.cuda.empty_cache()
