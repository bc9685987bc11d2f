"""GPU parity over the compiled variants the benchmark workloads do not reach.

Every kernel family (2/3/4-bit Lloyd-Max + QJL keys, MSE-only Lloyd-Max keys, per-block
affine keys at 8/5/4/2 bits, group-32 and rotated Lloyd-Max values, head_dim 64/128/256/512, n_rep 1..8, fp16/bf16 inputs) is
encoded and decoded at a small, ragged size against the CPU oracle, and degenerate
vectors (all zero, constant, a single non-zero element, signed zeros, subnormals) go
through both sides.
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

# d, key kind/bits, value kind/bits, Hq, Hkv, input dtype, context, recent tokens
VARIANTS = [
    (64, "lm_qjl", 2, "group_sym", 2, 4, 2, "f16", 300, 17),
    (64, "lm_qjl", 4, "group_sym", 4, 24, 3, "bf16", 260, 0),
    (128, "lm_qjl", 2, "group_sym", 4, 6, 2, "f16", 200, 64),
    (128, "lm_qjl", 4, "group_sym", 2, 12, 2, "bf16", 333, 5),
    (256, "lm_qjl", 3, "group_sym", 2, 2, 2, "f16", 150, 31),
    (256, "lm_qjl", 2, "group_sym", 4, 8, 1, "f16", 190, 0),
    (256, "lm_qjl", 4, "group_sym", 4, 10, 2, "bf16", 150, 9),      # 4-bit single-code operands
    (64, "affine8", 8, "lm_rot", 2, 8, 2, "f16", 280, 0),
    (64, "affine8", 8, "lm_rot", 4, 2, 2, "bf16", 200, 20),
    (128, "affine8", 8, "lm_rot", 2, 14, 2, "f16", 222, 100),
    (256, "affine8", 8, "lm_rot", 4, 6, 3, "bf16", 170, 9),
    # MSE-only keys (no QJL term) with rotated LM and group values
    (64, "lm_mse", 3, "lm_rot", 3, 4, 2, "f16", 300, 17),
    (64, "lm_mse", 2, "group_sym", 2, 16, 2, "bf16", 260, 0),
    (128, "lm_mse", 4, "lm_rot", 4, 8, 1, "f16", 333, 64),
    (128, "lm_mse", 3, "group_sym", 4, 6, 2, "bf16", 222, 5),
    (128, "lm_mse", 4, "group_sym", 2, 10, 2, "f16", 200, 5),      # 4-bit single-code operands
    (256, "lm_mse", 4, "lm_rot", 2, 10, 2, "f16", 190, 31),
    (256, "lm_mse", 2, "group_sym", 2, 3, 3, "f16", 150, 0),
    # 16-bit keys (V-only mode)
    (64, "f16", 16, "lm_rot", 3, 4, 2, "f16", 300, 17),
    (64, "f16", 16, "group_sym", 4, 8, 1, "bf16", 250, 0),
    (128, "f16", 16, "lm_rot", 2, 14, 2, "bf16", 222, 40),
    (128, "f16", 16, "group_sym", 2, 2, 2, "f16", 180, 3),
    (64, "f16", 16, "group_sym", 2, 12, 2, "f16", 230, 9),       # fp16 keys, n_rep 6: matrix cores
    (64, "f16", 16, "lm_rot", 4, 10, 2, "f16", 190, 0),
    (256, "f16", 16, "lm_rot", 3, 4, 2, "f16", 200, 17),        # d 256: fp16 keys, 32-token tiles
    (256, "f16", 16, "group_sym", 2, 2, 2, "f16", 150, 0),
    (256, "f16", 16, "lm_rot", 3, 10, 2, "bf16", 210, 17),      # d 256 bf16 keys: bf16 products
    (256, "f16", 16, "group_sym", 4, 2, 2, "bf16", 150, 0),
    # group-32 min/max values (matrix cores at every n_rep)
    (64, "lm_qjl", 2, "group_asym", 2, 4, 2, "f16", 300, 17),
    (64, "lm_qjl", 3, "group_asym", 2, 2, 2, "f16", 200, 5),
    (128, "lm_qjl", 3, "group_asym", 4, 10, 2, "bf16", 260, 0),
    (128, "lm_qjl", 2, "group_asym", 2, 16, 2, "f16", 222, 64),
    # 5/4/2-bit affine keys with rotated values (matrix cores at every n_rep)
    (128, "affine8", 5, "lm_rot", 3, 16, 4, "f16", 300, 17),
    (64, "affine8", 5, "lm_rot", 2, 2, 2, "bf16", 230, 0),
    (128, "affine8", 4, "lm_rot", 3, 4, 2, "bf16", 260, 9),
    (64, "affine8", 4, "lm_rot", 4, 14, 2, "f16", 222, 40),
    (128, "affine8", 2, "lm_rot", 3, 8, 1, "f16", 333, 5),
    (128, "affine8", 2, "lm_rot", 2, 6, 2, "bf16", 190, 64),
    (64, "affine8", 2, "lm_rot", 2, 10, 2, "f16", 250, 0),
    # head_dim 512 (vector-ALU kernels: one wave per token), every key and value kind
    (512, "lm_qjl", 3, "group_sym", 2, 8, 2, "f16", 200, 17),
    (512, "lm_qjl", 2, "lm_rot", 3, 2, 2, "bf16", 150, 0),
    (512, "lm_qjl", 4, "group_asym", 4, 16, 2, "f16", 1200, 5),     # several splits
    (512, "lm_mse", 3, "lm_rot", 4, 4, 1, "bf16", 170, 9),
    (512, "lm_mse", 2, "group_sym", 4, 2, 2, "f16", 100, 0),
    (512, "affine8", 8, "lm_rot", 2, 6, 2, "f16", 130, 31),
    (512, "affine8", 5, "group_asym", 2, 4, 2, "bf16", 120, 0),
    (512, "affine8", 4, "group_sym", 2, 2, 1, "f16", 100, 3),
    (512, "affine8", 2, "lm_rot", 3, 8, 2, "f16", 90, 0),
    (512, "f16", 16, "lm_rot", 3, 4, 2, "bf16", 110, 7),
    (512, "f16", 16, "group_sym", 4, 16, 2, "f16", 120, 0),
]


def make(v, seed=4242):
    d, kk, kb, vk, vb, hq, hkv, dt, n_ctx, n_rec = v
    return W.Workload(name=f"var_d{d}_{kk}{kb}_{vk}{vb}_h{hq}x{hkv}_{dt}", seed=seed, batch=2, n_q_heads=hq,
                      n_kv_heads=hkv, head_dim=d, n_ctx=n_ctx, n_recent=n_rec, k_kind=kk, k_bits=kb, v_kind=vk,
                      v_bits=vb, in_dtype=dt, recent_dtype="f16")


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: make(v).name)
def test_variant_encode_and_decode(v):
    wl = make(v)
    s = H.Setup(wl)
    K, V = s.kv()
    n = wl.n_compressed
    off, cap = 3, n + 7
    H.log(f"[variant] {wl.name} n_c={n} n_recent={wl.n_recent}")
    cache = s.gpu_encode(K[:, :, :n], V[:, :, :n], n, cap, dst_offset=off)
    gpu = H.download(cache, wl, K.shape[0], cap)
    planes, ek, ev = s.oracle_encode(K[:, :, :n], V[:, :, :n])
    st = H.compare_encode(wl, gpu, ek, ev, rows=slice(off, off + n))
    H.log(f"  encode {st}")
    assert H.untouched(gpu, slice(off, off + n), cap)
    rk, rv, R = s.recent(K, V)
    for variant in ("normal", "needle"):
        Q = W.q_bits(wl, variant)
        c2 = s.tq.alloc_cache(s.layout, K.shape[0], n)
        H.upload_planes(c2, planes)
        out = s.gpu_decode(c2, Q, n, rk, rv, R)
        ref = s.oracle_decode(planes, Q, n, rk, rv, R)
        err = H.rel_err(out, ref)
        H.log(f"  decode {variant}: max rel err {err:.3e}")
        assert err <= H.ATTN_TOL


def _bits(dt, x):
    return int(W.to_storage(np.array([x], dtype=np.float32), dt)[0])


DEGENERATE = ["llama1b_h32x8_d64_t32k", "qwen0p6b_h16x4_d128_b8_t64k", "qwen32b_h40x8_d128_b4_t128k",
              (512, "lm_qjl", 3, "lm_rot", 3, 4, 2, "bf16", 200, 0),
              (512, "lm_mse", 4, "group_sym", 2, 4, 2, "f16", 200, 0)]


@pytest.mark.parametrize("name", DEGENERATE, ids=lambda v: v if isinstance(v, str) else make(v).name)
def test_degenerate_vectors(name):
    """Zero, constant, one-hot, signed-zero and subnormal vectors through encode and decode."""
    wl = W.WORKLOADS[name] if isinstance(name, str) else make(name)
    wl = dataclasses.replace(wl.scaled(200, batch=1), n_recent=0)
    s = H.Setup(wl)
    K, V = s.kv()
    dt, d = wl.in_dtype, wl.head_dim
    one, big, neg_small = _bits(dt, 1.0), _bits(dt, 6.0e4), _bits(dt, -3.0e-3)
    tiny = 0x0001                                   # the smallest subnormal of either format
    for X in (K, V):
        X[:, :, 0] = 0                              # all zero
        X[:, :, 1] = one                            # constant
        X[:, :, 2] = 0
        X[:, :, 2, 5] = big                         # one non-zero element, large
        X[:, :, 3] = 0x8000                         # negative zeros
        X[:, :, 4] = tiny                           # subnormals
        X[:, :, 4, 1::2] = tiny | 0x8000
        X[:, :, 5] = neg_small                      # constant negative
        X[:, :, 6, : d // 2] = one                  # half constant, half random
    n = wl.n_compressed
    cache = s.gpu_encode(K[:, :, :n], V[:, :, :n], n, n)
    gpu = H.download(cache, wl, 1, n)
    planes, ek, ev = s.oracle_encode(K[:, :, :n], V[:, :, :n])
    st = H.compare_encode(wl, gpu, ek, ev)
    H.log(f"[degenerate] {name}: {st}")
    Q = W.q_bits(wl)
    c2 = s.tq.alloc_cache(s.layout, 1, n)
    H.upload_planes(c2, planes)
    out = s.gpu_decode(c2, Q, n)
    ref = s.oracle_decode(planes, Q, n)
    err = H.rel_err(out, ref)
    H.log(f"  decode max rel err {err:.3e}")
    assert err <= H.ATTN_TOL


EXTREME = [(64, "lm_qjl", 4, "lm_rot", 3, 4, 2, "bf16", 100, 0),
           (128, "lm_qjl", 3, "lm_rot", 2, 4, 2, "bf16", 100, 0),
           (256, "lm_mse", 3, "lm_rot", 4, 2, 2, "bf16", 100, 0),
           (512, "lm_qjl", 3, "lm_rot", 3, 4, 2, "bf16", 100, 0),
           (512, "lm_mse", 4, "lm_rot", 2, 2, 1, "bf16", 100, 0)]


@pytest.mark.parametrize("v", EXTREME, ids=lambda v: make(v).name)
def test_encode_extreme_bf16_magnitudes(v):
    """bf16 tokens whose float32 square sum leaves float32's range (a one-hot 1e38, constant
    rows of 3e38, 1e30 and +-1e-30, a random row with one 2e37 element) encode like the oracle's
    float64 path: identical codes and signs, norms within the side values' tolerance (an fp16
    norm of a QJL key overflows to inf on both sides; decoding such a key is outside the
    format's range and is not checked)."""
    wl = dataclasses.replace(make(v), n_recent=0)
    s = H.Setup(wl)
    K, V = s.kv()
    d = wl.head_dim
    for X in (K, V):
        X[:, :, 0] = 0
        X[:, :, 0, 5] = _bits("bf16", 1.0e38)
        X[:, :, 1] = _bits("bf16", 3.0e38)
        X[:, :, 2] = _bits("bf16", 1.0e30)
        X[:, :, 3] = _bits("bf16", -1.0e-30)
        X[:, :, 3, ::3] = _bits("bf16", 1.0e-30)
        X[:, :, 4, d // 3] = _bits("bf16", 2.0e37)
    n = wl.n_compressed
    cache = s.gpu_encode(K[:, :, :n], V[:, :, :n], n, n)
    gpu = H.download(cache, wl, K.shape[0], n)
    _, ek, ev = s.oracle_encode(K[:, :, :n], V[:, :, :n])
    st = H.compare_encode(wl, gpu, ek, ev)
    H.log(f"[extreme] {wl.name}: {st}")


def _set_codebook(s, role, c, t):
    """Give both sides the same (float32) codebook for `role` ("k" or "v")."""
    import torch
    tq = s.tq
    s.dstate.tensors[f"{role}_centroids"] = torch.from_numpy(np.ascontiguousarray(c, np.float32)).cuda()
    s.dstate.tensors[f"{role}_thresholds"] = torch.from_numpy(np.ascontiguousarray(t, np.float32)).cuda()
    s.dstate.struct = tq.tq_state(*[(s.dstate.tensors[n].data_ptr() if n in s.dstate.tensors else None)
                                    for n, _ in tq.tq_state._fields_])
    s.ostate[f"cb_{role}"] = (np.asarray(c, np.float32), np.asarray(t, np.float32))


def _crowded(c, t):
    """Two thresholds 0.003 apart (closer than the encoder's finest decision cell, 2^-7 of
    the unit coordinate): the encoder decides by counting the thresholds below y."""
    t = t.copy()
    m = len(t) // 2
    t[m + 1] = t[m] + np.float32(0.003)
    return c, t


def _shifted(c, t):
    """Every centroid and threshold moved by +0.01: no longer symmetric about 0."""
    return c + np.float32(0.01), t + np.float32(0.01)


# (variant, codebook transform, roles)
CODEBOOKS = [((128, "lm_qjl", 4, "group_sym", 2, 12, 2, "bf16", 150, 0), _crowded, "k"),
             ((64, "lm_qjl", 2, "group_sym", 2, 4, 2, "f16", 150, 0), _crowded, "k"),
             ((256, "lm_qjl", 3, "group_sym", 2, 2, 2, "f16", 120, 0), _crowded, "k"),
             ((64, "lm_mse", 3, "lm_rot", 3, 4, 2, "f16", 150, 0), _crowded, "kv"),
             ((256, "lm_mse", 4, "lm_rot", 2, 10, 2, "f16", 120, 0), _crowded, "v"),
             ((128, "lm_mse", 4, "lm_rot", 4, 8, 1, "f16", 150, 0), _shifted, "kv"),
             ((128, "lm_qjl", 3, "group_asym", 4, 10, 2, "bf16", 150, 0), _shifted, "k"),
             ((512, "lm_qjl", 2, "lm_rot", 3, 2, 2, "bf16", 100, 0), _shifted, "kv")]


@pytest.mark.parametrize("case", CODEBOOKS, ids=lambda c: f"{make(c[0]).name}-{c[1].__name__.strip('_')}")
def test_custom_codebooks(case):
    """Ascending codebooks other than the Lloyd-Max ones (crowded thresholds, or shifted off
    symmetry) give the oracle's indices idx = #{i : t_i < y}, signs and side values, and the
    decode of the oracle's planes matches."""
    v, transform, roles = case
    wl = dataclasses.replace(make(v), n_recent=0)
    s = H.Setup(wl)
    for role in roles:
        kind = wl.k_kind if role == "k" else wl.v_kind
        if kind not in ("lm_qjl", "lm_mse", "lm_rot"):
            continue
        c, t = s.ostate[f"cb_{role}"]
        _set_codebook(s, role, *transform(c, t))
    K, V = s.kv()
    n = wl.n_compressed
    cache = s.gpu_encode(K[:, :, :n], V[:, :, :n], n, n)
    gpu = H.download(cache, wl, K.shape[0], n)
    planes, ek, ev = s.oracle_encode(K[:, :, :n], V[:, :, :n])
    st = H.compare_encode(wl, gpu, ek, ev)
    H.log(f"[codebook] {wl.name} {transform.__name__}: {st}")
    Q = W.q_bits(wl)
    c2 = s.tq.alloc_cache(s.layout, K.shape[0], n)
    H.upload_planes(c2, planes)
    out = s.gpu_decode(c2, Q, n)
    ref = s.oracle_decode(planes, Q, n)
    err = H.rel_err(out, ref)
    H.log(f"  decode max rel err {err:.3e}")
    assert err <= H.ATTN_TOL
