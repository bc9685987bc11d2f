"""C-ABI host side, no GPU: the library loads, exports every declared symbol, its host
math matches the oracle, and every argument check fails loudly before any HIP call."""
import os
import re

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import layout as OL
from oracle import rotation as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tq = pytest.importorskip("compressed_decode_attention_encode_amd.tq",
                         reason="libtq.so not built (run __graft_entry__.build())")


def declared_symbols():
    """Every entry point declared in include/*.h."""
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(tq_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert set(names) == set(tq.EXPORTED)
    for n in names:
        assert hasattr(tq._lib, n)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle(d, bits):
    c, t, dist = tq.tq_make_codebook(d, bits)
    c2, t2 = cb.codebook_f32(d, bits)
    # independent solvers (quadrature vs incomplete beta) agree to the last float32 bit
    assert np.array_equal(c, c2) and np.array_equal(t, t2)
    c64, _ = cb.lloyd_max(d, bits)
    assert abs(dist - cb.distortion(c64, d)) < 1e-12


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_state_matches_reference_generator(d):
    s, q = tq.tq_make_rotation(d, 20260101 + d)
    s2, q2 = R.reference_rotation_state(d, 20260101 + d)
    assert np.array_equal(s, s2)
    # both round the same float64 Box-Muller value to fp16 (libm and Python may differ in
    # the last float64 bit, which moves an fp16 result only at an exact rounding tie)
    assert q.dtype == np.float16 and q2.dtype == np.float16
    assert np.array_equal(q.view(np.uint16), q2.view(np.uint16))


CONFIGS = [(64, "lm_qjl", 3, "group_sym", 2), (128, "lm_qjl", 4, "group_sym", 4), (128, "affine8", 8, "lm_rot", 3),
           (128, "affine8", 5, "lm_rot", 3), (64, "affine8", 4, "lm_rot", 2), (128, "affine8", 2, "lm_rot", 2),
           (256, "lm_qjl", 4, "group_sym", 4), (128, "lm_qjl", 2, "lm_rot", 2), (128, "lm_qjl", 2, "group_asym", 2),
           (64, "lm_qjl", 3, "group_asym", 4)]


@pytest.mark.parametrize("cfg", CONFIGS)
def test_plane_bytes_match_layout(cfg):
    d, kk, kb, vk, vb = cfg
    L = tq.make_layout(d, 8, 2, kk, kb, vk, vb)
    got = tq.tq_cache_plane_bytes(L, 3, 17)
    per = OL.bytes_per_token_head(d, kk, kb, vk, vb)
    rows = 3 * 2 * 17
    assert got == [rows * per[n] for n in ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")]


# ------------------------------------------------------------------------- argument checks
FAKE = 0x10000      # aligned non-null address: never dereferenced, checks fail first


def _layout(**kw):
    base = dict(head_dim=128, n_q_heads=8, n_kv_heads=2, k_kind="lm_qjl", k_bits=3, v_kind="group_sym", v_bits=2)
    base.update(kw)
    return tq.make_layout(**base)


def _state():
    return tq.tq_state(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def _cache(batch=1, cap=256):
    return tq.tq_cache(FAKE, FAKE, FAKE, FAKE, FAKE, batch, cap)


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=96), tq.TQ_ERR_UNSUPPORTED),
    (dict(n_q_heads=7), tq.TQ_ERR_UNSUPPORTED),
    (dict(k_bits=5), tq.TQ_ERR_UNSUPPORTED),
    (dict(k_kind="affine8", k_bits=3), tq.TQ_ERR_UNSUPPORTED),
    (dict(k_kind="affine8", k_bits=6), tq.TQ_ERR_UNSUPPORTED),
    (dict(v_bits=3), tq.TQ_ERR_UNSUPPORTED),
    (dict(v_kind="lm_rot", v_bits=5), tq.TQ_ERR_UNSUPPORTED),
    (dict(n_kv_heads=0), tq.TQ_ERR_INVALID),
    (dict(in_dtype=7), tq.TQ_ERR_UNSUPPORTED),
])
def test_encode_rejects_bad_layouts(bad, code):
    with pytest.raises(tq.TQError) as e:
        tq.tq_encode(_layout(**bad), _state(), FAKE, FAKE, 1, 16, 0, _cache())
    assert e.value.status == code
    assert tq.tq_last_error()


def test_encode_rejects_bad_arguments():
    L = _layout()
    cases = [
        (dict(k=None, v=None), tq.TQ_ERR_INVALID),
        (dict(k=FAKE + 4), tq.TQ_ERR_INVALID),                    # misaligned input
        (dict(batch=2), tq.TQ_ERR_INVALID),                       # != cache batch
        (dict(n_tokens=-1), tq.TQ_ERR_INVALID),
        (dict(dst_offset=250, n_tokens=16), tq.TQ_ERR_CAPACITY),  # 266 > 256
        (dict(cache=tq.tq_cache(None, FAKE, FAKE, FAKE, FAKE, 1, 256)), tq.TQ_ERR_INVALID),
        (dict(state=tq.tq_state(FAKE, FAKE, None, None, FAKE, None, None)), tq.TQ_ERR_INVALID),  # no QJL matrix
    ]
    for over, code in cases:
        a = dict(k=FAKE, v=FAKE, batch=1, n_tokens=16, dst_offset=0, cache=_cache(), state=_state())
        a.update(over)
        with pytest.raises(tq.TQError) as e:
            tq.tq_encode(L, a["state"], a["k"], a["v"], a["batch"], a["n_tokens"], a["dst_offset"], a["cache"])
        assert e.value.status == code, (over, e.value)


def test_encode_unsupported_head_dim_is_loud():
    """head_dim 64 / 128 / 256 / 512 are the supported set; 1024 fails before any HIP call."""
    with pytest.raises(tq.TQError) as e:
        tq.tq_encode(_layout(head_dim=1024), _state(), FAKE, FAKE, 1, 16, 0, _cache())
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED


def test_head_dim_512_decode_limits():
    """head_dim 512 decodes every key / value kind up to n_rep 8; n_rep 9 fails loudly before any
    HIP call, and the plane sizes follow the row layouts at d = 512."""
    ws = 1 << 30
    with pytest.raises(tq.TQError) as e:
        tq.tq_decode_attn(_layout(head_dim=512, n_q_heads=18, n_kv_heads=2), _state(), FAKE, _cache(), 100,
                          None, None, 0, 0, FAKE, FAKE, ws)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    sizes = tq.tq_cache_plane_bytes(_layout(head_dim=512, k_kind="lm_qjl", k_bits=3, v_kind="lm_rot", v_bits=3), 1, 10)
    per = 10 * 2                                            # 10 tokens, 2 kv-heads
    assert sizes == [4 * 52 * per, 4 * 16 * per, 4 * per, 4 * 52 * per, 4 * per]   # 52 words of ten 3-bit codes
    sizes = tq.tq_cache_plane_bytes(_layout(head_dim=512, k_kind="affine8", k_bits=5, v_kind="group_sym", v_bits=4), 1, 10)
    assert sizes == [4 * (64 + 16) * per, 0, 4 * 16 * per, 4 * 64 * per, 2 * 16 * per]


def test_decode_rejects_bad_arguments():
    L = _layout()
    ws = tq.tq_decode_workspace_bytes(L, 1, 256)
    assert ws > 0
    base = dict(q=FAKE, n_c=100, rk=FAKE, rv=FAKE, n_r=8, rcap=128, out=FAKE, ws=FAKE, wsb=ws, cache=_cache())
    cases = [
        (dict(n_c=0, n_r=0), tq.TQ_ERR_INVALID),
        (dict(n_r=129, rcap=256), tq.TQ_ERR_INVALID),
        (dict(rk=None), tq.TQ_ERR_INVALID),
        (dict(rcap=4), tq.TQ_ERR_INVALID),
        (dict(wsb=16), tq.TQ_ERR_INVALID),
        (dict(n_c=300), tq.TQ_ERR_CAPACITY),
        (dict(out=FAKE + 8), tq.TQ_ERR_INVALID),
        (dict(q=None), tq.TQ_ERR_INVALID),
    ]
    for over, code in cases:
        a = dict(base)
        a.update(over)
        with pytest.raises(tq.TQError) as e:
            tq.tq_decode_attn(L, _state(), a["q"], a["cache"], a["n_c"], a["rk"], a["rv"], a["n_r"], a["rcap"],
                              a["out"], a["ws"], a["wsb"])
        assert e.value.status == code, (over, e.value)
    with pytest.raises(tq.TQError) as e:
        tq.tq_decode_attn(_layout(n_q_heads=18, n_kv_heads=2), _state(), FAKE, _cache(), 100, None, None, 0, 0,
                          FAKE, FAKE, 1 << 30)       # n_rep 9: no kernel compiled
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    with pytest.raises(tq.TQError) as e:              # LM + QJL keys with rotated values: not compiled
        tq.tq_decode_attn(_layout(v_kind="lm_rot", v_bits=3), _state(), FAKE, _cache(), 100, None, None, 0, 0,
                          FAKE, FAKE, 1 << 30)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED


def test_multi_query_decode_rejects_bad_arguments():
    """Host-side checks of tq_decode_attn_multi: every rejection happens before any HIP call."""
    L = _layout(head_dim=64, n_q_heads=8, n_kv_heads=2)       # n_rep 4
    ws = tq.tq_decode_multi_workspace_bytes(L, 1, 4, 256)
    assert ws > tq.tq_decode_multi_workspace_bytes(L, 1, 2, 256) > 0
    assert tq.tq_decode_multi_workspace_bytes(L, 1, 2, 256) == 2 * tq.tq_decode_workspace_bytes(L, 1, 256)
    assert tq.tq_decode_multi_workspace_bytes(L, 1, 0, 256) == 0
    assert tq.tq_decode_multi_workspace_bytes(L, 1, 9, 256) == 0
    base = dict(L=L, nq=4, q=FAKE, n_c=100, rk=FAKE, rv=FAKE, n_r=8, rcap=128, out=FAKE, ws=FAKE, wsb=ws, cache=_cache())
    cases = [
        (dict(nq=0), tq.TQ_ERR_INVALID),
        (dict(nq=9), tq.TQ_ERR_INVALID),
        (dict(n_r=3), tq.TQ_ERR_INVALID),                # fewer recent tokens than queries
        (dict(n_r=129, rcap=256), tq.TQ_ERR_INVALID),
        (dict(rk=None), tq.TQ_ERR_INVALID),
        (dict(wsb=ws - 1), tq.TQ_ERR_INVALID),
        (dict(n_c=300), tq.TQ_ERR_CAPACITY),
        (dict(q=FAKE + 4), tq.TQ_ERR_INVALID),
        (dict(nq=8), tq.TQ_ERR_UNSUPPORTED),             # 8 x 4 rows > 16
        (dict(nq=3), tq.TQ_ERR_UNSUPPORTED),
        (dict(nq=4, L=_layout(head_dim=64, n_q_heads=6, n_kv_heads=2)), tq.TQ_ERR_UNSUPPORTED),   # 4 x 3 rows: not compiled
        (dict(L=_layout(head_dim=256, n_q_heads=4, n_kv_heads=2)), tq.TQ_ERR_UNSUPPORTED),
        (dict(L=_layout(head_dim=64, k_kind="affine8", k_bits=8, v_kind="lm_rot", v_bits=3)), tq.TQ_ERR_UNSUPPORTED),
    ]
    for over, code in cases:
        a = dict(base)
        a.update(over)
        with pytest.raises(tq.TQError) as e:
            tq.tq_decode_attn_multi(a["L"], _state(), a["q"], a["nq"], a["cache"], a["n_c"], a["rk"], a["rv"], a["n_r"],
                                    a["rcap"], a["out"], a["ws"], a["wsb"])
        assert e.value.status == code, (over, e.value)


def test_materialize_rejects_bad_arguments():
    """Host-side checks of tq_materialize: every rejection happens before any HIP call."""
    L = _layout()
    base = dict(t0=0, n=16, ok=FAKE, ov=FAKE, dt=tq.TQ_F16, cache=_cache(), state=_state())
    cases = [
        (dict(ok=None, ov=None), tq.TQ_ERR_INVALID),
        (dict(ok=FAKE + 4), tq.TQ_ERR_INVALID),                     # misaligned output
        (dict(t0=-1), tq.TQ_ERR_INVALID),
        (dict(n=-2), tq.TQ_ERR_INVALID),
        (dict(t0=250, n=16), tq.TQ_ERR_CAPACITY),                   # 266 > 256
        (dict(dt=7), tq.TQ_ERR_UNSUPPORTED),
        (dict(cache=tq.tq_cache(None, FAKE, FAKE, FAKE, FAKE, 1, 256)), tq.TQ_ERR_INVALID),
        (dict(state=tq.tq_state(FAKE, FAKE, None, None, FAKE, None, None)), tq.TQ_ERR_INVALID),  # no QJL matrix
    ]
    for over, code in cases:
        a = dict(base)
        a.update(over)
        with pytest.raises(tq.TQError) as e:
            tq.tq_materialize(L, a["state"], a["cache"], a["t0"], a["n"], a["ok"], a["ov"], a["dt"])
        assert e.value.status == code, (over, e.value)
    with pytest.raises(tq.TQError) as e:
        tq.tq_materialize(_layout(head_dim=1024), _state(), _cache(), 0, 16, FAKE, FAKE, tq.TQ_F16)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED


def test_mse_only_keys_arguments():
    """MSE-only LM keys: k_bits 2..4, no QJL matrix or sign plane needed, key rotation needed."""
    L = _layout(k_kind="lm_mse", k_bits=5)
    with pytest.raises(tq.TQError) as e:
        tq.tq_encode(L, _state(), FAKE, None, 1, 16, 0, _cache())
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    L = _layout(k_kind="lm_mse", k_bits=3)
    sizes = tq.tq_cache_plane_bytes(L, 1, 100)
    assert sizes[1] == 0 and sizes[2] == 4 * 100 * L.n_kv_heads      # no sign plane; fp32 n per row
    with pytest.raises(tq.TQError) as e:                               # no key rotation signs
        tq.tq_encode(L, tq.tq_state(FAKE, FAKE, None, None, None, None, None), FAKE, None, 1, 16, 0,
                     tq.tq_cache(FAKE, None, FAKE, FAKE, FAKE, 1, 256))
    assert e.value.status == tq.TQ_ERR_INVALID


def test_sixteen_bit_keys_arguments():
    """16-bit keys (V-only mode): k_bits 16, no aux plane; decode compiled for d 64/128/256/512 in
    either storage type, n_rep <= 8."""
    with pytest.raises(tq.TQError) as e:
        tq.tq_encode(_layout(k_kind="f16", k_bits=8), _state(), FAKE, None, 1, 16, 0, _cache())
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    L = _layout(k_kind="f16", k_bits=16, v_kind="lm_rot", v_bits=3)
    sizes = tq.tq_cache_plane_bytes(L, 1, 10)
    assert sizes[:3] == [2 * 128 * 10 * L.n_kv_heads, 0, 0]
    ws = tq.tq_decode_workspace_bytes(L, 1, 100)
    cache = tq.tq_cache(FAKE, None, None, FAKE, FAKE, 1, 256)
    with pytest.raises(tq.TQError) as e:          # n_rep 9 has no 16-bit-key decode at any head_dim
        tq.tq_decode_attn(_layout(head_dim=256, n_q_heads=18, k_kind="f16", k_bits=16, v_kind="lm_rot", v_bits=3,
                                  in_dtype="bf16"),
                          _state(), FAKE, cache, 100, None, None, 0, 0, FAKE, FAKE, 1 << 30)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    assert ws > 0


def test_workspace_bound_covers_every_length():
    L = _layout(head_dim=64, n_q_heads=32, n_kv_heads=8)
    import ctypes
    bound = tq.tq_decode_workspace_bytes(L, 1, 40000)
    # the plan for any shorter cache never needs more than the bound
    for n in list(range(1, 3000, 37)) + [32640, 32768, 40000]:
        need = tq.tq_decode_workspace_bytes(L, 1, n)
        assert need <= bound
    assert tq.tq_strerror(tq.TQ_ERR_CAPACITY) == "cache capacity exceeded"


def test_one_hip_runtime_in_process():
    # libtq must share torch's HIP runtime (device pointers and streams come from torch)
    loaded = tq._hip_runtimes_loaded()
    assert len(loaded) == 1, loaded


def test_narrow_affine_key_decode_limits():
    """5/4/2-bit affine keys decode with rotated values at head_dim 64/128; other combinations
    fail loudly before any HIP call."""
    ws = 1 << 30
    for bad in (dict(head_dim=256, k_kind="affine8", k_bits=4, v_kind="lm_rot", v_bits=3),
                dict(head_dim=128, k_kind="affine8", k_bits=5, v_kind="group_sym", v_bits=2)):
        with pytest.raises(tq.TQError) as e:
            tq.tq_decode_attn(_layout(**bad), _state(), FAKE, _cache(), 100, None, None, 0, 0, FAKE, FAKE, ws)
        assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    sizes = tq.tq_cache_plane_bytes(_layout(head_dim=128, k_kind="affine8", k_bits=5, v_kind="lm_rot", v_bits=3), 1, 10)
    assert sizes[0] == 4 * (128 // 8 + 128 // 32) * 10 * 2 and sizes[1] == 0   # 5 bits per code, 2 kv-heads

