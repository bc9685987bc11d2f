"""tq_decode_attn_noalloc (decode with the library's static scratch instead of a caller
workspace) against tq_decode_attn on the same inputs: two calls in a row, the second
smaller, each checked against the workspace entry point's output (the same kernels and
split plan, so bit-identical) and against the oracle's attention (2e-3)."""
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


def _case(name, n_ctx, batch, n_recent):
    base = W.WORKLOADS[name]
    wl = dataclasses.replace(base.scaled(n_ctx, batch=batch), n_recent=n_recent)
    s = H.Setup(wl)
    K, V = s.kv()
    n = wl.n_compressed
    rk, rv, R = s.recent(K, V)
    Q = W.q_bits(wl)
    planes, _, _ = s.oracle_encode(K[:, :, :n], V[:, :, :n])
    cache = s.tq.alloc_cache(s.layout, K.shape[0], n)
    H.upload_planes(cache, planes)
    return wl, s, cache, Q, rk, rv, R, planes


def _noalloc(s, cache, Q, n, rk, rv, R):
    import torch
    out = torch.full((Q.shape[0], s.wl.n_q_heads, s.wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    rkd = H.dev_u16(rk) if rk is not None else None
    rvd = H.dev_u16(rv) if rv is not None else None
    s.tq.tq_decode_attn_noalloc(s.layout, s.dstate.struct, H.dev_u16(Q), cache.struct, n, rkd, rvd, R,
                                rk.shape[2] if rk is not None else 0, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_noalloc_matches_workspace_entry_point_twice():
    big = _case("qwen7b_h28x4_d128_b16_t32k", 6000 + 128, 4, 128)
    small = _case("llama1b_h32x8_d64_t32k", 700 + 5, 1, 5)
    for (wl, s, cache, Q, rk, rv, R, planes) in (big, small):
        n = wl.n_compressed
        H.log(f"[noalloc] {wl.name} B={Q.shape[0]} n_c={n} n_recent={R}")
        got = _noalloc(s, cache, Q, n, rk, rv, R)
        want = s.gpu_decode(cache, Q, n, rk, rv, R)
        assert np.array_equal(got, want), "noalloc output differs from tq_decode_attn"
        ref = s.oracle_decode(planes, Q, n, rk, rv, R)
        err = H.rel_err(got, ref)
        H.log(f"  max rel err vs oracle {err:.3e}")
        assert err <= H.ATTN_TOL


def test_noalloc_rejects_a_decode_above_its_scratch():
    tq = __import__("compressed_decode_attention_encode_amd.tq", fromlist=["tq"])
    assert tq.tq_decode_noalloc_max_scratch_bytes() == 16 << 20
    L = tq.make_layout(256, 64, 8, "lm_qjl", 4, "group_sym", 4)
    B, n_c = 64, 1 << 20
    assert tq.tq_decode_workspace_bytes(L, B, n_c) > 16 << 20
    fake = 1 << 20
    cache = tq.tq_cache(fake, fake, fake, fake, fake, B, n_c)
    st = tq.tq_state(fake, fake, None, None, fake, None, fake)
    with pytest.raises(tq.TQError) as e:
        tq.tq_decode_attn_noalloc(L, st, fake, cache, n_c, None, None, 0, 0, fake)
    assert e.value.status == tq.TQ_ERR_CAPACITY
