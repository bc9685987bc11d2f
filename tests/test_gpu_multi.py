"""GPU parity of the multi-query decode (several consecutive queries per step against one pass
over the packed cache; the last n_query recent tokens are the queries' own, causal inside the
suffix) against the CPU oracle, on identical codes (the oracle's packed planes uploaded)."""
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
from oracle import decode as OD  # noqa: E402

# (workload, n_rep override or None, n_query, context incl. the recent buffer, batch)
CASES = [
    ("llama1b_h32x8_d64_t32k", None, 2, 357 + 128, 1),      # d 64, LM3 + sym2, n_rep 4
    ("llama1b_h32x8_d64_t32k", None, 4, 357 + 128, 2),      # 16 query rows per kv-head
    ("llama1b_h32x8_d64_t32k", 1, 8, 700 + 128, 1),
    ("qwen7b_h28x4_d128_b16_t32k", 2, 4, 357 + 128, 2),     # d 128, bf16 inputs, LM3 + sym2
    ("qwen32b_h40x8_d128_b4_t128k", 4, 2, 421, 2),          # d 128, LM4 + sym4, recent = own tokens only
    ("qwen32b_h40x8_d128_b4_t128k", 2, 8, 300, 1),
    ("qwen7b_h28x4_d128_b16_t32k", None, 2, 357 + 128, 2),   # n_rep 7: 14 query rows
    ("qwen32b_h40x8_d128_b4_t128k", None, 2, 300, 1),        # n_rep 5
]


def _case(name, nrep, n_ctx, batch, nq):
    wl = W.WORKLOADS[name]
    if nrep is not None:
        wl = dataclasses.replace(wl, n_q_heads=wl.n_kv_heads * nrep)
    wl = wl.scaled(n_ctx, batch=batch)
    if wl.n_recent < nq:      # the queries' own tokens end the recent buffer
        wl = dataclasses.replace(wl, n_recent=nq)
    return wl


@pytest.mark.parametrize("name,nrep,nq,n_ctx,batch", CASES)
def test_multi_query_parity(name, nrep, nq, n_ctx, batch):
    torch = H.torch_mod()
    wl = _case(name, nrep, n_ctx, batch, nq)
    s = H.Setup(wl)
    K, V = s.kv()
    n = wl.n_compressed
    planes, _, _ = s.oracle_encode(K[:, :, :n], V[:, :, :n])
    rk, rv, R = s.recent(K, V)
    Q = W.q_bits_multi(wl, nq)
    H.log(f"[multi-query parity] {wl.name} n_rep={wl.n_rep} n_query={nq} n_c={n} n_recent={R} B={wl.batch}")
    cache = s.tq.alloc_cache(s.layout, wl.batch, n)
    H.upload_planes(cache, planes)
    ws_bytes = s.tq.tq_decode_multi_workspace_bytes(s.layout, wl.batch, nq, n)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.full((wl.batch, nq, wl.n_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    s.tq.tq_decode_attn_multi(s.layout, s.dstate.struct, H.dev_u16(Q), nq, cache.struct, n, H.dev_u16(rk),
                              H.dev_u16(rv), R, rk.shape[2], out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    q = W.storage_to_f64(Q, wl.in_dtype)
    rkf = W.storage_to_f64(rk[:, :, :R], wl.recent_dtype)
    rvf = W.storage_to_f64(rv[:, :, :R], wl.recent_dtype)
    ref = OD.decode_attention_multi(wl, q, planes, n, s.ostate, rkf, rvf)
    err = max(H.rel_err(got[:, j], ref[:, j]) for j in range(nq))
    H.log(f"  max rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= H.ATTN_TOL


def test_multi_query_one_query_is_single_decode():
    """n_query = 1 goes through the single-query path: identical output."""
    torch = H.torch_mod()
    wl = W.WORKLOADS["llama1b_h32x8_d64_t32k"].scaled(357 + 128, batch=1)
    s = H.Setup(wl)
    K, V = s.kv()
    n = wl.n_compressed
    cache = s.gpu_encode(K[:, :, :n], V[:, :, :n], n, n)
    rk, rv, R = s.recent(K, V)
    Q = W.q_bits(wl)
    single = s.gpu_decode(cache, Q, n, rk, rv, R)
    ws_bytes = s.tq.tq_decode_multi_workspace_bytes(s.layout, 1, 1, n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 1, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    s.tq.tq_decode_attn_multi(s.layout, s.dstate.struct, H.dev_u16(Q), 1, cache.struct, n, H.dev_u16(rk),
                              H.dev_u16(rv), R, rk.shape[2], out, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy()[:, 0].astype(np.float64), single)
