#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV encode + decode-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|targets] [--reps R]

One step = one pass of the whole hot path over one batch of synthetic input:
tq_encode of the workload's compressed history (keys, then values) followed by one
tq_decode_attn (query preparation, split-K attention on the packed cache, merge with the
exact recent buffer, one inverse butterfly).  Codebooks and rotation state are built once
before timing (they are per-layer constants).

By default every 32K-128K target workload is measured in turn (Llama-3.2-1B-like 32K,
Qwen3-0.6B-like 64K, Qwen2.5-7B-like 32K, Qwen2.5-32B-like 128K at head_dim 128 and 256);
the line's top-level figures are the 128K head_dim-128 workload's.  For each workload:
  * exactly K steps after W warm-up steps, bracketed by synchronisation, give ms_per_step;
  * R further event-timed steps (R >= 50, >= 200 on the 32K Llama-like layer) give the
    median and p10/p90 of each kernel group (HIP events on the stream the library
    launches on);
  * inputs and packed caches rotate over >= 1 GiB of distinct copies so the 256 MB
    Infinity Cache cannot serve a repeat: step i encodes input copy i into cache copy i and
    decodes a cache written half a ring earlier;
  * the decode is also timed as a captured HIP graph of 8 decodes (no launch gaps);
  * the deviation of the decode output from exact softmax attention on the original K/V
    (fp32 on the GPU, every (b, h)) is reported, next to the oracle parity figures that the
    cpu_baseline leg measures on the slices it times.

Prints one JSON line on stdout (value = decode KV GB/s of the 128K head_dim-128 workload).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from compressed_decode_attention_encode_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "decode-attn KV GB/s (% of HBM peak) + encode tokens/s, at 32K–128K context"
TARGETS = ["llama1b_h32x8_d64_t32k", "qwen0p6b_h16x4_d128_b8_t64k", "qwen7b_h28x4_d128_b16_t32k",
           "qwen32b_h40x8_d128_b4_t128k", "qwen32b_h40x8_d256_b4_t128k"]
HEADLINE = "qwen32b_h40x8_d128_b4_t128k"
GRAPH_DECODES = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_decode_attention_encode_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stats(ms: list[float]) -> dict:
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "mean_ms": float(a.mean()), "reps": int(a.size)}


def plane_bytes_per_token_head(wl) -> dict:
    """Bytes of each packed plane for one token of one kv-head (the library's own layout
    accounting, tq_cache_plane_bytes)."""
    from compressed_decode_attention_encode_amd import tq
    names = ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")
    cap = 4096
    sizes = tq.tq_cache_plane_bytes(tq.layout_of(wl), 1, cap)
    return {nm: sz // (wl.n_kv_heads * cap) for nm, sz in zip(names, sizes)}


def algorithmic(wl):
    """Bytes / flops the method must move or compute per step, per kernel group."""
    B, Hkv, Hq, d, n, R = wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.n_compressed, wl.n_recent
    per = plane_bytes_per_token_head(wl)
    rows = B * Hkv * n
    k_out = rows * (per["k_codes"] + per["k_signs"] + per["k_aux"])
    v_out = rows * (per["v_codes"] + per["v_aux"])
    inb = rows * d * 2
    dec = rows * sum(per.values()) + 2 * B * Hkv * R * d * 2 + B * Hq * d * 2 + B * Hq * d * 4
    qjl_flops = 2.0 * d * d * rows if wl.k_kind == "lm_qjl" else 0.0
    return {"encode_k_bytes": inb + k_out, "encode_v_bytes": inb + v_out, "decode_bytes": dec,
            "encode_k_qjl_flops": qjl_flops, "vectors": rows, "bytes_per_token_head": sum(per.values())}


def decode_kernel_name(wl) -> str:
    """The split kernel the library picks for this layout: the matrix-core kernel from 3 query
    heads per kv-head (LM, MSE-only and affine keys; min/max values at every n_rep), for
    fp16-stored 16-bit keys at head_dim 64 from 3 heads and at head_dim 256 always; otherwise
    (bf16 16-bit keys, MSE-only keys with rotated values, n_rep 1-2) the vector-ALU kernel."""
    n_rep = wl.n_q_heads // wl.n_kv_heads
    if wl.k_kind == "f16":
        mma = wl.in_dtype == "f16" and (wl.head_dim == 256 or (wl.head_dim == 64 and n_rep >= 3))
    elif wl.k_kind == "lm_mse":
        mma = wl.v_kind != "lm_rot" and (n_rep >= 3 or wl.v_kind == "group_asym")
    else:
        mma = n_rep >= 3 or wl.v_kind == "group_asym"
    return "decode_mma_kernel" if mma else "decode_main_kernel"


def read_profile_kv(path: str, digest: str) -> dict:
    """`key = value` lines of a committed counter summary, or {} when it is absent or was
    taken on different kernel sources."""
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv if kv.get("source_digest") == digest else {}


def read_traffic(workload: str, digest: str) -> dict:
    """HBM bytes per launch of each kernel group (key encode, value encode, decode) from the
    copy-calibrated FETCH_SIZE / WRITE_SIZE summary in profiles/."""
    kv = read_profile_kv(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt"), digest)
    out = {}
    for k, v in kv.items():
        if k.startswith("group.") and k.endswith(".hbm_bytes_per_launch"):
            try:
                out[k[len("group."):-len(".hbm_bytes_per_launch")]] = float(v)
            except ValueError:
                pass
    return out


def read_instr(workload: str, digest: str) -> dict:
    """Per-launch instruction counters (VALU, MFMA, LDS, busy cycles) of each kernel group
    from the committed rocprofv3 --pmc summary in profiles/."""
    kv = read_profile_kv(os.path.join(ROOT, "profiles", f"instr_counters_{workload}.txt"), digest)
    out: dict = {}
    for k, v in kv.items():
        if k.startswith("group."):
            parts = k.split(".")
            if len(parts) == 3:
                try:
                    out.setdefault(parts[1], {})[parts[2]] = float(v)
                except ValueError:
                    pass
    return out


def timed(stream, fn, reps: int, warmup: int) -> list[float]:
    import torch
    for i in range(warmup):
        fn(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def stream_read_ceiling(tq, gib: float = 4.0, reps: int = 20) -> dict:
    """Streaming HBM read rate measured on this GPU: tq_probe_stream_read over a buffer
    far larger than the Infinity Cache (median of `reps` passes)."""
    import torch
    n = int(gib * (1 << 30))
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ms = timed(stream, lambda i: tq.tq_probe_stream_read(buf, n, sink, stream), reps, 3)
    med = float(np.median(ms))
    del buf
    torch.cuda.empty_cache()
    return {"gbps": n / (med * 1e-3) / 1e9, "bytes": n, "reps": reps, "frac_of_peak": n / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel": "stream_read_kernel (tq_probe_stream_read: 16-byte non-temporal loads over the whole GPU)"}


def exact_deviation(wl, k0, v0, rk, rv, q, out) -> dict:
    """Deviation of the decode output from exact softmax attention on the original K/V
    (fp32 on the GPU, every (b, h)); recent tokens as the buffer stores them.  Per (b, h):
    max_j |o - o_exact| / max_j |o_exact| (max and median over (b, h)) and the cosine
    similarity of the two output vectors (median and min).  This is the method's own error
    (the oracle shows the same figures), not a parity measure: with N(0,1) queries over 32K+
    synthetic keys the softmax is nearly flat, the output is a small average, and the key
    quantisation error moves it by a large fraction of its size."""
    import torch
    d, n, R, nrep = wl.head_dim, wl.n_compressed, wl.n_recent, wl.n_rep
    tdt = torch.float16 if wl.in_dtype == "f16" else torch.bfloat16
    rdt = torch.float16 if wl.recent_dtype == "f16" else torch.bfloat16
    errs, coss = [], []
    qf = q.view(tdt).float()
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            kk = k0[b, g].view(tdt).float()
            vv = v0[b, g].view(tdt).float()
            if R:
                kk = torch.cat([kk, rk[b, g, :R].view(rdt).float()], 0)
                vv = torch.cat([vv, rv[b, g, :R].view(rdt).float()], 0)
            qq = qf[b, g * nrep:(g + 1) * nrep].contiguous()
            s = torch.mm(kk, qq.t().contiguous()) / float(np.sqrt(d))       # [N, n_rep]
            p = torch.softmax(s, dim=0)
            o = torch.mm(p.t().contiguous(), vv)                           # [n_rep, d]
            got = out[b, g * nrep:(g + 1) * nrep]
            e = (got - o).abs().amax(dim=1) / o.abs().amax(dim=1).clamp_min(1e-30)
            errs.append(e)
            coss.append(torch.nn.functional.cosine_similarity(got.double(), o.double(), dim=1))
    e = torch.cat(errs).double().cpu().numpy()
    c = torch.cat(coss).cpu().numpy()
    return {"max": float(e.max()), "median": float(np.median(e)), "heads": int(e.size),
            "cosine_median": float(np.median(c)), "cosine_min": float(c.min()),
            "reference": "softmax(q K^T / sqrt(d)) V in fp32 on the original fp16/bf16 K, V (recent tokens as stored)"}


def bench_materialize(tq, lay, state, caches, wl, stream, reps: int, warmup: int) -> dict:
    """tq_materialize of the whole compressed history (keys and values, fp16 rows), timed
    apart from the step: caches and output buffers rotate over more than the Infinity Cache."""
    import torch
    B, Hkv, d, n = wl.batch, wl.n_kv_heads, wl.head_dim, wl.n_compressed
    rows = B * Hkv * n
    per = plane_bytes_per_token_head(wl)
    out_bytes = 2 * rows * d * 2
    alg = rows * sum(per.values()) + out_bytes
    n_out = max(1, min(8, -(-(512 << 20) // out_bytes)))
    outs = [(torch.empty((B, Hkv, n, d), dtype=torch.int16, device="cuda"),
             torch.empty((B, Hkv, n, d), dtype=torch.int16, device="cuda")) for _ in range(n_out)]

    def run(i):
        ok, ov = outs[i % n_out]
        tq.tq_materialize(lay, state.struct, caches[(3 * i + 1) % len(caches)].struct, 0, n, ok, ov, tq.TQ_F16,
                          stream)

    st = stats(timed(stream, run, reps, warmup))
    ms = st["median_ms"]
    gb = alg / (ms * 1e-3) / 1e9
    res = {"us": ms * 1e3, "gbps": gb, "algorithmic_bytes": alg, "timing": st,
           "kernels": {"lm_qjl": "materialize_lm_kernel (keys, QJL term on fp16 matrix cores)",
                       "lm_mse": "materialize_lm_kernel (keys)",
                       "affine8": "materialize_elem_kernel (keys)",
                       "f16": "materialize_elem_kernel (16-bit keys, copy)"}[wl.k_kind] + " + " +
                      ("materialize_elem_kernel (values)" if wl.v_kind in ("group_sym", "group_asym")
                       else "materialize_lm_kernel (values)"),
           "roofline": {"bound": "hbm", "achieved": gb, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gb / HBM_PEAK_GBS, "traffic": None}}
    if wl.k_kind == "lm_qjl":
        res["qjl_tflops_fp16"] = 2.0 * d * d * rows / (ms * 1e-3) / 1e12
    del outs
    return res


def bench_multi(tq, lay, state, caches, wl, stream, rk, rv, reps: int, warmup: int) -> dict | None:
    """tq_decode_attn_multi with 4 queries (a speculative step: the last n_query recent tokens
    are the drafts' own; 2 where 4 x n_rep rows exceed the compiled set) against n_query
    single-query decodes of the same cache, timed apart from the step; None where the layout
    has no multi-query kernel."""
    for nq in (4, 2):
        r = _bench_multi(tq, lay, state, caches, wl, stream, rk, rv, reps, warmup, nq)
        if r is not None:
            return r
    return None


def _bench_multi(tq, lay, state, caches, wl, stream, rk, rv, reps: int, warmup: int, n_query: int) -> dict | None:
    import torch
    B, n, R = wl.batch, wl.n_compressed, wl.n_recent
    if R < n_query:
        return None
    qm = torch.from_numpy(np.ascontiguousarray(W.q_bits_multi(wl, n_query)).view(np.int16)).cuda()
    ws_m = tq.tq_decode_multi_workspace_bytes(lay, B, n_query, n)
    if ws_m == 0:
        return None
    wsm = torch.empty(ws_m, dtype=torch.uint8, device="cuda")
    outm = torch.empty((B, n_query, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    ws_s = tq.tq_decode_workspace_bytes(lay, B, n)
    wss = torch.empty(ws_s, dtype=torch.uint8, device="cuda")
    outs = torch.empty((B, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    q1 = [qm[:, j].contiguous() for j in range(n_query)]

    def multi(i):
        c = caches[(5 * i + 2) % len(caches)]
        tq.tq_decode_attn_multi(lay, state.struct, qm, n_query, c.struct, n, rk, rv, R, R, outm, wsm, ws_m, stream)

    def singles(i):
        c = caches[(5 * i + 2) % len(caches)]
        for j in range(n_query):
            tq.tq_decode_attn(lay, state.struct, q1[j], c.struct, n, rk, rv, R - n_query + j + 1, R, outs, wss, ws_s,
                              stream)

    try:
        multi(0)
    except tq.TQError:
        return None
    res = {name: stats(timed(stream, fn, reps, warmup))["median_ms"] * 1e3
           for name, fn in (("multi", multi), ("singles", singles))}
    per = plane_bytes_per_token_head(wl)
    kv_bytes = B * wl.n_kv_heads * n * sum(per.values()) + 2 * B * wl.n_kv_heads * R * wl.head_dim * 2
    return {"n_query": n_query, "us": res["multi"], "single_query_decodes_us": res["singles"],
            "speedup_vs_single_decodes": res["singles"] / res["multi"],
            "kv_gbps": kv_bytes / (res["multi"] * 1e-6) / 1e9,
            "kernels": "decode_mma_kernel (n_query x n_rep query rows) + decode_finish_kernel"}


def bench_flush(tq, lay, state, wl, stream, reps: int, warmup: int) -> dict:
    """One 128-token flush (keys and values of every (batch, kv-head), appended at the end of
    the history; benchmark page: 128-token flushes) timed on its own."""
    import torch
    B, Hkv, d, T = wl.batch, wl.n_kv_heads, wl.head_dim, wl.flush_tokens
    cap = wl.n_compressed
    n_buf = 64
    ks = [torch.randn((B, Hkv, T, d), device="cuda").to(torch.float16).view(torch.int16) for _ in range(n_buf)]
    vs = [torch.randn((B, Hkv, T, d), device="cuda").to(torch.float16).view(torch.int16) for _ in range(n_buf)]
    cache = tq.alloc_cache(lay, B, cap)

    def run(i):
        tq.tq_encode(lay, state.struct, ks[i % n_buf], vs[i % n_buf], B, T, cap - T - (i % 200) * T % (cap - T), cache.struct,
                     stream)

    st = stats(timed(stream, run, reps, warmup))
    return {"tokens_per_call": B * T, "vectors_per_call": B * Hkv * T, "timing": st,
            "tokens_per_s": B * T / (st["median_ms"] * 1e-3)}


def bench_graph(tq, lay, state, caches, wl, stream, q, rk, rv, out, reps: int) -> dict:
    """GRAPH_DECODES decodes of distinct caches captured into one HIP graph and replayed:
    the per-decode time without host launch gaps."""
    import torch
    n, R = wl.n_compressed, wl.n_recent
    ng = min(GRAPH_DECODES, len(caches))
    wss = [torch.empty(tq.tq_decode_workspace_bytes(lay, wl.batch, n), dtype=torch.uint8, device="cuda")
           for _ in range(ng)]
    outs = [torch.empty_like(out) for _ in range(ng)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for j in range(ng):          # eager run on the capture stream first
            tq.tq_decode_attn(lay, state.struct, q, caches[j].struct, n, rk, rv, R, R, outs[j], wss[j], wss[j].numel(), s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for j in range(ng):
            tq.tq_decode_attn(lay, state.struct, q, caches[j].struct, n, rk, rv, R, R, outs[j], wss[j], wss[j].numel(), s)
    cur = torch.cuda.current_stream()
    ms = timed(cur, lambda i: g.replay(), reps, 3)
    same = all(torch.equal(a, b) for a, b in zip(outs, ref))
    st = stats([m / ng for m in ms])
    return {"decodes_per_graph": ng, "per_decode": st, "replay_matches_eager": bool(same)}


def cpu_baseline(wl, gpu_planes_fn, gpu_out, budget_s: float = 15.0, max_slices: int | None = None):
    """Time the CPU oracle (as it stands) on whole (batch, kv-head) slices of the workload
    until about `budget_s` of CPU work: encode of the slice's keys and values, then decode of
    its n_rep query heads.  Reported in the metric's unit (decode GB/s).  The same run compares
    the oracle's planes and outputs with the GPU's on those slices (parity of the timed sample:
    codes and signs outside the 1e-6 band, max relative attention error end to end)."""
    from oracle import cache as OC
    from oracle import decode as OD
    from oracle import layout as OL
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_harness as H
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    sk, sv, S = W.rotation_signs(wl, "k"), W.rotation_signs(wl, "v"), W.qjl_matrix(wl)
    st = OC.make_state(wl, sk, sv, S)
    sub = dataclasses.replace(wl, batch=1, n_q_heads=wl.n_rep, n_kv_heads=1)
    n, d, R = wl.n_compressed, wl.head_dim, wl.n_recent
    per = sum(OL.bytes_per_token_head(d, wl.k_kind, wl.k_bits, wl.v_kind, wl.v_bits).values())
    t_enc = t_dec = 0.0
    done = []
    par = {"mismatch": 0, "excluded": 0, "excluded_differ": 0, "max_rel_err_end_to_end": 0.0}
    q_all = W.storage_to_f64(W.q_bits(wl), wl.in_dtype)
    order = [(wl.batch - 1, wl.n_kv_heads - 1)] + [(b, g) for b in range(wl.batch) for g in range(wl.n_kv_heads)]
    seen = set()
    start = time.time()
    for (b, g) in order:
        if (b, g) in seen:
            continue
        seen.add((b, g))
        Kb = W.kv_slice_bits(wl, W.ROLE_K, b, g)
        Vb = W.kv_slice_bits(wl, W.ROLE_V, b, g)
        k = W.storage_to_f64(Kb[None, None, :n], wl.in_dtype)
        v = W.storage_to_f64(Vb[None, None, :n], wl.in_dtype)
        t0 = time.perf_counter()
        ek = OC.encode_k(sub, k, st)
        ev = OC.encode_v(sub, v, st)
        t1 = time.perf_counter()
        planes = {nm: a for nm, a in {**ek, **ev}.items() if nm in ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")}
        rk = rv = None
        if R:
            rk = W.storage_to_f64(W.to_storage(W.storage_to_f64(Kb[None, None, n:], wl.in_dtype).astype(np.float32),
                                               wl.recent_dtype), wl.recent_dtype)
            rv = W.storage_to_f64(W.to_storage(W.storage_to_f64(Vb[None, None, n:], wl.in_dtype).astype(np.float32),
                                               wl.recent_dtype), wl.recent_dtype)
        q = q_all[b:b + 1, g * wl.n_rep:(g + 1) * wl.n_rep]
        t2 = time.perf_counter()
        ref = OD.decode_attention(sub, q, planes, n, st, rk, rv)
        t3 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t3 - t2
        done.append((b, g))
        # parity of this slice (outside the timed oracle work)
        gp = gpu_planes_fn(b, g)
        try:
            cs = H.compare_encode(wl, gp, ek, ev)
        except AssertionError as ex:
            cs = ex.args[0][1] if ex.args and isinstance(ex.args[0], tuple) else {"error": str(ex)}
        for key, val in cs.items():
            for tag in ("mismatch", "excluded_differ", "excluded"):
                if isinstance(val, int) and key.endswith(tag):
                    par[tag] += val
                    break
        got = gpu_out[b:b + 1, g * wl.n_rep:(g + 1) * wl.n_rep]
        par["max_rel_err_end_to_end"] = max(par["max_rel_err_end_to_end"], H.rel_err(got, ref))
        if time.time() - start > budget_s or (max_slices and len(done) >= max_slices):
            break
    dec_bytes = len(done) * (n * per + 2 * R * d * 2 + wl.n_rep * d * 6)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"value": dec_bytes / t_dec / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cores_affinity": affinity, "blas_threads": int(threads),
            "sample": f"{len(done)} of {wl.batch * wl.n_kv_heads} (batch, kv-head) slices (first {done[0]}), "
                      f"{n} compressed + {R} recent tokens each: oracle encode of keys+values, then decode of the "
                      f"slice's {wl.n_rep} query heads",
            "encode_tokens_per_s": len(done) * n / t_enc, "decode_s": t_dec, "encode_s": t_enc,
            "parity": dict(par, slices=[list(x) for x in done], tolerance=2e-3)}


def run_workload(tq, wl, a, digest: str, headline: bool) -> dict:
    import torch
    dev = torch.device("cuda", 0)
    B, n, R = wl.batch, wl.n_compressed, wl.n_recent
    lay = tq.layout_of(wl)
    state = tq.upload_state(lay, W.signs_to_mask(W.rotation_signs(wl, "k")), W.signs_to_mask(W.rotation_signs(wl, "v")),
                            W.qjl_matrix(wl), device=dev)
    t0 = time.time()
    K = W.kv_bits(wl, W.ROLE_K, threads=16)
    V = W.kv_bits(wl, W.ROLE_V, threads=16)
    log(f"[bench] {wl.name}: inputs {K.shape} generated in {time.time() - t0:.1f}s")

    def dev16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)

    k0, v0 = dev16(K[:, :, :n]), dev16(V[:, :, :n])
    rk = rv = None
    if R:
        conv = lambda X: W.to_storage(W.storage_to_f64(X[:, :, n:], wl.in_dtype).astype(np.float32), wl.recent_dtype)
        rk, rv = dev16(conv(K)), dev16(conv(V))
    q = dev16(W.q_bits(wl))
    del K, V

    in_bytes = 2 * k0.numel() * 2
    cache_bytes = sum(tq.tq_cache_plane_bytes(lay, B, n))
    ring = int(a.ring_gib * (1 << 30))
    n_in = max(1, min(16, -(-ring // in_bytes)))
    n_cache = max(2, min(256, -(-ring // cache_bytes)))
    ins = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n_in - 1)]
    caches = [tq.alloc_cache(lay, B, n, device=dev) for _ in range(n_cache)]
    ws_bytes = tq.tq_decode_workspace_bytes(lay, B, n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] ring: {n_in} input copies ({in_bytes / 2**20:.1f} MiB each), {n_cache} caches "
        f"({cache_bytes / 2**20:.1f} MiB each)")

    def enc_k(i):
        kk, _ = ins[i % n_in]
        tq.tq_encode(lay, state.struct, kk, None, B, n, 0, caches[i % n_cache].struct, stream)

    def enc_v(i):
        _, vv = ins[i % n_in]
        tq.tq_encode(lay, state.struct, None, vv, B, n, 0, caches[i % n_cache].struct, stream)

    def dec(i):
        c = caches[(i + n_cache // 2) % n_cache]
        tq.tq_decode_attn(lay, state.struct, q, c.struct, n, rk, rv, R, R, out, ws, ws_bytes, stream)

    # every cache holds a valid encoding before the timed region
    for i in range(n_cache):
        enc_k(i)
        enc_v(i)
    for i in range(a.warmup):
        enc_k(i), enc_v(i), dec(i)
    torch.cuda.synchronize()

    # exactly K steps, synchronised on both sides
    steps = a.steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        enc_k(i)
        enc_v(i)
        dec(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert torch.isfinite(out).all(), "non-finite attention output"

    # per-kernel-group statistics over R further event-timed steps
    reps = a.reps if a.step_only else max(a.reps, 200 if wl.n_ctx * wl.batch * wl.n_kv_heads <= 8 * 32768 else 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        e = evs[i]
        e[0].record(stream)
        enc_k(steps + i)
        e[1].record(stream)
        enc_v(steps + i)
        e[2].record(stream)
        dec(steps + i)
        e[3].record(stream)
    torch.cuda.synchronize()
    st = {g: stats([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(reps)])
          for j, g in enumerate(("encode_k", "encode_v", "decode"))}
    t_ek, t_ev, t_dec = (st[g]["median_ms"] for g in ("encode_k", "encode_v", "decode"))
    alg = algorithmic(wl)
    dec_gbs = alg["decode_bytes"] / (t_dec * 1e-3) / 1e9
    enc_tok = B * n / ((t_ek + t_ev) * 1e-3)

    kernels = {
        "encode_k": {"lm_qjl": "encode_lm_kernel (keys, QJL projection on fp16 matrix cores)",
                     "lm_mse": "encode_lm_kernel (keys)", "affine8": "encode_affine8_kernel",
                     "f16": "encode_copy16_kernel"}[wl.k_kind],
        "encode_v": {"group_sym": "encode_group_kernel", "group_asym": "encode_affine8_kernel (min/max values)",
                     "lm_rot": "encode_lm_kernel (values)"}[wl.v_kind],
        "decode": decode_kernel_name(wl) + " + decode_finish_kernel",
    }
    byts = {"encode_k": alg["encode_k_bytes"], "encode_v": alg["encode_v_bytes"], "decode": alg["decode_bytes"]}
    tr = read_traffic(wl.name, digest)
    ins_c = read_instr(wl.name, digest)
    rl = {}
    for g in ("encode_k", "encode_v", "decode"):
        ms = st[g]["median_ms"]
        gb = byts[g] / (ms * 1e-3) / 1e9
        rl[g] = {"bound": "hbm", "achieved": gb, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gb / HBM_PEAK_GBS,
                 "traffic": tr.get(g), "algorithmic_per_launch": byts[g], "kernel": kernels[g],
                 "ms_per_launch": ms, "p10_ms": st[g]["p10_ms"], "p90_ms": st[g]["p90_ms"], "reps": reps}
        if g in ins_c:
            rl[g]["counters_per_launch"] = ins_c[g]
    if wl.k_kind == "lm_qjl":
        # the QJL contraction (fp16 S times the fp16 hi and lo halves of the residual) is far
        # below its matrix-core peak; its fp32-product rate is reported beside the HBM figure
        rl["encode_k"]["qjl_tflops_fp32_products"] = alg["encode_k_qjl_flops"] / (t_ek * 1e-3) / 1e12
    dom = max(("encode_k", "encode_v", "decode"), key=lambda g: st[g]["median_ms"])

    res = {
        "workload": wl.name,
        "config": {"workload": wl.name, "batch": B, "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "context": wl.n_ctx, "compressed_tokens": n, "recent_tokens": R,
                   "keys": f"{wl.k_kind}{wl.k_bits}", "values": f"{wl.v_kind}{wl.v_bits}", "input_dtype": wl.in_dtype,
                   "bytes_per_token_head": alg["bytes_per_token_head"], "parallelism": "single-gpu"},
        "steps": steps, "ms_per_step": wall * 1e3 / steps,
        "decode_gbps": dec_gbs, "decode_pct_hbm_peak": 100.0 * dec_gbs / HBM_PEAK_GBS,
        "encode_tokens_per_s": enc_tok,
        "kernel_ms": {g: st[g]["median_ms"] for g in st}, "kernel_stats": st,
        "roofline": {k: rl[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} | {
            "kernel": rl[dom]["kernel"], "group": dom},
        "rooflines": rl,
    }
    if a.step_only:
        del caches, ins, k0, v0, ws
        torch.cuda.empty_cache()
        return res
    dec(0)
    torch.cuda.synchronize()
    res["deviation_from_exact_attention"] = exact_deviation(wl, k0, v0, rk, rv, q, out)
    try:
        res["decode_graph"] = bench_graph(tq, lay, state, caches, wl, stream, q, rk, rv, out, max(20, reps // 4))
        gms = res["decode_graph"]["per_decode"]["median_ms"]
        res["decode_graph"]["gbps"] = alg["decode_bytes"] / (gms * 1e-3) / 1e9
    except Exception as ex:          # capture unsupported: reported, not fatal
        res["decode_graph"] = {"error": repr(ex)}
    if wl.flush_tokens:
        res["flush_encode"] = bench_flush(tq, lay, state, wl, stream, max(50, reps // 2), 5)
    if not a.no_materialize:
        res["materialize"] = bench_materialize(tq, lay, state, caches, wl, stream, max(20, reps // 4), 3)
        mq = bench_multi(tq, lay, state, caches, wl, stream, rk, rv, max(20, reps // 4), 3)
        if mq is not None:
            res["multi_query"] = mq
    if not a.no_cpu_baseline:
        log(f"[bench] {wl.name}: timing the CPU oracle on a bounded sample ...")
        dec(0)
        torch.cuda.synchronize()
        out_np = out.double().cpu().numpy()
        c0 = caches[(0 + n_cache // 2) % n_cache]

        def planes_of(b, g):
            from compressed_decode_attention_encode_amd import tq as _tq
            names = ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")
            sizes = _tq.tq_cache_plane_bytes(lay, B, n)
            outp = {}
            for nm, sz in zip(names, sizes):
                if sz == 0:
                    continue
                row = sz // (B * wl.n_kv_heads * n)
                off = (b * wl.n_kv_heads + g) * n * row
                outp[nm] = c0.planes[nm][off:off + n * row].cpu().numpy()
            return _slice_views(wl, outp, n)

        res["cpu_baseline"] = cpu_baseline(wl, planes_of, out_np, budget_s=15.0 if headline else 4.0)
    del caches, ins, k0, v0, ws
    torch.cuda.empty_cache()
    return res


def _slice_views(wl, raw: dict, n: int) -> dict:
    """Typed [1, 1, n, ...] views of one slice's raw plane bytes (the layout in tq.h)."""
    d = wl.head_dim
    out = {}
    for nm, r in raw.items():
        if nm in ("k_codes", "k_signs", "v_codes"):
            out[nm] = r.view(np.uint32).reshape(1, 1, n, -1)
        elif nm == "k_aux":
            if wl.k_kind == "lm_qjl":
                out[nm] = r.view(np.uint16).reshape(1, 1, n, 2)
            elif wl.k_kind == "lm_mse":
                out[nm] = r.view(np.float32).reshape(1, 1, n)
            else:
                out[nm] = r.view(np.uint16).reshape(1, 1, n, d // 32, 2)
        elif nm == "v_aux":
            if wl.v_kind == "group_sym":
                out[nm] = r.view(np.uint16).reshape(1, 1, n, d // 32)
            elif wl.v_kind == "group_asym":
                out[nm] = r.view(np.uint16).reshape(1, 1, n, d // 32, 2)
            else:
                out[nm] = r.view(np.float32).reshape(1, 1, n)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=50, help="event-timed steps per workload for median/p10/p90 "
                                                         "(at least 50; 200 on the 32K Llama-like layer)")
    ap.add_argument("--workload", default="targets", choices=["targets"] + sorted(W.WORKLOADS),
                    help="one workload, or 'targets': the five 32K-128K workloads")
    ap.add_argument("--ring-gib", type=float, default=1.0, help="distinct input/cache bytes to rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-materialize", action="store_true",
                    help="skip the separate timing of tq_materialize and of the multi-query decode")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step (no ceiling, graph, flush, materialise, multi-query, exact-attention or "
                         "oracle legs): the command the profiler summaries are taken with")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device-to-device copies of MIB MiB (counter calibration) and exit")
    a = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}, "
              f"WORLD_SIZE {world}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from compressed_decode_attention_encode_amd import tq

    if a.calibrate_copy:
        # a copy of known size: each launch reads and writes MIB MiB, for scaling the HBM
        # byte counters of the profiled kernels
        n = a.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 10}))
        return

    torch.cuda.set_device(0)
    digest = source_digest()
    names = TARGETS if a.workload == "targets" else [a.workload]
    head = HEADLINE if HEADLINE in names else names[0]
    if a.step_only:
        a.no_ceiling = a.no_cpu_baseline = a.no_materialize = True
    ceiling = None if a.no_ceiling else stream_read_ceiling(tq)
    if ceiling:
        log(f"[bench] streaming-read ceiling {ceiling['gbps']:.0f} GB/s")
    per = {}
    for nm in names:
        per[nm] = run_workload(tq, W.WORKLOADS[nm], a, digest, headline=(nm == head))
        r = per[nm]
        log(f"[bench] {nm}: decode {r['kernel_ms']['decode'] * 1e3:.1f} us ({r['decode_pct_hbm_peak']:.1f}% HBM), "
            f"encode K {r['kernel_ms']['encode_k'] * 1e3:.1f} us, V {r['kernel_ms']['encode_v'] * 1e3:.1f} us, "
            f"{r['encode_tokens_per_s'] / 1e6:.0f} Mtok/s")
    h = per[head]
    line = {
        "metric": METRIC, "value": h["decode_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 products, fp32 accumulation", "data": "synthetic",
        "config": h["config"],
        "decode_pct_hbm_peak": h["decode_pct_hbm_peak"],
        "encode_tokens_per_s": h["encode_tokens_per_s"],
        "kernel_ms": h["kernel_ms"],
        "roofline": h["roofline"],
        "rooflines": h["rooflines"],
        "stream_read_ceiling": ceiling,
        "parity": {"deviation_from_exact_attention": h.get("deviation_from_exact_attention"),
                   "oracle_sample": h.get("cpu_baseline", {}).get("parity")},
        "source_digest": digest,
        "workloads": {nm: {k: v for k, v in r.items() if k != "cpu_baseline"} |
                      ({"cpu_oracle": r["cpu_baseline"]} if "cpu_baseline" in r and nm != head else {})
                      for nm, r in per.items()},
    }
    if ceiling:
        line["decode_frac_of_stream_ceiling"] = h["decode_gbps"] / ceiling["gbps"]
    if "cpu_baseline" in h:
        cb = dict(h["cpu_baseline"])
        line["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")} | {
            "cores_affinity": cb["cores_affinity"], "blas_threads": cb["blas_threads"],
            "encode_tokens_per_s": cb["encode_tokens_per_s"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
