#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV encode + decode-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path over one batch of synthetic input:
tq_encode of the workload's compressed history (keys, then values) followed by one
tq_decode_attn (query prep, split-K attention on the packed cache, combine with the
exact recent buffer).  Codebooks and rotation state are built once before timing.

Inputs and packed caches rotate over >= 1 GiB of distinct copies so that the 256 MB
Infinity Cache cannot serve a repeat: step i encodes input copy i into cache copy i
and decodes a cache copy written half a ring earlier.  Kernel durations come from HIP
events recorded on the stream the library launches on; the whole-step time from a
synchronized wall clock around exactly K steps.

Prints one JSON line on stdout:
  value       decode-attention KV GB/s (algorithmic bytes / decode kernel time)
  roofline    the dominant kernel against its MI355X peak
  materialize tq_materialize of the whole history to fp16 rows (timed apart from the
              step: the dequantise path ahead of a dense prefill)
  multi_query tq_decode_attn_multi with 4 queries (2 where 4 x n_rep rows are not compiled;
              a speculative step) against as many single-query decodes of the same cache
              (timed apart from the step)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_decode_attention_encode_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


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
            "encode_k_qjl_flops": qjl_flops, "vectors": rows}


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


def read_traffic(workload: str, digest: str):
    """HBM bytes per launch of each kernel group (key encode, value encode, decode) from
    the committed counter summary, or {} when it is absent or was taken on different
    kernel sources.  Lines `group.<name>.hbm_bytes_per_launch = <bytes>`."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != digest:
        return {}
    out = {}
    for k, v in kv.items():
        if k.startswith("group.") and k.endswith(".hbm_bytes_per_launch"):
            try:
                out[k[len("group."):-len(".hbm_bytes_per_launch")]] = float(v)
            except ValueError:
                pass
    return out


def bench_materialize(tq, lay, state, caches, wl, stream, steps: int, warmup: int) -> dict:
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

    for i in range(warmup):
        run(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record(stream)
        run(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    gb = alg / (ms * 1e-3) / 1e9
    res = {"us": ms * 1e3, "gbps": gb, "algorithmic_bytes": alg, "steps": steps,
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


def bench_multi(tq, lay, state, caches, wl, stream, rk, rv, steps: int, warmup: int) -> dict | None:
    """tq_decode_attn_multi with 4 queries (a speculative step: the last n_query recent tokens
    are the drafts' own; 2 where 4 x n_rep query rows exceed the compiled set) against
    n_query single-query decodes of the same cache, timed apart from the step; None where the
    layout has no multi-query kernel."""
    for nq in (4, 2):
        r = _bench_multi(tq, lay, state, caches, wl, stream, rk, rv, steps, warmup, nq)
        if r is not None:
            return r
    return None


def _bench_multi(tq, lay, state, caches, wl, stream, rk, rv, steps: int, warmup: int, n_query: int) -> dict | None:
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
    res = {}
    for name, fn in (("multi", multi), ("singles", singles)):
        for i in range(warmup):
            fn(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            evs[i][0].record(stream)
            fn(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        res[name] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
    per = plane_bytes_per_token_head(wl)
    kv_bytes = B * wl.n_kv_heads * n * sum(per.values()) + 2 * B * wl.n_kv_heads * R * wl.head_dim * 2
    return {"n_query": n_query, "us": res["multi"], "single_query_decodes_us": res["singles"],
            "speedup_vs_single_decodes": res["singles"] / res["multi"],
            "kv_gbps": kv_bytes / (res["multi"] * 1e-6) / 1e9,
            "kernels": "decode_mma_kernel (n_query x n_rep query rows) + decode_finish_kernel"}


def cpu_baseline(wl, budget_s: float = 15.0):
    """Time the CPU oracle (as it stands) on whole (batch, kv-head) slices of the workload
    until about `budget_s` of CPU work: encode of the slice's keys and values, then
    decode of its n_rep query heads.  Reported in the metric's unit (decode GB/s)."""
    from oracle import cache as OC
    from oracle import decode as OD
    from oracle import layout as OL
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
    done = 0
    q_all = W.storage_to_f64(W.q_bits(wl), wl.in_dtype)
    start = time.time()
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
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
            OD.decode_attention(sub, q, planes, n, st, rk, rv)
            t3 = time.perf_counter()
            t_enc += t1 - t0
            t_dec += t3 - t2
            done += 1
            if time.time() - start > budget_s:
                break
        else:
            continue
        break
    dec_bytes = done * (n * per + 2 * R * d * 2 + wl.n_rep * d * 6)
    return {"value": dec_bytes / t_dec / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {wl.batch * wl.n_kv_heads} (batch, kv-head) slices, {n} compressed + {R} recent "
                      f"tokens each: oracle encode of keys+values, then decode of the slice's {wl.n_rep} query heads",
            "encode_tokens_per_s": done * n / t_enc, "decode_s": t_dec, "encode_s": t_enc}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=W.BENCH_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--ring-gib", type=float, default=1.0, help="distinct input/cache bytes to rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-materialize", action="store_true",
                    help="skip the separate timing of tq_materialize (dequantisation of the whole cache)")
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

    wl = W.WORKLOADS[a.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    B, n, R = wl.batch, wl.n_compressed, wl.n_recent
    lay = tq.layout_of(wl)
    state = tq.upload_state(lay, W.signs_to_mask(W.rotation_signs(wl, "k")), W.signs_to_mask(W.rotation_signs(wl, "v")),
                            W.qjl_matrix(wl), device=dev)

    t0 = time.time()
    K = W.kv_bits(wl, W.ROLE_K)
    V = W.kv_bits(wl, W.ROLE_V)
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

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(a.steps):
        e = evs[i]
        e[0].record(stream)
        enc_k(i)
        e[1].record(stream)
        enc_v(i)
        e[2].record(stream)
        dec(i)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert torch.isfinite(out).all(), "non-finite attention output"

    ms = lambda j: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(a.steps)]))
    t_ek, t_ev, t_dec = ms(0), ms(1), ms(2)
    alg = algorithmic(wl)
    dec_gbs = alg["decode_bytes"] / (t_dec * 1e-3) / 1e9
    enc_tok = B * n / ((t_ek + t_ev) * 1e-3)

    digest = source_digest()
    groups = {
        "encode_k": {"kernel": {"lm_qjl": "encode_lm_kernel (keys)", "lm_mse": "encode_lm_kernel (keys)",
                                "affine8": "encode_affine8_kernel", "f16": "encode_copy16_kernel"}[wl.k_kind],
                     "ms": t_ek},
        "encode_v": {"kernel": {"group_sym": "encode_group_kernel", "group_asym": "encode_affine8_kernel (min/max values)",
                                "lm_rot": "encode_lm_kernel (values)"}[wl.v_kind],
                     "ms": t_ev},
        "decode": {"kernel": decode_kernel_name(wl) + " + decode_finish_kernel", "ms": t_dec},
    }
    rl = {}
    # key encode: the QJL contraction runs on the fp16 matrix cores (fp16 S times the fp16
    # hi and lo halves of the residual: 2 x 2 d^2 flops per vector, ~1.7 us at 2.5 PFLOP/s
    # on the bench workload) -- below the time its bytes take at 8 TB/s, so HBM is the
    # binding roofline; the fp32-equivalent QJL rate is reported beside it
    gb = alg["encode_k_bytes"] / (t_ek * 1e-3) / 1e9
    rl["encode_k"] = {"bound": "hbm", "achieved": gb, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": gb / HBM_PEAK_GBS, "traffic": None, "algorithmic_per_launch": alg["encode_k_bytes"]}
    if wl.k_kind == "lm_qjl":
        rl["encode_k"]["qjl_tflops_fp32_products"] = alg["encode_k_qjl_flops"] / (t_ek * 1e-3) / 1e12
    gb = alg["encode_v_bytes"] / (t_ev * 1e-3) / 1e9
    rl["encode_v"] = {"bound": "hbm", "achieved": gb, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gb / HBM_PEAK_GBS,
                      "traffic": None, "algorithmic_per_launch": alg["encode_v_bytes"]}
    rl["decode"] = {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dec_gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_per_launch": alg["decode_bytes"]}
    dom = max(groups, key=lambda g: groups[g]["ms"])
    tr = read_traffic(wl.name, digest)
    for g in rl:
        rl[g]["traffic"] = tr.get(g)
    for g in rl:
        rl[g]["kernel"] = groups[g]["kernel"]
        rl[g]["ms_per_launch"] = groups[g]["ms"]

    line = {
        "metric": METRIC, "value": dec_gbs, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": wall * 1e3 / a.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "context": wl.n_ctx, "compressed_tokens": n, "recent_tokens": R,
                   "keys": f"{wl.k_kind}{wl.k_bits}", "values": f"{wl.v_kind}{wl.v_bits}", "input_dtype": wl.in_dtype,
                   "parallelism": "single-gpu"},
        "decode_pct_hbm_peak": 100.0 * dec_gbs / HBM_PEAK_GBS,
        "encode_tokens_per_s": enc_tok,
        "kernel_ms": {g: groups[g]["ms"] for g in groups},
        "roofline": {k: rl[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} | {
            "kernel": rl[dom]["kernel"], "group": dom},
        "rooflines": rl,
        "source_digest": digest,
    }
    if not a.no_materialize:
        line["materialize"] = bench_materialize(tq, lay, state, caches, wl, stream, max(10, a.steps // 4),
                                                max(2, a.warmup // 4))
    if not a.no_materialize:
        mq = bench_multi(tq, lay, state, caches, wl, stream, rk, rv, max(10, a.steps // 4), max(2, a.warmup // 4))
        if mq is not None:
            line["multi_query"] = mq
    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
