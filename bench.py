"""Benchmark of the LLSA hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input already resident in HBM:
pyramid -> hierarchical selection -> enriched attention forward -> CSR->CSC transpose -> backward,
each through the C ABI of libllsa.so on torch's current stream, except the transpose, which needs only the
selection and runs on a second stream beside the forward (the backward waits for it).  The workload is the N = 65536
forward+backward configuration (batch 1, 16 heads, head dim 64, bf16, B = 16, K = 8, L = 3, smooth
2-D Gaussian-random-field inputs on a 256x256 grid plus 0.1 noise, dO ~ N(0, 1)).

Prints ONE JSON line: the metric (ms per fwd+bwd step, lower is better), a per-stage breakdown, the
roofline of the dominant kernel (algorithmic bytes / its average launch time, timed with events on
the launch stream) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "LLSA fwd+bwd ms at N=65536 (MFMA util %, selection HBM GB/s)"
COPY_PROBE_BYTES = 256 << 20
WORKLOAD = "fwdbwd_bf16_n65536"
WARM_STEPS = 50                # steps of the per-step (median, min, max) distributions


KERNEL_SYMBOL = {"pool": "pool_levels12", "select": "select_level", "attn_fwd": "attn_fwd_bf16",
                 "transpose": "csc_*", "bwd_dq": "bwd_dq_bf16", "bwd_reduce": "coarse_reduce",
                 "bwd_dkdv": "bwd_dkdv_bf16"}


def algorithmic(w, levels, enrich):
    """Algorithmic bytes and flops per step of every kernel family: each tensor is counted once (a gathered
    K/V block read by many query blocks counts once), products at their exact sizes (no padding)."""
    bh, n, d, B, K = w.bh, w.n, w.d, w.block, w.topk
    s = 2  # bf16 bytes
    tokens = bh * n
    rows = [n // B ** l for l in range(1, levels + 1)]
    R = sum(rows)
    pooled_frac = sum(B ** -l for l in range(1, levels + 1))
    fine = K * B                                       # raw keys per query
    coarse = K * enrich                                # enrichment tokens per query
    nhigh = K * max(0, enrich - 1)                     # enrichment tokens of levels >= 2 per query
    pooled_kv = 2 * bh * R * d * s                     # the bf16 copies of the K and V pyramids
    out = {}
    # pyramid: read Q, K, V once, write three fp32 pyramids and the bf16 copies of two
    out["pool"] = dict(bytes=tokens * (3 * d * s + (3 * d * 4 + 2 * d * s) * pooled_frac), flops=0.0)
    # selection: per pooled query unit read its pooled query and key rows (fp32), its parent row and write
    # K indices; flops of the scored (unit, block) pairs
    out["select"] = dict(bytes=bh * R * (2 * d * 4 + 2 * K * 4),
                         flops=2.0 * d * bh * (rows[-1] ** 2 + sum(rows[l - 1] * K * B for l in range(1, levels))))
    # forward: read Q, K, V, write O (bf16), write LSE, read the pooled K/V once; QK^T and PV products
    out["attn_fwd"] = dict(bytes=tokens * (4 * d * s + 4) + pooled_kv, flops=4.0 * d * (fine + coarse) * tokens)
    # transpose: read each CSR entry, write it to the CSC, write col_ptr
    T = max(1, min(enrich, levels))
    nnz = bh * sum(rows[l - 1] * K for l in range(1, T + 1))
    out["transpose"] = dict(bytes=8.0 * nnz + 4.0 * bh * sum(rows[l - 1] + 1 for l in range(1, T + 1)), flops=0.0)
    # backward dQ kernel: read Q, K, V, O, dO, LSE, pooled K/V; write dQ, Delta, pooled-token partials;
    # products S, dP, dQ over every entry plus the pooled dK/dV partials of levels >= 2
    n2 = rows[1] if levels >= 2 else 0
    part = 2 * bh * n2 * nhigh * d * 4
    out["bwd_dq"] = dict(bytes=tokens * (6 * d * s + 8) + pooled_kv + part,
                         flops=6.0 * d * (fine + coarse) * tokens + 4.0 * d * nhigh * tokens)
    # pooled-gradient reduction: read the partials, write the reduced pooled gradients of levels >= 2
    out["bwd_reduce"] = dict(bytes=part + 2 * bh * (R - rows[0]) * d * 4, flops=0.0)
    # backward dK/dV kernel: read K, V, Q, dO, LSE, Delta, level-1 pooled K/V and reduced gradients; write dK, dV;
    # products S, dP, dV, dK over the fine entries plus the level-1 pooled token
    out["bwd_dkdv"] = dict(bytes=tokens * (6 * d * s + 8) + 2 * bh * rows[0] * d * s + 2 * bh * (R - rows[0]) * d * 4,
                           flops=8.0 * d * fine * tokens + 6.0 * d * K * tokens)
    return out


def complement_algorithmic(w, levels, enrich):
    """Complement-partition reading of the enrichment: entries per fine block, list ints per slice, and the
    algorithmic bytes / flops of the list kernel and of its forward (each tensor counted once)."""
    bh, n, d, B, K = w.bh, w.n, w.d, w.block, w.topk
    rows = [n // B ** l for l in range(1, levels + 1)]
    m = [rows[-1] - K if l == levels else (B - 1) * K for l in range(1, enrich + 1)]
    total, ints = sum(m), sum(rows[l - 1] * m[l - 1] for l in range(1, enrich + 1))
    tokens, R = bh * n, sum(rows)
    lists = dict(bytes=bh * (R * K * 4 + ints * 4), flops=0.0)
    fwd = dict(bytes=tokens * (4 * d * 2 + 4) + 2 * bh * R * d * 2 + bh * ints * 4,
               flops=4.0 * d * (K * B + total) * tokens)
    return total, ints, lists, fwd


def oracle_baseline(w, x, budget_s=20.0):
    """Oracle chain timed on whole (batch, head) slices until ~budget_s of CPU work; scaled to one step."""
    import oracle
    t_all = 0.0
    done = 0
    for h in range(w.bh):
        q, k, v, do = (x[nm].exact.reshape(w.bh, w.n, w.d)[h:h + 1] for nm in ("q", "k", "v", "dout"))
        t0 = time.perf_counter()
        oracle.run(q, k, v, w.block, w.topk, levels=w.levels, dout=do)
        t_all += time.perf_counter() - t0
        done += 1
        if t_all >= budget_s:
            break
    ms_full = t_all / done * w.bh * 1e3
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(ms_full, 1), "unit": "ms", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": model,
            "sample": f"{done} of {w.bh} (batch, head) slices of the {WORKLOAD} workload, full chain "
                      f"(pool, select, forward, transpose, backward) in fp64; {t_all:.1f} s measured, "
                      f"scaled by {w.bh}/{done} to one step"}


def dense_sdpa(w, q, k, v, do, steps, llsa_fwd_ms, llsa_step_ms):
    """Dense attention at the same shapes with PyTorch SDPA (flash or memory-efficient backend only -- the math
    backend would materialise n x n scores), timed for the forward and the forward+backward; the ratio to the
    LLSA chain puts the sparse path beside dense attention."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    shape = (w.batch, w.heads, w.n, w.d)
    qq, kk, vv, gg = (t.view(shape) for t in (q, k, v, do))
    errors = {}
    for backend in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([backend]):
                F.scaled_dot_product_attention(qq, kk, vv)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    F.scaled_dot_product_attention(qq, kk, vv)
                e1.record()
                torch.cuda.synchronize()
                fwd_ms = e0.elapsed_time(e1) / steps
                ql, kl, vl = (t.detach().requires_grad_(True) for t in (qq, kk, vv))
                F.scaled_dot_product_attention(ql, kl, vl).backward(gg)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(steps):
                    F.scaled_dot_product_attention(ql, kl, vl).backward(gg)
                e1.record()
                torch.cuda.synchronize()
                fb_ms = e0.elapsed_time(e1) / steps
            return {"backend": backend.name, "fwd_ms": round(fwd_ms, 3), "fwdbwd_ms": round(fb_ms, 3),
                    "llsa_fwd_chain_ms": round(llsa_fwd_ms, 4), "llsa_fwdbwd_ms": round(llsa_step_ms, 4),
                    "speedup_fwd": round(fwd_ms / llsa_fwd_ms, 2), "speedup_fwdbwd": round(fb_ms / llsa_step_ms, 2)}
        except RuntimeError as e:  # backend not available for these shapes / this device
            errors[backend.name] = str(e).splitlines()[0][:200]
    return {"error": errors}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--reorder", action="store_true",
                    help="also time the chain on 2-D-locally reordered inputs (reorder Q, K, V, dO in; O, dQ, dK, "
                         "dV back out)")
    ap.add_argument("--exhaustive", action="store_true",
                    help="also time the single-level exhaustive Top-K and report the hierarchy's routing recall")
    ap.add_argument("--dense", action="store_true",
                    help="also time dense PyTorch SDPA (flash / memory-efficient backend) at the same shapes")
    ap.add_argument("--complement", action="store_true",
                    help="also time the forward under the complement-partition reading of the enrichment")
    ap.add_argument("--configs", action="store_true",
                    help="also time the other workloads: the forward chain (pool, select, forward) of the N = 4096 "
                         "fp32, N = 16384 and N = 65536 forward workloads, the whole step of the N = 262144 one")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the per-step timings that each follow a 1 GiB buffer write (L2 and MALL flushed)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain device copy of COPY_PROBE_BYTES after the warm-up (calibrates rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE; see hierarchical_sparse_attention_mean_amd/profiling.py)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path shards by "
              "(batch x heads) with no exchange, but only the one-GPU share is built and measured)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hierarchical_sparse_attention_mean_amd import inputs, llsa, profiling

    w = inputs.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    x = inputs.make_inputs(w, with_dout=True)
    gen_s = time.perf_counter() - t0

    def dev(t):
        return torch.from_numpy(t.store.view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    b = llsa.Buffers(llsa.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels))
    p = b.prob
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority, like every stream here

    def step():
        # pyramid -> selection -> forward, the index transpose on the second stream beside the forward -> backward
        b.forward_backward(q, k, v, do, stream, side)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"timed {args.steps} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    # Second timed region over the same work with the library's per-kernel event timing switched on: every
    # kernel launch is bracketed by hipEvents recorded on the stream it is launched on.
    llsa.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step_events = (time.perf_counter() - t0) * 1e3 / args.steps
    fam = llsa.timing_read()
    llsa.timing_enable(False)

    alg = algorithmic(w, p.levels, p.enrich_levels)
    kernels = {}
    for nm, (tot, cnt) in fam.items():
        if cnt == 0:
            continue
        per_step = tot / args.steps
        a = alg[nm]
        kernels[nm] = {"ms_per_step": round(per_step, 4), "launches_per_step": cnt // args.steps,
                       "avg_launch_ms": round(tot / cnt, 4),
                       "alg_GBps": round(a["bytes"] / (per_step * 1e-3) / 1e9, 1),
                       "alg_TFLOPs": round(a["flops"] / (per_step * 1e-3) / 1e12, 2)}
    dom = max(kernels, key=lambda nm: kernels[nm]["ms_per_step"])
    dk = kernels[dom]
    a_gbs = alg[dom]["bytes"] / (dk["avg_launch_ms"] * 1e-3) / 1e9 if dk["launches_per_step"] == 1 else dk["alg_GBps"]
    # HBM bytes per launch measured by rocprofv3 FETCH_SIZE + WRITE_SIZE (calibrated by a plain copy), from the
    # committed summary under profiles/; None when absent or when the kernel's sources changed since
    traffic = profiling.read_traffic(KERNEL_SYMBOL[dom], w.name)
    roofline = {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": KERNEL_SYMBOL[dom], "kernel_avg_ms": dk["avg_launch_ms"],
                "alg_bytes_per_launch": alg[dom]["bytes"], "alg_flops_per_launch": alg[dom]["flops"],
                "mfma_frac": round(alg[dom]["flops"] / (dk["avg_launch_ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}
    attn = ("attn_fwd", "bwd_dq", "bwd_reduce", "bwd_dkdv")
    attn_flops = sum(alg[nm]["flops"] for nm in attn)
    attn_ms = sum(kernels[nm]["ms_per_step"] for nm in attn if nm in kernels)
    mfma_util = attn_flops / (attn_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    sel_gbs = kernels["select"]["alg_GBps"]
    pool_gbs = kernels["pool"]["alg_GBps"]

    exhaustive = None
    if args.exhaustive:
        n1 = w.n // w.block
        idx1 = torch.empty((w.bh, n1, w.topk), dtype=torch.int32, device="cuda")
        llsa.select_exhaustive(p, b.pq, b.pk, idx1, stream)
        torch.cuda.synchronize()
        reps = max(3, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            llsa.select_exhaustive(p, b.pq, b.pk, idx1, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        hier = b.idx[:, :n1]
        hit = (hier[..., :, None] == idx1[..., None, :]).any(-1).sum(-1).float()
        exhaustive = {"exhaustive_select_ms": round(e0.elapsed_time(e1) / reps, 4),
                      "hierarchical_select_ms": kernels["select"]["ms_per_step"],
                      "routing_recall": round(float(hit.mean()) / w.topk, 4),
                      "units_fully_recalled": round(float((hit == w.topk).float().mean()), 4)}

    reordered = None
    if args.reorder:
        H, W = w.grid
        qr, kr, vr, dr = (torch.empty_like(t) for t in (q, k, v, do))
        o2, dq2, dk2, dv2 = (torch.empty_like(t) for t in (q, q, q, q))

        def step_reordered():
            for a, z in ((q, qr), (k, kr), (v, vr), (do, dr)):
                llsa.reorder(p, H, W, True, a, z, stream)
            b.forward_backward(qr, kr, vr, dr, stream, side)
            for a, z in ((b.o, o2), (b.dq, dq2), (b.dk, dk2), (b.dv, dv2)):
                llsa.reorder(p, H, W, False, a, z, stream)

        for _ in range(args.warmup):
            step_reordered()
        torch.cuda.synchronize()
        llsa.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_reordered()
        torch.cuda.synchronize()
        ms_r = (time.perf_counter() - t0) * 1e3 / args.steps
        fam_r = llsa.timing_read()
        llsa.timing_enable(False)
        if args.exhaustive:  # routing recall of the hierarchy on the reordered sequence
            n1 = w.n // w.block
            idx1 = torch.empty((w.bh, n1, w.topk), dtype=torch.int32, device="cuda")
            llsa.select_exhaustive(p, b.pq, b.pk, idx1, stream)
            torch.cuda.synchronize()
            hit = (b.idx[:, :n1][..., :, None] == idx1[..., None, :]).any(-1).sum(-1).float()
            recall_r = round(float(hit.mean()) / w.topk, 4)
        else:
            recall_r = None
        reordered = {"grid": [H, W], "ms_per_step": round(ms_r, 4), "routing_recall": recall_r,
                     "reorder_ms_per_step": round(fam_r["reorder"][0] / args.steps, 4),
                     "kernels_ms_per_step": {nm: round(tc[0] / args.steps, 4) for nm, tc in fam_r.items() if tc[1]}}

    complement = None
    if args.complement:
        total, ints, a_lists, a_fwd = complement_algorithmic(w, p.levels, p.enrich_levels)
        ws_c = torch.empty(max(1, llsa.workspace_bytes(p, llsa.OP_ATTN_FWD_COMPLEMENT)), dtype=torch.uint8,
                           device="cuda")
        o_c, lse_c = torch.empty_like(b.o), torch.empty_like(b.lse)
        for _ in range(2):
            llsa.attn_fwd_complement(p, q, k, v, b.pka, b.pva, b.idx, o_c, lse_c, ws_c, stream)
        torch.cuda.synchronize()
        reps = max(3, args.steps // 2)
        llsa.timing_enable(True)
        for _ in range(reps):
            llsa.attn_fwd_complement(p, q, k, v, b.pka, b.pva, b.idx, o_c, lse_c, ws_c, stream)
        torch.cuda.synchronize()
        fam_c = llsa.timing_read()
        llsa.timing_enable(False)
        lists_ms, fwd_ms = fam_c["complement"][0] / reps, fam_c["attn_fwd"][0] / reps
        # the whole step under this reading: pyramid, selection, forward, backward (which builds its own lists
        # and CSC of levels 1..min(L_e + 1, L))
        ws_cb = torch.empty(max(1, llsa.workspace_bytes(p, llsa.OP_ATTN_BWD_COMPLEMENT)), dtype=torch.uint8,
                            device="cuda")
        dq_c, dk_c, dv_c = (torch.empty_like(q) for _ in range(3))

        def step_c():
            b.pyramid(q, k, v, stream)
            llsa.select(p, b.pq, b.pk, b.idx, stream)
            llsa.attn_fwd_complement(p, q, k, v, b.pka, b.pva, b.idx, o_c, lse_c, ws_c, stream)
            llsa.attn_bwd_complement(p, q, k, v, o_c, lse_c, do, b.pka, b.pva, b.idx, dq_c, dk_c, dv_c, ws_cb,
                                     stream)

        for _ in range(2):
            step_c()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            step_c()
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) * 1e3 / reps
        llsa.timing_enable(True)
        for _ in range(reps):
            step_c()
        torch.cuda.synchronize()
        fam_s = llsa.timing_read()
        llsa.timing_enable(False)
        complement = {"entries_per_fine_block": total, "selected_entries_per_fine_block": p.topk * p.enrich_levels,
                      "lists_ms": round(lists_ms, 4), "attn_fwd_ms": round(fwd_ms, 4),
                      "attn_fwd_alg_GBps": round(a_fwd["bytes"] / (fwd_ms * 1e-3) / 1e9, 1),
                      "attn_fwd_alg_TFLOPs": round(a_fwd["flops"] / (fwd_ms * 1e-3) / 1e12, 2),
                      "selected_reading_attn_fwd_ms": kernels["attn_fwd"]["ms_per_step"],
                      "fwdbwd_ms_per_step": round(step_ms, 4),
                      "fwdbwd_kernels_ms_per_step": {nm: round(tc[0] / reps, 4) for nm, tc in fam_s.items() if tc[1]},
                      "workspace_bytes_bwd": ws_cb.numel()}
        del ws_c, o_c, lse_c, ws_cb, dq_c, dk_c, dv_c

    # per-step distributions (hipEvents on the main stream, which joins the side stream before the backward):
    # warm = steps back to back as above, each timed alone; cold = each step right after a 1 GiB buffer write,
    # which flushes the L2s and the MALL
    def step_times(n, flush=None):
        times = []
        for _ in range(n):
            if flush is not None:
                flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return {"median_ms": round(float(np.median(times)), 4), "min_ms": round(min(times), 4),
                "max_ms": round(max(times), 4), "steps": n}

    warm = step_times(WARM_STEPS)
    cold = None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold = step_times(WARM_STEPS, flush)
        del flush

    configs = None
    if args.configs:
        configs = {}
        for name in ("tiny_fwd_f32_n4096", "fwd_bf16_n16384", "fwd_bf16_n65536", "fwdbwd_bf16_n262144"):
            wc = inputs.WORKLOADS[name]
            xc = inputs.make_inputs(wc)
            tc = {}
            for nm, tt in xc.items():
                arr = tt.store
                tc[nm] = (torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16) if arr.dtype == np.uint16
                          else torch.from_numpy(np.ascontiguousarray(arr)).cuda())
            bc = llsa.Buffers(llsa.problem(wc.batch, wc.heads, wc.n, wc.d, wc.block, wc.topk, wc.levels,
                                           dtype=llsa.BF16 if wc.dtype == "bf16" else llsa.F32),
                              backward=wc.backward)
            if wc.backward:
                def run_c():
                    bc.forward_backward(tc["q"], tc["k"], tc["v"], tc["dout"], stream, side)
            else:
                def run_c():
                    bc.forward(tc["q"], tc["k"], tc["v"], stream)
            for _ in range(3):
                run_c()
            torch.cuda.synchronize()
            reps = max(5, args.steps // 2)
            t0 = time.perf_counter()
            for _ in range(reps):
                run_c()
            torch.cuda.synchronize()
            configs[name] = {"ms_per_step": round((time.perf_counter() - t0) * 1e3 / reps, 4),
                             "step": "pool+select+forward+transpose+backward" if wc.backward
                             else "pool+select+forward",
                             "batch": wc.batch, "heads": wc.heads, "seq_len": wc.n, "dtype": wc.dtype, "topk": wc.topk,
                             "levels": wc.levels}
            del bc, tc, xc
            torch.cuda.empty_cache()

    dense = None
    if args.dense:
        fwd_chain = sum(kernels[nm]["ms_per_step"] for nm in ("pool", "select", "attn_fwd"))
        dense = dense_sdpa(w, q, k, v, do, max(3, args.steps // 4), fwd_chain, ms_step)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_baseline(w, x)

    rec = {
        "metric": METRIC, "value": round(ms_step, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.n, "head_dim": w.d,
                   "block": w.block, "topk": w.topk, "levels": p.levels, "enrich_levels": p.enrich_levels,
                   "grid": list(w.grid), "inputs": "2-D Gaussian random field (l=16 px) projected to 64 dims + 0.1 noise",
                   "parallelism": "none (one GPU)"},
        "mfma_util_pct_attention": round(100 * mfma_util, 2),
        "selection_alg_GBps": round(sel_gbs, 1),
        "pyramid_alg_GBps": round(pool_gbs, 1),
        "ms_per_step_with_kernel_events": round(ms_step_events, 4),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_sdpa": dense,
        "exhaustive_selection": exhaustive,
        "reordered_chain": reordered,
        "complement_forward": complement,
        "warm_steps": warm,
        "cold_steps": cold,
        "other_workloads": configs,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
