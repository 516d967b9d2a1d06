"""Benchmark of the LLSA hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input already resident in HBM:
pyramid -> hierarchical selection -> enriched attention forward -> CSR->CSC transpose -> backward,
each through the C ABI of libllsa.so on torch's current stream, except the transpose, which needs only the
selection and runs on a second stream beside the forward (the backward waits for it).  The headline workload is
the N = 65536 forward+backward configuration (batch 1, 16 heads, head dim 64, bf16, B = 16, K = 8, L = 3, smooth
2-D Gaussian-random-field inputs on a 256x256 grid plus 0.1 noise, dO ~ N(0, 1)).

Prints ONE JSON line: the metric (ms per fwd+bwd step, lower is better), a per-kernel breakdown, the roofline of
the dominant kernel (algorithmic bytes / its average launch time, timed with events on the launch stream), the
fp64 CPU oracle timed on the same workload, and -- unless --headline-only -- the other four workloads (each with
its own breakdown and roofline) and the measurements beside the hot path: dense attention at the same shapes,
routing recall against exhaustive Top-K, the chain on 2-D-locally reordered inputs and the complement reading.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, TFLOP/s
METRIC = "LLSA fwd+bwd ms at N=65536 (MFMA util %, selection HBM GB/s)"
COPY_PROBE_BYTES = 256 << 20
WORKLOAD = "fwdbwd_bf16_n65536"
OTHER_WORKLOADS = ("tiny_fwd_f32_n4096", "fwd_bf16_n16384", "fwd_bf16_n65536", "fwdbwd_bf16_n262144")
WARM_STEPS = 50                # steps of the per-step (median, min, max) distributions
ATTN = ("attn_fwd", "bwd_dq", "bwd_reduce", "bwd_dkdv")


def kernel_symbol(name, w, enrich):
    """The kernel a family runs on workload w: the bf16 forward pairs fine blocks when n_1 is even, K <= 32 and
    K * L_e <= 64 (the limits of attn_fwd_pair_bf16), else runs one block per wave."""
    if w.dtype == "bf16":
        pair = (w.n // w.block) % 2 == 0 and w.topk <= 32 and w.topk * enrich <= 64
        fwd = "attn_fwd_pair_bf16" if pair else "attn_fwd_bf16"
    else:
        fwd = "attn_fwd_f32"
    return {"pool": "pool_levels12", "select": "select_level", "attn_fwd": fwd,
            "transpose": "csc_*", "bwd_dq": "bwd_dq_bf16", "bwd_reduce": "reduce_and_order",
            "bwd_dkdv": "bwd_dkdv_bf16"}[name]


def algorithmic(w, levels, enrich):
    """Algorithmic bytes and flops per step of every kernel family: each tensor is counted once (a gathered
    K/V block read by many query blocks counts once), products at their exact sizes (no padding)."""
    bh, n, d, B, K = w.bh, w.n, w.d, w.block, w.topk
    s = 2 if w.dtype == "bf16" else 4  # bytes per raw element
    tokens = bh * n
    rows = [n // B ** l for l in range(1, levels + 1)]
    R = sum(rows)
    pooled_frac = sum(B ** -l for l in range(1, levels + 1))
    fine = K * B                                       # raw keys per query
    coarse = K * enrich                                # enrichment tokens per query
    nhigh = K * max(0, enrich - 1)                     # enrichment tokens of levels >= 2 per query
    pooled_kv = 2 * bh * R * d * s                     # the pooled K and V the attention reads (raw dtype)
    copies = 2 * d * s if s == 2 else 0                # bf16 problems: the bf16 copies of the pooled K, V
    out = {}
    # pyramid: read Q, K, V once, write three fp32 pyramids (and the bf16 copies of two)
    out["pool"] = dict(bytes=tokens * (3 * d * s + (3 * d * 4 + copies) * pooled_frac), flops=0.0)
    # selection: per pooled query unit read its pooled query and key rows (fp32), its parent row and write
    # K indices; flops of the scored (unit, block) pairs
    out["select"] = dict(bytes=bh * R * (2 * d * 4 + 2 * K * 4),
                         flops=2.0 * d * bh * (rows[-1] ** 2 + sum(rows[l - 1] * K * B for l in range(1, levels))))
    # forward: read Q, K, V, write O, write LSE, read the pooled K/V once; QK^T and PV products
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        return None


def oracle_baseline(w, x, budget_s=20.0):
    """The oracle chain, after one untimed warm-up run on the first slice, timed on whole (batch, head) slices
    until ~budget_s of CPU work; scaled to one step."""
    import oracle
    sl = lambda nm, h: x[nm].exact.reshape(w.bh, w.n, w.d)[h:h + 1]
    oracle.run(sl("q", 0), sl("k", 0), sl("v", 0), w.block, w.topk, levels=w.levels, dout=sl("dout", 0))
    t_all = 0.0
    done = 0
    for h in range(w.bh):
        t0 = time.perf_counter()
        oracle.run(sl("q", h), sl("k", h), sl("v", h), w.block, w.topk, levels=w.levels, dout=sl("dout", h))
        t_all += time.perf_counter() - t0
        done += 1
        if t_all >= budget_s:
            break
    ms_full = t_all / done * w.bh * 1e3
    return {"value": round(ms_full, 1), "unit": "ms", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} of {w.bh} (batch, head) slices of the {w.name} workload after one untimed warm-up "
                      f"slice, full chain (pool, select, forward, transpose, backward) in fp64; {t_all:.1f} s "
                      f"measured, scaled by {w.bh}/{done} to one step"}


def device_inputs(x):
    import torch
    out = {}
    for nm, t in x.items():
        a = t.store
        out[nm] = (torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if a.dtype == np.uint16
                   else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    return out


class Chain:
    """Buffers and the step of one workload: pool -> select -> forward, and for forward+backward workloads the
    transpose on a second stream beside the forward, then the backward.  The inputs are row-major token grids,
    and the problem says so (grid_w: the dK/dV work-list order hint)."""

    def __init__(self, llsa, w, t, stream, side):
        self.llsa, self.w, self.t, self.stream, self.side = llsa, w, t, stream, side
        self.b = llsa.Buffers(llsa.problem(w.batch, w.heads, w.n, w.d, w.block, w.topk, w.levels,
                                           dtype=llsa.BF16 if w.dtype == "bf16" else llsa.F32,
                                           grid_w=w.grid[1] if w.grid[1] else 0),
                              backward=w.backward)
        self.p = self.b.prob

    def step(self):
        t = self.t
        if self.w.backward:
            self.b.forward_backward(t["q"], t["k"], t["v"], t["dout"], self.stream, self.side)
        else:
            self.b.forward(t["q"], t["k"], t["v"], self.stream)

    def timed(self, steps):
        import torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def kernel_times(self, steps):
        """Second timed region with the library's event timer on: every kernel launch is bracketed by hipEvents
        recorded on the stream it is launched on.  Returns (ms per step of that region, {family: (ms, launches)})."""
        import torch
        self.llsa.timing_enable(True)
        ms = self.timed(steps)
        fam = self.llsa.timing_read()
        self.llsa.timing_enable(False)
        torch.cuda.synchronize()
        return ms, fam


def breakdown(w, p, fam, steps):
    """Per-kernel-family figures, the dominant kernel's roofline and the target fractions of one workload."""
    from hierarchical_sparse_attention_mean_amd import profiling
    alg = algorithmic(w, p.levels, p.enrich_levels)
    kernels = {}
    for nm, (tot, cnt) in fam.items():
        if cnt == 0 or nm not in alg:
            continue
        per_step = tot / steps
        a = alg[nm]
        k = {"ms_per_step": round(per_step, 4), "launches_per_step": cnt // steps,
             "avg_launch_ms": round(tot / cnt, 4),
             "alg_GBps": round(a["bytes"] / (per_step * 1e-3) / 1e9, 1),
             "alg_TFLOPs": round(a["flops"] / (per_step * 1e-3) / 1e12, 2)}
        if nm in ATTN and a["flops"] > 0 and w.dtype == "bf16":
            # algorithmic intensity below the MFMA ridge caps the MFMA fraction at AI x HBM peak / MFMA peak
            k["mfma_frac"] = round(a["flops"] / (per_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)
            k["mfma_ceiling_frac"] = round(min(1.0, a["flops"] / a["bytes"] * HBM_PEAK_GBS / (BF16_PEAK_TFLOPS * 1e3)),
                                           4)
        kernels[nm] = k
    dom = max(kernels, key=lambda nm: kernels[nm]["ms_per_step"])
    dk = kernels[dom]
    sym = kernel_symbol(dom, w, p.enrich_levels)
    a_gbs = alg[dom]["bytes"] / (dk["avg_launch_ms"] * 1e-3) / 1e9 if dk["launches_per_step"] == 1 else dk["alg_GBps"]
    # HBM bytes per launch measured by rocprofv3 FETCH_SIZE + WRITE_SIZE (calibrated by a plain copy), from the
    # committed summary under profiles/; None when absent or when the kernel's sources changed since
    traffic = profiling.read_traffic(sym, w.name)
    roofline = {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": sym, "kernel_avg_ms": dk["avg_launch_ms"],
                "alg_bytes_per_launch": alg[dom]["bytes"], "alg_flops_per_launch": alg[dom]["flops"]}
    if w.dtype == "bf16":
        roofline["mfma_frac"] = round(alg[dom]["flops"] / (dk["avg_launch_ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)
    attn_flops = sum(alg[nm]["flops"] for nm in ATTN if nm in kernels)
    attn_ms = sum(kernels[nm]["ms_per_step"] for nm in ATTN if nm in kernels)
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VALU_PEAK_TFLOPS
    out = {"kernels": kernels, "roofline": roofline,
           "selection_alg_GBps": kernels["select"]["alg_GBps"], "pyramid_alg_GBps": kernels["pool"]["alg_GBps"]}
    out["mfma_util_pct_attention" if w.dtype == "bf16" else "fp32_valu_util_pct_attention"] = \
        round(100 * attn_flops / (attn_ms * 1e-3) / (peak * 1e12), 2)
    return out


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
                    "speedup_fwd": round(fwd_ms / llsa_fwd_ms, 2), "speedup_fwdbwd": round(fb_ms / llsa_step_ms, 2),
                    "pages_context": "28.27x attention inference / 6.09x DiT training at 256x256 pixel tokens, "
                                     "against FlashAttention2 on hardware the pages do not state"}
        except RuntimeError as e:  # backend not available for these shapes / this device
            errors[backend.name] = str(e).splitlines()[0][:200]
    return {"error": errors}


def routing_recall(llsa, p, b, w, stream):
    """Share of the exhaustive single-level Top-K picks (level-1 query unit x all level-1 key blocks) that the
    hierarchical selection keeps, and the exhaustive selection's time."""
    import torch
    n1 = w.n // w.block
    idx1 = torch.empty((w.bh, n1, w.topk), dtype=torch.int32, device="cuda")
    llsa.select_exhaustive(p, b.pq, b.pk, idx1, stream)
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        llsa.select_exhaustive(p, b.pq, b.pk, idx1, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    hit = (b.idx[:, :n1][..., :, None] == idx1[..., None, :]).any(-1).sum(-1).float()
    return {"exhaustive_select_ms": round(e0.elapsed_time(e1) / reps, 4),
            "routing_recall": round(float(hit.mean()) / w.topk, 4),
            "units_fully_recalled": round(float((hit == w.topk).float().mean()), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload: no other workloads, no dense / recall / reordered / "
                         "complement measurements (the profiling runs pass it)")
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
    from hierarchical_sparse_attention_mean_amd import inputs, llsa

    w = inputs.WORKLOADS[args.workload]
    extras = not args.headline_only and w.name == WORKLOAD
    t0 = time.perf_counter()
    x = inputs.make_inputs(w, with_dout=w.backward)
    gen_s = time.perf_counter() - t0
    t = device_inputs(x)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority, like every stream here
    ch = Chain(llsa, w, t, stream, side)
    b, p = ch.b, ch.p

    for _ in range(args.warmup):
        ch.step()
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_step = ch.timed(args.steps)
    print(f"timed {args.steps} steps of {w.name}: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    ms_step_events, fam = ch.kernel_times(args.steps)
    head = breakdown(w, p, fam, args.steps)
    kernels = head["kernels"]

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
            ch.step()
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

    dense = exhaustive = reordered = complement = None
    if extras:
        # routing recall of the hierarchy against exhaustive single-level Top-K (row-major order)
        exhaustive = routing_recall(llsa, p, b, w, stream)
        exhaustive["hierarchical_select_ms"] = kernels["select"]["ms_per_step"]

        # dense attention at the same shapes
        fwd_chain = sum(kernels[nm]["ms_per_step"] for nm in ("pool", "select", "attn_fwd"))
        dense = dense_sdpa(w, t["q"], t["k"], t["v"], t["dout"], 3, fwd_chain, ms_step)
        print(f"dense SDPA: {dense}", file=sys.stderr, flush=True)

        # the chain on 2-D-locally reordered inputs (reorder Q, K, V, dO in; O, dQ, dK, dV back out); the
        # reordered tokens are no longer a row-major grid, so the problem carries no grid hint meanwhile
        H, W = w.grid
        b.prob.grid_w = 0
        qr, kr, vr, dr = (torch.empty_like(t["q"]) for _ in range(4))
        o2, dq2, dk2, dv2 = (torch.empty_like(t["q"]) for _ in range(4))

        def step_reordered():
            for a, z in ((t["q"], qr), (t["k"], kr), (t["v"], vr), (t["dout"], dr)):
                llsa.reorder(p, H, W, True, a, z, stream)
            b.forward_backward(qr, kr, vr, dr, stream, side)
            for a, z in ((b.o, o2), (b.dq, dq2), (b.dk, dk2), (b.dv, dv2)):
                llsa.reorder(p, H, W, False, a, z, stream)

        for _ in range(5):
            step_reordered()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_reordered()
        torch.cuda.synchronize()
        ms_r = (time.perf_counter() - t0) * 1e3 / args.steps
        llsa.timing_enable(True)
        for _ in range(args.steps):
            step_reordered()
        torch.cuda.synchronize()
        fam_r = llsa.timing_read()
        llsa.timing_enable(False)
        rec_r = routing_recall(llsa, p, b, w, stream)
        reordered = {"grid": [H, W], "ms_per_step": round(ms_r, 4), "routing_recall": rec_r["routing_recall"],
                     "units_fully_recalled": rec_r["units_fully_recalled"],
                     "reorder_ms_per_step": round(fam_r["reorder"][0] / args.steps, 4),
                     "kernels_ms_per_step": {nm: round(tc[0] / args.steps, 4) for nm, tc in fam_r.items() if tc[1]}}
        del qr, kr, vr, dr, o2, dq2, dk2, dv2

        # the complement-partition reading of the enrichment: forward alone, then the whole step
        total, ints, a_lists, a_fwd = complement_algorithmic(w, p.levels, p.enrich_levels)
        q, k, v, do = t["q"], t["k"], t["v"], t["dout"]
        b.pyramid(q, k, v, stream)
        llsa.select(p, b.pq, b.pk, b.idx, stream)
        ws_c = torch.empty(max(1, llsa.workspace_bytes(p, llsa.OP_ATTN_FWD_COMPLEMENT)), dtype=torch.uint8,
                           device="cuda")
        o_c, lse_c = torch.empty_like(b.o), torch.empty_like(b.lse)
        for _ in range(2):
            llsa.attn_fwd_complement(p, q, k, v, b.pka, b.pva, b.idx, o_c, lse_c, ws_c, stream)
        torch.cuda.synchronize()
        reps = 5
        llsa.timing_enable(True)
        for _ in range(reps):
            llsa.attn_fwd_complement(p, q, k, v, b.pka, b.pva, b.idx, o_c, lse_c, ws_c, stream)
        torch.cuda.synchronize()
        fam_c = llsa.timing_read()
        llsa.timing_enable(False)
        lists_ms, fwd_ms = fam_c["complement"][0] / reps, fam_c["attn_fwd"][0] / reps
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
        complement = {"entries_per_fine_block": total, "selected_entries_per_fine_block": p.topk * p.enrich_levels,
                      "lists_ms": round(lists_ms, 4), "attn_fwd_ms": round(fwd_ms, 4),
                      "attn_fwd_alg_GBps": round(a_fwd["bytes"] / (fwd_ms * 1e-3) / 1e9, 1),
                      "selected_reading_attn_fwd_ms": kernels["attn_fwd"]["ms_per_step"],
                      "fwdbwd_ms_per_step": round(step_ms, 4), "workspace_bytes_bwd": ws_cb.numel()}
        del ws_c, o_c, lse_c, ws_cb, dq_c, dk_c, dv_c
        torch.cuda.synchronize()

    others = None
    if extras:
        others = {}
        for name in OTHER_WORKLOADS:
            wc = inputs.WORKLOADS[name]
            tc = device_inputs(inputs.make_inputs(wc))
            cc = Chain(llsa, wc, tc, stream, side)
            for _ in range(5):
                cc.step()
            steps = max(10, args.steps)
            ms = cc.timed(steps)
            _, fam_o = cc.kernel_times(steps)
            rec = {"ms_per_step": round(ms, 4), "steps": steps,
                   "step": "pool+select+forward+transpose+backward" if wc.backward else "pool+select+forward",
                   "batch": wc.batch, "heads": wc.heads, "seq_len": wc.n, "dtype": wc.dtype, "topk": wc.topk,
                   "levels": cc.p.levels}
            rec.update(breakdown(wc, cc.p, fam_o, steps))
            others[name] = rec
            print(f"{name}: {ms:.4f} ms/step", file=sys.stderr, flush=True)
            del cc, tc
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and w.backward:
        cpu = oracle_baseline(w, x)

    rec = {
        "metric": METRIC, "value": round(ms_step, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.n, "head_dim": w.d,
                   "block": w.block, "topk": w.topk, "levels": p.levels, "enrich_levels": p.enrich_levels,
                   "grid": list(w.grid), "inputs": "2-D Gaussian random field (l=16 px) projected to 64 dims + 0.1 noise"
                   if w.kind == "field" else "i.i.d. N(0, 1)", "parallelism": "none (one GPU)"},
        "value_protocol": "K back-to-back steps on inputs resident in HBM, as a training loop runs them; "
                          "cold_steps is the distribution with the L2s and the MALL flushed before every step",
        "mfma_util_pct_attention": head.get("mfma_util_pct_attention"),
        "selection_alg_GBps": head["selection_alg_GBps"],
        "pyramid_alg_GBps": head["pyramid_alg_GBps"],
        "ms_per_step_with_kernel_events": round(ms_step_events, 4),
        "kernels": kernels,
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "dense_sdpa": dense,
        "exhaustive_selection": exhaustive,
        "reordered_chain": reordered,
        "complement": complement,
        "warm_steps": warm,
        "cold_steps": cold,
        "other_workloads": others,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
