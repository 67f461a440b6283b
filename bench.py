"""Benchmark: MatMul-free LM block forward on one MI355X.

Default (the largest single-GPU workload, `2.7B-longctx`): a step is one prefill of the
32-layer 2.7B-shaped stack over 2 sequences x 32768 tokens -- in every layer RMSNorm + int8
quantization, the i|f|g ternary BitLinear, the chunked MLGRU scan with the RMSNorm-swish
gate, o_proj + residual, the GLU with SiLU(gate)*up and down + residual -- on synthetic
bf16 activations already resident in HBM and ternary weights from N(0, 0.02^2) latents.

Prints one JSON line.  `roofline` describes the dominant kernel (the gate|up int8-MFMA GEMM)
with its launch durations from HIP events recorded on the launch stream during the timed
steps; `cpu_baseline` is the CPU oracle timed on a bounded causal sample of the same
workload.  `extra_workloads` carries the other shapes measured the same way: the 2.7B block
(16 x 2048 tokens), the same block with HGRN's forget-gate lower bound (`+hgrn`), the 370M
block (8 x 2048 tokens) and the 24-layer 1.3B decode stack at
batch 1 and 64 (bound by HBM bandwidth; roofline of the decode BitLinear launches), then a
block's backward (block_backward: forward recomputed, every gradient; straight-through
BitLinear backwards on bf16 MFMA) at the 370M and 2.7B block sizes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block tokens/s; % peak HBM GB/s (decode), % int8 MFMA util (prefill)"
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, tera-ops/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
CSRC = os.path.join(ROOT, "ternary_weight_matmul_bitlinear_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
DEFAULT_EXTRAS = "2.7B-block,2.7B-block+hgrn,370M-block,1.3B-decode@1,1.3B-decode@64"
DEFAULT_BACKWARD = "370M-block,2.7B-block"
DATA = "synthetic (seeded N(0,1) activations / uniform token ids, ternary weights from N(0,0.02^2) latents)"


# ------------------------------------------------------------------------ helpers

def _src_hash(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(kernel_id: str, workload: str, srcs: tuple, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch (or per step) of a kernel from its committed counter summary
    (profiles/<kernel_id>_<workload>_traffic.json), or None when the summary is missing or
    the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel_id}_{workload}_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != _src_hash(*srcs):
        return None
    return t.get(key)


def cpu_info(orc) -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"cores": orc.max_threads(), "nproc": nproc, "cpu_model": model}


def spin_up(fn, seconds: float) -> None:
    """Untimed steps for `seconds` of wall time: the GPU reaches its steady clock only under
    sustained load, which a handful of warm-up steps of a few hundred microseconds each does
    not provide (the 370M block measured 0.37 ms/step after 5 steps, 0.33 after ~100)."""
    if seconds <= 0:
        return
    import torch
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-6)
    batch = max(1, min(50, int(0.02 / per)))  # ~20 ms of queued work between host checks
    t_end = t0 + seconds
    while time.perf_counter() < t_end:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()


def log(msg: str) -> None:
    print(f"# {msg}", file=sys.stderr, flush=True)


def rel_err(got, ref) -> float:
    """max |got - ref| / (|ref| + rms of ref's row)."""
    import numpy as np
    got = np.asarray(got, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(got.shape)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + rms)))


def timed_events(fams, fn, steps: int):
    """Run fn(i) for `steps` steps with the library's HIP events around every launch of the
    given kernel families; returns (wall ms per step, {family: (launches, total ms)})."""
    import torch

    from ternary_weight_matmul_bitlinear_amd import api
    api.timing_reset()
    api.timing_families(fams)
    api.timing_enable(True)
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    api.timing_enable(False)
    return wall, {f: api.timing_query(f) for f in fams}


def gemm_families(M: int, D: int, F: int, ab: int, per_step_layers: int = 1):
    """Algorithmic work per step of each kernel family of a prefill block: int8 ops of the
    GEMMs; bytes of the HBM-bound kernels (the scan reads the i|f|g pre-activations once
    and writes the int8 o_proj input with its scale and code sum; the row quantizers read x,
    y1 (D wide) and the GLU hidden (F wide) and write int8 codes + 8 bytes per row)."""
    L = per_step_layers
    return {"gemm_ifg": ("mfma", L * 2.0 * M * D * 3 * D), "gemm_o": ("mfma", L * 2.0 * M * D * D),
            "gemm_gateup": ("mfma", L * 2.0 * M * D * 2 * F),
            "gemm_down": ("mfma", L * 2.0 * M * F * D),
            "scan": ("hbm", L * M * (3 * D * ab + D + 8.0)),
            "quant": ("hbm", L * M * (2 * D * (ab + 1) + F * (ab + 1) + 24.0))}


def family_breakdown(fn, nb: int, work: dict) -> dict:
    """A separate pass with events around every launch: per-family launch counts, durations
    and fractions of their roofline."""
    _, q = timed_events(["quant", "gemm_ifg", "gemm_o", "gemm_gateup", "gemm_down", "scan"], fn, nb)
    fams = {}
    for fam, (n, ms) in q.items():
        if not n:
            continue
        d = {"launches_per_step": n / nb, "ms_per_launch": ms / n, "ms_per_step": ms / nb}
        if fam in work:
            bound, amount = work[fam]
            sec = ms / nb * 1e-3
            if bound == "mfma":
                d.update(tops=amount / sec / 1e12, mfma_frac=amount / sec / 1e12 / PEAK_INT8_TOPS)
            else:
                d.update(gbs=amount / sec / 1e9, hbm_frac=amount / sec / 1e9 / PEAK_HBM_GBS)
        fams[fam] = d
    return fams


def gateup_roofline(w, M: int, n: int, ms: float, note: str) -> dict:
    ops = 2.0 * M * w.D * (2 * w.F)
    achieved = ops / (ms / n * 1e-3) / 1e12 if n else None
    return {"kernel": f"gemm_gateup (int8 MFMA, SiLU(gate)*up epilogue){note}", "bound": "mfma",
            "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_INT8_TOPS if achieved else None,
            "traffic": traffic("gemm_gateup", w.name, ("gemm_prefill.hip",)),
            "algorithmic_ops_per_launch": ops, "launches_timed": n,
            "us_per_launch": ms / n * 1e3 if n else None}


# ------------------------------------------------------------------ prefill block

HGRN_LAYERS, HGRN_LAYER = 32, 16


def bench_block(w, args, orc, hgrn: bool = False) -> dict:
    """One block over B x T tokens (the 370M and 2.7B blocks).  hgrn: with HGRN's forget-gate
    lower bound of layer 16 of a 32-layer stack (bounds from per-layer logits ~ N(0, 1))."""
    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api, synth

    dt = torch.bfloat16 if w.bf16 else torch.float32
    lat = synth.layer_latents(w, 0)
    fb = np.full(w.D, w.f_bias, np.float32) if w.f_bias else None
    lb = None
    if hgrn:
        logits = synth.gaussian(w.seed + 201, (HGRN_LAYERS, w.D))
        lb = np.ascontiguousarray(api.hgrn_lower_bounds(logits)[HGRN_LAYER])
    blk = api.Block.from_latents(lat, "cuda", f_bias=fb, f_lower=lb)
    name = w.name + ("+hgrn" if hgrn else "")
    x_np = synth.activations(w)
    x = torch.from_numpy(x_np).to("cuda").to(dt)
    y = torch.empty_like(x)
    h = torch.zeros((w.B, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(api.block_workspace_bytes(blk, w.B, w.T), dtype=torch.uint8, device="cuda")
    M = w.M
    log(f"workload {name}: B={w.B} T={w.T} D={w.D} F={w.F}")

    def step(i):
        api.block_forward(blk, x, h_state=h, y=y, ws=ws)

    spin_up(lambda: step(0), args.spin_up)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: HIP events only around the dominant kernel (gate|up GEMM), on the stream
    # it is launched on, so the measured stream stays close to an untimed one
    ms_step, q = timed_events(["gemm_gateup"], step, args.steps)
    n, ms = q["gemm_gateup"]
    log(f"{name}: timed {args.steps} steps: {ms_step:.3f} ms/step")
    fams = family_breakdown(step, min(args.steps, 10), gemm_families(M, w.D, w.F, 2 if w.bf16 else 4))
    cfg = {"workload": name, "B": w.B, "T": w.T, "D": w.D, "F": w.F, "layers": 1,
           "activations": "bf16" if w.bf16 else "fp32", "state": "fp32"}
    if hgrn:
        cfg["f_lower"] = (f"HGRN bounds of layer {HGRN_LAYER} of {HGRN_LAYERS} "
                          f"(per-layer logits N(0, 1), mean bound {float(lb.mean()):.3f})")
    out = {"workload": name, "value": M / (ms_step * 1e-3), "unit": "tokens/s",
           "ms_per_step": ms_step, "steps": args.steps, "config": cfg,
           "roofline": gateup_roofline(w, M, n, ms, ""), "kernels": fams}
    if orc is not None:
        # the timed steps chained the state; the sample is checked on a fresh prefill
        h.zero_()
        step(0)
        torch.cuda.synchronize()
        ct = args.cpu_tokens or (128 if w.D <= 1024 else 16)
        B0, T0 = min(w.B, args.cpu_seqs), min(ct, w.T)
        W = {k: orc.ternarize(lat[k]) for k in ("i", "f", "g", "o", "gate", "up", "down")}
        xs = np.ascontiguousarray(x_np[:B0, :T0])
        orc.block(np.ascontiguousarray(xs[:1, :2]), W, f_bias=fb, resid_bf16=w.bf16, f_lower=lb)  # warm-up
        t = time.perf_counter()
        r = orc.block(xs, W, f_bias=fb, resid_bf16=w.bf16, f_lower=lb)
        cdt = time.perf_counter() - t
        got = y.float().cpu().numpy()[:B0, :T0]
        out["cpu_baseline"] = {
            "value": B0 * T0 / cdt, "unit": "tokens/s", **cpu_info(orc), "kind": "oracle",
            "sample": f"causal prefix: first {T0} tokens of {B0} of the {w.B} sequences "
                      f"({B0 * T0} tokens), one block, {cdt:.1f} s",
            "sample_max_rel_err_vs_gpu": rel_err(got, r["y"])}
    return out


# ------------------------------------------------------------- long-context stack

def build_stack(w, with_oracle: bool, orc):
    import numpy as np

    from ternary_weight_matmul_bitlinear_amd import api, synth

    fb = np.full(w.D, w.f_bias, np.float32) if w.f_bias else None
    t0 = time.perf_counter()
    blocks, Ws = [], []
    for l in range(w.layers):
        lat = synth.layer_latents(w, l)
        blocks.append(api.Block.from_latents(lat, "cuda", f_bias=fb))
        if with_oracle:
            Ws.append({k: orc.ternarize(lat[k]) for k in ("i", "f", "g", "o", "gate", "up", "down")})
        del lat
        if (l + 1) % 8 == 0:
            log(f"{w.name}: {l + 1} of {w.layers} layers built")
    emb = head = None
    qe = qh = None
    if w.vocab:
        E, H = synth.embedding_latents(w)
        emb = api.TernaryLinear.from_latent(E)
        head = api.TernaryLinear.from_latent(H)
        if with_oracle:
            qe, qh = orc.ternarize(E), orc.ternarize(H)
        del E, H
    log(f"{w.name}: {w.layers} layers built in {time.perf_counter() - t0:.1f} s")
    return api.Stack(blocks, emb, head), Ws, qe, qh, fb


def bench_longctx(w, args, orc) -> dict:
    """The 32-layer 2.7B stack prefill over 2 x 32768 tokens."""
    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api, synth

    stack, Ws, _, _, fb = build_stack(w, orc is not None, orc)
    B, T, D, F, L = w.B, w.T, w.D, w.F, w.layers
    x_np = synth.activations(w)
    x = torch.from_numpy(x_np).to("cuda").to(torch.bfloat16)
    y = torch.empty_like(x)
    ws = torch.empty(stack.workspace_bytes(B, T), dtype=torch.uint8, device="cuda")

    def step(i):
        api.stack_forward(stack, B, T, x=x, ws=ws, y=y)

    spin_up(lambda: step(0), args.spin_up)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step, q = timed_events(["gemm_gateup"], step, args.steps)
    n, ms = q["gemm_gateup"]
    log(f"{w.name}: timed {args.steps} steps: {ms_step:.3f} ms/step")
    M = B * T
    fams = family_breakdown(step, min(args.steps, 3), gemm_families(M, D, F, 2, L))
    out = {"workload": w.name, "value": M / (ms_step * 1e-3), "unit": "tokens/s",
           "ms_per_step": ms_step, "steps": args.steps,
           "layer_tokens_per_s": M * L / (ms_step * 1e-3),
           "config": {"workload": w.name, "B": B, "T": T, "D": D, "F": F, "layers": L,
                      "forget_bias": w.f_bias, "activations": "bf16", "state": "fp32"},
           "roofline": gateup_roofline(w, M, n, ms, f", one launch per layer"), "kernels": fams}
    if orc is not None:
        P = min(args.cpu_tokens_stack, T)
        xo = np.ascontiguousarray(x_np[:, :P])
        orc.block(np.ascontiguousarray(xo[:1, :1]), Ws[0], f_bias=fb, resid_bf16=True)  # warm-up
        t = time.perf_counter()
        for l in range(L):
            xo = orc.block(xo, Ws[l], f_bias=fb, resid_bf16=True)["y"].astype(np.float32)
        cdt = time.perf_counter() - t
        got = y.float().cpu().numpy()[:, :P]
        out["cpu_baseline"] = {
            "value": B * P / cdt, "unit": "tokens/s", **cpu_info(orc), "kind": "oracle",
            "sample": f"causal prefix: first {P} tokens of each of the {B} sequences through all "
                      f"{L} layers ({B * P} tokens), {cdt:.1f} s",
            "sample_max_rel_err_vs_gpu": rel_err(got, xo),
            "sample_err_note": "independent 32-layer runs: near-tie int8 flips compound layer by layer"}
    return out


# ------------------------------------------------------------------- decode stack

def decode_bytes(B: int, D: int, F: int, V: int, L: int):
    """Algorithmic bytes of a decode step's BitLinear launches (N*K/4 packed weights + rows
    in + rows out, residual where added) and of the whole step (plus embedding rows and the
    fp32 state read and written per layer).  Up to 4 rows the weight-streaming kernel
    quantizes the bf16 rows itself; above, the k-split kernel reads int8 rows written by the
    row quantizer."""
    def bl(N, K, in_b, out_b, resid=0):
        return N * K // 4 + B * K * in_b + B * N * out_b + B * N * resid
    xin = 2 if B <= 4 else 1
    per_layer = (bl(3 * D, D, xin, 2) + bl(D, D, 1, 2, 2) + bl(2 * F, D, xin, 0) + B * F * 2
                 + bl(D, F, xin, 2, 2))
    gemv = L * per_layer + bl(V, D, xin, 4)
    return gemv, gemv + B * D // 4 + B * D * 2 + L * B * D * 4 * 2


def bench_decode(w, args, batches, orc) -> list:
    """The 24-layer 1.3B stack + ternary embedding and head, one token per sequence per
    step, state carried; steps replayed from a captured HIP graph (a step is ~100-200
    small launches whose host-side launch cost would otherwise dominate)."""
    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api, synth

    stack, Ws, qe, qh, _ = build_stack(w, orc is not None, orc)
    D, F, L, V = w.D, w.F, w.layers, w.vocab
    outs = []
    fams = ["gemv", "gemm_ifg", "gemm_o", "gemm_gateup", "gemm_down", "gemm"]
    for B in batches:
        steps = args.steps
        hs = torch.zeros((L, B, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(stack.workspace_bytes(B, 1), dtype=torch.uint8, device="cuda")
        ids_all = torch.from_numpy(synth.token_ids(w, args.warmup + steps, B)).to("cuda")
        logits = torch.empty((B, V), dtype=torch.float32, device="cuda")

        def eager(i):
            api.stack_forward(stack, B, 1, ids=ids_all[i], h_state=hs, want_y=False,
                              want_logits=True, ws=ws, logits=logits)

        for i in range(2):
            eager(i)
        torch.cuda.synchronize()
        # per-launch durations of the decode BitLinear launches: an eager pass with events
        eager_ms, q = timed_events(fams, lambda i: eager(args.warmup + i), steps)
        n = sum(v[0] for v in q.values())
        ms = sum(v[1] for v in q.values())
        if args.no_graph:   # profiler runs: eager steps only
            ms_step = eager_ms
        else:
            # timed loop: graph replay of one captured step
            ids_static = ids_all[0].clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                api.stack_forward(stack, B, 1, ids=ids_static, h_state=hs, want_y=False,
                                  want_logits=True, ws=ws, logits=logits)
            spin_up(lambda: g.replay(), args.spin_up)
            for i in range(args.warmup):
                ids_static.copy_(ids_all[i])
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                ids_static.copy_(ids_all[args.warmup + i])
                g.replay()
            torch.cuda.synchronize()
            ms_step = (time.perf_counter() - t0) * 1e3 / steps
            del g
        gemv_bytes, step_bytes = decode_bytes(B, D, F, V, L)
        achieved = gemv_bytes * steps / (ms * 1e-3) / 1e9 if n else None
        name = f"{w.name}@{B}"
        one = None
        if B == 1 and args.one_launch:
            # the whole step in one cooperative launch (stack_decode_step): its kernel
            # duration from HIP events on the launch stream is the step's BitLinear time
            ds = api.DecodeStep(stack)
            h1 = torch.zeros((L, 1, D), dtype=torch.float32, device="cuda")
            lg1 = torch.empty((1, V), dtype=torch.float32, device="cuda")
            run1 = lambda i: ds.step(ids_all[i % (args.warmup + steps)], h1, logits=lg1)
            spin_up(lambda: run1(0), args.spin_up)
            for i in range(args.warmup):
                run1(i)
            torch.cuda.synchronize()
            wall1, q1 = timed_events(["gemv"], lambda i: run1(args.warmup + i), steps)
            ds.status()
            n1, ms1 = q1["gemv"]
            k1 = ms1 / n1 if n1 else None
            one = {"kernel": "one cooperative launch per step (embedding, 24 blocks, head)",
                   "ms_per_step": wall1, "kernel_ms": k1,
                   "achieved_gbs": gemv_bytes / (k1 * 1e-3) / 1e9 if k1 else None}
            one["hbm_frac"] = one["achieved_gbs"] / PEAK_HBM_GBS if k1 else None
            log(f"{name}: one-launch step {wall1:.4f} ms (kernel {k1:.4f} ms)")
            del ds, h1, lg1
        log(f"{name}: graph-replayed step {ms_step:.4f} ms, eager {eager_ms:.4f} ms")
        res = {"workload": name, "value": B / (ms_step * 1e-3), "unit": "tokens/s",
               "ms_per_step": ms_step, "steps": steps,
               "config": {"workload": w.name, "B": B, "T": 1, "D": D, "F": F, "layers": L,
                          "vocab": V, "activations": "bf16", "state": "fp32"},
               "roofline": {"kernel": "decode BitLinear (dot4 weight streaming up to 4 rows, "
                                      "k-split MFMA above), all launches of a step",
                            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS if achieved else None,
                            "traffic": traffic("decode_bitlinear", name,
                                               ("gemv_decode.hip", "gemm_mid.hip"),
                                               "hbm_bytes_per_step"),
                            "algorithmic_bytes_per_step": gemv_bytes,
                            "launches_per_step": n / steps},
               "step_hbm_fraction": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "step_algorithmic_bytes": step_bytes, "eager_ms_per_step": eager_ms}
        if one is not None:
            # the one-launch step is the batch-1 path: it becomes the line's value and roofline,
            # the graph-replayed launch-per-stage step is kept beside it
            res["launch_per_stage"] = {"ms_per_step": ms_step, "roofline": res["roofline"]}
            res["value"] = B / (one["ms_per_step"] * 1e-3)
            res["ms_per_step"] = one["ms_per_step"]
            res["roofline"] = {"kernel": one["kernel"], "bound": "hbm", "achieved": one["achieved_gbs"],
                               "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": one["hbm_frac"],
                               "traffic": None, "algorithmic_bytes_per_step": gemv_bytes,
                               "kernel_ms": one["kernel_ms"]}
            res["step_hbm_fraction"] = step_bytes / (one["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS
        if orc is not None:
            Bs = min(B, args.cpu_seqs_decode)
            ids_np = synth.token_ids(w, 1, B)[0][:Bs]
            t = time.perf_counter()
            xo = orc.embedding(qe[0], qe[1], ids_np, resid_bf16=True).reshape(Bs, 1, D)
            for l in range(L):
                xo = orc.block(xo, Ws[l], resid_bf16=True)["y"].astype(np.float32)
            orc.bitlinear(xo.reshape(Bs, D), *qh)
            cdt = time.perf_counter() - t
            res["cpu_baseline"] = {
                "value": Bs / cdt, "unit": "tokens/s", **cpu_info(orc), "kind": "oracle",
                "sample": f"one decode step (embedding, {L} layers, head) of {Bs} of the {B} "
                          f"sequences, {cdt:.1f} s"}
        outs.append(res)
        del hs, ws, logits
        torch.cuda.empty_cache()
    return outs


def decode_kernel_sweep(B: int, D: int, F: int, V: int) -> list:
    """One BitLinear launch per (N, K) at B token rows, cycling through enough copies of random
    packed weights (>= 512 MB) that none is in the 256 MB MALL when it is read again; durations
    from the library's events.  Shapes: the 1.3B projections, the head, and one large matrix
    whose streaming is not dominated by the per-launch latency."""
    import torch

    from ternary_weight_matmul_bitlinear_amd import api

    out = []
    fams = ["gemv", "gemm_ifg", "gemm_o", "gemm_gateup", "gemm_down", "gemm"]
    for N, K in ((3 * D, D), (2 * F, D), (D, F), (V, D), (65536, 8192)):
        wbytes = N * K // 4
        copies = max(2, -(-(512 << 20) // wbytes))
        gen = torch.Generator(device="cuda").manual_seed(N * 131 + K)
        ws = []
        for _ in range(copies):
            r0 = torch.randint(-2**31, 2**31 - 1, (N, K // 16), dtype=torch.int32, device="cuda", generator=gen)
            r1 = torch.randint(-2**31, 2**31 - 1, (N, K // 16), dtype=torch.int32, device="cuda", generator=gen)
            lo = r0 & 0x55555555                    # code bit 0
            hi = (r1 & 0x55555555) & ~lo            # code bit 1 where bit 0 is clear: codes 0, 1, 2
            ws.append(api.TernaryLinear(lo | (hi << 1), 0.016, K, N))
        x = torch.randn((B, K), device="cuda").to(torch.bfloat16)
        for i in range(copies):
            api.bitlinear_forward(ws[i], x)
        torch.cuda.synchronize()
        reps = max(copies, 40)
        _, q = timed_events(fams, lambda i: api.bitlinear_forward(ws[i % copies], x), reps)
        n = sum(v[0] for v in q.values())
        ms = sum(v[1] for v in q.values())
        bytes_ = wbytes + B * K * 2 + B * N * 2
        gbs = bytes_ * n / (ms * 1e-3) / 1e9
        res = {"N": N, "K": K, "rows": B, "weight_copies": copies,
               "us_per_launch": ms / n * 1e3, "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
        del ws
        torch.cuda.empty_cache()
        if B <= 16 and K <= 10240:
            # the same shape with base-3 packed weights (five per byte): random valid bytes
            # b = ceil(256 v / 243), v uniform in [0, 243)
            rb = api.trit_row_bytes(K)
            tbytes = N * rb
            tcopies = max(2, -(-(512 << 20) // tbytes))
            wt = []
            for _ in range(tcopies):
                v = torch.randint(0, 243, (N, rb), dtype=torch.int32, device="cuda", generator=gen)
                b = ((v * 256 + 242) // 243).to(torch.uint8)
                wt.append(api.TernaryLinearTrits(b, 0.016, K, N))
            for i in range(tcopies):
                api.bitlinear_forward_trits(wt[i], x)
            torch.cuda.synchronize()
            reps = max(tcopies, 40)
            _, q = timed_events(["gemv"], lambda i: api.bitlinear_forward_trits(wt[i % tcopies], x), reps)
            n3, ms3 = q["gemv"]
            tb = tbytes + B * K * 2 + B * N * 2
            res["trits"] = {"weight_bytes": tbytes, "weight_copies": tcopies,
                            "us_per_launch": ms3 / n3 * 1e3,
                            "gbs": tb * n3 / (ms3 * 1e-3) / 1e9,
                            "hbm_frac": tb * n3 / (ms3 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            "weights_per_s_vs_2bit": (ms / n) / (ms3 / n3)}
            del wt
            torch.cuda.empty_cache()
        out.append(res)
    return out


# ---------------------------------------------------------------------------- main

# ------------------------------------------------------------------ backward

def bench_backward(w, args, orc) -> dict:
    """One block's backward at the block workload's size (block_backward): the forward
    recomputed on the prefill kernels, then every gradient -- the seven straight-through
    BitLinear backwards (g = s_w dy T and dW = (dy a)^T q_x on bf16 MFMA, dx with the
    RMSNorm backward, dgamma, db), the GLU product's and the MLGRU + output gate's
    backwards.  bf16 activations and dy, fp32 gradients, layer 0's weights."""
    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api, synth

    M, D, F = w.B * w.T, w.D, w.F
    lat = synth.layer_latents(w, 0)
    fb = np.full(D, w.f_bias, np.float32) if w.f_bias else None
    blk = api.Block.from_latents(lat, "cuda", f_bias=fb)
    x = torch.from_numpy(synth.activations(w)).to("cuda").to(torch.bfloat16)
    dy_np = synth.round_to_bf16(synth.gaussian(w.seed + 101, (w.B, w.T, D)))
    dy = torch.from_numpy(dy_np).to("cuda").to(torch.bfloat16)

    def step(_i):
        api.block_backward(blk, x, dy)

    spin_up(lambda: step(0), args.spin_up)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    steps = args.steps
    fams = ["bwd_g", "bwd_dw", "bwd_scan", "quant", "gemm_ifg", "gemm_o", "gemm", "scan"]
    wall, q = timed_events(fams, step, steps)
    ops = 2.0 * M * D * (4 * D + 3 * F)          # the seven contractions of g (and of dW) per step
    kern = {}
    for fam, (n, ms) in q.items():
        if not n:
            continue
        d = {"launches_per_step": n / steps, "ms_per_step": ms / steps}
        sec = ms / steps * 1e-3
        if fam in ("bwd_g", "bwd_dw"):
            d.update(bound="mfma", algorithmic_flops_per_step=ops, tflops=ops / sec / 1e12,
                     mfma_frac=ops / sec / 1e12 / PEAK_BF16_TFLOPS)
        elif fam == "bwd_scan":
            nb = M * D * (4 * 2 + 12.0)   # read i|f|g (bf16) and do (fp32 counted as 2 x bf16), write d_ifg
            d.update(bound="hbm", algorithmic_bytes_per_step=nb, gbs=nb / sec / 1e9,
                     hbm_frac=nb / sec / 1e9 / PEAK_HBM_GBS)
        kern[fam] = d
    n_g, ms_g = q["bwd_g"]
    tf = ops / (ms_g / steps * 1e-3) / 1e12 if n_g else None
    res = {"workload": f"{w.name} backward", "value": M / (wall * 1e-3), "unit": "tokens/s",
           "ms_per_step": wall, "steps": steps,
           "config": {"workload": f"{w.name} backward", "B": w.B, "T": w.T, "D": D, "F": F,
                      "step": "block_backward (forward recomputed, every gradient)",
                      "inputs": "bf16", "gradients": "fp32"},
           "roofline": {"kernel": "bwd_g: the seven g = s_w dy T contractions of a step (bf16 MFMA)",
                        "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / PEAK_BF16_TFLOPS if tf else None,
                        "traffic": traffic("bwd_g", f"{w.name}-backward", ("backward.hip",),
                                           key="hbm_bytes_per_step"),
                        "traffic_per": "step (the four g launches)",
                        "algorithmic_flops_per_step": ops, "launches_per_step": n_g / steps},
           "kernels": kern}
    if orc is not None:
        # oracle on a bounded sample: the block backward of a causal prefix of one sequence
        P = 32 if D <= 1024 else 8
        W = {}
        for k in ("i", "f", "g", "o", "gate", "up", "down"):
            W[k] = orc.ternarize(lat[k])
        xs = synth.activations(w)[:1, :P]
        t = time.perf_counter()
        orc.block_backward(xs, W, dy_np[:1, :P].astype(np.float64), f_bias=fb, resid_bf16=True)
        dt = time.perf_counter() - t
        res["cpu_baseline"] = {"value": P / dt, "unit": "tokens/s", **cpu_info(orc), "kind": "oracle",
                               "sample": f"block backward of the first {P} tokens of one sequence "
                                         f"({dt:.2f} s), fp64"}
    log(f"{w.name} backward: {wall:.3f} ms/step; bwd_g {tf / PEAK_BF16_TFLOPS if tf else 0:.3f} of bf16 peak")
    del x, dy
    return res


def library_gemm_reference() -> list:
    """The vendor library's own GEMMs (hipBLASLt through torch: int8 x int8 -> int32 with
    torch._int_mm, bf16 x bf16 -> bf16 with torch.matmul) next to the ternary int8 GEMM of
    this library (bitlinear_forward, GEMM launch timed with the library's events) at the
    shapes of the prefill and backward contractions, each as a fraction of its dense peak.
    Context for the roofline fractions: what a general-purpose GEMM reaches on this part."""
    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        spin_up(fn, 0.5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = []
    shapes = [("2.7B gate|up", 32768, 2560, 13824), ("square-ish", 16384, 8192, 8192),
              ("370M gate|up", 16384, 1024, 5632), ("2.7B down", 32768, 6912, 2560)]
    for name, M, K, N in shapes:
        ops = 2.0 * M * K * N
        r = {"shape": name, "M": M, "K": K, "N": N}
        g = torch.Generator(device="cuda").manual_seed(7)
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        b = torch.randint(-1, 2, (N, K), dtype=torch.int8, device="cuda", generator=g)
        bt = b.t()
        ms = timed(lambda: torch._int_mm(a, bt))
        r["hipblaslt_int8_ms"] = ms
        r["hipblaslt_int8_frac"] = ops / (ms * 1e-3) / (PEAK_INT8_TOPS * 1e12)
        del a, b, bt
        q = np.random.default_rng(7).integers(-1, 2, (N, K)).astype(np.int8)
        lin = api.TernaryLinear.from_ternary(q, 0.02, "cuda")
        x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        api.timing_reset()
        api.timing_families(["gemm"])
        api.timing_enable(True)
        timed(lambda: api.bitlinear_forward(lin, x))
        api.timing_enable(False)
        n, t = api.timing_query("gemm")
        r["ternary_int8_ms"] = t / n
        r["ternary_int8_frac"] = ops / (t / n * 1e-3) / (PEAK_INT8_TOPS * 1e12)
        del x, lin
        A = torch.randn(M, K, device="cuda", generator=g, dtype=torch.bfloat16)
        B = torch.randn(N, K, device="cuda", generator=g, dtype=torch.bfloat16)
        Bt = B.t()
        ms = timed(lambda: torch.matmul(A, Bt))
        r["hipblaslt_bf16_ms"] = ms
        r["hipblaslt_bf16_frac"] = ops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
        del A, B, Bt
        torch.cuda.empty_cache()
        log(f"library GEMMs {name}: ternary int8 {r['ternary_int8_frac']:.3f}, hipBLASLt int8 "
            f"{r['hipblaslt_int8_frac']:.3f}, hipBLASLt bf16 {r['hipblaslt_bf16_frac']:.3f}")
        out.append(r)
    return out


def run_workload(spec: str, args, orc):
    from ternary_weight_matmul_bitlinear_amd import synth
    name, _, b = spec.partition("@")
    name, hgrn = (name[:-len("+hgrn")], True) if name.endswith("+hgrn") else (name, False)
    w = synth.WORKLOADS[name]
    if hgrn:
        return [bench_block(w, args, orc, hgrn=True)]
    if w.vocab:
        batches = [int(b)] if b else ([args.batch] if args.batch else [1, 64])
        return bench_decode(w, args, batches, orc)
    if w.layers > 1:
        return [bench_longctx(w, args, orc)]
    return [bench_block(w, args, orc)]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spin-up", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="2.7B-longctx",
                    help="headline workload (a name of synth.WORKLOADS, decode stacks as "
                         "NAME@BATCH, a block with HGRN bounds as NAME+hgrn)")
    ap.add_argument("--extras", default=DEFAULT_EXTRAS,
                    help="comma-separated workloads measured after the headline ('' for none)")
    ap.add_argument("--no-extras", dest="extras", action="store_const", const="")
    ap.add_argument("--backward", default=DEFAULT_BACKWARD,
                    help="block workloads whose whole backward (block_backward) is measured "
                         "after the extras ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="block workloads: tokens per sequence of the causal CPU sample "
                         "(default: 128 at hidden size <= 1024, else 16)")
    ap.add_argument("--cpu-seqs", type=int, default=16,
                    help="block workloads: sequences of the causal CPU sample")
    ap.add_argument("--cpu-tokens-stack", type=int, default=8,
                    help="long-context stack: tokens per sequence of the causal CPU sample")
    ap.add_argument("--cpu-seqs-decode", type=int, default=16,
                    help="decode stack: sequences of the one-step CPU sample")
    ap.add_argument("--batch", type=int, default=None,
                    help="decode stack without @BATCH: sequences per step")
    ap.add_argument("--regime", choices=("auto", "decode", "prefill", "tiles"), default="auto",
                    help="BitLinear kernel choice (auto: by token count; decode: weight "
                         "streaming; prefill: MFMA kernels; tiles: 128-row MFMA tiles only)")
    ap.add_argument("--kernel-sweep", action="store_true",
                    help="decode stacks: also time single BitLinear launches on rotated weights")
    ap.add_argument("--one-launch", action="store_true",
                    help="decode stack at batch 1: also time the one-launch step (stack_decode_step)")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode stacks: time eager steps only (no HIP graph replay)")
    ap.add_argument("--library-gemm", dest="library_gemm", action="store_true", default=None,
                    help="time the vendor library's int8 and bf16 GEMMs (hipBLASLt) next to the "
                         "ternary GEMM at the prefill and backward shapes (default: with the "
                         "extra workloads, so single-workload profiling runs leave it out)")
    ap.add_argument("--no-library-gemm", dest="library_gemm", action="store_false")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"asked for --gpus {args.gpus} / WORLD_SIZE={world}", file=sys.stderr)
        return 2

    import torch

    from ternary_weight_matmul_bitlinear_amd import api

    torch.cuda.set_device(0)
    api.set_regime({"auto": 0, "decode": 1, "prefill": 2, "tiles": 3}[args.regime])
    orc = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        orc = O.get()

    res = run_workload(args.workload, args, orc)
    head, rest = res[0], res[1:]
    extras = list(rest)
    for spec in [s for s in args.extras.split(",") if s and s != args.workload]:
        extras.extend(run_workload(spec, args, orc))
        torch.cuda.empty_cache()
    from ternary_weight_matmul_bitlinear_amd import synth as _synth
    for spec in [s for s in args.backward.split(",") if s]:
        extras.append(bench_backward(_synth.WORKLOADS[spec], args, orc))
        torch.cuda.empty_cache()
    if args.kernel_sweep:
        from ternary_weight_matmul_bitlinear_amd import synth
        w3 = synth.WORKLOADS["1.3B-decode"]
        head["decode_bitlinear_kernels"] = {
            f"rows={b}": decode_kernel_sweep(b, w3.D, w3.F, w3.vocab) for b in (1, 64)}
    if args.library_gemm is None:
        args.library_gemm = bool(args.extras)
    if args.library_gemm:
        try:
            head["library_gemm_reference"] = library_gemm_reference()
        except Exception as e:  # context only: never lose the measured line over it
            head["library_gemm_reference"] = {"error": f"{type(e).__name__}: {e}"[:300]}
        torch.cuda.empty_cache()
    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    line = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": DATA, "config": head["config"], "roofline": head["roofline"],
            "cpu_baseline": head.get("cpu_baseline")}
    for k, v in head.items():
        if k not in line and k not in ("workload", "unit", "steps"):
            line[k] = v
    line["extra_workloads"] = extras
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
