"""Benchmark: MatMul-free LM block forward on one MI355X.

A step is one pass of the whole block (RMSNorm + int8 quantization, i|f|g ternary
BitLinear, chunked MLGRU scan with RMSNorm-swish gate, o_proj + residual, GLU with
SiLU(gate)*up, down + residual) over one batch of synthetic input already resident in
HBM.  Default workload: the 370M-shaped block, 8 sequences x 2048 tokens, hidden 1024,
GLU 2816, bf16 activations, ternary weights from N(0, 0.02^2) latents.

Prints one JSON line.  `roofline` describes the dominant kernel (the gate|up int8-MFMA
GEMM), timed with HIP events on the launch stream during the timed steps;
`cpu_baseline` is the CPU oracle timed on a causal prefix of the same workload.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gateup_370M-block_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "ternary_weight_matmul_bitlinear_amd", "csrc", "gemm_prefill.hip")


def _src_hash(path: str) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _traffic(per_launch_key: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or
    None when the summary is missing or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != _src_hash(KERNEL_SRC):
        return None
    return t.get(per_launch_key)


def cpu_baseline(w, x_np, W, B0: int, T0: int):
    """Oracle block forward on the causal prefix x[:B0, :T0] (bounded CPU sample)."""
    import numpy as np
    from oracle import oracle as O
    orc = O.get()
    xs = np.ascontiguousarray(x_np[:B0, :T0])
    orc.block(np.ascontiguousarray(xs[:1, :8]), W, resid_bf16=w.bf16)  # warm-up
    t = time.perf_counter()
    r = orc.block(xs, W, resid_bf16=w.bf16)
    dt = time.perf_counter() - t
    return r, dt, orc.max_threads()


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spin-up", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="370M-block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=128,
                    help="tokens per sequence of the causal prefix timed on the CPU")
    ap.add_argument("--batch", type=int, default=None,
                    help="decode stack: sequences per step (default: the workload's B)")
    ap.add_argument("--regime", choices=("auto", "decode", "prefill", "tiles"), default="auto",
                    help="BitLinear kernel choice (auto: by token count; decode: weight "
                         "streaming; prefill: MFMA kernels; tiles: 128-row MFMA tiles only)")
    ap.add_argument("--no-kernel-sweep", dest="kernel_sweep", action="store_false",
                    help="decode stacks: skip the per-kernel BitLinear streaming sweep")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"asked for --gpus {args.gpus} / WORLD_SIZE={world}", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api, synth

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    api.set_regime({"auto": 0, "decode": 1, "prefill": 2, "tiles": 3}[args.regime])
    if w.layers != 1 or w.vocab:
        return bench_stack(args, w)
    dt = torch.bfloat16 if w.bf16 else torch.float32
    lat = synth.layer_latents(w, 0)
    fb = np.full(w.D, w.f_bias, np.float32) if w.f_bias else None
    blk = api.Block.from_latents(lat, "cuda", f_bias=fb)
    x_np = synth.activations(w)
    x = torch.from_numpy(x_np).to("cuda").to(dt)
    y = torch.empty_like(x)
    h = torch.zeros((w.B, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(api.block_workspace_bytes(blk, w.B, w.T), dtype=torch.uint8, device="cuda")
    M, D, F = w.M, w.D, w.F
    print(f"# workload {w.name}: B={w.B} T={w.T} D={D} F={F} dtype={dt}", file=sys.stderr,
          flush=True)

    spin_up(lambda: api.block_forward(blk, x, h_state=h, y=y, ws=ws), args.spin_up)
    for _ in range(args.warmup):
        h.zero_()
        api.block_forward(blk, x, h_state=h, y=y, ws=ws)
    torch.cuda.synchronize()

    # timed region: HIP events only around the dominant kernel (gate|up GEMM), on the
    # stream it is launched on, so the measured stream stays close to an untimed one
    api.timing_reset()
    api.timing_families(["gemm_gateup"])
    api.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        api.block_forward(blk, x, h_state=h, y=y, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    api.timing_enable(False)
    elapsed = t1 - t0
    ms_step = elapsed * 1e3 / args.steps
    value = M * args.steps / elapsed
    print(f"# timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)
    gn, gms = api.timing_query("gemm_gateup")

    # per-family breakdown: a separate, shorter pass with events around every launch
    fams = {}
    nb = min(args.steps, 10)
    api.timing_reset()
    api.timing_families(None)
    api.timing_enable(True)
    for _ in range(nb):
        api.block_forward(blk, x, h_state=h, y=y, ws=ws)
    torch.cuda.synchronize()
    api.timing_enable(False)
    # algorithmic work per step of each family: int8 ops of the GEMMs; bytes of the HBM-bound
    # kernels (the scan reads the bf16 i|f|g pre-activations once and writes the int8 o_proj
    # input with its scale and code sum; the row quantizers read x, y1 (D wide) and the GLU
    # hidden (F wide) and write int8 codes + 8 bytes per row)
    ab = 2 if w.bf16 else 4
    work = {"gemm_ifg": ("mfma", 2.0 * M * D * 3 * D), "gemm_o": ("mfma", 2.0 * M * D * D),
            "gemm_gateup": ("mfma", 2.0 * M * D * 2 * F), "gemm_down": ("mfma", 2.0 * M * F * D),
            "scan": ("hbm", M * (3 * D * ab + D + 8.0)),
            "quant": ("hbm", M * (2 * D * (ab + 1) + F * (ab + 1) + 24.0))}
    for fam in ("quant", "gemm_ifg", "gemm_o", "gemm_gateup", "gemm_down", "gemv", "scan"):
        n, ms = api.timing_query(fam)
        if n:
            fams[fam] = {"launches_per_step": n / nb, "ms_per_launch": ms / n,
                         "ms_per_step": ms / nb}
            if fam in work:
                bound, amount = work[fam]
                sec = ms / nb * 1e-3
                if bound == "mfma":
                    fams[fam].update(tops=amount / sec / 1e12, mfma_frac=amount / sec / 1e12 / PEAK_INT8_TOPS)
                else:
                    fams[fam].update(gbs=amount / sec / 1e9, hbm_frac=amount / sec / 1e9 / PEAK_HBM_GBS)

    # dominant kernel: gate|up GEMM, 2*M*K*N dense int8 ops per launch
    ops = 2.0 * M * D * (2 * F)
    achieved = ops / (gms / gn * 1e-3) / 1e12 if gn else None
    traffic = _traffic("hbm_bytes_per_launch")
    roofline = {"kernel": "gemm_gateup (int8 MFMA, SiLU(gate)*up epilogue)", "bound": "mfma",
                "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                "frac": (achieved / PEAK_INT8_TOPS) if achieved else None, "traffic": traffic,
                "algorithmic_ops_per_launch": ops}

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        # the timed steps chained the state; parity is checked on a fresh prefill (h0 = 0)
        h.zero_()
        api.block_forward(blk, x, h_state=h, y=y, ws=ws)
        torch.cuda.synchronize()
        B0, T0 = w.B, min(args.cpu_sample_tokens, w.T)
        W = {}
        from oracle import oracle as O
        orc = O.get()
        for k in ("i", "f", "g", "o", "gate", "up", "down"):
            W[k] = orc.ternarize(lat[k])
        r, cdt, threads = cpu_baseline(w, x_np, W, B0, T0)
        ref = r["y"]
        got = y.float().cpu().numpy()[:B0, :T0].astype(np.float64)
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        err = float(np.max(np.abs(got - ref) / (np.abs(ref) + rms)))
        cpu = {"value": B0 * T0 / cdt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"causal prefix: first {T0} tokens of each of the {B0} sequences "
                         f"({B0 * T0} tokens), one block, {cdt:.1f} s",
               "sample_max_rel_err_vs_gpu": err}

    line = {"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": "synthetic (seeded N(0,1) activations, ternary weights from N(0,0.02^2) latents)",
            "config": {"workload": w.name, "B": w.B, "T": w.T, "D": D, "F": F,
                       "activations": "bf16" if w.bf16 else "fp32", "state": "fp32"},
            "roofline": roofline, "cpu_baseline": cpu,
            "kernels": fams, "kernels_note": f"separate {nb}-step pass, events around every launch; "
                                             "mfma_frac / hbm_frac: the family's algorithmic work per "
                                             "step over its summed launch time"}
    print(json.dumps(line))
    return 0


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
        api.timing_reset()
        api.timing_families(fams)
        api.timing_enable(True)
        reps = max(copies, 40)
        for i in range(reps):
            api.bitlinear_forward(ws[i % copies], x)
        torch.cuda.synchronize()
        api.timing_enable(False)
        n = ms = 0
        for f in fams:
            nf, msf = api.timing_query(f)
            n, ms = n + nf, ms + msf
        bytes_ = wbytes + B * K * 2 + B * N * 2
        gbs = bytes_ * n / (ms * 1e-3) / 1e9
        out.append({"N": N, "K": K, "rows": B, "weight_copies": copies,
                    "us_per_launch": ms / n * 1e3, "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS})
        del ws
        torch.cuda.empty_cache()
    return out


def bench_stack(args, w) -> int:
    """Stack workloads.  1.3B-decode: one step = one token for each of B sequences through
    the ternary embedding, 24 blocks (state carried) and the LM head; the weights (about
    325 MB packed) exceed the 256 MB MALL, so every step streams them from HBM.
    2.7B-longctx: one step = the 32-block prefill of 2 x 32768 tokens."""
    import numpy as np
    import torch

    from ternary_weight_matmul_bitlinear_amd import api, synth

    D, F, L = w.D, w.F, w.layers
    fb = np.full(D, w.f_bias, np.float32) if w.f_bias else None
    t_build = time.perf_counter()
    blocks = []
    for l in range(L):
        blocks.append(api.Block.from_latents(synth.layer_latents(w, l), "cuda", f_bias=fb))
    emb = head = None
    if w.vocab:
        E, H = synth.embedding_latents(w)
        emb = api.TernaryLinear.from_latent(E)
        head = api.TernaryLinear.from_latent(H)
        del E, H
    stack = api.Stack(blocks, emb, head)
    print(f"# workload {w.name}: {L} layers, D={D} F={F}; weights built in "
          f"{time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)

    decode = bool(w.vocab)
    B = args.batch or w.B
    T = 1 if decode else w.T
    steps = args.steps
    hs = torch.zeros((L, B, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(stack.workspace_bytes(B, T), dtype=torch.uint8, device="cuda")
    if decode:
        ids_all = torch.from_numpy(synth.token_ids(w, args.warmup + steps, B)).to("cuda")
        logits = torch.empty((B, w.vocab), dtype=torch.float32, device="cuda")

        def step(i):
            api.stack_forward(stack, B, 1, ids=ids_all[i], h_state=hs, want_y=False,
                              want_logits=True, ws=ws, logits=logits)
    else:
        x = torch.from_numpy(synth.activations(w)).to("cuda").to(torch.bfloat16)
        y = torch.empty_like(x)

        def step(i):
            hs.zero_()
            api.stack_forward(stack, B, T, x=x, ws=ws, y=y)

    spin_up(lambda: step(0), args.spin_up)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch durations of the dominant kernel family: an eager pass with events
    # decode: every BitLinear launch of the step (the dot4 kernel for a few rows, the k-split
    # MFMA kernel for more, both under their own family names)
    fams = (["gemv", "gemm_ifg", "gemm_o", "gemm_gateup", "gemm_down", "gemm"] if decode
            else ["gemm_gateup"])
    api.timing_reset()
    api.timing_families(fams)
    api.timing_enable(True)
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    api.timing_enable(False)
    n, ms = 0, 0.0
    for f in fams:
        nf, msf = api.timing_query(f)
        n, ms = n + nf, ms + msf
    graph_ms = None
    if decode:
        # the timed loop replays one captured step (a HIP graph): a decode step is ~120 small
        # launches, whose host-side launch cost would otherwise dominate
        ids_static = ids_all[0].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            api.stack_forward(stack, B, 1, ids=ids_static, h_state=hs, want_y=False,
                              want_logits=True, ws=ws, logits=logits)
        for i in range(args.warmup):
            ids_static.copy_(ids_all[i])
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ids_static.copy_(ids_all[args.warmup + i])
            g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        graph_ms = elapsed * 1e3 / steps
    else:
        elapsed = eager_ms * steps / 1e3
    ms_step = elapsed * 1e3 / steps
    value = B * T * steps / elapsed

    if decode:
        # algorithmic bytes of the decode BitLinear launches (N*K/4 packed weights + rows in
        # + rows out, residual where added), and of the whole step (plus embedding rows and
        # the fp32 state read and written per layer)
        def bl(N, K, in_b, out_b, resid=0):
            return N * K // 4 + B * K * in_b + B * N * out_b + B * N * resid
        # the dot4 kernel (up to 4 rows) quantizes bf16 rows itself; the k-split kernel reads
        # int8 rows written by the row quantizer
        xin = 2 if B <= 4 else 1
        per_layer = (bl(3 * D, D, xin, 2) + bl(D, D, 1, 2, 2) + bl(2 * F, D, xin, 0) + B * F * 2
                     + bl(D, F, xin, 2, 2))
        gemv_bytes = L * per_layer + bl(w.vocab, D, xin, 4)
        step_bytes = gemv_bytes + B * D // 4 + B * D * 2 + L * B * D * 4 * 2
        achieved = gemv_bytes * steps / (ms * 1e-3) / 1e9 if n else None
        roofline = {"kernel": "decode BitLinear (dot4 weight streaming up to 4 rows, k-split "
                              "MFMA above), all launches of a step",
                    "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS if achieved else None, "traffic": None,
                    "algorithmic_bytes_per_step": gemv_bytes}
        extra = {"step_hbm_fraction": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
                 "step_algorithmic_bytes": step_bytes, "eager_ms_per_step": eager_ms,
                 "graph_ms_per_step": graph_ms}
        if args.kernel_sweep:
            extra["decode_bitlinear_kernels"] = decode_kernel_sweep(B, D, F, w.vocab)
    else:
        ops = 2.0 * (B * T) * D * (2 * F)
        achieved = ops * n / (ms * 1e-3) / 1e12 if n else None
        roofline = {"kernel": "gemm_gateup (int8 MFMA, SiLU(gate)*up epilogue), all layers",
                    "bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_INT8_TOPS if achieved else None,
                    "traffic": None, "algorithmic_ops_per_launch": ops}
        extra = {}
    line = {"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": "synthetic (seeded ids / N(0,1) activations, ternary weights from N(0,0.02^2) latents)",
            "config": {"workload": w.name, "B": B, "T": T, "D": D, "F": F, "layers": L,
                       "vocab": w.vocab or None, "activations": "bf16", "state": "fp32"},
            "roofline": roofline, "cpu_baseline": None, **extra}
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
