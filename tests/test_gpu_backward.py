"""Straight-through BitLinear backward and MLGRU + output-gate backward on the GPU against the
oracle (reading R14).

BitLinear: every output is compared element by element with a bound derived from the
kernel's arithmetic: the contractions run on bf16 matrix cores with fp32 accumulation, so
an output is a sum of n terms each rounded once to bf16 (relative 2^-9: dy when it is fp32,
dy*a for dW; bf16 dy and the codes are exact) plus n fp32 additions (n*2^-24 relative), all
relative to the sum of the terms' absolute values (computed here in fp64 from the same
inputs); dx inherits g's bound through its formula.  The MLGRU backward is fp32 throughout
and is held to the fp32 tolerance 1e-3 (relative to |ref| + the row's rms)."""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import dev, host, note, rel_check

pytestmark = pytest.mark.gpu

U_BF16 = 2.0**-9
U_F32 = 2.0**-24


def _bl_inputs(seed, M, K, N, x_bf, dy_bf, with_gamma):
    x = synth.gaussian(seed, (M, K))
    if x_bf:
        x = synth.round_to_bf16(x)
    lat = synth.gaussian(seed + 1, (N, K), 0.02)
    dy = synth.gaussian(seed + 2, (M, N))
    if dy_bf:
        dy = synth.round_to_bf16(dy)
    gamma = (1.0 + 0.2 * synth.gaussian(seed + 3, (K,))).astype(np.float32) if with_gamma else None
    return x, lat, dy, gamma


def _bounds(orc, x, q, s, dy, gamma, dy_bf, eps=1e-6):
    """Per-element error bounds of the GPU's g, dx, dgamma, dw, db (fp64)."""
    M, K = x.shape
    N = q.shape[0]
    xs = x.astype(np.float64)
    ady = np.abs(dy.astype(np.float64))
    aq = np.abs(q.astype(np.float64))
    gm = np.ones(K) if gamma is None else gamma.astype(np.float64)
    eg = (0.0 if dy_bf else U_BF16) + N * U_F32
    gb = eg * s * (ady @ aq)                         # bound of g
    r = 1.0 / np.sqrt((xs * xs).mean(axis=1) + eps)
    g_ref = s * (dy.astype(np.float64) @ q.astype(np.float64))
    mag = r[:, None] * np.abs(gm) * np.abs(g_ref) + np.abs(xs) * (r**3 / K)[:, None] * np.abs(
        (g_ref * gm * xs).sum(axis=1))[:, None]
    dxb = (r[:, None] * np.abs(gm) * gb
           + np.abs(xs) * (r**3 / K)[:, None] * (gb * np.abs(gm * xs)).sum(axis=1)[:, None]
           + 1e-5 * mag)
    dgb = (gb * np.abs(xs) * r[:, None]).sum(axis=0) + M * U_F32 * (np.abs(g_ref * xs) * r[:, None]).sum(axis=0)
    qx, a, _ = orc.act_quant(x, gamma, eps)
    dwb = (U_BF16 + 2 * U_F32 + M * U_F32) * ((ady * a[:, None]).T @ np.abs(qx.astype(np.float64)))
    dbb = M * U_F32 * ady.sum(axis=0) + (0.0 if dy_bf else U_BF16) * ady.sum(axis=0)
    return {"dx": dxb, "dgamma": dgb, "dw": dwb, "db": dbb}


def _bound_check(got, ref, bound, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - ref)
    # factor 2 over the bound; the floor covers exact zeros of the reference
    lim = 2.0 * bound + 1e-30
    ratio = err / lim
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: err {err[worst]:.3e} > 2 x bound {bound[worst]:.3e} at {worst} "
                                f"(got {got[worst]:.6e}, ref {ref[worst]:.6e})")
    return float(ratio.max())


BL_CASES = [(1, 64, 8), (37, 128, 40), (300, 704, 256), (257, 1024, 2816), (64, 2816, 1024)]


@pytest.mark.parametrize("with_gamma", [True, False], ids=["gamma", "nogamma"])
@pytest.mark.parametrize("x_bf,dy_bf", [(False, False), (True, True), (True, False)],
                         ids=["x32-dy32", "x16-dy16", "x16-dy32"])
@pytest.mark.parametrize("M,K,N", BL_CASES, ids=[f"M{m}K{k}N{n}" for m, k, n in BL_CASES])
def test_bitlinear_backward_parity(orc, M, K, N, x_bf, dy_bf, with_gamma):
    note(f"bitlinear_backward M={M} K={K} N={N} x_bf16={x_bf} dy_bf16={dy_bf} gamma={with_gamma}")
    x, lat, dy, gamma = _bl_inputs(M * 7 + K + N, M, K, N, x_bf, dy_bf, with_gamma)
    q, s = orc.ternarize(lat)
    w = api.TernaryLinear.from_ternary(q, s, "cuda", norm_w=gamma)
    xdt = torch.bfloat16 if x_bf else torch.float32
    ydt = torch.bfloat16 if dy_bf else torch.float32
    got = api.bitlinear_backward(w, dev(x, xdt), dev(dy, ydt))
    torch.cuda.synchronize()
    ref = orc.bitlinear_backward(x, q, s, dy.astype(np.float64), gamma=gamma)
    b = _bounds(orc, x, q, s, dy, gamma, dy_bf)
    for k in ("dx", "dgamma", "dw", "db"):
        _bound_check(host(got[k]), ref[k], b[k], k)


@pytest.mark.parametrize("M,K,N", [(16384, 1024, 2816), (32768, 2560, 6912)], ids=["370M", "2.7B"])
def test_bitlinear_backward_full_size_sampled(orc, M, K, N):
    """The gate projection at the benchmark's block sizes (370M: 16384 tokens, K 1024,
    N 2816; 2.7B: 32768 tokens, K 2560, N 6912; bf16): dx on sampled rows (rows are
    independent), dW on sampled entries, db whole."""
    note(f"bitlinear_backward full size M={M} K={K} N={N}")
    x, lat, dy, gamma = _bl_inputs(4242 + K, M, K, N, True, True, True)
    q, s = orc.ternarize(lat)
    w = api.TernaryLinear.from_ternary(q, s, "cuda", norm_w=gamma)
    got = api.bitlinear_backward(w, dev(x, torch.bfloat16), dev(dy, torch.bfloat16), want_dgamma=False)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 4095, 9000, M - 2, M - 1])
    ref = orc.bitlinear_backward(x[rows], q, s, dy[rows].astype(np.float64), gamma=gamma)
    b = _bounds(orc, x[rows], q, s, dy[rows], gamma, True)
    _bound_check(host(got["dx"])[rows], ref["dx"], b["dx"], "dx rows")
    qx, a, _ = orc.act_quant(x, gamma)
    rng = np.random.default_rng(5)
    ns, ks = rng.integers(0, N, 64), rng.integers(0, K, 64)
    dws = host(got["dw"])[ns, ks]
    dyd = dy.astype(np.float64)
    ref_dw = np.array([np.dot(dyd[:, n] * a, qx[:, k].astype(np.float64)) for n, k in zip(ns, ks)])
    bnd = np.array([(U_BF16 + (M + 2) * U_F32) * np.dot(np.abs(dyd[:, n]) * a, np.abs(qx[:, k].astype(np.float64)))
                    for n, k in zip(ns, ks)])
    _bound_check(dws, ref_dw, bnd, "dw sampled")
    db_ref = dyd.sum(axis=0)
    _bound_check(host(got["db"]), db_ref, M * U_F32 * np.abs(dyd).sum(axis=0), "db")


def test_bitlinear_backward_empty(orc):
    """m = 0: the parameter gradients are empty sums (zero)."""
    q, s = orc.ternarize(synth.gaussian(1, (16, 64), 0.02))
    w = api.TernaryLinear.from_ternary(q, s, "cuda")
    got = api.bitlinear_backward(w, torch.empty((0, 64), device="cuda"), torch.empty((0, 16), device="cuda"))
    torch.cuda.synchronize()
    for k in ("dgamma", "dw", "db"):
        assert float(got[k].abs().max()) == 0.0, k


MG_CASES = [(1, 1, 64), (1, 16, 128), (2, 37, 256), (2, 200, 1024), (1, 33, 2560), (1, 20, 4096),
            (8, 2048, 1024), (16, 2048, 2560)]


@pytest.mark.parametrize("gate_mode", [0, 1], ids=["swish_rmsnorm", "sigmoid"])
@pytest.mark.parametrize("bf", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", MG_CASES, ids=[f"B{b}T{t}D{d}" for b, t, d in MG_CASES])
def test_mlgru_backward_parity(orc, B, T, D, bf, gate_mode):
    note(f"mlgru_backward B={B} T={T} D={D} bf16={bf} gate={gate_mode}")
    seed = B * 1000 + T * 10 + D
    ifg = synth.gaussian(seed, (B, T, 3 * D), 1.5)
    dout = synth.gaussian(seed + 1, (B, T, D))
    if bf:
        ifg, dout = synth.round_to_bf16(ifg), synth.round_to_bf16(dout)
    fb = synth.gaussian(seed + 2, (D,), 0.5)
    h0 = synth.gaussian(seed + 3, (B, D))
    gw = (1.0 + 0.2 * synth.gaussian(seed + 4, (D,))).astype(np.float32)
    lb = orc.hgrn_lower_bounds(synth.gaussian(seed + 5, (3, D)))[1].astype(np.float32)
    dl = synth.gaussian(seed + 6, (B, D))
    dt = torch.bfloat16 if bf else torch.float32
    got = api.mlgru_backward(dev(ifg, dt), dev(dout, dt), f_bias=dev(fb), h0=dev(h0), gnorm_w=dev(gw),
                             gate_mode=gate_mode, f_lower=dev(lb), dh_last=dev(dl))
    torch.cuda.synchronize()
    ref = orc.mlgru_backward(ifg.astype(np.float64), dout.astype(np.float64), f_bias=fb, h0=h0,
                             gnorm_w=gw, gate_mode=gate_mode, f_lower=lb, dh_last=dl)
    rel_check(host(got["d_ifg"]), ref["d_ifg"], 1e-3, "d_ifg")
    rel_check(host(got["dh0"]), ref["dh0"], 1e-3, "dh0")
    rel_check(host(got["df_bias"]), ref["df_bias"], 1e-3, "df_bias")
    if gate_mode == 0:
        rel_check(host(got["dgnorm_w"]), ref["dgnorm_w"], 1e-3, "dgnorm_w")
    else:
        assert float(got["dgnorm_w"].abs().max()) == 0.0


def test_mlgru_backward_no_options(orc):
    """No forget bias, bound, gain, initial state or final-state gradient (all NULL)."""
    B, T, D = 2, 50, 256
    ifg = synth.gaussian(77, (B, T, 3 * D), 1.5)
    dout = synth.gaussian(78, (B, T, D))
    got = api.mlgru_backward(dev(ifg), dev(dout))
    torch.cuda.synchronize()
    ref = orc.mlgru_backward(ifg.astype(np.float64), dout)
    rel_check(host(got["d_ifg"]), ref["d_ifg"], 1e-3, "d_ifg")
    rel_check(host(got["dh0"]), ref["dh0"], 1e-3, "dh0")


def test_mlgru_backward_empty(orc):
    """T = 0: dh0 = dh_last, the parameter gradients are zero."""
    D = 128
    dl = synth.gaussian(3, (2, D))
    got = api.mlgru_backward(torch.empty((2, 0, 3 * D), device="cuda"), torch.empty((2, 0, D), device="cuda"),
                             dh_last=dev(dl))
    torch.cuda.synchronize()
    assert np.array_equal(host(got["dh0"]), dl.astype(np.float32).astype(np.float64))
    assert float(got["df_bias"].abs().max()) == 0.0


# ------------------------------------------------------------------ block backward

def _block(orc, seed, D, F, with_extras):
    """A device block (gains and biases when with_extras; i|f|g and gate|up share their gains)
    and the oracle's weight dict (q, scale, gamma, bias) for the same ternary weights."""
    lat = synth.layer_latents(synth.Workload("bb", D=D, F=F, B=1, T=1, seed=seed), 0)
    gains = {}
    if with_extras:
        gx = (1 + 0.2 * synth.gaussian(seed + 50, (D,))).astype(np.float32)
        ggu = (1 + 0.2 * synth.gaussian(seed + 51, (D,))).astype(np.float32)
        gains = {"i": gx, "f": gx, "g": gx, "gate": ggu, "up": ggu,
                 "o": (1 + 0.2 * synth.gaussian(seed + 52, (D,))).astype(np.float32),
                 "down": (1 + 0.2 * synth.gaussian(seed + 53, (F,))).astype(np.float32)}
    lins, W = {}, {}
    dev_gain = {}   # one device tensor per distinct gain: the block shares them by pointer
    for j, k in enumerate(api.BLOCK_LINEARS):
        q, s = orc.ternarize(lat[k])
        g = gains.get(k)
        b = (0.05 * synth.gaussian(seed + 60 + j, (q.shape[0],))).astype(np.float32) if with_extras else None
        gd = None
        if g is not None:
            gd = dev_gain.setdefault(id(g), dev(g))
        lins[k] = api.TernaryLinear.from_ternary(q, s, "cuda", norm_w=gd, bias=b)
        W[k] = (q, s, g, b)
    kw = {}
    if with_extras:
        kw = dict(f_bias=synth.gaussian(seed + 70, (D,), 0.5),
                  gnorm_w=(1 + 0.2 * synth.gaussian(seed + 71, (D,))).astype(np.float32),
                  f_lower=orc.hgrn_lower_bounds(synth.gaussian(seed + 72, (3, D)))[1].astype(np.float32))
    blk = api.Block(**lins, **{k: (dev(v) if v is not None else None) for k, v in kw.items()})
    return blk, W, kw


def _grad_check(got, ref, tol, what):
    """Independent-run criterion (as for the forward's end-to-end runs): the recomputed
    forward takes its own int8 decisions (a near-tie can flip one code against the oracle's
    fp64 run) and every gradient passes through up to three bf16 roundings of matrix-core
    operands, so p99.9 of the element error (relative to |ref| + the row's rms) and every
    row's norm-wise error are held to tol, and the maximum to 5 tol."""
    got = np.atleast_2d(np.asarray(got, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    ratio = np.abs(got - ref) / (np.abs(ref) + rms + 1e-30)
    p999 = float(np.quantile(ratio, 0.999))
    rowerr = float(np.max(np.linalg.norm(got - ref, axis=-1) / (np.linalg.norm(ref, axis=-1) + 1e-30)))
    assert p999 <= tol and rowerr <= tol and ratio.max() <= 5 * tol, \
        f"{what}: p99.9 {p999:.3e}, row {rowerr:.3e}, max {ratio.max():.3e} (tol {tol})"
    return p999, rowerr, float(ratio.max())


def _block_checks(got, ref, D, tol, rows=None, what=""):
    """Every block gradient against the oracle's (rows: the dx rows compared)."""
    dx = host(got["dx"]).reshape(-1, D)
    worst = {"dx": _grad_check(dx if rows is None else dx[rows], ref["dx"].reshape(-1, D), tol, what + "dx"),
             "dh0": _grad_check(host(got["dh0"]), ref["dh0"], tol, what + "dh0")}
    for k in api.BLOCK_LINEARS:
        worst["dw " + k] = _grad_check(host(got["dw"][k]), ref["dw"][k], tol, f"{what}dw[{k}]")
        worst["db " + k] = _grad_check(host(got["db"][k]), ref["db"][k], tol, f"{what}db[{k}]")
    groups = {"x": ("i", "f", "g"), "o": ("o",), "y1": ("gate", "up"), "m": ("down",)}
    for name, ks in groups.items():
        worst["dgamma " + name] = _grad_check(host(got["dgamma"][name]), sum(ref["dgamma"][k] for k in ks),
                                              tol, f"{what}dgamma[{name}]")
    worst["dgnorm_w"] = _grad_check(host(got["dgnorm_w"]), ref["dgnorm_w"], tol, what + "dgnorm_w")
    worst["df_bias"] = _grad_check(host(got["df_bias"]), ref["df_bias"], tol, what + "df_bias")
    note("  worst (p99.9, row, max): " + ", ".join(f"{k} {v[2]:.1e}" for k, v in worst.items() if v[2] > 2e-3))


BB_TOL = 2e-2   # the bf16 tolerance: the backward's contractions run on bf16 matrix cores


@pytest.mark.parametrize("gate_mode", [0, 1], ids=["swish_rmsnorm", "sigmoid"])
@pytest.mark.parametrize("bf", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("B,T,D,F,extras", [(2, 37, 256, 704, True), (1, 16, 128, 384, False),
                                            (3, 50, 512, 1408, True)],
                         ids=["B2T37D256", "B1T16D128-plain", "B3T50D512"])
def test_block_backward_parity(orc, B, T, D, F, extras, bf, gate_mode):
    note(f"block_backward B={B} T={T} D={D} F={F} extras={extras} bf16={bf} gate={gate_mode}")
    seed = B * 100 + T + D
    blk, W, kw = _block(orc, seed, D, F, extras)
    blk.gate_mode = gate_mode
    x = synth.gaussian(seed + 1, (B, T, D))
    dy = synth.gaussian(seed + 2, (B, T, D))
    if bf:
        x, dy = synth.round_to_bf16(x), synth.round_to_bf16(dy)
    h0 = synth.gaussian(seed + 3, (B, D)) if extras else None
    dl = synth.gaussian(seed + 4, (B, D)) if extras else None
    dt = torch.bfloat16 if bf else torch.float32
    got = api.block_backward(blk, dev(x, dt), dev(dy, dt), h0=dev(h0) if h0 is not None else None,
                             dh_last=dev(dl) if dl is not None else None)
    torch.cuda.synchronize()
    ref = orc.block_backward(x, W, dy.astype(np.float64), gate_mode=gate_mode, resid_bf16=bf,
                             h0=h0, dh_last=dl, **kw)
    _block_checks(got, ref, D, BB_TOL)


def test_block_backward_mixed_dtypes(orc):
    """bf16 activations with an fp32 output gradient: down's g then runs on the fp32-operand
    contraction, its dy*a transpose reads fp32 and the gate|up row kernel adds an fp32
    residual."""
    B, T, D, F = 2, 29, 256, 704
    note(f"block_backward bf16 x, fp32 dy, B={B} T={T} D={D} F={F}")
    blk, W, kw = _block(orc, 4040, D, F, True)
    x = synth.round_to_bf16(synth.gaussian(4041, (B, T, D)))
    dy = synth.gaussian(4042, (B, T, D))
    h0 = synth.gaussian(4043, (B, D))
    got = api.block_backward(blk, dev(x, torch.bfloat16), dev(dy, torch.float32), h0=dev(h0))
    torch.cuda.synchronize()
    ref = orc.block_backward(x, W, dy.astype(np.float64), resid_bf16=True, h0=h0, **kw)
    _block_checks(got, ref, D, BB_TOL)


@pytest.mark.parametrize("name,P", [("370M-block", 64), ("2.7B-block", 8)])
def test_block_backward_full_size_prefix(orc, name, P):
    """A block at the benchmark's size (370M: 8 x 2048 tokens, 2.7B: 16 x 2048, bf16), with
    dy non-zero only on the first P tokens of every sequence and no final-state gradient: the
    reverse recurrence then carries nothing from the later tokens and their rows contribute
    nothing to the parameter gradients, so every gradient equals the oracle's on the B x P
    prefix, and dx is zero beyond it."""
    w = synth.WORKLOADS[name]
    B, T, D, F = w.B, w.T, w.D, w.F
    note(f"block_backward full size B={B} T={T} D={D} F={F}, dy on the first {P} tokens")
    blk, W, kw = _block(orc, 4321, D, F, True)
    x = synth.activations(w)
    dy = np.zeros((B, T, D), np.float32)
    dy[:, :P] = synth.round_to_bf16(synth.gaussian(4322, (B, P, D)))
    h0 = synth.gaussian(4323, (B, D))
    got = api.block_backward(blk, dev(x, torch.bfloat16), dev(dy, torch.bfloat16), h0=dev(h0))
    torch.cuda.synchronize()
    ref = orc.block_backward(x[:, :P], W, dy[:, :P].astype(np.float64), resid_bf16=True, h0=h0, **kw)
    dx = host(got["dx"])
    assert float(np.abs(dx[:, P:]).max()) == 0.0, "dx beyond the prefix"
    rows = (np.arange(B)[:, None] * T + np.arange(P)[None, :]).reshape(-1)
    got["dx"] = got["dx"].reshape(B * T, D)
    _block_checks(got, ref, D, BB_TOL, rows=rows)


def test_block_backward_some_gradients(orc):
    """Only some parameter gradients asked for (the others NULL): one row block of the stacked
    gate|up and i|f|g dW launches, single bias and gain gradients (o's bias without its
    weights), df_bias without dgnorm_w.
    Each equals the same call's gradient with everything asked for (the same kernels; the
    fp32 atomic sums may differ in order only)."""
    B, T, D, F = 2, 40, 256, 704
    blk, _, _ = _block(orc, 77, D, F, True)
    x = dev(synth.round_to_bf16(synth.gaussian(78, (B, T, D))), torch.bfloat16)
    dy = dev(synth.round_to_bf16(synth.gaussian(79, (B, T, D))), torch.bfloat16)
    full = api.block_backward(blk, x, dy)
    # o: its bias gradient without its weight gradient (the column-sum path)
    want = {"dw/up", "dw/f", "dw/down", "db/g", "db/gate", "db/o", "dgamma/y1", "df_bias"}
    part = api.block_backward(blk, x, dy, grads=want)
    torch.cuda.synchronize()
    assert set(part["dw"]) == {"up", "f", "down"} and set(part["db"]) == {"g", "gate", "o"}
    assert set(part["dgamma"]) == {"y1"} and "dgnorm_w" not in part and "df_bias" in part
    pairs = [(part["dx"], full["dx"]), (part["dh0"], full["dh0"]), (part["df_bias"], full["df_bias"])]
    pairs += [(part["dw"][k], full["dw"][k]) for k in part["dw"]]
    pairs += [(part["db"][k], full["db"][k]) for k in part["db"]]
    pairs += [(part["dgamma"]["y1"], full["dgamma"]["y1"])]
    for a, b in pairs:
        a, b = host(a), host(b)
        assert np.all(np.isfinite(a))
        assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(b) + 1e-30


def test_block_backward_empty(orc):
    """T = 0: dh0 = dh_last and every parameter gradient is zero."""
    blk, _, _ = _block(orc, 7, 128, 384, False)
    dl = synth.gaussian(8, (2, 128))
    got = api.block_backward(blk, torch.empty((2, 0, 128), device="cuda"),
                             torch.empty((2, 0, 128), device="cuda"), dh_last=dev(dl))
    torch.cuda.synchronize()
    assert np.array_equal(host(got["dh0"]), dl.astype(np.float32).astype(np.float64))
    for k in api.BLOCK_LINEARS:
        assert float(got["dw"][k].abs().max()) == 0.0 and float(got["db"][k].abs().max()) == 0.0
