"""Shared helpers of the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth

TOL = {torch.float32: 1e-3, torch.bfloat16: 2e-2}


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a crashed run)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_check(got, ref, tol: float, what: str = "") -> dict:
    """Pass when |got - ref| <= tol * (|ref| + rms of ref's row) everywhere."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    ratio = np.abs(got - ref) / (np.abs(ref) + rms + 1e-30)
    stats = {"max": float(ratio.max()), "p999": float(np.quantile(ratio, 0.999))}
    assert stats["max"] <= tol, f"{what}: max rel err {stats['max']:.3e} > {tol} (p99.9 {stats['p999']:.3e})"
    return stats


def stage_recheck(orc, st: dict, w_cat: np.ndarray, gamma=None, eps: float = 1e-6,
                  what: str = "") -> None:
    """Capture protocol: rerun the oracle quantizer and accumulator on the captured fp32
    stage input; int8 codes and int32 accumulators must match bit for bit."""
    q, a, _ = orc.act_quant(st["x_in"], gamma=gamma, eps=eps)
    assert np.array_equal(q, st["q"]), f"{what}: q differs at {np.argwhere(q != st['q'])[:5]}"
    np.testing.assert_allclose(st["a"], a, rtol=2e-5, err_msg=f"{what}: a")
    acc = orc.accumulate(st["q"], w_cat)
    bad = np.argwhere(acc != st["acc"])
    assert bad.size == 0, f"{what}: acc differs at {bad[:5]} ({len(bad)} elements)"


def make_block(orc, lat: dict, device="cuda", f_bias=None, gnorm_w=None, gate_mode=0,
               eps=1e-6, f_lower=None):
    """Device block from latent weights (library host quantizer) and the oracle's own
    ternarization of the same latents (asserted identical)."""
    blk = api.Block.from_latents(lat, device, f_bias=f_bias, gnorm_w=gnorm_w, eps=eps,
                                 gate_mode=gate_mode, f_lower=f_lower)
    W = {}
    for k in ("i", "f", "g", "o", "gate", "up", "down"):
        q, s = orc.ternarize(lat[k])
        W[k] = (q, s)
    return blk, W


def cat_weights(W: dict) -> dict:
    return {"ifg": np.concatenate([W["i"][0], W["f"][0], W["g"][0]]), "o": W["o"][0],
            "gateup": np.concatenate([W["gate"][0], W["up"][0]]), "down": W["down"][0]}


def small_latents(seed: int, D: int, F: int) -> dict:
    w = synth.Workload("t", D=D, F=F, B=1, T=1, seed=seed)
    return synth.layer_latents(w, 0)


def round_act(orc, v, bf16: bool) -> np.ndarray:
    """Round fp64 values to the activation dtype (the oracle's single rounding)."""
    v = np.asarray(v, np.float64)
    return orc.round_bf16(v) if bf16 else v.astype(np.float32).astype(np.float64)


def block_stage_checks(orc, cap: dict, W: dict, x_rows: np.ndarray, bf16: bool, *,
                       seq_rows: tuple | None = None, f_bias=None, gnorm_w=None,
                       gate_mode: int = 0, h0=None, h_last=None, y_rows=None,
                       f_lower=None) -> dict:
    """Stage-wise parity of one block run from its capture (host dicts per stage).

    Integers: every stage's int8 codes and int32 accumulators must be bit-exact against the
    oracle's quantizer and accumulator applied to the stage input the GPU captured.
    Floating point: every stage's stored output must match the oracle applied to the GPU's
    own stage inputs (tolerance of the stored dtype).  seq_rows = (B, T) when the capture
    window holds whole sequences from t = 0, which enables the recurrence check."""
    tol = 2e-2 if bf16 else 1e-3
    stats = {}
    cw = cat_weights(W)
    D = x_rows.shape[-1]
    F = W["gate"][0].shape[0]
    x_rows = np.asarray(x_rows, np.float32).reshape(-1, D)
    # i|f|g: input is x itself
    st = cap["ifg"]
    assert np.array_equal(st["x_in"], x_rows), "ifg x_in is not x"
    stage_recheck(orc, st, cw["ifg"], what="ifg")
    ifg_ref = np.concatenate([orc.bitlinear(x_rows, *W[k])[0] for k in ("i", "f", "g")], axis=1)
    stats["ifg"] = rel_check(st["y_out"], round_act(orc, ifg_ref, bf16), tol, "ifg pre-activations")
    # recurrence + g_norm from the GPU's stored pre-activations
    o_in = cap["o"]["x_in"]
    assert np.array_equal(round_act(orc, o_in, bf16).astype(np.float32), o_in), \
        "g_norm output is not a value of the activation dtype"
    if seq_rows is not None:
        B, T = seq_rows
        o_ref, h_ref = orc.mlgru(st["y_out"].astype(np.float64).reshape(B, T, 3 * D),
                                 f_bias=f_bias, h0=h0, gnorm_w=gnorm_w, gate_mode=gate_mode,
                                 f_lower=f_lower)
        # g_norm's output is materialised in the activation dtype before o_proj
        stats["mlgru"] = rel_check(o_in, round_act(orc, o_ref.reshape(-1, D), bf16), tol,
                                   "g_norm output")
        if h_last is not None:
            stats["h_T"] = rel_check(h_last, h_ref, 1e-3, "h_T")
    # o_proj + residual
    stage_recheck(orc, cap["o"], cw["o"], what="o")
    y1_ref = round_act(orc, x_rows + orc.bitlinear(o_in, *W["o"])[0], bf16)
    y1 = cap["o"]["y_out"]
    stats["y1"] = rel_check(y1, y1_ref, tol, "y1")
    # GLU
    assert np.array_equal(cap["gateup"]["x_in"], y1), "GLU input is not the stored y1"
    stage_recheck(orc, cap["gateup"], cw["gateup"], what="gateup")
    _, m_ref = orc.glu(y1, W["gate"], W["up"], W["down"], act_bf16=bf16)
    m = cap["gateup"]["y_out"]
    stats["m"] = rel_check(m, m_ref, tol, "GLU hidden")
    assert np.array_equal(cap["down"]["x_in"], m), "down input is not the stored GLU hidden"
    stage_recheck(orc, cap["down"], cw["down"], what="down")
    y_ref = round_act(orc, y1 + orc.bitlinear(m, *W["down"])[0], bf16)
    stats["y"] = rel_check(cap["down"]["y_out"], y_ref, tol, "block output")
    if y_rows is not None:
        assert np.array_equal(np.asarray(y_rows, np.float32).reshape(-1, D),
                              cap["down"]["y_out"]), "returned y differs from the captured output"
    return stats


def e2e_checks(got_y, ref_y, bf16: bool, cap: dict | None = None, rec: dict | None = None,
               got_h=None, ref_h=None, decisions_agree: bool = False) -> dict:
    """Independent end-to-end comparison (GPU vs oracle from the same x).  Downstream int8
    codes may flip by one where fp32 and fp64 land on opposite sides of a rounding point,
    and such a flip propagates.  While every downstream int8 decision agrees (the captured
    codes equal the oracle's, or the caller established it: decisions_agree) every element
    is held to the tolerance; after a flip the bound is statistical: p99.9 of the element
    error and every row's norm-wise relative error within the tolerance, flips <= 1e-3,
    and the maximum is reported."""
    tol = 2e-2 if bf16 else 1e-3
    g = np.asarray(got_y, np.float64).reshape(-1, got_y.shape[-1])
    r = np.asarray(ref_y, np.float64).reshape(g.shape)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    el = np.abs(g - r) / (np.abs(r) + rms)
    rowwise = np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)
    out = {"max": float(el.max()), "p999": float(np.quantile(el, 0.999)),
           "row_norm_max": float(rowwise.max())}
    assert out["p999"] <= tol, out
    assert out["row_norm_max"] <= tol, out
    if cap is not None and rec is not None:
        n_flips = 0
        for name in ("o", "gateup", "down"):
            ne = cap[name]["q"] != rec[name]["q"]
            f = float(np.mean(ne))
            n_flips += int(np.count_nonzero(ne))
            d = np.abs(cap[name]["q"].astype(np.int32) - rec[name]["q"].astype(np.int32))
            out[f"flips_{name}"] = f
            assert f <= 1e-3, (name, f)
            assert d.max() <= 1 or name != "o", (name, int(d.max()))
        decisions_agree = decisions_agree or n_flips == 0
    if decisions_agree:
        assert out["max"] <= tol, out
    if got_h is not None:
        out["h_T"] = rel_check(got_h, ref_h, tol, "h_T end to end")["max"]
    note(f"  end to end: {out}")
    return out
