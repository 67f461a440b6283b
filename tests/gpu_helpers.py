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
               eps=1e-6):
    """Device block from latent weights (library host quantizer) and the oracle's own
    ternarization of the same latents (asserted identical)."""
    blk = api.Block.from_latents(lat, device, f_bias=f_bias, gnorm_w=gnorm_w, eps=eps,
                                 gate_mode=gate_mode)
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
