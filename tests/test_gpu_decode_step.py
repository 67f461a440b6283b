"""One-launch decode step of a stack (stack_decode_step) on the GPU against the oracle,
layer by layer: every layer's input is read back from the exchange area of the workspace
(bf16 values the next layer consumed), each layer's output and new state are compared with
the oracle block fed that layer's GPU input and state, and the logits with the oracle head
fed the last layer's GPU output; the state is carried over several steps.  The error path
is forced from the host (timeout flag set before a step: nothing runs, status reports it)."""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import e2e_checks, note, rel_check, stage_recheck

pytestmark = pytest.mark.gpu


def _stack(orc, w, f_lower=None, f_bias=None, gains=False):
    blocks, Ws = [], []
    for l in range(w.layers):
        lat = synth.layer_latents(w, l)
        gw = (1 + 0.2 * synth.gaussian(l + 9, (w.D,))).astype(np.float32) if gains else None
        lb = None if f_lower is None else f_lower[l]
        blocks.append(api.Block.from_latents(lat, "cuda", f_bias=f_bias, gnorm_w=gw, f_lower=lb))
        Ws.append(({k: orc.ternarize(lat[k]) for k in ("i", "f", "g", "o", "gate", "up", "down")}, gw, lb))
    E, H = synth.embedding_latents(w)
    emb, head = api.TernaryLinear.from_latent(E), api.TernaryLinear.from_latent(H)
    return api.Stack(blocks, emb, head), Ws, orc.ternarize(E), orc.ternarize(H)


def _layer_inputs(ds, L, D, F):
    S = 5 * D // 2 + F // 2
    nbytes = -(-(L + 1) * S * 8 // 256) * 256
    words = ds.ws[ds.ws.numel() - nbytes:].view(torch.int64).cpu().numpy()
    lo = (words & 0xFFFFFFFF).astype(np.uint32)
    xs = []
    for l in range(1, L + 1):
        w = lo[l * S:l * S + D // 2]
        pair = np.stack([(w & 0xFFFF) << 16, w & 0xFFFF0000], axis=1).astype(np.uint32)
        xs.append(pair.reshape(D).view(np.float32))
    return xs


CASES = {
    "tiny": dict(w=synth.Workload("tiny-stack", D=256, F=704, B=1, T=1, layers=3, vocab=1000, seed=11),
                 extras=True, steps=4),
    "1.3B": dict(w=synth.WORKLOADS["1.3B-decode"], extras=False, steps=3),
    # the 2.7B widths: D > 2048 and F > 6144 take the kernel instance sized for D <= 4096
    "wide": dict(w=synth.Workload("wide-stack", D=2560, F=6912, B=1, T=1, layers=2, vocab=2000, seed=12),
                 extras=True, steps=2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_decode_step_layer_by_layer(orc, case):
    c = CASES[case]
    w = c["w"]
    D, F, L, V = w.D, w.F, w.layers, w.vocab
    note(f"one-launch decode step {case}: building {L} layers")
    fl = fb = None
    if c["extras"]:
        fl = orc.hgrn_lower_bounds(synth.gaussian(3, (L, D), 1.0))
        fb = np.full(D, 0.4, np.float32)
    stack, Ws, (qe, se), (qh, sh) = _stack(orc, w, f_lower=fl, f_bias=fb, gains=c["extras"])
    ds = api.DecodeStep(stack)
    ids = synth.token_ids(w, c["steps"], 1)
    h = torch.zeros((L, 1, D), device="cuda")
    logits = torch.empty((1, V), device="cuda")
    y = torch.empty((1, D), dtype=torch.bfloat16, device="cuda")
    for s in range(c["steps"]):
        note(f"  step {s}")
        h_before = h.cpu().numpy().copy()
        ds.step(torch.from_numpy(ids[s]).cuda(), h, logits=logits, y=y)
        ds.status()
        torch.cuda.synchronize()
        h_after = h.cpu().numpy()
        xs = [orc.embedding(qe, se, ids[s], resid_bf16=True).reshape(D)] + _layer_inputs(ds, L, D, F)
        assert np.array_equal(xs[-1], y.float().cpu().numpy().reshape(D)), "y is not the head's input"
        for l in range(L):
            W, gw, lb = Ws[l]
            r = orc.block(xs[l].reshape(1, 1, D), W, f_bias=fb, gnorm_w=gw, f_lower=lb,
                          resid_bf16=True, h0=h_before[l].astype(np.float64))
            e2e_checks(xs[l + 1].reshape(1, 1, D), r["y"], True, got_h=h_after[l],
                       ref_h=r["h_last"])
        ref = orc.bitlinear(xs[L].reshape(1, D), qh, sh)[0]
        rel_check(logits.cpu().numpy(), ref, 1e-3, "logits")


def test_decode_step_matches_launch_per_stage_path(orc):
    """The same steps through stack_forward (one launch per stage): equal to the bf16
    tolerance, layer outputs and states included through the logits."""
    w = CASES["tiny"]["w"]
    D, L, V = w.D, w.layers, w.vocab
    note("one-launch decode step vs stack_forward")
    stack, _, _, _ = _stack(orc, w)
    ds = api.DecodeStep(stack)
    ids = synth.token_ids(w, 5, 1)
    h1 = torch.zeros((L, 1, D), device="cuda")
    h2 = torch.zeros((L, 1, D), device="cuda")
    lg1 = torch.empty((1, V), device="cuda")
    for s in range(5):
        idt = torch.from_numpy(ids[s]).cuda()
        ds.step(idt, h1, logits=lg1)
        _, lg2 = api.stack_forward(stack, 1, 1, ids=idt, h_state=h2, want_y=False, want_logits=True)
        torch.cuda.synchronize()
        e2e_checks(lg1.cpu().numpy(), lg2.cpu().numpy().astype(np.float64), True)
        rel_check(h1.cpu().numpy().reshape(L, D), h2.cpu().numpy().reshape(L, D).astype(np.float64), 2e-2, "h")
    ds.status()


def test_decode_step_error_flag_from_host(orc):
    """A timeout flag set by the host before a step: the kernel runs nothing, the status call
    reports it, outputs and state stay untouched; re-initialising clears it."""
    w = CASES["tiny"]["w"]
    D, L, V = w.D, w.layers, w.vocab
    note("one-launch decode step: forced error flag")
    stack, _, _, _ = _stack(orc, w)
    ds = api.DecodeStep(stack)
    h = torch.zeros((L, 1, D), device="cuda")
    logits = torch.full((1, V), 7.0, device="cuda")
    ds.ws[8:12].fill_(1)          # the timeout flag (bytes 8..11)
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ds.step(ids, h, logits=logits)
    with pytest.raises(Exception):
        ds.status()
    torch.cuda.synchronize()
    assert torch.all(logits == 7.0) and not h.any()
    ds.init()
    ds.step(ids, h, logits=logits)
    ds.status()
    torch.cuda.synchronize()
    assert not torch.all(logits == 7.0) and h.any()
