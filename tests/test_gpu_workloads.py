"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot run these sizes whole, so each test combines:
  * stage-wise checks on captured token windows (integers bit-exact, each fp stage against
    the oracle fed the GPU's own inputs), including windows deep inside long sequences;
  * an end-to-end comparison on a causal prefix the oracle can run (outputs of a prefix
    depend only on the prefix);
  * determinism (two runs bit-identical) and stack_forward == the layer-by-layer path.
"""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import (block_stage_checks, cat_weights, dev, e2e_checks, host, note,
                               rel_check, stage_recheck)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _layer(orc, w, layer, f_bias=None):
    lat = synth.layer_latents(w, layer)
    blk = api.Block.from_latents(lat, "cuda", f_bias=f_bias)
    W = {k: orc.ternarize(lat[k]) for k in ("i", "f", "g", "o", "gate", "up", "down")}
    for k in W:  # the library's host quantizer and the oracle agree bit for bit
        assert getattr(blk, k).scale == W[k][1], k
    return blk, W


def _caps(cap):
    return {k: getattr(cap, k).host() for k in ("ifg", "o", "gateup", "down")}


def _block_run(blk, x, B, T, D, F, row0, row1, ws):
    h = torch.zeros((B, D), device="cuda")
    cap = api.BlockCapture.alloc(row0, row1, D, F)
    y = api.block_forward(blk, x, h_state=h, ws=ws, capture=cap)
    torch.cuda.synchronize()
    return y, h, _caps(cap)


@pytest.mark.timeout(600)  # full-size launches checked against the CPU oracle
@pytest.mark.parametrize("name,win", [("370M-block", 256), ("2.7B-block", 64)])
def test_block_workload(orc, name, win):
    w = synth.WORKLOADS[name]
    B, T, D, F = w.B, w.T, w.D, w.F
    note(f"workload {name}: B={B} T={T} D={D} F={F}")
    blk, W = _layer(orc, w, 0)
    x_np = synth.activations(w)
    x = dev(x_np, torch.bfloat16)
    ws = torch.empty(api.block_workspace_bytes(blk, B, T), dtype=torch.uint8, device="cuda")
    outs = []
    # windows: start of the first and of the last sequence (recurrence checked from t = 0),
    # and a late window of a middle sequence (state carried through every chunk seam)
    b_mid = B // 2
    for (r0, seq) in ((0, True), ((B - 1) * T, True), (b_mid * T + T - win, False)):
        y, h, ch = _block_run(blk, x, B, T, D, F, r0, r0 + win, ws)
        outs.append(y)
        b, t0 = divmod(r0, T)
        xw = x_np[b, t0:t0 + win]
        block_stage_checks(orc, ch, W, xw, True, seq_rows=(1, win) if seq else None,
                           y_rows=host(y[b, t0:t0 + win]))
    assert all(torch.equal(outs[0], o) for o in outs[1:]), "runs are not bit-identical"
    # end to end on the causal prefix of the first and last sequence
    pre = np.ascontiguousarray(x_np[[0, B - 1], :win])
    r = orc.block(pre, W, resid_bf16=True)
    e2e_checks(host(outs[0][[0, B - 1], :win]), r["y"], True)


@pytest.mark.timeout(900)  # 24 oracle layers per step at five batch sizes
def test_decode_stack_1p3b(orc):
    """24 layers + ternary embedding and head, one token per step with carried state."""
    w = synth.WORKLOADS["1.3B-decode"]
    D, F, V, L = w.D, w.F, w.vocab, w.layers
    note("1.3B decode stack: building 24 layers")
    blocks, Ws = [], []
    for l in range(L):
        b, W = _layer(orc, w, l)
        blocks.append(b)
        Ws.append(W)
    E, H = synth.embedding_latents(w)
    qe, se = orc.ternarize(E)
    qh, sh = orc.ternarize(H)
    emb = api.TernaryLinear.from_latent(E)
    head = api.TernaryLinear.from_latent(H)
    assert emb.scale == se and head.scale == sh
    stack = api.Stack(blocks, emb, head)
    # 1: fused one-token path; 4: four-token weight streaming; 16, 32: k-split MFMA kernel
    # with one 32-row token block; 64: two token blocks (the batch the decode profile times).
    # Sequences are independent in a decode step, so above 16 the oracle follows 8 of them
    # (spread over the batch, both token blocks) while the GPU runs all of them.
    for B in (1, 4, 16, 32, 64):
        steps = 3 if B == 1 else 2
        sel = np.arange(B) if B <= 16 else np.linspace(0, B - 1, 8).round().astype(int)
        note(f"1.3B decode B={B}: {steps} steps, oracle rows {sel.tolist()}")
        ids = synth.token_ids(w, steps, B)
        hs = torch.zeros((L, B, D), device="cuda")
        hs_ref = torch.zeros((L, B, D), device="cuda")
        ref_state = [None] * L
        for s in range(steps):
            idt = torch.from_numpy(ids[s]).to("cuda")
            _, logits = api.stack_forward(stack, B, 1, ids=idt, h_state=hs, want_y=False,
                                          want_logits=True)
            # the same step layer by layer through the public entry points, with captures
            x = api.embedding_forward(emb.packed, emb.scale, V, D, idt)
            x = x.reshape(B, 1, D)
            xs_gpu, hb_gpu, ha_gpu = [host(x)], [], []
            for l in range(L):
                capt = api.BlockCapture.alloc(0, B, D, F) if l in (0, L - 1) else None
                h_before = hs_ref[l].cpu().numpy().copy()
                x = api.block_forward(blocks[l], x, h_state=hs_ref[l], capture=capt)
                torch.cuda.synchronize()
                xs_gpu.append(host(x))
                hb_gpu.append(h_before)
                ha_gpu.append(hs_ref[l].cpu().numpy().copy())
                if capt is not None:
                    block_stage_checks(orc, _caps(capt), Ws[l], capt.ifg.host()["x_in"].reshape(B, D),
                                       True, seq_rows=(B, 1), h0=h_before,
                                       h_last=ha_gpu[-1], y_rows=xs_gpu[-1].reshape(B, D))
            # every layer against the oracle block fed the same input and state
            note(f"  B={B} step {s}: layer by layer against the oracle")
            for l in range(L):
                r = orc.block(xs_gpu[l][sel].astype(np.float32), Ws[l], resid_bf16=True,
                              h0=hb_gpu[l][sel])
                e2e_checks(xs_gpu[l + 1][sel], r["y"], True, got_h=ha_gpu[l][sel],
                           ref_h=r["h_last"])
            hc = api.StageCapture.alloc(0, B, D, V)
            lg = api.bitlinear_forward(head, x.reshape(B, D), out_dtype=torch.float32, capture=hc)
            torch.cuda.synchronize()
            assert torch.equal(lg, logits), "stack_forward differs from the layer-by-layer path"
            assert torch.equal(hs, hs_ref)
            c = hc.host()
            stage_recheck(orc, c, qh, what="head")
            rel_check(host(lg), orc.bitlinear(c["x_in"], qh, sh)[0], 1e-3, "logits (stage)")
            # fully independent oracle stack (teacher-forced ids): the embedding is exact;
            # afterwards near-tie int8 flips are amplified layer by layer through the random
            # weights, so this divergence is reported per layer, and bounded only loosely
            nb = len(sel)
            xo = orc.embedding(qe, se, ids[s][sel], resid_bf16=True).reshape(nb, 1, D)
            assert np.array_equal(xo, xs_gpu[0][sel].astype(np.float32))
            div = []
            for l in range(L):
                r = orc.block(xo, Ws[l], resid_bf16=True, h0=ref_state[l])
                ref_state[l] = r["h_last"]
                xo = r["y"].astype(np.float32)
                g = xs_gpu[l + 1][sel].reshape(nb, D)
                div.append(float(np.max(np.linalg.norm(g - xo.reshape(nb, D), axis=1) /
                                        np.linalg.norm(xo.reshape(nb, D), axis=1))))
            print(f"B={B} step {s}: independent stack divergence by layer",
                  " ".join(f"{d:.1e}" for d in div), flush=True)
            # measured: at most 0.12 after 24 layers (batch 1-64, 3 steps); bound at ~2x
            assert div[0] <= 2e-2 and max(div) <= 0.25, div


@pytest.mark.timeout(900)  # 32 oracle layers
def test_longctx_stack_2p7b(orc):
    """32 layers over 2 x 32768 tokens with b_f = ln 9: captured windows at the start and
    deep in the second sequence for the first and last layer, a causal-prefix end-to-end
    check, and stack_forward == the layer-by-layer path."""
    w = synth.WORKLOADS["2.7B-longctx"]
    B, T, D, F, L = w.B, w.T, w.D, w.F, w.layers
    fb = np.full(D, w.f_bias, np.float32)
    note("2.7B long context: building 32 layers")
    blocks, Ws = [], []
    for l in range(L):
        b, W = _layer(orc, w, l, f_bias=fb)
        blocks.append(b)
        Ws.append(W)
    x_np = synth.activations(w)
    x = dev(x_np, torch.bfloat16)
    stack = api.Stack(blocks)
    ws = torch.empty(stack.workspace_bytes(B, T), dtype=torch.uint8, device="cuda")
    note("2.7B long context: stack_forward")
    y_stack, _ = api.stack_forward(stack, B, T, x=x, ws=ws)
    torch.cuda.synchronize()
    win = 32
    late = T + T - 3 * win  # second sequence, near its end
    note("2.7B long context: layer by layer with captures")
    cur = x
    bws = torch.empty(api.block_workspace_bytes(blocks[0], B, T), dtype=torch.uint8, device="cuda")
    P = 8
    pre_gpu = [host(cur[:, :P])]
    for l in range(L):
        nxt = torch.empty_like(cur)
        if l in (0, L - 1):
            for r0, seq in ((0, True), (late, False)):
                cap = api.BlockCapture.alloc(r0, r0 + win, D, F)
                api.block_forward(blocks[l], cur, y=nxt, ws=bws, capture=cap)
                torch.cuda.synchronize()
                b, t0 = divmod(r0, T)
                xw = host(cur[b, t0:t0 + win]).astype(np.float32)
                block_stage_checks(orc, _caps(cap), Ws[l], xw, True, seq_rows=(1, win) if seq else None,
                                   f_bias=fb, y_rows=host(nxt[b, t0:t0 + win]))
        else:
            api.block_forward(blocks[l], cur, y=nxt, ws=bws)
        cur = nxt
        pre_gpu.append(host(cur[:, :P]))
    torch.cuda.synchronize()
    assert torch.equal(cur, y_stack), "stack_forward differs from the layer-by-layer path"
    # causal prefix of both sequences: every layer against the oracle block fed the GPU's
    # input of that layer, then the fully independent 32-layer run (reported per layer)
    div = []
    xo = np.ascontiguousarray(x_np[:, :P])
    for l in range(L):
        r = orc.block(pre_gpu[l].astype(np.float32), Ws[l], f_bias=fb, resid_bf16=True)
        e2e_checks(pre_gpu[l + 1], r["y"], True)
        xo = orc.block(xo, Ws[l], f_bias=fb, resid_bf16=True)["y"].astype(np.float32)
        g, o = pre_gpu[l + 1].reshape(-1, D), xo.reshape(-1, D)
        div.append(float(np.max(np.linalg.norm(g - o, axis=1) / np.linalg.norm(o, axis=1))))
    print("independent 32-layer divergence by layer", " ".join(f"{d:.1e}" for d in div), flush=True)
    # measured: 0.095 after 32 layers; bound at ~2x the largest stack divergence measured
    assert div[0] <= 2e-2 and max(div) <= 0.25, div
