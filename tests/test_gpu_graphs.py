"""Calls captured into a HIP graph (torch.cuda.graph) and replayed: the library launches no
allocation, memset or synchronization inside a call, so a decode step of a stack and a whole
block backward can be captured.  Every replay is compared with the eager result, with the
program's own eager work and synchronizations between the replays."""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import dev, host, note

pytestmark = pytest.mark.gpu

GRAPH_STACK = synth.Workload("graph-tiny", D=256, F=704, B=1, T=1, layers=2, vocab=512, seed=11)


def _stack(w):
    blocks = [api.Block.from_latents(synth.layer_latents(w, l), "cuda") for l in range(w.layers)]
    E, H = synth.embedding_latents(w)
    return api.Stack(blocks, api.TernaryLinear.from_latent(E), api.TernaryLinear.from_latent(H))


@pytest.mark.parametrize("B", [1, 64])
def test_graph_replay_decode_steps(B):
    """Teacher-forced decode steps: the graph-replayed steps (state carried in place, token ids
    copied into the captured buffer) give the eager steps' logits and states bit for bit."""
    w = GRAPH_STACK
    L, D, V = w.layers, w.D, w.vocab
    note(f"graph replay of stack_forward decode steps, B={B}")
    stack = _stack(w)
    ids = synth.token_ids(w, 5, B)
    ws = torch.empty(stack.workspace_bytes(B, 1), dtype=torch.uint8, device="cuda")
    h_e = torch.zeros((L, B, D), device="cuda")
    ref_logits = []
    for s in range(5):
        _, lg = api.stack_forward(stack, B, 1, ids=torch.from_numpy(ids[s]).cuda(), h_state=h_e,
                                  want_y=False, want_logits=True, ws=ws)
        ref_logits.append(host(lg).copy())
    torch.cuda.synchronize()

    h_g = torch.zeros((L, B, D), device="cuda")
    ids_static = torch.from_numpy(ids[0]).cuda()
    lg_g = torch.empty((B, V), device="cuda")
    ws_g = torch.empty_like(ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.stack_forward(stack, B, 1, ids=ids_static, h_state=h_g, want_y=False, want_logits=True,
                          ws=ws_g, logits=lg_g)
    h_g.zero_()   # the capture did not run the step; start from the same state as the eager run
    scratch_h = torch.zeros((L, B, D), device="cuda")
    for s in range(5):
        ids_static.copy_(torch.from_numpy(ids[s]).cuda())
        g.replay()
        # eager work of the program between replays, on other buffers
        api.stack_forward(stack, B, 1, ids=torch.from_numpy(ids[(s + 2) % 5]).cuda(), h_state=scratch_h,
                          want_y=False, want_logits=True, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(lg_g), ref_logits[s]), f"replay {s}: logits differ from the eager step"
    assert np.array_equal(host(h_g), host(h_e)), "replayed state differs from the eager state"


def test_graph_replay_block_backward(orc):
    """A captured block_backward replayed three times, eager calls on other inputs between the
    replays: every replay gives the eager call's gradients (equal up to the order of the fp32
    atomic sums)."""
    from tests.test_gpu_backward import _block

    B, T, D, F = 2, 37, 256, 704
    note("graph replay of block_backward")
    blk, _, _ = _block(orc, 91, D, F, True)
    x = dev(synth.round_to_bf16(synth.gaussian(92, (B, T, D))), torch.bfloat16)
    dy = dev(synth.round_to_bf16(synth.gaussian(93, (B, T, D))), torch.bfloat16)
    h0 = dev(synth.gaussian(94, (B, D)))
    x2 = dev(synth.round_to_bf16(synth.gaussian(95, (B, T, D))), torch.bfloat16)
    dy2 = dev(synth.round_to_bf16(synth.gaussian(96, (B, T, D))), torch.bfloat16)
    ref = api.block_backward(blk, x, dy, h0=h0)
    torch.cuda.synchronize()

    def flat(d):
        out = []
        for k, v in sorted(d.items()):
            if isinstance(v, dict):
                out += [(f"{k}[{j}]", host(t)) for j, t in sorted(v.items())]
            else:
                out.append((k, host(v)))
        return out

    ref_f = flat(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = api.block_backward(blk, x, dy, h0=h0)
    for r in range(3):
        g.replay()
        api.block_backward(blk, x2, dy2)   # eager work between the replays
        torch.cuda.synchronize()
        for (name, a), (_, b) in zip(flat(got), ref_f):
            assert np.all(np.isfinite(a)), f"replay {r}: {name} not finite"
            assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(b) + 1e-30, f"replay {r}: {name} differs"
