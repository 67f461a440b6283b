"""block_forward_noalloc (static per-GPU scratch, no device allocation by the library)
against block_forward with a caller workspace: identical outputs and states on two calls in
a row, the second with a smaller input, so the second runs on scratch the first left
behind."""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import _lib as L
from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import note, small_latents

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,F,shapes", [(256, 704, [(4, 300), (2, 37)]),
                                        (1024, 2816, [(8, 96), (1, 1)]),
                                        (2048, 5632, [(64, 1), (3, 1)])],
                         ids=["d256", "d1024", "d2048-decode"])
def test_noalloc_matches_block_forward(D, F, shapes):
    blk = api.Block.from_latents(small_latents(D + F, D, F), "cuda",
                                 f_bias=np.full(D, 0.4, np.float32))
    for i, (B, T) in enumerate(shapes):
        note(f"block_forward_noalloc D={D} F={F} call {i}: B={B} T={T}")
        x = torch.from_numpy(synth.round_to_bf16(synth.gaussian(i + D, (B, T, D)))).cuda().to(torch.bfloat16)
        h0 = torch.from_numpy(synth.gaussian(i + 3, (B, D))).cuda()
        h_ref, h_na = h0.clone(), h0.clone()
        y_ref = api.block_forward(blk, x, h_state=h_ref)
        y_na = api.block_forward_noalloc(blk, x, h_state=h_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ref), f"call {i}: outputs differ"
        assert torch.equal(h_na, h_ref), f"call {i}: states differ"


def test_noalloc_rejects_inputs_beyond_the_scratch():
    D, F = 2048, 5632
    blk = api.Block.from_latents(small_latents(9, D, F), "cuda")
    cap = L.lib().block_scratch_bytes()
    B, T = 1, 4096
    assert api.block_workspace_bytes(blk, B, T) > cap
    x = torch.zeros((B, T, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.MMFError) as ei:
        api.block_forward_noalloc(blk, x)
    assert ei.value.code == -5
