"""Decode BitLinear over base-3 packed weights (five per byte) on the GPU against the oracle:
int8 codes and int32 accumulators bit-exact, outputs within the dtype's tolerance, and the
same accumulators as the 2-bit weight-streaming kernel on the same weights."""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import TOL, dev, note, rel_check

pytestmark = pytest.mark.gpu

CASES = [(1, 64, 16), (3, 256, 100), (1, 2048, 6144), (4, 2048, 11264), (2, 5632, 2048),
         (16, 8192, 512), (5, 1024, 37), (7, 10240, 300)]


@pytest.mark.parametrize("xdt,ydt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32)], ids=["bf16", "f32", "bf16-f32"])
@pytest.mark.parametrize("m,K,N", CASES, ids=[f"m{m}K{k}N{n}" for m, k, n in CASES])
def test_trit_bitlinear_parity(orc, m, K, N, xdt, ydt):
    note(f"trit bitlinear m={m} K={K} N={N} x={xdt} y={ydt}")
    lat = synth.gaussian(K + N, (N, K), 0.02)
    q, s = orc.ternarize(lat)
    gamma = (1.0 + 0.1 * synth.gaussian(K, (K,))).astype(np.float32)
    bias = synth.gaussian(N, (N,), 0.1)
    packed = orc.pack_trits(q)
    assert np.array_equal(api.pack_trits(q), packed)   # library and oracle pack agree
    w = api.TernaryLinearTrits.from_ternary(q, s, norm_w=gamma, bias=bias)
    x = synth.gaussian(m * 7 + K, (m, K))
    if xdt == torch.bfloat16:
        x = synth.round_to_bf16(x)
    cap = api.StageCapture.alloc(0, m, K, N)
    y = api.bitlinear_forward_trits(w, dev(x, xdt), out_dtype=ydt, capture=cap)
    torch.cuda.synchronize()
    c = cap.host()
    y_o, qx, a, acc = orc.bitlinear(x, orc.unpack_trits(packed, K), s, gamma=gamma, bias=bias)
    assert np.array_equal(c["x_in"], x)
    assert np.array_equal(c["q"], qx), "int8 codes differ"
    np.testing.assert_allclose(c["a"], a, rtol=2e-5)
    bad = np.argwhere(c["acc"] != acc)
    assert bad.size == 0, f"accumulators differ at {bad[:5]}"
    rel_check(y.float().cpu().numpy(), y_o, TOL[ydt], "y")
    assert np.array_equal(c["y_out"], y.float().cpu().numpy())


def test_trit_matches_two_bit_kernel(orc):
    """The same weights through both formats: identical int32 accumulators."""
    m, K, N = 2, 2048, 2048
    note("trit vs 2-bit decode kernel")
    q, s = orc.ternarize(synth.gaussian(5, (N, K), 0.02))
    x = dev(synth.round_to_bf16(synth.gaussian(6, (m, K))), torch.bfloat16)
    c3 = api.StageCapture.alloc(0, m, K, N)
    c2 = api.StageCapture.alloc(0, m, K, N)
    api.bitlinear_forward_trits(api.TernaryLinearTrits.from_ternary(q, s), x, capture=c3)
    prev = api.set_regime(1)
    try:
        api.bitlinear_forward(api.TernaryLinear.from_ternary(q, s), x, capture=c2)
    finally:
        api.set_regime(prev)
    torch.cuda.synchronize()
    assert np.array_equal(c3.host()["acc"], c2.host()["acc"])
    assert np.array_equal(c3.host()["q"], c2.host()["q"])


def test_trit_edge_cases(orc):
    note("trit edge cases")
    q = np.zeros((8, 64), np.int8)
    w = api.TernaryLinearTrits.from_ternary(q, 0.5)
    y = api.bitlinear_forward_trits(w, torch.zeros((0, 64), device="cuda"))
    assert y.shape == (0, 8)
    # all-zero weights and an all-zero activation row: exactly zero output
    y = api.bitlinear_forward_trits(w, torch.zeros((2, 64), device="cuda"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not y.any()
    with pytest.raises(Exception):
        api.bitlinear_forward_trits(w, torch.zeros((17, 64), device="cuda"))
