"""BitLinear parity on the GPU: int8 codes and int32 accumulators bit-exact against the
oracle, rescaled outputs within tolerance, for every kernel (decode weight streaming, the
k-split MFMA kernel for up to 64 rows, the 128-row MFMA tiles) at shapes spanning several
tiles, ragged tails and the real layer shapes."""
import numpy as np
import pytest
import torch

from ternary_weight_matmul_bitlinear_amd import api, synth
from tests.gpu_helpers import TOL, dev, host, note, rel_check

pytestmark = pytest.mark.gpu

CASES = [
    # M, K, N, dtype, gamma, bias
    (1, 256, 256, torch.float32, False, False),
    (64, 256, 256, torch.float32, True, True),
    (3, 2048, 6144, torch.bfloat16, False, False),
    (8, 1024, 200, torch.bfloat16, True, False),
    (300, 512, 384, torch.bfloat16, False, True),
    (129, 1024, 130, torch.float32, False, False),
    (16, 5632, 2048, torch.bfloat16, False, False),
    (1, 6912, 2560, torch.bfloat16, True, False),
    (257, 2816, 1024, torch.bfloat16, False, False),
    # k-split MFMA kernel: ragged k-tiles (K % 128 == 64), k-tiles per wave 1..16, one and two
    # 32-row token blocks, ragged N
    (33, 192, 100, torch.bfloat16, True, True),
    (64, 64, 40, torch.float32, False, False),
    (50, 2048, 6144, torch.bfloat16, False, False),
    (64, 5632, 2048, torch.bfloat16, False, True),
    (17, 4096, 96, torch.float32, True, False),
    (48, 2048, 32000, torch.bfloat16, False, False),
    (24, 6912, 320, torch.bfloat16, False, False),  # 14 k-tiles per wave (2.7B down width)
    (40, 8192, 160, torch.float32, True, True),     # 16 k-tiles per wave
    # one token, rows of 8192 and more: the long-row weight-streaming variant (two passes of
    # weight chunks at K = 16384)
    (1, 8192, 300, torch.bfloat16, True, True),
    (1, 16384, 130, torch.float32, False, False),
    # one token, rows shorter than 8192: 1, 2, 4, 6 or 8 chunks per lane, ragged last group
    (1, 1088, 96, torch.bfloat16, False, True),
    (1, 2048, 6144, torch.bfloat16, False, False),
    (1, 3136, 200, torch.float32, True, True),
    (1, 5632, 2048, torch.bfloat16, False, False),
    (1, 7232, 68, torch.bfloat16, True, False),
    # two to four tokens, bf16: the group's rows held in registers (1, 4, 6 or 8 chunks per
    # lane of weights, 1-4 slices of the row per thread), ragged rows and groups
    (4, 320, 96, torch.bfloat16, False, True),
    (2, 2048, 200, torch.bfloat16, True, False),
    (4, 5632, 300, torch.bfloat16, True, True),
    (3, 7232, 130, torch.bfloat16, False, False),
    # one token, 16384 rows and more (bf16): persistent streaming over 16-row blocks with the
    # next block's weights in flight; ragged last block, 1/2/6/8 chunks per lane
    (1, 320, 16390, torch.bfloat16, False, True),
    (1, 2048, 20000, torch.bfloat16, False, False),
    (1, 5632, 16384, torch.bfloat16, True, False),
    (1, 8192, 16400, torch.bfloat16, True, True),
]


@pytest.fixture(autouse=True)
def _restore_regime():
    prev = api.set_regime(0)
    yield
    api.set_regime(prev)


@pytest.mark.parametrize("regime", [1, 2, 3], ids=["decode", "mfma", "tiles"])
@pytest.mark.parametrize("M,K,N,dt,use_gamma,use_bias", CASES,
                         ids=[f"M{c[0]}K{c[1]}N{c[2]}{'bf' if c[3] == torch.bfloat16 else 'f'}"
                              for c in CASES])
def test_bitlinear_parity(orc, regime, M, K, N, dt, use_gamma, use_bias):
    note(f"bitlinear regime={regime} M={M} K={K} N={N} dt={dt}")
    seed = M * 7919 + K * 31 + N
    x = synth.gaussian(seed, (M, K))
    if dt == torch.bfloat16:
        x = synth.round_to_bf16(x)
    lat = synth.gaussian(seed + 1, (N, K), 0.02)
    gamma = (1.0 + 0.2 * synth.gaussian(seed + 2, (K,))).astype(np.float32) if use_gamma else None
    bias = synth.gaussian(seed + 3, (N,)) if use_bias else None
    q_l, s_l = api.quantize_ternary(lat)
    q_o, s_o = orc.ternarize(lat)
    assert s_l == s_o and np.array_equal(q_l, q_o)
    w = api.TernaryLinear.from_ternary(q_l, s_l, norm_w=gamma, bias=bias)
    api.set_regime(regime)
    cap = api.StageCapture.alloc(0, M, K, N)
    y = api.bitlinear_forward(w, dev(x, dt), out_dtype=torch.float32, capture=cap)
    torch.cuda.synchronize()
    c = cap.host()
    y_o, qx_o, a_o, acc_o = orc.bitlinear(x, q_o, s_o, gamma=gamma, bias=bias)
    assert np.array_equal(c["x_in"], x)
    assert np.array_equal(c["q"], qx_o), "int8 activations differ"
    assert np.array_equal(c["acc"], acc_o), "int32 accumulators differ"
    np.testing.assert_allclose(c["a"], a_o, rtol=2e-5)
    rel_check(host(y), y_o, TOL[torch.float32], "y")


@pytest.mark.parametrize("regime", [1, 2, 3], ids=["decode", "mfma", "tiles"])
def test_bitlinear_bf16_output_and_zero_rows(orc, regime):
    """bf16 output; an all-zero input row gives exactly the bias (acc = 0)."""
    M, K, N = 40, 512, 320
    note(f"bitlinear zero rows regime={regime}")
    x = synth.round_to_bf16(synth.gaussian(5, (M, K)))
    x[7] = 0.0
    lat = synth.gaussian(6, (N, K), 0.02)
    bias = synth.gaussian(7, (N,))
    q, s = api.quantize_ternary(lat)
    w = api.TernaryLinear.from_ternary(q, s, bias=bias)
    api.set_regime(regime)
    y = api.bitlinear_forward(w, dev(x, torch.bfloat16), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y_o, _, _, acc_o = orc.bitlinear(x, q, s, bias=bias)
    assert not acc_o[7].any()
    rel_check(host(y), y_o, TOL[torch.bfloat16], "y bf16")
    assert np.array_equal(host(y)[7], host(torch.from_numpy(bias).to(torch.bfloat16)))


def test_bitlinear_empty_is_noop():
    lat = synth.gaussian(8, (64, 256), 0.02)
    w = api.TernaryLinear.from_latent(lat)
    y = api.bitlinear_forward(w, torch.zeros((0, 256), device="cuda"))
    assert y.shape == (0, 64)


def test_regimes_agree_bit_exact_on_integers():
    """All three kernels produce identical int8 codes and accumulators."""
    M, K, N = 24, 2048, 700
    note("bitlinear regimes agree")
    x = synth.round_to_bf16(synth.gaussian(9, (M, K)))
    w = api.TernaryLinear.from_latent(synth.gaussian(10, (N, K), 0.02))
    out = {}
    for r in (1, 2, 3):
        api.set_regime(r)
        cap = api.StageCapture.alloc(0, M, K, N)
        api.bitlinear_forward(w, dev(x, torch.bfloat16), capture=cap)
        torch.cuda.synchronize()
        out[r] = cap.host()
    for r in (2, 3):
        assert np.array_equal(out[1]["q"], out[r]["q"])
        assert np.array_equal(out[1]["acc"], out[r]["acc"])
