"""The CPU oracle against hand-worked cases, closed forms, invariants and brute force."""
import pytest

from tests.oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(orc, pin):
    pin(orc)


def test_deep_stack_sensitivity_is_inherent(orc):
    """The oracle against itself: one bf16 ulp in one input element of a stack of blocks
    with random ternary weights flips a few downstream int8 codes, and the flips cascade:
    after a few layers the two runs differ by ~1e-2 norm-wise.  Hence deep stacks are
    compared layer by layer (each block fed the same input), not end to end."""
    import numpy as np
    from ternary_weight_matmul_bitlinear_amd import synth
    w = synth.Workload("sens", D=512, F=1408, B=1, T=1, layers=6, seed=7)
    Ws = []
    for l in range(w.layers):
        lat = synth.layer_latents(w, l)
        Ws.append({k: orc.ternarize(lat[k]) for k in lat})
    rng = np.random.default_rng(3)
    a = synth.round_to_bf16(rng.standard_normal((8, 1, 512)).astype(np.float32))
    b = a.copy()
    bits = b[:, 0, 10].view(np.uint32) + np.uint32(1 << 16)
    b[:, 0, 10] = bits.view(np.float32)
    div = []
    for l in range(w.layers):
        a = orc.block(a, Ws[l], resid_bf16=True)["y"].astype(np.float32)
        b = orc.block(b, Ws[l], resid_bf16=True)["y"].astype(np.float32)
        A, B = a.reshape(8, -1), b.reshape(8, -1)
        div.append(float(np.max(np.linalg.norm(A - B, axis=1) / np.linalg.norm(A, axis=1))))
    # a 2^-8 relative change of one of 4096 inputs becomes a ~1e-2 change of the output
    assert max(div) > 5e-3, div
