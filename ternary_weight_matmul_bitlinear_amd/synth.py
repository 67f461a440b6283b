"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module only draws random numbers and rounds fp32 inputs to bf16; it holds none of the
method's arithmetic (no ternarization, quantization, recurrence or accumulation).

Recipe (stands in for trained checkpoints and real text, which are not used):
  * activations x ~ N(0, 1), generated as fp32, rounded to bf16 (ties to even) when the
    workload's activation dtype is bf16;
  * latent weights ~ N(0, 0.02^2) fp32, later absmean-ternarized by each side on its own
    (about 31 % of the ternary weights come out zero);
  * token ids uniform in [0, vocab);
  * generator: numpy PCG64 seeded through SeedSequence(seed).spawn(n), one child stream per
    tensor, in the fixed order x, then per layer W_i, W_f, W_g, W_o, W_gate, W_up, W_down,
    then the embedding E, the head W_head and the ids.
"""
from __future__ import annotations

import dataclasses

import numpy as np

WEIGHT_STD = 0.02
PER_LAYER = ("i", "f", "g", "o", "gate", "up", "down")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload (names follow the model-zoo sizes on the pages)."""
    name: str
    D: int            # hidden size
    F: int            # GLU intermediate size
    B: int            # sequences
    T: int            # tokens per sequence
    layers: int = 1
    vocab: int = 0    # > 0: ternary embedding + head present
    bf16: bool = True
    f_bias: float = 0.0   # forget-gate bias (sigmoid(ln 9) = 0.9)
    seed: int = 0

    @property
    def M(self) -> int:
        return self.B * self.T


WORKLOADS = {
    # single fused BitLinear + MLGRU at a tiny shape, fp32 activations
    "tiny-d256": Workload("tiny-d256", D=256, F=704, B=1, T=64, bf16=False, seed=0),
    # one block at the 370M shape: 8 sequences x 2048 tokens
    "370M-block": Workload("370M-block", D=1024, F=2816, B=8, T=2048, seed=1),
    # 24-layer 1.3B-shaped stack, one token per step, batch 1..64
    "1.3B-decode": Workload("1.3B-decode", D=2048, F=5632, B=1, T=1, layers=24,
                            vocab=32000, seed=2),
    # one block at the 2.7B shape: 16 sequences x 2048 tokens
    "2.7B-block": Workload("2.7B-block", D=2560, F=6912, B=16, T=2048, seed=3),
    # 32-layer 2.7B-shaped long-context prefill, forget-gate bias ln 9
    "2.7B-longctx": Workload("2.7B-longctx", D=2560, F=6912, B=2, T=32768, layers=32,
                             f_bias=float(np.log(9.0)), seed=4),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def n_streams(w: Workload) -> int:
    return 1 + len(PER_LAYER) * w.layers + 3


def activations(w: Workload, B: int | None = None, T: int | None = None) -> np.ndarray:
    """x [B, T, D] fp32 (values exact in bf16 when the workload is bf16)."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    rng = _streams(w.seed, n_streams(w))[0]
    x = rng.standard_normal((B, T, w.D), dtype=np.float32)
    return round_to_bf16(x) if w.bf16 else x


def layer_latents(w: Workload, layer: int) -> dict:
    """Latent fp32 weights of one layer: i, f, g, o [D, D]; gate, up [F, D]; down [D, F]."""
    rngs = _streams(w.seed, n_streams(w))
    base = 1 + len(PER_LAYER) * layer
    shapes = {"i": (w.D, w.D), "f": (w.D, w.D), "g": (w.D, w.D), "o": (w.D, w.D),
              "gate": (w.F, w.D), "up": (w.F, w.D), "down": (w.D, w.F)}
    out = {}
    for j, name in enumerate(PER_LAYER):
        out[name] = (rngs[base + j].standard_normal(shapes[name], dtype=np.float32)
                     * np.float32(WEIGHT_STD))
    return out


def embedding_latents(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Latent embedding E [vocab, D] and head W_head [vocab, D] (fp32)."""
    rngs = _streams(w.seed, n_streams(w))
    base = 1 + len(PER_LAYER) * w.layers
    E = rngs[base].standard_normal((w.vocab, w.D), dtype=np.float32) * np.float32(WEIGHT_STD)
    H = rngs[base + 1].standard_normal((w.vocab, w.D), dtype=np.float32) * np.float32(WEIGHT_STD)
    return E, H


def token_ids(w: Workload, steps: int, B: int) -> np.ndarray:
    """Teacher-forced token ids [steps, B] int32, uniform in [0, vocab)."""
    rngs = _streams(w.seed, n_streams(w))
    return rngs[-1].integers(0, w.vocab, size=(steps, B), dtype=np.int32)


def gaussian(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, std^2) fp32 tensor for unit tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
